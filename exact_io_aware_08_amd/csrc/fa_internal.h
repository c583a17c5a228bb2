// Internal interface between the C-ABI shim (fa_api.cpp) and the kernel
// translation units (fa_fwd_kernel.hip, fa_fp8_kernel.hip, fa_bwd_kernel.hip).
// Not installed, not part of the ABI.
#pragma once

#include <cfloat>

#include <hip/hip_runtime_api.h>

namespace fa {

// Exponent factor of the scores, c = scale * log2(e) (the exp2 form of exp).
// The kernels mask a score with -inf and form fma(S, c, -m), which is NaN
// for c = 0, so a factor below FLT_MIN (in practice scale = 0) is raised to
// FLT_MIN = 2^-126: every score with |S| < 2^101 then has an exponent within
// 2^-25 of its row's reference, exp2 of it is exactly 1 in fp32, and every
// visible key weighs the same, which is the result for scale = 0.
inline float exp2_factor(double scale_log2e) {
    const float c = (float)scale_log2e;
    return c < FLT_MIN ? FLT_MIN : c;
}

enum class DType { BF16 = 0, F32 = 1 };

// Compute units of the current device (cached per device); 0 if the query
// fails.
int cu_count();

// Tile geometry of one compiled instantiation.
struct TileConfig {
    int block_m;   // query rows per workgroup
    int block_n;   // keys per K/V tile
    int threads;   // threads per workgroup
};

// Geometry for (dtype, d); returns false if no instantiation exists.
bool tile_config(DType dt, int d, TileConfig* out);

// Enqueue the forward kernel.  Arguments were validated by the caller.
// Returns the hipError_t of the launch.
hipError_t launch_fwd(DType dt, const void* q, const void* k, const void* v,
                      void* o, float* lse, int B, int H, int Lq, int Lk,
                      int d, bool causal, float scale, hipStream_t stream);

// bf16 sliding window: key j visible to query i iff i - wl <= j <= i + wr
// (and j < Lk); wl, wr >= 0, already clamped to at most Lq + Lk.
hipError_t launch_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int Lq, int Lk, int d, int wl, int wr, float scale,
                             hipStream_t stream);

// bf16 key-split forward: nsplit partial results in fp32 (opart
// [nsplit][B*H][Lq][d], lpart [nsplit][B*H][Lq]) then their merge into o and
// lse; two kernels on `stream`.
hipError_t launch_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Lq, int Lk, int d, bool causal, float scale,
                            int nsplit, float* opart, float* lpart, hipStream_t stream);

// Every argument check of fa_fwd_splitkv except those of the workspace;
// enqueues nothing.  FA_OK or the status fa_fwd_splitkv would return.
int splitkv_check(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int H, int Lq, int Lk, int d, int causal, float scale, int num_splits);

// FP8 (E4M3) forward: tile geometry for head dim d (false: no instantiation).
bool fp8_tile_config(int d, TileConfig* out);

// FP8 forward: q, k, v E4M3 codes, o bf16, lse fp32.  c = scale * q_descale *
// k_descale * log2(e) (the exponent factor of S), vd = v_descale.
hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int Lq, int Lk, int d, bool causal, float c, float vd,
                          hipStream_t stream);

// Backward (bf16): head dims with a backward instantiation.
bool bwd_supported(int d);

// Backward: -Delta and -LSE / scale into ndelta / nlse ([B*H][Lq] fp32 each,
// caller-provided), then dK/dV and dQ; three kernels on `stream`.
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      int B, int H, int Lq, int Lk, int d, bool causal, float scale,
                      float* ndelta, float* nlse, hipStream_t stream);

}  // namespace fa
