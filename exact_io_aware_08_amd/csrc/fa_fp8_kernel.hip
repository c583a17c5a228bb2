// FP8 (OCP E4M3) attention forward for gfx950 (MI355X, CDNA4).
//
// The pages' FP8 variant ("Flash Attention 原理与实现详解" (tbr8.org), section
// 4.3 "FP8 支持": the same tiled method on FP8 matrix units) with the reading
// the pages leave open: Q, K, V are E4M3 codes with one fp32 descale factor
// per tensor; S = scale (Q K^T) q_descale k_descale; P is multiplied by 2^8
// and rounded to E4M3 (nearest even) for the PV product, which keeps P down
// to 2^-14 of the row maximum in E4M3's normal range, while the row sum l
// takes the unrounded P (the factor cancels in O / l); O = v_descale (P V) /
// l in bf16 and LSE = ln(sum_j exp(s_ij)) in fp32.  The online softmax is
// the bf16 kernel's: per key tile a new running max, O and l rescaled by
// exp2(m - m_new) (skipped exactly when it is 1), tiles in ascending order.
//
// gfx950 mapping (d = 128):
//  * every product is v_mfma_f32_32x32x64_f8f6f4 with both operands E4M3:
//    lane l holds row / column l % 32 and 32 bytes; byte b of lane half h of
//    the A operand meets byte b of lane half h of the B operand, and any
//    labelling of the 64 contraction indices by (h, b) works as long as both
//    operands use it;
//  * S^T = K Q^T: A = 32 key rows, 32 d-bytes per lane (two ds_read_b128 of
//    the K tile, d = 64 s + 32 h + b), B = the wave's 32 query rows, held in
//    registers in the same order;
//  * the S^T accumulator leaves lane (query, h) the keys 32 mb + 8 (i/4) +
//    4 h + i % 4 (element i); two consecutive 32-key blocks, rounded to E4M3
//    four at a time with v_cvt_pk_fp8_f32, are the B operand of one PV
//    product (byte b: block b / 16, element b % 16);
//  * O^T = V^T P^T: A = 32 d-rows of V^T; four ds_read_b64_tr_b8 give lane
//    (d, h) the 32 keys in exactly that labelling.  In a 16-lane group, lane
//    j receives byte j % 8 of the 8-byte pieces addressed by lanes 2 i + j / 8
//    (i = 0..7), so the addressing lane 2 i + t points at key row (i's key)
//    and d-bytes 8 t .. 8 t + 7 of its half of the 32-d block;
//  * K and V tiles are copied HBM -> LDS with buffer_load_dwordx4 ... lds
//    (16 bytes per lane, no registers), rows in natural order, the 16-byte chunks of row r
//    XOR-swizzled: K by (r >> 1) & 7 (a 16-lane pass of row reads then hits
//    16 different bank groups), V by 2 ((r >> 1) & 1 | ((r >> 3) & 1) << 1)
//    (the 32 8-byte pieces of a 32-lane transposed read cover all 64 banks).
//  * 8 waves (two per SIMD) of 32 queries share double-buffered 128-key tiles.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
constexpr float kPShift = 8.0f;   // P is rounded as P * 2^8

// 32x32x64 product of E4M3 operands (format code 0 for A and B, no block
// scales), fp32 accumulate
__device__ inline f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// four fp32 values -> four E4M3 bytes (round to nearest even), a in the low
// byte.  The first conversion keeps the upper half of its destination, which
// the second overwrites, so a's own register serves as that destination (no
// move of a zero first).
__device__ inline int pack4(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

template <int D> struct F8Geom {
    static constexpr int NW = 8, NT = 64 * NW, WPE = 2;
    static constexpr int BN = 128;          // keys per K/V tile
    static constexpr int BM = NW * 32;      // query rows per workgroup
    static constexpr int NS = D / 64;       // 64-byte d steps of S^T
    static constexpr int NMB = BN / 32;     // 32-key blocks (S^T accumulators)
    static constexpr int NPC = BN / 64;     // 64-key chunks (PV contraction steps)
    static constexpr int NDB = D / 32;      // 32-d blocks of O^T
    static constexpr int TILE = BN * D;     // bytes per K or V tile
    static constexpr int NBLK = TILE / 1024;
    static constexpr int BPW = NBLK / NW;   // 1 KB copy blocks per wave per tile
    static_assert(D == 128, "FP8 forward: d = 128");
    static_assert(BPW * NW == NBLK && BPW >= 1, "tile / waves");
    __device__ static inline int fk(int r) { return (r >> 1) & 7; }
    __device__ static inline int fv(int r) { return (((r >> 1) & 1) | (((r >> 3) & 1) << 1)) << 1; }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(F8Geom<D>::NT)
__attribute__((amdgpu_waves_per_eu(F8Geom<D>::WPE, F8Geom<D>::WPE)))
void fa_fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                       const uint8_t* __restrict__ V, uint16_t* __restrict__ O,
                       float* __restrict__ LSE, int BH, int Lq, int Lk, int nqb, float c,
                       float vd)
{
    using G = F8Geom<D>;
    constexpr int BN = G::BN, BM = G::BM, NS = G::NS, NMB = G::NMB, NPC = G::NPC;
    constexpr int NDB = G::NDB, NW = G::NW;

    __shared__ __attribute__((aligned(1024))) uint8_t Kb0[G::TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t Kb1[G::TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t Vb0[G::TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t Vb1[G::TILE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, half = lane >> 5;

    // work decode: every query block of a head on one XCD (block p runs on
    // XCD p % 8), causal: the longest rows first
    int bh, lvl;
    xcd_decode(blockIdx.x, BH, bh, lvl);
    const int qb = CAUSAL ? (nqb - 1 - lvl) : lvl;
    const int q0 = qb * BM;
    const int q0w = q0 + wave * 32;          // this wave's rows q0w .. q0w + 31
    const int qi = q0w + col;                // this lane's query (accumulator column)
    const uint8_t* Kh = K + (size_t)bh * Lk * D;
    const uint8_t* Vh = V + (size_t)bh * Lk * D;

    // Q^T fragments (B operand of S^T): d-bytes 64 s + 32 h .. + 31 of row qi
    i32x8 qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if (qi < Lq) {
            const i32x4* src = reinterpret_cast<const i32x4*>(Q + ((size_t)bh * Lq + qi) * D + 64 * s + 32 * half);
            const i32x4 a = src[0], b = src[1];
            qf[s] = i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        } else {
            qf[s] = i32x8{};
        }
    }
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
    float m_run = -__builtin_inff(), l_run = 0.f;

    const int kv_end = CAUSAL ? min(Lk, q0 + BM) : Lk;
    const int nt = (kv_end + BN - 1) / BN;

    // ---- tile copy: HBM -> LDS, 16 bytes per lane, no registers ----------
    // physical 16-byte chunk pc of tile row r holds logical chunk pc ^ f(r)
    unsigned kofs[G::BPW], vofs[G::BPW];
#pragma unroll
    for (int i = 0; i < G::BPW; ++i) {
        const int pbyte = (wave + NW * i) * 1024 + 16 * lane;
        const int row = pbyte / D, pch = (pbyte % D) / 16;
        kofs[i] = (unsigned)(row * D + (pch ^ G::fk(row)) * 16);
        vofs[i] = (unsigned)(row * D + (pch ^ G::fv(row)) * 16);
    }
    // Through a buffer resource per tile that starts at its first row and
    // covers only its rows below Lk (none for the prefetch after the last
    // tile): rows outside read zeros (finite values the mask gives weight
    // 0) without touching memory, so every step issues the same copies with
    // loop-constant lane offsets; the LDS destination comes from a scalar
    // copy of the wave index.
    const int swave = __builtin_amdgcn_readfirstlane(wave);
    auto issue = [&](int j, const uint8_t* base, const unsigned (&ofs)[G::BPW], uint8_t* dst) {
        const int jc = min(j, nt - 1);
        const int bytes = j < nt ? min(BN, Lk - jc * BN) * D : 0;
        const uint8_t* src = base + (size_t)jc * BN * D;
#pragma unroll
        for (int i = 0; i < G::BPW; ++i)
            buffer_copy<16>(src, bytes, ofs[i], (FA_LDS void*)(dst + (swave + NW * i) * 1024));
    };

    // K fragment (A operand of S^T) for key block mb, d step s: row 32 mb +
    // col, logical chunks 4 s + 2 h + t (t = 0, 1); f_k(32 mb + col) = f_k(col)
    int kfo[NS][2];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t) kfo[s][t] = col * D + ((4 * s + 2 * half + t) ^ G::fk(col)) * 16;
    auto k_frag = [&](const uint8_t* Ks, int mb, int s) {
        const i32x4 a = *reinterpret_cast<const i32x4*>(Ks + mb * 32 * D + kfo[s][0]);
        const i32x4 b = *reinterpret_cast<const i32x4*>(Ks + mb * 32 * D + kfo[s][1]);
        return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    };
    // V^T fragment (A operand of O^T) for key chunk pc, d block db: read u
    // (bytes 8 u .. 8 u + 7 of every lane) is addressed by lane (g, s) of its
    // 16-lane group at key 64 pc + 32 (u / 2) + 16 (u % 2) + 8 a + 4 h + e
    // (a = s / 8, e = (s / 2) % 4, h = g / 2) and d-bytes 32 db + 16 (g % 2) +
    // 8 (s % 2).  The row's swizzle depends on a and e only, i.e. on the lane.
    const int g16 = lane >> 4, s16 = lane & 15;
    const int va = s16 >> 3, ve = (s16 >> 1) & 3, vhh = g16 >> 1, vg1 = g16 & 1, vt = s16 & 1;
    const int vrow = 8 * va + 4 * vhh + ve;
    const int vfh = G::fv(vrow) >> 1;
    int vlane[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        vlane[db] = vrow * D + 32 * (db ^ vfh) + 16 * vg1 + 8 * vt;
    auto v_frag = [&](const uint8_t* Vs, int pc, int db) {
        i32x2 u[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint8_t* a = Vs + (64 * pc + 32 * (r >> 1) + 16 * (r & 1)) * D + vlane[db];
            u[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA_LDS i32x2*)(FA_LDS void*)a);
        }
        return i32x8{u[0][0], u[0][1], u[1][0], u[1][1], u[2][0], u[2][1], u[3][0], u[3][1]};
    };

    // Wait until this wave's copies and LDS reads are done, then barrier;
    // the empty asm statements keep memory accesses from moving across.
    auto sync_tiles = [&]() {
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) expcnt(7) lgkmcnt(0)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    auto step = [&](int j, const uint8_t* Kc, const uint8_t* Vc, uint8_t* Kn, uint8_t* Vn) {
        const int kv0 = j * BN;
        issue(j + 1, Kh, kofs, Kn);
        issue(j + 1, Vh, vofs, Vn);
        // a wave whose rows all precede this tile skips its math
        if (!CAUSAL || kv0 <= q0w + 31) {
            // S^T = K Q^T
            f32x16 sacc[NMB];
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) sacc[mb] = f32x16{};
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) sacc[mb] = mfma8(k_frag(Kc, mb, s), qf[s], sacc[mb]);
            // masks: element i of block mb is key kv0 + 4 h + 32 mb + 8 (i/4)
            // + i % 4; this lane's query sees keys up to min(Lk - 1, qi)
            if (kv0 + BN > Lk || (CAUSAL && kv0 + BN - 1 > q0w)) {
                int hi = CAUSAL ? min(Lk - 1, qi) : Lk - 1;
                hi -= kv0 + 4 * half;     // visible iff offset <= hi
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (32 * mb + 8 * (i / 4) + (i % 4) > hi) sacc[mb][i] = -__builtin_inff();
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // running max, rescale, exponentials (times 2^8)
            float pm[NMB];
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
                float a = fmaxf(fmaxf(sacc[mb][0], sacc[mb][1]), sacc[mb][2]);
#pragma unroll
                for (int i = 3; i < 15; i += 2) a = fmaxf(fmaxf(a, sacc[mb][i]), sacc[mb][i + 1]);
                pm[mb] = fmaxf(a, sacc[mb][15]);
            }
#pragma unroll
            for (int mb = 1; mb < NMB; ++mb) pm[0] = fmaxf(pm[0], pm[mb]);
            const float m_new = fmaxf(m_run, half_max(pm[0]) * c);
            const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
            }
            m_run = m_new;
            const float off = kPShift - m_use;
            float rs = 0.f;
            i32x8 pb[NPC];
#pragma unroll
            for (int pc = 0; pc < NPC; ++pc) {
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    const int mb = 2 * pc + (w >> 2), e = 4 * (w & 3);
                    float p[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        p[x] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mb][e + x], c, off));
                    rs += (p[0] + p[1]) + (p[2] + p[3]);
                    pb[pc][w] = pack4(p[0], p[1], p[2], p[3]);
                }
            }
            l_run = l_run * alpha + rs;
            // O^T += V^T P^T
#pragma unroll
            for (int pc = 0; pc < NPC; ++pc)
#pragma unroll
                for (int db = 0; db < NDB; ++db) oacc[db] = mfma8(v_frag(Vc, pc, db), pb[pc], oacc[db]);
        }
        sync_tiles();   // this wave's copies of tile j + 1 landed; reads of tile j done
    };
    issue(0, Kh, kofs, Kb0);
    issue(0, Vh, vofs, Vb0);
    sync_tiles();
    for (int j = 0; j < nt; j += 2) {
        step(j, Kb0, Vb0, Kb1, Vb1);
        if (j + 1 < nt) step(j + 1, Kb1, Vb1, Kb0, Vb0);
    }

    // epilogue: O = v_descale O_acc / l, LSE = ln2 (m + log2 l - 8); the
    // cross-half sum runs on every lane
    const float lt = half_sum(l_run);
    if (qi < Lq) {
        const float inv = vd / lt;
        uint16_t* Or = O + ((size_t)bh * Lq + qi) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 v4 = {oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]};
                v4 *= inv;
                *reinterpret_cast<bf16x4*>(Or + 32 * db + 8 * g + 4 * half) =
                    __builtin_convertvector(v4, bf16x4);
            }
        if (half == 0)
            LSE[(size_t)bh * Lq + qi] = (m_run + __builtin_amdgcn_logf(lt) - kPShift) * kLn2;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_fp8_d(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int Lq, int Lk, float c, float vd, hipStream_t stream)
{
    using G = F8Geom<D>;
    const int BH = B * H;
    const int nqb = (Lq + G::BM - 1) / G::BM;
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)(nqb * BH)), dim3(G::NT), 0,
                       stream, static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(k),
                       static_cast<const uint8_t*>(v), static_cast<uint16_t*>(o), lse, BH, Lq, Lk,
                       nqb, c, vd);
    return hipGetLastError();
}

}  // namespace

bool fp8_tile_config(int d, TileConfig* out)
{
    if (d != 128) return false;
    *out = TileConfig{F8Geom<128>::BM, F8Geom<128>::BN, F8Geom<128>::NT};
    return true;
}

hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int Lq, int Lk, int d, bool causal, float c, float vd,
                          hipStream_t stream)
{
    if (d != 128) return hipErrorInvalidValue;
    return causal ? launch_fp8_d<128, true>(q, k, v, o, lse, B, H, Lq, Lk, c, vd, stream)
                  : launch_fp8_d<128, false>(q, k, v, o, lse, B, H, Lq, Lk, c, vd, stream);
}

}  // namespace fa
