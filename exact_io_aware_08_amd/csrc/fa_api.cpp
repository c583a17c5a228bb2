// C-ABI entry points of libfa_fwd.so (declared in include/fa.h).
//
// Every argument check runs here, on the host, before any HIP call: a
// nonzero status means nothing was enqueued.  The only HIP calls are the
// kernel launch and hipGetLastError right after it.

#include <algorithm>
#include <atomic>
#include <initializer_list>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "fa.h"
#include "fa_internal.h"

namespace {

bool aligned16(const void* p) {
    return (reinterpret_cast<std::uintptr_t>(p) & 15u) == 0;
}

// The kernels take the scores' exponent factor scale * log2(e) as an fp32
// value; a scale above FLT_MAX / log2(e) would make it infinite.
bool factor_finite(float scale) {
    return std::isfinite((float)((double)scale * 1.4426950408889634));
}

// [p, p + bytes) overlaps [r, r + rbytes)
bool overlaps(const void* p, std::size_t bytes, const void* r, std::size_t rbytes) {
    const auto a = reinterpret_cast<std::uintptr_t>(p);
    const auto b = reinterpret_cast<std::uintptr_t>(r);
    return a < b + rbytes && b < a + bytes;
}

// Workspace of fa_fwd_splitkv: fp32 partial O [nsplit][B*H][Lq][d], then
// fp32 partial LSE [nsplit][B*H][Lq], each part starting on 256 bytes.
std::size_t round256(std::size_t n) { return (n + 255) & ~(std::size_t)255; }
std::size_t split_opart_bytes(long long bh, int Lq, int d, int nsplit) {
    return round256((std::size_t)nsplit * bh * Lq * d * sizeof(float));
}
std::size_t split_workspace_bytes(long long bh, int Lq, int d, int nsplit) {
    return split_opart_bytes(bh, Lq, d, nsplit) +
           round256((std::size_t)nsplit * bh * Lq * sizeof(float));
}
constexpr int kMaxSplits = 64;

// Which keys each query sees (after the ABI arguments are checked).
struct MaskSpec {
    bool causal = false;   // fa_fwd / fa_fwd_f32
    bool window = false;   // fa_fwd_window with a bound the causal flag cannot express
    int wl = 0, wr = 0;    // window bounds, clamped to [0, Lq + Lk]
    int nsplit = 0;        // fa_fwd_splitkv: key splits (>= 1), else 0
    void* workspace = nullptr;
    std::size_t workspace_bytes = 0;
    bool check_only = false;   // run the argument checks (not the workspace's), launch nothing
};

int validate_and_launch(fa::DType dt, std::size_t esize, const void* q,
                        const void* k, const void* v, void* o, float* lse,
                        int B, int H, int Lq, int Lk, int d, int mask_status,
                        const MaskSpec& mask, float scale, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || H < 1 || Lq < 1 || Lk < 1) return FA_ERR_SHAPE;
    fa::TileConfig tc;
    if (!fa::tile_config(dt, d, &tc)) return FA_ERR_UNSUPPORTED_D;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        !aligned16(lse))
        return FA_ERR_ALIGN;
    if (!std::isfinite(scale) || !(scale >= 0.f) || !factor_finite(scale)) return FA_ERR_SCALE;
    if (mask_status != FA_OK) return mask_status;   // causal / window / split arguments
    if (mask.nsplit && !mask.check_only) {
        if (!mask.workspace) return FA_ERR_NULL;
        if (!aligned16(mask.workspace)) return FA_ERR_ALIGN;
    }

    // sizes: element counts must fit the kernel's 64-bit offsets and the
    // per-head int arithmetic; the grid must fit one dimension.
    const long long bh = (long long)B * H;
    const long long nqb = ((long long)Lq + tc.block_m - 1) / tc.block_m;
    const long long grid = nqb * bh;
    if (bh > (1LL << 30) || grid > 0x7fffffffLL) return FA_ERR_SHAPE;
    if ((long long)Lq * d > 0x7fffffffLL || (long long)Lk * d > 0x7fffffffLL)
        return FA_ERR_SHAPE;
    const std::size_t qbytes = (std::size_t)bh * Lq * d * esize;
    const std::size_t kbytes = (std::size_t)bh * Lk * d * esize;
    const std::size_t lbytes = (std::size_t)bh * Lq * sizeof(float);
    if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kbytes) ||
        overlaps(o, qbytes, v, kbytes) || overlaps(lse, lbytes, q, qbytes) ||
        overlaps(lse, lbytes, k, kbytes) || overlaps(lse, lbytes, v, kbytes) ||
        overlaps(lse, lbytes, o, qbytes))
        return FA_ERR_ARG;
    if (mask.check_only) return FA_OK;
    if (mask.nsplit) {
        const std::size_t wbytes = split_workspace_bytes(bh, Lq, d, mask.nsplit);
        if (mask.workspace_bytes < wbytes) return FA_ERR_WORKSPACE;
        const void* w = mask.workspace;
        if (overlaps(w, wbytes, q, qbytes) || overlaps(w, wbytes, k, kbytes) ||
            overlaps(w, wbytes, v, kbytes) || overlaps(w, wbytes, o, qbytes) ||
            overlaps(w, wbytes, lse, lbytes))
            return FA_ERR_ARG;
        float* opart = static_cast<float*>(mask.workspace);
        float* lpart = reinterpret_cast<float*>(static_cast<char*>(mask.workspace) +
                                                split_opart_bytes(bh, Lq, d, mask.nsplit));
        const hipError_t err = fa::launch_fwd_split(q, k, v, o, lse, B, H, Lq, Lk, d,
                                                    mask.causal, scale, mask.nsplit, opart,
                                                    lpart, stream);
        return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
    }

    const hipError_t err =
        mask.window ? fa::launch_fwd_window(q, k, v, o, lse, B, H, Lq, Lk, d, mask.wl, mask.wr,
                                            scale, stream)
                    : fa::launch_fwd(dt, q, k, v, o, lse, B, H, Lq, Lk, d, mask.causal, scale,
                                     stream);
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// causal flag of fa_fwd / fa_fwd_f32
int causal_mask(int causal, MaskSpec* m) {
    if (causal != 0 && causal != 1) return FA_ERR_ARG;
    m->causal = causal == 1;
    return FA_OK;
}

// window pair of fa_fwd_window: -1 = unbounded on that side.  (-1, -1) is
// full attention and (-1, 0) the causal mask; both take those kernels.
int window_mask(int left, int right, int Lq, int Lk, MaskSpec* m) {
    if (left < -1 || right < -1) return FA_ERR_ARG;
    const long long cap = (long long)Lq + Lk;   // farther bounds change nothing
    if (left == -1 && right == -1) return FA_OK;
    if (left == -1 && right == 0) {
        m->causal = true;
        return FA_OK;
    }
    m->window = true;
    m->wl = (int)(left < 0 ? cap : std::min<long long>(left, cap));
    m->wr = (int)(right < 0 ? cap : std::min<long long>(right, cap));
    return FA_OK;
}

// Workspace of fa_bwd: -Delta then -LSE / scale, [B*H][Lq] fp32 each.
std::size_t bwd_workspace_bytes(long long bh, int Lq) {
    return 2 * round256((std::size_t)bh * Lq * sizeof(float));
}

}  // namespace

namespace fa {

int cu_count() {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cache[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDev) {
        const int n = cache[dev].load(std::memory_order_relaxed);
        if (n > 0) return n;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        return 0;
    if (dev < kMaxDev) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

int splitkv_check(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int H, int Lq, int Lk, int d, int causal, float scale, int num_splits) {
    MaskSpec m;
    int ms = causal_mask(causal, &m);
    if (ms == FA_OK && (num_splits < 1 || num_splits > kMaxSplits)) ms = FA_ERR_ARG;
    m.nsplit = num_splits;
    m.check_only = true;
    return validate_and_launch(DType::BF16, 2, q, k, v, o, lse, B, H, Lq, Lk, d, ms, m, scale,
                               nullptr);
}

}  // namespace fa

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Lq, int Lk, int d, int causal, float scale,
           hipStream_t stream) {
    MaskSpec m;
    const int ms = causal_mask(causal, &m);
    return validate_and_launch(fa::DType::BF16, 2, q, k, v, o, lse, B, H, Lq,
                               Lk, d, ms, m, scale, stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Lq, int Lk, int d, int causal, float scale,
               float q_descale, float k_descale, float v_descale, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || H < 1 || Lq < 1 || Lk < 1) return FA_ERR_SHAPE;
    fa::TileConfig tc;
    if (!fa::fp8_tile_config(d, &tc)) return FA_ERR_UNSUPPORTED_D;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_ALIGN;
    if (!std::isfinite(scale) || !(scale >= 0.f)) return FA_ERR_SCALE;
    for (float x : {q_descale, k_descale, v_descale})
        if (!std::isfinite(x) || !(x > 0.f)) return FA_ERR_SCALE;
    // the exponent factor of S: scale * q_descale * k_descale * log2(e)
    const double cd = (double)scale * q_descale * k_descale * 1.4426950408889634;
    if (!std::isfinite((float)cd)) return FA_ERR_SCALE;
    const float c = fa::exp2_factor(cd);
    if (causal != 0 && causal != 1) return FA_ERR_ARG;
    const long long bh = (long long)B * H;
    const long long grid = (((long long)Lq + tc.block_m - 1) / tc.block_m) * bh;
    if (bh > (1LL << 30) || grid > 0x7fffffffLL) return FA_ERR_SHAPE;
    if ((long long)Lq * d > 0x7fffffffLL || (long long)Lk * d > 0x7fffffffLL)
        return FA_ERR_SHAPE;
    const std::size_t qbytes = (std::size_t)bh * Lq * d;        // E4M3: 1 byte
    const std::size_t kbytes = (std::size_t)bh * Lk * d;
    const std::size_t obytes = (std::size_t)bh * Lq * d * 2;    // bf16
    const std::size_t lbytes = (std::size_t)bh * Lq * sizeof(float);
    if (overlaps(o, obytes, q, qbytes) || overlaps(o, obytes, k, kbytes) ||
        overlaps(o, obytes, v, kbytes) || overlaps(lse, lbytes, q, qbytes) ||
        overlaps(lse, lbytes, k, kbytes) || overlaps(lse, lbytes, v, kbytes) ||
        overlaps(lse, lbytes, o, obytes))
        return FA_ERR_ARG;
    const hipError_t err = fa::launch_fwd_fp8(q, k, v, o, lse, B, H, Lq, Lk, d, causal == 1, c,
                                              v_descale, stream);
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o,
               float* lse, int B, int H, int Lq, int Lk, int d, int causal,
               float scale, hipStream_t stream) {
    MaskSpec m;
    const int ms = causal_mask(causal, &m);
    return validate_and_launch(fa::DType::F32, 4, q, k, v, o, lse, B, H, Lq,
                               Lk, d, ms, m, scale, stream);
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Lq, int Lk, int d, int causal, float scale,
                   int num_splits, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
    MaskSpec m;
    int ms = causal_mask(causal, &m);
    if (ms == FA_OK && (num_splits < 1 || num_splits > kMaxSplits)) ms = FA_ERR_ARG;
    m.nsplit = num_splits;
    m.workspace = workspace;
    m.workspace_bytes = workspace_bytes;
    return validate_and_launch(fa::DType::BF16, 2, q, k, v, o, lse, B, H, Lq,
                               Lk, d, ms, m, scale, stream);
}

size_t fa_splitkv_workspace_size(int B, int H, int Lq, int d, int num_splits) {
    if (B < 1 || H < 1 || Lq < 1 || num_splits < 1 || num_splits > kMaxSplits) return 0;
    if (d != 64 && d != 128 && d != 256) return 0;
    return split_workspace_bytes((long long)B * H, Lq, d, num_splits);
}

int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Lq, int Lk, int d, int window_left, int window_right,
                  float scale, hipStream_t stream) {
    MaskSpec m;
    const int ms = window_mask(window_left, window_right, Lq, Lk, &m);
    return validate_and_launch(fa::DType::BF16, 2, q, k, v, o, lse, B, H, Lq,
                               Lk, d, ms, m, scale, stream);
}

size_t fa_bwd_workspace_size(int B, int H, int Lq) {
    if (B < 1 || H < 1 || Lq < 1) return 0;
    return bwd_workspace_bytes((long long)B * H, Lq);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, int B, int H, int Lq, int Lk,
           int d, int causal, float scale, void* workspace, size_t workspace_bytes,
           hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace)
        return FA_ERR_NULL;
    if (B < 1 || H < 1 || Lq < 1 || Lk < 1) return FA_ERR_SHAPE;
    if (!fa::bwd_supported(d)) return FA_ERR_UNSUPPORTED_D;
    for (const void* p : {q, k, v, o, static_cast<const void*>(lse), dout,
                          static_cast<const void*>(dq), static_cast<const void*>(dk),
                          static_cast<const void*>(dv), static_cast<const void*>(workspace)})
        if (!aligned16(p)) return FA_ERR_ALIGN;
    if (!std::isfinite(scale) || !(scale > 0.f) || !factor_finite(scale)) return FA_ERR_SCALE;
    if (causal != 0 && causal != 1) return FA_ERR_ARG;
    const long long bh = (long long)B * H;
    if (bh > (1LL << 30) || (long long)Lq * d > 0x7fffffffLL || (long long)Lk * d > 0x7fffffffLL ||
        bh * ((Lq + 255) / 256) > 0x7fffffffLL || bh * ((Lk + 127) / 128) > 0x7fffffffLL)
        return FA_ERR_SHAPE;
    const std::size_t qbytes = (std::size_t)bh * Lq * d * 2;
    const std::size_t kbytes = (std::size_t)bh * Lk * d * 2;
    const std::size_t lbytes = (std::size_t)bh * Lq * sizeof(float);
    const std::size_t wbytes = bwd_workspace_bytes(bh, Lq);
    if (workspace_bytes < wbytes) return FA_ERR_WORKSPACE;
    // outputs (dq, dk, dv, workspace) must not overlap any argument or each other
    struct Span { const void* p; std::size_t n; };
    const Span ins[] = {{q, qbytes}, {k, kbytes}, {v, kbytes}, {o, qbytes}, {lse, lbytes},
                        {dout, qbytes}};
    const Span outs[] = {{dq, qbytes}, {dk, kbytes}, {dv, kbytes}, {workspace, wbytes}};
    for (int i = 0; i < 4; ++i) {
        for (const Span& s : ins)
            if (overlaps(outs[i].p, outs[i].n, s.p, s.n)) return FA_ERR_ARG;
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return FA_ERR_ARG;
    }
    float* ndelta = static_cast<float*>(workspace);
    float* nlse = reinterpret_cast<float*>(static_cast<char*>(workspace) + wbytes / 2);
    const hipError_t err = fa::launch_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d,
                                          causal == 1, scale, ndelta, nlse, stream);
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

const char* fa_status_string(int status) {
    switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer argument";
    case FA_ERR_SHAPE: return "B, H, Lq and Lk must be >= 1 and sizes must fit";
    case FA_ERR_UNSUPPORTED_D: return "head dim d must be 64, 128 or 256";
    case FA_ERR_ALIGN: return "pointers must be 16-byte aligned";
    case FA_ERR_SCALE: return "scale must be finite and >= 0 (> 0 for fa_bwd; FP8 descales > 0), with scale * log2(e) finite in fp32";
    case FA_ERR_ARG: return "causal must be 0 or 1, window bounds >= -1, 1 <= num_splits <= 64, and outputs and workspace must not overlap inputs";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_WORKSPACE: return "workspace smaller than fa_splitkv_workspace_size";
    case FA_ERR_SCRATCH:
        return "the key-split partials exceed the library's fixed scratch "
               "(fa_noalloc_scratch_bytes)";
    default: return "unknown status";
    }
}

int fa_abi_version(void) { return FA_ABI_VERSION; }

int fa_splitkv_suggest(int B, int H, int Lq, int Lk, int d, int causal, int num_cus) {
    if (B < 1 || H < 1 || Lq < 1 || Lk < 1 || (causal != 0 && causal != 1)) return 0;
    fa::TileConfig tc;
    if (!fa::tile_config(fa::DType::BF16, d, &tc)) return 0;
    if (num_cus <= 0 && (num_cus = fa::cu_count()) <= 0) return 0;
    const long long nqb = ((long long)Lq + tc.block_m - 1) / tc.block_m;
    const long long base = (long long)B * H * nqb;
    // key tiles of the longest query block (causal: it sees min(Lk, Lq) keys)
    const long long keys = causal ? std::min<long long>(Lk, Lq) : Lk;
    const long long tiles = (keys + tc.block_n - 1) / tc.block_n;
    long long splits;
    if (!causal) {
        // equal blocks: enough workgroups for every compute unit
        if (base >= num_cus) return 1;
        splits = (num_cus + base - 1) / base;
    } else {
        // causal block i sees min(Lk, (i + 1) block_m) keys; the longest
        // block's share of tiles should not exceed the mean per compute unit
        long long total = 0;
        for (long long i = 0; i < nqb; ++i)
            total += (std::min<long long>(Lk, (i + 1) * tc.block_m) + tc.block_n - 1) / tc.block_n;
        total *= (long long)B * H;
        splits = (tiles * num_cus + total - 1) / total;
    }
    splits = std::min<long long>(splits, std::max<long long>(1, tiles / 8));
    // at d = 64 the unsplit kernel already runs two key halves per block on
    // grids of at most two workgroups per compute unit (merged on chip)
    if (d == 64 && base <= 2LL * num_cus && splits <= 2) return 1;
    return (int)std::max<long long>(1, std::min<long long>(splits, kMaxSplits));
}

int fa_tile_config(int dtype, int d, int* block_m, int* block_n, int* threads) {
    if (dtype < 0 || dtype > 2) return FA_ERR_ARG;
    fa::TileConfig tc;
    const bool ok = dtype == 2 ? fa::fp8_tile_config(d, &tc)
                               : fa::tile_config(dtype == 0 ? fa::DType::BF16 : fa::DType::F32, d, &tc);
    if (!ok) return FA_ERR_UNSUPPORTED_D;
    if (block_m) *block_m = tc.block_m;
    if (block_n) *block_n = tc.block_n;
    if (threads) *threads = tc.threads;
    return FA_OK;
}

}  // extern "C"
