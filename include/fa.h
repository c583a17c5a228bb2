/*
 * fa.h - C ABI of the MI355X (gfx950) FlashAttention-2 forward library
 *        (libfa_fwd.so).
 *
 * Operation (every forward entry point):  for every batch b < B,
 * head h < H and query row i < Lq,
 *
 *     s_ij   = scale * sum_t q[b,h,i,t] * k[b,h,j,t]        j < Lk
 *     A_i    = { j < Lk }                  (causal == 0)
 *            = { j < Lk : j <= i }         (causal == 1, top-left aligned)
 *            = { j < Lk : i - wl <= j <= i + wr }    (fa_fwd_window)
 *     o[b,h,i,:] = sum_{j in A_i} softmax_j(s_i.) * v[b,h,j,:]
 *     lse[b,h,i] = ln( sum_{j in A_i} exp(s_ij) )           natural log
 *
 * i.e. O = softmax(Q K^T * scale) V plus the per-row log-sum-exp, the
 * exact scaled dot-product attention result ("Flash Attention 原理与实现详解：
 * 如何通过 IO-Aware 算法突破注意力机制的计算瓶颈" (tbr8.org), section 一 and
 * section 3 "Flash Attention v2"; the LSE output of "第 08 章: Flash
 * Attention——分块注意力" (chuoer47.github.io), section 3 "LSE"; the causal
 * lower triangle including the diagonal, same page, section 4).  It is
 * computed tile by tile with the online-softmax update ("從零開始用自定義
 * Triton 內核編寫 FlashAttention-2" (digipub.cc), sections "流式注意力內核
 * _attn_fwd_inner" and "部分分數計算和在線更新"), so the Lq x Lk score matrix
 * never reaches device memory.
 *
 * Layout: q and o are [B, H, Lq, d], k and v are [B, H, Lk, d], all dense
 * row-major (d fastest) with no padding; lse is [B, H, Lq] fp32.  All five
 * are device pointers, 16-byte aligned.
 *
 * Ownership: the caller owns every buffer.  The library never allocates,
 * frees or synchronises; each call enqueues its kernels on `stream` (a
 * hipStream_t; 0 means the null stream) and returns: one kernel for the
 * forward entry points, two for the key split (partials, then merge), three
 * for the backward (preprocess, dK/dV, dQ).  o and lse must not
 * overlap q, k, v or each other.  Calls are thread-safe (no global mutable
 * state).
 *
 * Errors: every argument check runs on the host before any HIP call; on a
 * nonzero return nothing was enqueued.  FA_ERR_LAUNCH reports a failed
 * launch (hipGetLastError after the launch).  Faults during execution
 * surface at the caller's next synchronisation of `stream`.
 */
#ifndef FA_FWD_H
#define FA_FWD_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 7   /* 2: fa_fwd_window; 3: fa_fwd_splitkv; 4: fa_bwd;
                              5: fa_fwd_fp8; 6: fa_splitkv_suggest;
                              7: fa_fwd_splitkv_noalloc */

enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = 1,           /* a pointer argument is NULL                 */
    FA_ERR_SHAPE = 2,          /* B, H, Lq or Lk < 1, or a size overflows    */
    FA_ERR_UNSUPPORTED_D = 3,  /* d is not 64, 128 or 256                    */
    FA_ERR_ALIGN = 4,          /* a pointer is not 16-byte aligned           */
    FA_ERR_SCALE = 5,          /* scale not finite and >= 0 (fa_bwd: > 0;
                                  fa_fwd_fp8: descales finite and > 0), or
                                  its exponent factor past fp32's range     */
    FA_ERR_ARG = 6,            /* causal not 0/1, a window bound < -1, or
                                  outputs overlap inputs                     */
    FA_ERR_LAUNCH = 7,         /* the kernel launch failed                   */
    FA_ERR_WORKSPACE = 8,      /* workspace smaller than required            */
    FA_ERR_SCRATCH = 9         /* fa_fwd_splitkv_noalloc: the partials exceed
                                  the fixed scratch (fa_noalloc_scratch_bytes) */
};

/*
 * bf16 forward (the benchmarked entry point).  q, k, v, o hold bfloat16
 * values (raw 16-bit patterns); lse is fp32.  Products QK^T and PV run on
 * bf16 MFMA with fp32 accumulation; P is rounded to bf16 (round to nearest
 * even) before the PV product, as the pages cast P to V's dtype
 * ("FlashAttention的Triton实现：IO-aware注意力机制底层原理" (gitcode.csdn.net),
 * section "FlashAttention的Triton Kernel结构"); o is rounded to bf16 with
 * round to nearest even.
 *   d      : 64, 128 or 256
 *   causal : 0 (all keys) or 1 (key j visible to query i iff j <= i)
 *   scale  : multiplies QK^T; finite and >= 0 (usually 1/sqrt(d)), with
 *            scale * log2(e) finite in fp32 (else FA_ERR_SCALE).  scale = 0
 *            weighs every visible key the same (O the mean of the visible V
 *            rows, lse = ln of their count); the kernels then use the
 *            exponent factor FLT_MIN in place of 0 (exact for |q.k| < 2^101).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Lq, int Lk, int d, int causal, float scale,
           hipStream_t stream);

/*
 * fp32 forward: q, k, v, o are fp32; the same kernel template on the fp32
 * MFMA (P stays fp32).  Same arguments, layout, ownership and errors as
 * fa_fwd.
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o,
               float* lse, int B, int H, int Lq, int Lk, int d, int causal,
               float scale, hipStream_t stream);

/*
 * bf16 sliding-window forward: key j is visible to query i iff
 * i - window_left <= j <= i + window_right (and j < Lk), the (left, right)
 * window-size pair of "Flash Attention 原理与实现详解" (tbr8.org), section
 * 6.3 "滑动窗口注意力" ((1024, 0) together with causal masking: 1024 keys to
 * the left of each query and none to its right).  A bound of -1 means no
 * bound on that side, so (-1, 0) is fa_fwd with causal = 1 and (-1, -1) is
 * fa_fwd with causal = 0; a bound w >= 0 admits keys at distance up to and
 * including w.  A query row with no visible key (only possible when
 * i > Lk - 1 + window_left) gets o = 0 and lse = -inf.  Other arguments,
 * layout, ownership, precision and errors as fa_fwd; a bound below -1 is
 * FA_ERR_ARG.  Only tiles that intersect a query block's band are read.
 */
int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Lq, int Lk, int d, int window_left,
                  int window_right, float scale, hipStream_t stream);

/*
 * bf16 forward with the keys split among num_splits workgroups per query
 * block, for shapes with too few query blocks to fill the GPU (short Lq,
 * long Lk).  Each split computes the normalised partial result over its
 * share of the block's key tiles, in fp32, into `workspace`; a second
 * kernel merges the partials with the block-merge step of "Flash Attention
 * 原理与实现详解" (tbr8.org), section 2.1 "Tiling（分块计算）策略":
 * LSE = ln sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s.  The result
 * is the same quantity as fa_fwd's (rounding differs only in the order of
 * the sums).
 *   num_splits      : 1 .. 64
 *   workspace       : device memory of at least
 *                     fa_splitkv_workspace_size(B, H, Lq, d, num_splits)
 *                     bytes, 16-byte aligned, owned by the caller, not
 *                     overlapping any other argument; its contents are
 *                     scratch (overwritten, need not be initialised).
 *                     Concurrent calls need separate workspaces.
 * Both kernels are enqueued on `stream`.  Other arguments, layout,
 * ownership and errors as fa_fwd; a NULL workspace is FA_ERR_NULL, a
 * misaligned one FA_ERR_ALIGN, num_splits out of range FA_ERR_ARG, a small
 * one FA_ERR_WORKSPACE.
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Lq, int Lk, int d, int causal, float scale,
                   int num_splits, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/*
 * fa_fwd_splitkv without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The fp32 partials live in a
 * fixed device array of the library, fa_noalloc_scratch_bytes() bytes (40
 * MiB) on each GPU it runs on, held until the process ends; the call
 * itself allocates and frees nothing.  Every call on one GPU shares that
 * GPU's array, so calls that overlap in time on one GPU race; calls on
 * different GPUs do not.  All arguments, checks, results and errors as
 * fa_fwd_splitkv (same kernels, bit-identical output); a problem whose
 * partials, fa_splitkv_workspace_size(B, H, Lq, d, num_splits) bytes,
 * exceed the array returns FA_ERR_SCRATCH before any HIP call.
 */
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Lq, int Lk, int d, int causal, float scale,
                           int num_splits, hipStream_t stream);

/* Bytes of the fixed scratch fa_fwd_splitkv_noalloc uses per GPU.  Host-only. */
size_t fa_noalloc_scratch_bytes(void);

/* Workspace bytes fa_fwd_splitkv needs, or 0 for invalid arguments
 * (B, H, Lq < 1, d not 64/128/256, num_splits outside 1 .. 64).  Host-only. */
size_t fa_splitkv_workspace_size(int B, int H, int Lq, int d, int num_splits);

/* A num_splits for fa_fwd_splitkv on this shape.  Non-causal: 1 when the
 * unsplit grid (B * H * query blocks) already gives every compute unit a
 * workgroup, else enough splits that the (query block, split) workgroups
 * cover `num_cus` compute units.  Causal (blocks of unequal length): enough
 * splits that the longest block's share of key tiles is at most the mean
 * number of tiles per compute unit.  Either way at least 8 key tiles per
 * split and at most 64 splits; 1 instead of 2 at d = 64 when the unsplit
 * kernel already splits each block's keys in two (grids of at most two
 * workgroups per compute unit).  num_cus <= 0 reads the current device's
 * count.  Returns 0 for invalid arguments (as fa_fwd's shape checks) or
 * when the device cannot be queried.  Host-only; no GPU work. */
int fa_splitkv_suggest(int B, int H, int Lq, int Lk, int d, int causal, int num_cus);

/*
 * bf16 backward: the gradients dq, dk, dv of sum(dout * o) for the forward
 * o = fa_fwd(q, k, v, causal, scale), following "第 08 章: Flash Attention——
 * 分块注意力" (chuoer47.github.io), section 6 "反向":
 *     Delta_i = sum_t dout[i,t] o[i,t]
 *     P_ij    = exp(scale q_i.k_j - lse_i)      (recomputed, j in A_i)
 *     dv = P^T dout,   dP = dout v^T,   dS = P (dP - Delta),
 *     dq = scale dS k,  dk = scale dS^T q
 * o and lse must be the outputs of fa_fwd for the same q, k, v, causal and
 * scale (lse is the natural-log LSE fa_fwd writes; scale > 0 here).  Products run on bf16
 * MFMA with fp32 accumulation (P and dS rounded to bf16 for their second
 * product); dq, dk, dv are written in bf16, round to nearest even.
 *   layout    : q, o, dout, dq [B, H, Lq, d]; k, v, dk, dv [B, H, Lk, d];
 *               lse [B, H, Lq] fp32; dense row-major, 16-byte aligned
 *   d         : 64 or 128 (other values: FA_ERR_UNSUPPORTED_D)
 *   workspace : device memory of at least fa_bwd_workspace_size(B, H, Lq)
 *               bytes, 16-byte aligned, caller-owned scratch (holds Delta);
 *               concurrent calls need separate workspaces
 * Three kernels are enqueued on `stream`.  dq, dk, dv and the workspace must
 * not overlap any other argument or each other.  Errors as fa_fwd, plus
 * FA_ERR_WORKSPACE for a small workspace.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, int B, int H, int Lq, int Lk,
           int d, int causal, float scale, void* workspace, size_t workspace_bytes,
           hipStream_t stream);

/*
 * FP8 forward: the same operation on FP8 inputs, the pages' FP8 variant
 * ("Flash Attention 原理与实现详解" (tbr8.org), section 4.3 "FP8 支持"; the
 * page warns that it loses more precision, section 6.1 "精度问题").
 *   q, k, v   : OCP FP8 E4M3 codes (1 byte each: sign, 4 exponent bits with
 *               bias 7, 3 mantissa bits; 448 the largest finite value),
 *               [B, H, Lq, d] / [B, H, Lk, d]; the value of a code is
 *               decode(code) * q_descale (k_descale, v_descale for k, v)
 *   o         : bf16 [B, H, Lq, d];  lse: fp32 [B, H, Lq], natural log
 *   d         : 128 (other values: FA_ERR_UNSUPPORTED_D)
 *   descales  : finite and > 0; scale finite and >= 0, and scale * q_descale
 *               * k_descale * log2(e) finite in fp32 (else FA_ERR_SCALE); a
 *               product below FLT_MIN weighs every visible key the same
 * S = scale * q_descale * k_descale * (Q K^T) from the codes (their products
 * are exact, fp32 accumulation); the second product takes P multiplied by
 * 2^8 and rounded to E4M3 (nearest even), while the row sum uses the
 * unrounded P, so o differs from the exact result by at most
 * 2^-4 sum_j P_ij |v_jd| + 2^-18 sum_j |v_jd| / l_i (P the exact softmax
 * weights, l_i = sum_j exp(s_ij - max_j s_ij)) plus the bf16 rounding of o;
 * lse keeps fp32 accuracy.  One kernel on `stream`; layout, ownership,
 * overlap rules and errors as fa_fwd.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Lq, int Lk, int d, int causal, float scale,
               float q_descale, float k_descale, float v_descale, hipStream_t stream);

/* Workspace bytes fa_bwd needs (0 for B, H or Lq < 1).  Host-only. */
size_t fa_bwd_workspace_size(int B, int H, int Lq);

/* Static English text for a status code (never NULL). */
const char* fa_status_string(int status);

/* FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

/*
 * Tile geometry the library uses for (dtype, d): query rows per workgroup
 * (block_m), keys per K/V tile (block_n) and threads per workgroup.  dtype
 * is 0 for bf16, 1 for fp32, 2 for FP8 E4M3 (fa_fwd_fp8).  (A bf16 d = 64
 * grid of at most two workgroups per compute unit runs the same rows and
 * tiles with twice the threads: two sets of waves that split the key
 * tiles between them.)  Returns FA_OK,
 * or FA_ERR_UNSUPPORTED_D /
 * FA_ERR_ARG for an unknown combination.  Host-only; makes no HIP call.
 */
int fa_tile_config(int dtype, int d, int* block_m, int* block_n,
                   int* threads);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_H */
