// FlashAttention-2 backward kernels for gfx950 (MI355X, CDNA4), bf16.
//
// Gradients of sum(dO * O) for O = softmax(scale Q K^T) V, following "第 08 章:
// Flash Attention——分块注意力" (chuoer47.github.io), section 6 "反向":
//   Delta_i = sum_d dO_id O_id                                  (6.2)
//   P_ij    = exp(scale q_i.k_j - LSE_i)   recomputed from the forward's LSE
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - Delta),            (6.3, 6.4)
//   dK = scale dS^T Q,  dQ = scale dS K
// in three kernels, as the page divides the work: a preprocess pass for
// Delta, a pass with K/V resident that accumulates dK and dV over all query
// blocks, and a pass with Q resident that accumulates dQ over all key
// blocks (the page's two stages; a block's dQ needs every key, its dK/dV
// every query, so neither pass can produce the other's result).  With
// natural-exp logits the page's base-2 factor ln 2 does not appear.
//
// gfx950 mapping:
//  * every product is v_mfma_f32_32x32x16_bf16 on bf16 operands with fp32
//    accumulation; P and dS are rounded to bf16 for their second product;
//  * the resident operands (K and V fragments, or Q and dO fragments) stay
//    in registers as MFMA B operands for the whole loop;
//  * streamed tiles (Q and dO, or K and V) are copied HBM -> LDS without
//    registers (global_load_lds in the dK/dV pass, buffer_load ... lds in
//    the dQ pass), rows in natural order, the 16-byte
//    chunks of row r XOR-swizzled by a rotation f(r) of its low bits; the
//    same tile serves row fragments (ds_read_b128, contraction over d) and
//    transposed fragments (two ds_read_b64_tr_b16, contraction over rows),
//    both free of bank conflicts;
//  * the first product of a block leaves each lane one column of a 32x32
//    accumulator (a key in the dK/dV pass, a query in the dQ pass); element
//    i of lane half h is row 8 (i/4) + 4 h + i % 4.  Converted to bf16 it
//    is directly the B operand of the second product, whose A operand reads
//    tile rows in that same order (16 t + 8 w + 4 h + 0..3 for step t).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline bf16x8 cvt8(const float* x) {
    f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
    return __builtin_convertvector(v, bf16x8);
}
__device__ inline void store4_bf16(uint16_t* dst, f32x4 v) {
    *reinterpret_cast<bf16x4*>(dst) = __builtin_convertvector(v, bf16x4);
}
__device__ inline float bf16_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Wait for this wave's copies (vmcnt(0)) and LDS reads, then barrier; the
// empty asm statements keep the compiler from moving memory accesses
// across it (a workgroup-scope fence would add nothing the waits miss).
__device__ inline void sync_tiles() {
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) expcnt(7) lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---- streamed tile geometry ----------------------------------------------
template <int D, int ROWS, int NW> struct Tile {
    static constexpr int CPR = D / 8;                  // 16-byte chunks per row
    static constexpr int ELEMS = ROWS * D;
    static constexpr int NBLK = ROWS * CPR / 64;       // 1 KB copy blocks
    static constexpr int BPW = NBLK / NW;              // blocks per wave
    static_assert(BPW * NW == NBLK && BPW >= 1, "tile / waves");
    static_assert(ROWS % 32 == 0, "tile rows");
    // chunk swizzle: a rotation of the row's low bits (d >= 128: bits 0-3,
    // d = 64: bits 1-3, where two rows share one 256-byte bank line)
    __device__ static inline int f(int r) {
        return CPR >= 16 ? (((r & 3) << 2) | ((r >> 2) & 3))
                         : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
    }
};

// Per-lane parts of a tile's addresses (element offsets inside the tile).
template <int D, int ROWS, int NW> struct TileLane {
    using T = Tile<D, ROWS, NW>;
    static constexpr int NS = D / 16, NDB = D / 32;
    static constexpr int NTL = NDB < 4 ? NDB : 4;
    unsigned cp_ofs[T::BPW];   // copy: byte offset of this lane's chunk in the tile
    int cp_row[T::BPW];        // copy: its tile row
    int rfo[NS];          // row fragment of step s (add blk * 32 * D)
    int tlane[2][NTL];    // transposed fragment, read w, d-block db & 3

    __device__ void init(int wave, int lane) {
        const int col = lane & 31, h = lane >> 5;
#pragma unroll
        for (int i = 0; i < T::BPW; ++i) {
            const int p = (wave + NW * i) * 64 + lane;
            const int row = p / T::CPR;
            cp_ofs[i] = (unsigned)(row * D + ((p % T::CPR) ^ T::f(row)) * 8) * 2u;
            cp_row[i] = row;
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) rfo[s] = col * D + (((2 * s + h) ^ T::f(col)) * 8);
        const int g16 = lane >> 4, rr = lane & 15;
        const int vh = g16 >> 1, vdh = g16 & 1, vi = rr >> 2, vq = rr & 3;
        const int lrow = 4 * vh + vi;          // row inside the 8-row group
#pragma unroll
        for (int w = 0; w < 2; ++w)
#pragma unroll
            for (int x = 0; x < NTL; ++x) {
                const int lc = 4 * x + 2 * vdh + (vq >> 1);
                // f depends on the row's low 4 bits only: (8 w + lrow)
                tlane[w][x] = lrow * D + (lc ^ T::f(8 * w + lrow)) * 8 + (vq & 1) * 4;
            }
    }
    // copy tile rows [r0, r0 + ROWS) of a [n, D] matrix.  BUF: through a
    // buffer resource that covers only rows below n, so rows >= n read
    // zeros without touching memory; else with global_load_lds from a
    // wave-uniform base plus a 32-bit lane offset, rows >= n reading row
    // n - 1.  Either way the values are finite and the masks give them
    // weight 0.  (The dK/dV pass keeps the second form: its hand-placed
    // schedule measured 3 % slower with the first; the dQ pass takes the
    // first, which needs no per-tile lane arithmetic.)  `wave` must be
    // wave-uniform.
    template <bool BUF>
    __device__ void copy(const uint16_t* base, int r0, int n, uint16_t* dst, int wave) const {
        if constexpr (BUF) {
            const int bytes = max(0, min(ROWS, n - r0)) * D * 2;
#pragma unroll
            for (int i = 0; i < T::BPW; ++i)
                buffer_copy<16>(base + (size_t)r0 * D, bytes, cp_ofs[i],
                                (FA_LDS void*)(dst + (wave + NW * i) * 512));
        } else {
            const char* src = reinterpret_cast<const char*>(base + (size_t)r0 * D);
            const int last = n - 1 - r0;
#pragma unroll
            for (int i = 0; i < T::BPW; ++i) {
                const unsigned o =
                    cp_ofs[i] + (unsigned)((min(cp_row[i], last) - cp_row[i]) * D * 2);
                __builtin_amdgcn_global_load_lds(src + o, (FA_LDS void*)(dst + (wave + NW * i) * 512),
                                                 16, 0, 0);
            }
        }
    }
    __device__ bf16x8 row_frag(const uint16_t* t, int blk, int s) const {
        return *reinterpret_cast<const bf16x8*>(t + blk * 32 * D + rfo[s]);
    }
    // A operand whose contraction runs over rows 16 t + 8 w + 4 h + (0..3)
    // of 32-row block blk, for d columns 32 db + lane % 32
    __device__ bf16x8 tr_frag(const uint16_t* tl, int blk, int t, int db) const {
        s16x4 u[2];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const uint16_t* a = tl + (32 * blk + 16 * t + 8 * w) * D + (db & ~3) * 32 +
                                tlane[w][db & (NTL - 1)];
            u[w] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(FA_LDS void*)a);
        }
        const s16x8 v8 = __builtin_shufflevector(u[0], u[1], 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, v8);
    }
};

// ===========================================================================
// Preprocess: per query row, -Delta_i = -sum_d dO_id O_id and -LSE_i / scale,
// the starting values of the dP and S accumulators (so that the products
// give dP - Delta and S - LSE / scale directly, and P = exp2(c (S - LSE /
// scale)) with c = scale log2(e)).  D/8 lanes per row, one 16-byte chunk
// each, reduced across the lanes of the row.
// ===========================================================================
template <int D>
__global__ __launch_bounds__(256)
void fa_bwd_pre_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                       const float* __restrict__ LSE, float* __restrict__ ndelta,
                       float* __restrict__ nlse, int rows, float scale)
{
    constexpr int TPR = D / 8;            // lanes per row (8 or 16)
    const int row = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
    const int ch = threadIdx.x % TPR;
    float acc = 0.f;
    if (row < rows) {
        const u16x8 o = *reinterpret_cast<const u16x8*>(O + (size_t)row * D + ch * 8);
        const u16x8 g = *reinterpret_cast<const u16x8*>(dO + (size_t)row * D + ch * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += bf16_to_f32(o[e]) * bf16_to_f32(g[e]);
    }
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, TPR);
    if (row < rows && ch == 0) {
        ndelta[row] = -acc;
        nlse[row] = -LSE[row] / scale;
    }
}

// ===========================================================================
// dK, dV: each wave keeps 32 keys' K and V fragments in registers and their
// dK^T, dV^T accumulators (at d = 128 one wave per SIMD, so the
// accumulators can live in AGPRs; at d = 64 everything fits in 256
// registers and two workgroups share a CU, two waves per SIMD, measured
// 9-12 % faster than one); the workgroup streams Q and dO tiles of BQ
// queries.  Per 32-query block: S = Q K^T and dP = dO V^T (lane = key), P
// and dS, then dV^T += dO^T P and dK^T += Q^T dS.
//
// With one wave per SIMD (d = 128) nothing else hides a wave's LDS
// latency, so each block is software-pipelined: its S and dP products run
// on row fragments read during the previous block's products, while its
// transposed fragments and statistics are read; its dV and dK products run
// while the next block's row fragments are read.  The next tile's row fragments are read
// before its first block, so the tile barrier sits just before the second
// block's dV/dK products, and the copy it guards goes into the tile just
// finished (two buffers suffice).
// ===========================================================================
constexpr int kKVWaves = 4;                 // waves per workgroup, 32 keys each
constexpr int kKVKeys = 32 * kKVWaves;      // keys per workgroup
constexpr int kKVBQ = 64;                   // queries per streamed tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kKVWaves)
__attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1, D == 64 ? 2 : 1)))
void fa_bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                        const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                        const float* __restrict__ nlse, const float* __restrict__ ndelta,
                        uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                        int BH, int Lq, int Lk, int nkb, float c, float scale)
{
    constexpr int NW = kKVWaves, BQ = kKVBQ;
    using L = TileLane<D, BQ, NW>;
    constexpr int NS = L::NS, NDB = L::NDB;
    __shared__ __attribute__((aligned(1024))) uint16_t Qb0[L::T::ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t Qb1[L::T::ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t Ob0[L::T::ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t Ob1[L::T::ELEMS];
    // the tile's -LSE / scale and -Delta values, copied with it (4 bytes per
    // lane)
    static_assert(BQ == 64, "one 64-lane copy per vector, two 32-query blocks per tile");
    __shared__ __attribute__((aligned(256))) float Sb0[2 * BQ];
    __shared__ __attribute__((aligned(256))) float Sb1[2 * BQ];

    // the wave index is uniform: keeping it in a scalar register makes every
    // per-wave condition below a scalar branch
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, h = lane >> 5;

    // key blocks of a head on one XCD; causal: the first key blocks (seen by
    // the most queries) start first
    int bh, kb;
    xcd_decode(blockIdx.x, BH, bh, kb);
    const int key0 = kb * kKVKeys;
    const int kw0 = key0 + wave * 32;          // this wave's keys kw0 .. kw0 + 31
    const int key = kw0 + col;                 // this lane's key (accumulator column)
    const uint16_t* Qh = Q + (size_t)bh * Lq * D;
    const uint16_t* Oh = dO + (size_t)bh * Lq * D;
    const float* nlseh = nlse + (size_t)bh * Lq;
    const float* ndelh = ndelta + (size_t)bh * Lq;

    // resident B operands: K^T and V^T fragments (lane = key, 8 d values)
    bf16x8 kf[NS], vf[NS];
    {
        const uint16_t* Kr = K + ((size_t)bh * Lk + key) * D;
        const uint16_t* Vr = V + ((size_t)bh * Lk + key) * D;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            kf[s] = key < Lk ? *reinterpret_cast<const bf16x8*>(Kr + 16 * s + 8 * h) : bf16x8{};
            vf[s] = key < Lk ? *reinterpret_cast<const bf16x8*>(Vr + 16 * s + 8 * h) : bf16x8{};
        }
    }
    f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) { dkt[db] = f32x16{}; dvt[db] = f32x16{}; }

    L ln;
    ln.init(wave, lane);
    // query tiles that can see a key of this block: causal, q >= key0.  Every
    // wave runs every block of these tiles (a block wholly before a wave's
    // keys, or past Lq, is masked to zero), so the waves stay in step.
    const int jt0 = CAUSAL ? key0 / BQ : 0;
    const int jt1 = (Lq + BQ - 1) / BQ;

    // copy query tile jt (Q, dO rows and their statistics); wave 0 copies
    // the -LSE / scale values, wave 1 the -Delta values
    auto copy_tile = [&](int jt, uint16_t* Qd, uint16_t* Od, float* Sd) {
        ln.template copy<false>(Qh, jt * BQ, Lq, Qd, wave);
        ln.template copy<false>(Oh, jt * BQ, Lq, Od, wave);
        if (wave < 2) {
            const float* src = (wave == 0 ? nlseh : ndelh) + min(jt * BQ + lane, Lq - 1);
            __builtin_amdgcn_global_load_lds(src, (FA_LDS void*)(Sd + wave * BQ), 4, 0, 0);
        }
    };

    // carried from one block to the next: the next block's Q row fragments
    // (contraction over d) and the start of its S accumulator (-LSE / scale
    // of its queries: element i is query 8 (i/4) + 4 h + i % 4 of the block,
    // four runs of four consecutive values in the tile's statistics)
    bf16x8 rq[NS];
    f32x16 s_init;
    auto read_stats = [&](const float* St, int qb, f32x16& dst) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(St + 32 * qb + 8 * g + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[4 * g + e] = a[e];
        }
    };

    // Block qb (0 or 1) of tile jt, held in (Qc, Oc, Sc); (Qn, On, Sn) hold
    // the next tile.  Each product below is one step followed by a
    // scheduling fence, with the reads (and exponentials) issued beside it
    // placed by hand.  Block 1 ends the tile: halfway through its dV/dK
    // products it waits at the barrier (tile jt + 1 has landed and every
    // wave is done with tile jt) and starts the copy of tile jt + 2 into
    // (Qc, Oc, Sc).
    auto block = [&](int jt, auto qbc, uint16_t* Qc, uint16_t* Oc, float* Sc,
                     const uint16_t* Qn, const uint16_t* On, const float* Sn) {
        constexpr int qb = decltype(qbc)::value;
        const int q0 = jt * BQ + 32 * qb;
        // X: S = Q K^T (from the carried fragments), then dP = dO V^T; the
        // dO row fragments are read two steps ahead, then the t = 0 halves
        // of the transposed fragments; the exponentials start two steps
        // after S is complete.  s_acc = S - LSE / scale, dp_acc = dP - Delta.
        f32x16 s_acc = s_init, dp_acc;
        read_stats(Sc + BQ, qb, dp_acc);
        bf16x8 ro[NS], to0[NDB], tq0[NDB];
        ro[0] = ln.row_frag(Oc, qb, 0);
        ro[1] = ln.row_frag(Oc, qb, 1);
        float p[16];
#pragma unroll
        for (int m = 0; m < 2 * NS; ++m) {
            if (m < NS) s_acc = mfma(rq[m], kf[m], s_acc);
            else dp_acc = mfma(ro[m - NS], vf[m - NS], dp_acc);
            if (m + 2 < NS) {
                ro[m + 2] = ln.row_frag(Oc, qb, m + 2);
            } else if (m + 2 - NS < 2 * NDB) {
                const int f = m + 2 - NS;
                if (f & 1) tq0[f >> 1] = ln.tr_frag(Qc, qb, 0, f >> 1);
                else to0[f >> 1] = ln.tr_frag(Oc, qb, 0, f >> 1);
            }
            if (m >= NS + 2) {
                constexpr int kSteps = NS - 2;
                const int e0 = (m - NS - 2) * 16 / kSteps, e1 = (m - NS - 1) * 16 / kSteps;
#pragma unroll
                for (int e = e0; e < e1; ++e) p[e] = __builtin_amdgcn_exp2f(s_acc[e] * c);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // Masks, on the blocks that need them (a wave-uniform test).  A key
        // past Lk needs none: its lane's column of dK, dV is never stored and
        // no product mixes columns.  Element i holds query q0 + off + 4h with
        // off = 8 (i/4) + i%4; it is visible iff lo <= off < hi.
        if ((q0 + 31 >= Lq) || (CAUSAL && q0 < kw0 + 31)) {
            const int lo = CAUSAL ? key - q0 - 4 * h : 0;   // query >= key
            const int hi = Lq - q0 - 4 * h;                  // query < Lq
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int off = 8 * (i / 4) + (i % 4);
                p[i] = (off < lo || off >= hi) ? 0.f : p[i];
            }
        }
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) ds[i] = p[i] * dp_acc[i];
        const bf16x8 pf[2] = {cvt8(p), cvt8(p + 8)};
        const bf16x8 sf[2] = {cvt8(ds), cvt8(ds + 8)};
        // Y: dV^T += dO^T P, dK^T += Q^T dS, the t = 0 half then the t = 1
        // half; the t = 1 transposed fragments are read during the first
        // half, the next block's Q row fragments and S start during the
        // second.
        bf16x8 to1[NDB], tq1[NDB];
        const uint16_t* Qx = qb == 1 ? Qn : Qc;
        const float* Sx = qb == 1 ? Sn : Sc;
        constexpr int kY = 4 * NDB, kHalf = 2 * NDB;
#pragma unroll
        for (int m = 0; m < kY; ++m) {
            const int t = m / kHalf, db = (m % kHalf) >> 1;
            if ((m & 1) == 0) dvt[db] = mfma(t ? to1[db] : to0[db], pf[t], dvt[db]);
            else dkt[db] = mfma(t ? tq1[db] : tq0[db], sf[t], dkt[db]);
            if (m < kHalf) {
                if (m & 1) tq1[m >> 1] = ln.tr_frag(Qc, qb, 1, m >> 1);
                else to1[m >> 1] = ln.tr_frag(Oc, qb, 1, m >> 1);
            } else {
                // NS fragments and the 4 statistics reads over kHalf steps
                const int r0 = (m - kHalf) * (NS + 4) / kHalf, r1 = (m - kHalf + 1) * (NS + 4) / kHalf;
#pragma unroll
                for (int r = r0; r < r1; ++r) {
                    if (r < NS) rq[r] = ln.row_frag(Qx, qb ^ 1, r);
                    else {
                        const f32x4 a = *reinterpret_cast<const f32x4*>(
                            Sx + 32 * (qb ^ 1) + 8 * (r - NS) + 4 * h);
#pragma unroll
                        for (int e = 0; e < 4; ++e) s_init[4 * (r - NS) + e] = a[e];
                    }
                }
            }
            if (qb == 1 && m == kHalf - 1) {
                sync_tiles();
                if (jt + 2 < jt1) copy_tile(jt + 2, Qc, Oc, Sc);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (jt0 < jt1) {
        copy_tile(jt0, Qb0, Ob0, Sb0);
        if (jt0 + 1 < jt1) copy_tile(jt0 + 1, Qb1, Ob1, Sb1);
        sync_tiles();
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) rq[s2] = ln.row_frag(Qb0, 0, s2);
        read_stats(Sb0, 0, s_init);
        using B0 = std::integral_constant<int, 0>;
        using B1 = std::integral_constant<int, 1>;
        // tiles in pairs (even tiles in buffer 0, odd in buffer 1), then a
        // last odd one out: a loop body without a join keeps the carried
        // registers in place
        int jt = jt0;
        for (; jt + 1 < jt1; jt += 2) {
            block(jt, B0{}, Qb0, Ob0, Sb0, Qb1, Ob1, Sb1);
            block(jt, B1{}, Qb0, Ob0, Sb0, Qb1, Ob1, Sb1);
            block(jt + 1, B0{}, Qb1, Ob1, Sb1, Qb0, Ob0, Sb0);
            block(jt + 1, B1{}, Qb1, Ob1, Sb1, Qb0, Ob0, Sb0);
        }
        if (jt < jt1) {
            block(jt, B0{}, Qb0, Ob0, Sb0, Qb1, Ob1, Sb1);
            block(jt, B1{}, Qb0, Ob0, Sb0, Qb1, Ob1, Sb1);
        }
    }
    // dK = scale dS^T Q, dV = P^T dO; lane = key, rows = d
    if (key < Lk) {
        uint16_t* dKr = dK + ((size_t)bh * Lk + key) * D;
        uint16_t* dVr = dV + ((size_t)bh * Lk + key) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dc = db * 32 + 8 * g + 4 * h;
                f32x4 k4 = {dkt[db][4 * g], dkt[db][4 * g + 1], dkt[db][4 * g + 2], dkt[db][4 * g + 3]};
                f32x4 v4 = {dvt[db][4 * g], dvt[db][4 * g + 1], dvt[db][4 * g + 2], dvt[db][4 * g + 3]};
                store4_bf16(dKr + dc, k4 * scale);
                store4_bf16(dVr + dc, v4);
            }
    }
}

// ===========================================================================
// dQ: each wave keeps 32 queries' Q and dO fragments in registers and their
// dQ^T accumulator; the workgroup streams K and V tiles of BK keys, as in
// the forward.  Per 32-key block: S^T = K Q^T and dP^T = V dO^T (lane =
// query), P^T and dS^T, then dQ^T += K^T dS^T.
// ===========================================================================
// Waves per workgroup (32 queries each) and per SIMD: at d = 128 eight
// waves, two per SIMD (246 registers); at d = 64 (149 registers) four, with
// three workgroups per CU (three waves per SIMD), 2.5-4 % faster on the
// whole d = 64 backward than eight waves at two per SIMD.
template <int D> struct QCfg {
    static constexpr int W = D == 64 ? 4 : 8, ROWS = 32 * W, WPE = D == 64 ? 3 : 2;
};
constexpr int kQBK = 64;                    // keys per streamed tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * QCfg<D>::W)
__attribute__((amdgpu_waves_per_eu(QCfg<D>::WPE, QCfg<D>::WPE)))
void fa_bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                      const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                      const float* __restrict__ nlse, const float* __restrict__ ndelta,
                      uint16_t* __restrict__ dQ, int BH, int Lq, int Lk, int nqb, float c,
                      float scale)
{
    constexpr int NW = QCfg<D>::W, BK = kQBK, NKB = BK / 32, kQRows = QCfg<D>::ROWS;
    using L = TileLane<D, BK, NW>;
    constexpr int NS = L::NS, NDB = L::NDB;
    __shared__ __attribute__((aligned(1024))) uint16_t Kb0[L::T::ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t Kb1[L::T::ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t Vb0[L::T::ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t Vb1[L::T::ELEMS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, h = lane >> 5;

    int bh, lvl;
    xcd_decode(blockIdx.x, BH, bh, lvl);
    const int qb = CAUSAL ? (nqb - 1 - lvl) : lvl;
    const int q0 = qb * kQRows;
    const int q0w = q0 + wave * 32;
    const int qi = q0w + col;                  // this lane's query (accumulator column)
    const uint16_t* Kh = K + (size_t)bh * Lk * D;
    const uint16_t* Vh = V + (size_t)bh * Lk * D;

    bf16x8 qf[NS], of[NS];
    {
        const uint16_t* Qr = Q + ((size_t)bh * Lq + qi) * D;
        const uint16_t* Or = dO + ((size_t)bh * Lq + qi) * D;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            qf[s] = qi < Lq ? *reinterpret_cast<const bf16x8*>(Qr + 16 * s + 8 * h) : bf16x8{};
            of[s] = qi < Lq ? *reinterpret_cast<const bf16x8*>(Or + 16 * s + 8 * h) : bf16x8{};
        }
    }
    // this lane's query: c (-LSE / scale) = -LSE log2(e), and -Delta
    const float lqc = qi < Lq ? nlse[(size_t)bh * Lq + qi] * c : 0.f;
    const float nd = qi < Lq ? ndelta[(size_t)bh * Lq + qi] : 0.f;
    f32x16 dqt[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dqt[db] = f32x16{};

    L ln;
    ln.init(wave, lane);
    const int kv_end = CAUSAL ? min(Lk, q0 + kQRows) : Lk;
    const int nt = (kv_end + BK - 1) / BK;

    auto step = [&](int j, const uint16_t* Kc, const uint16_t* Vc, uint16_t* Kn, uint16_t* Vn) {
        if (j + 1 < nt) {
            ln.template copy<true>(Kh, (j + 1) * BK, Lk, Kn, wave);
            ln.template copy<true>(Vh, (j + 1) * BK, Lk, Vn, wave);
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const int k0 = j * BK + 32 * kb;
            if ((CAUSAL && k0 > q0w + 31) || k0 >= Lk) continue;
            f32x16 s_acc = f32x16{}, dp_acc = f32x16{};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                s_acc = mfma(ln.row_frag(Kc, kb, s), qf[s], s_acc);
                dp_acc = mfma(ln.row_frag(Vc, kb, s), of[s], dp_acc);
            }
            float p[16], ds[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_acc[i], c, lqc));
            // Masks, on the blocks that need them (a wave-uniform test).  A
            // query past Lq needs none: its lane's column of dQ is never
            // stored.  Element i holds key k0 + off + 4h with off = 8 (i/4) +
            // i%4; it is visible iff off < hi.
            if ((k0 + 31 >= Lk) || (CAUSAL && k0 + 31 > q0w)) {
                const int hi = CAUSAL ? min(Lk, qi + 1) - k0 - 4 * h : Lk - k0 - 4 * h;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int off = 8 * (i / 4) + (i % 4);
                    p[i] = off < hi ? p[i] : 0.f;
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) ds[i] = p[i] * (dp_acc[i] + nd);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const bf16x8 sf = cvt8(ds + 8 * t);
#pragma unroll
                for (int db = 0; db < NDB; ++db) dqt[db] = mfma(ln.tr_frag(Kc, kb, t, db), sf, dqt[db]);
            }
        }
        sync_tiles();
    };
    ln.template copy<true>(Kh, 0, Lk, Kb0, wave);
    ln.template copy<true>(Vh, 0, Lk, Vb0, wave);
    sync_tiles();
    for (int j = 0; j < nt; j += 2) {
        step(j, Kb0, Vb0, Kb1, Vb1);
        if (j + 1 < nt) step(j + 1, Kb1, Vb1, Kb0, Vb0);
    }
    // dQ = scale dS K; lane = query, rows = d
    if (qi < Lq) {
        uint16_t* dQr = dQ + ((size_t)bh * Lq + qi) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 v4 = {dqt[db][4 * g], dqt[db][4 * g + 1], dqt[db][4 * g + 2], dqt[db][4 * g + 3]};
                store4_bf16(dQr + db * 32 + 8 * g + 4 * h, v4 * scale);
            }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_d(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        int B, int H, int Lq, int Lk, float scale, float* ndelta, float* nlse,
                        hipStream_t stream)
{
    const int BH = B * H;
    const int rows = BH * Lq;
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((fa_bwd_pre_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256),
                       0, stream, static_cast<const uint16_t*>(o),
                       static_cast<const uint16_t*>(dout), lse, ndelta, nlse, rows, scale);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const float c = scale * kLog2e;
    const int nkb = (Lk + kKVKeys - 1) / kKVKeys;
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)(nkb * BH)),
                       dim3(64 * kKVWaves), 0, stream, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                       static_cast<const uint16_t*>(dout), nlse, ndelta,
                       static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), BH, Lq, Lk, nkb,
                       c, scale);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int nqb = (Lq + QCfg<D>::ROWS - 1) / QCfg<D>::ROWS;
    hipLaunchKernelGGL((fa_bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)(nqb * BH)),
                       dim3(64 * QCfg<D>::W), 0, stream, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                       static_cast<const uint16_t*>(dout), nlse, ndelta,
                       static_cast<uint16_t*>(dq), BH, Lq, Lk, nqb, c, scale);
    return hipGetLastError();
}

}  // namespace

bool bwd_supported(int d) { return d == 64 || d == 128; }

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      int B, int H, int Lq, int Lk, int d, bool causal, float scale,
                      float* ndelta, float* nlse, hipStream_t stream)
{
    switch (d) {
    case 64:
        return causal ? launch_bwd_d<64, true>(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, scale, ndelta, nlse, stream)
                      : launch_bwd_d<64, false>(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, scale, ndelta, nlse, stream);
    case 128:
        return causal ? launch_bwd_d<128, true>(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, scale, ndelta, nlse, stream)
                      : launch_bwd_d<128, false>(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, scale, ndelta, nlse, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace fa
