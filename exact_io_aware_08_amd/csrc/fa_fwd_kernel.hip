// FlashAttention-2 forward kernel for gfx950 (MI355X, CDNA4).
//
// Computes O = softmax(Q K^T * scale) V and LSE = ln(sum_j exp(s_ij)) for
// each (batch, head, query row), streaming K/V tiles through LDS with the
// online-softmax update so the score matrix never leaves the chip.
//
// Method (the pages' schedule, re-derived for CDNA4):
//  * one workgroup per (query block, batch*head) with Q resident on chip
//    and K/V streamed in tiles ("從零開始用自定義 Triton 內核編寫
//    FlashAttention-2" (digipub.cc), sections "程序網格和並行化策略" and
//    "K 和 V 塊的流式循環");
//  * per tile: S = Q K^T * scale, running max m, P = exp(S - m),
//    alpha = exp(m_old - m), l = l*alpha + rowsum P, O = O*alpha + P V
//    ("第 08 章: Flash Attention——分块注意力" (chuoer47.github.io),
//    section 2 "在线 softmax", steps 1-7), in base 2 with scale * log2(e)
//    folded in (same page, section 1 "tl.exp2");
//  * O / l once after the last tile and LSE = m + log l (same page,
//    sections 2 and 3);
//  * causal: tiles right of the diagonal are never visited, tiles that
//    straddle it are masked element-wise (same page, section 4).
//
// Two kernels share that method.  fa_fwd_direct_kernel serves bf16: K and V
// tiles go from HBM straight into LDS (buffer_load ... lds, no registers), and
// the V^T operand is read with the transposing ds_read_b64_tr_b16.
// fa_fwd_kernel serves fp32: tiles are staged through registers and V is
// written to LDS transposed.
//
// gfx950 mapping (not the pages' Triton tiling):
//  * each wave owns 32*NBQ query rows; the NW waves of a workgroup share
//    one K/V tile in LDS;
//  * both products use v_mfma_f32_32x32x16_bf16 (fp32: 32x32x2f32) in the
//    transposed form S^T = K Q^T and O^T = V^T P^T.  In that form every
//    lane's accumulator column is one query, so the row max/sum are
//    in-lane plus one exchange between the two 32-lane halves, alpha
//    scales a lane's own O values, and the S^T accumulator registers are
//    already the P^T operand of the next MFMA (no LDS round trip for P);
//  * K rows are stored in LDS in a permuted order so that lane half h's
//    accumulator rows are the 16 consecutive keys 16h..16h+15 of each
//    32-key block, so every P^T operand is 8 consecutive keys;
//  * K/V tiles are double-buffered: the copy of tile j+1 runs while tile j
//    is computed;
//  * workgroup ids are remapped so that all query blocks of a head run on
//    one XCD (its L2 serves the K/V re-reads) and, for causal, the
//    heaviest query blocks start first.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {


template <class T, int N> struct VecOf {
    typedef T type __attribute__((ext_vector_type(N)));
};

constexpr float kLazy = 8.0f;   // bf16 direct kernel: reference-max slack (log2 units)

// ---- element traits -------------------------------------------------------

struct BF16 {
    using T = uint16_t;   // storage: raw bfloat16 bits
    using Frag = bf16x8;  // one MFMA A/B operand per lane
    static constexpr int KPL = 8;   // contraction elements per lane per MFMA
    static constexpr int VEC = 8;   // elements per 16-byte global chunk
    __device__ static inline f32x16 mfma(Frag a, Frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline Frag load(const T* p) {
        return *reinterpret_cast<const bf16x8*>(p);
    }
    // fp32 probabilities -> operand (round to nearest even)
    __device__ static inline Frag from_f32(const float* x) {
        f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
        return __builtin_convertvector(v, bf16x8);
    }
    __device__ static inline void store4(T* dst, f32x4 v) {
        bf16x4 b = __builtin_convertvector(v, bf16x4);
        *reinterpret_cast<bf16x4*>(dst) = b;
    }
};

struct F32 {
    using T = float;
    using Frag = float;
    static constexpr int KPL = 1;
    static constexpr int VEC = 4;
    __device__ static inline f32x16 mfma(Frag a, Frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    __device__ static inline Frag load(const T* p) { return *p; }
    __device__ static inline Frag from_f32(const float* x) { return x[0]; }
    __device__ static inline void store4(T* dst, f32x4 v) {
        *reinterpret_cast<f32x4*>(dst) = v;
    }
};

// ---- tile table of the register-staged kernel (fp32) ---------------------
// NBQ: 32-query blocks per wave; BN: keys per K/V tile; NW: waves per
// workgroup; WPE: waves per SIMD the register budget is sized for.
template <int NBQ_, int BN_, int NW_, int WPE_> struct CfgT {
    static constexpr int NBQ = NBQ_, BN = BN_, NW = NW_, WPE = WPE_;
};
template <class E, int D> struct Cfg;
template <int D> struct Cfg<F32, D> : CfgT<1, 32, 4, 1> {};

template <class E, int D> struct Geom {
    using T = typename E::T;
    static constexpr int NBQ = Cfg<E, D>::NBQ;   // 32-query blocks per wave
    static constexpr int BN = Cfg<E, D>::BN;     // keys per tile
    static constexpr int NW = Cfg<E, D>::NW;     // waves per workgroup
    static constexpr int WPE = Cfg<E, D>::WPE;   // waves per SIMD (target)
    static constexpr int NT = 64 * NW;           // threads per workgroup
    static constexpr int BM = NW * 32 * NBQ;     // query rows per workgroup
    static constexpr int KPL = E::KPL;
    static constexpr int KSTEP = 2 * KPL;        // contraction per MFMA
    static constexpr int NS = D / KSTEP;         // MFMAs along d for S
    static constexpr int NMB = BN / 32;          // 32-key blocks per tile
    static constexpr int NDB = D / 32;           // 32-wide d blocks of O
    static constexpr int NPV = 32 / KSTEP;       // PV MFMAs per key block
    static constexpr int VEC = E::VEC;
    // LDS rows padded by one 16-byte chunk
    static constexpr int KS = D + VEC;           // K row stride (elements)
    static constexpr int VS = BN + VEC;          // V^T row stride (elements)
    static constexpr int K_ELEMS = BN * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int STAGE_ELEMS = K_ELEMS + V_ELEMS;
    static constexpr int LDS_BYTES = 2 * STAGE_ELEMS * (int)sizeof(T);
    // cooperative loads: 16-byte chunks per thread per tensor per tile
    static constexpr int CH = BN * D / VEC / NT;
    static constexpr int NKG = BN / CH;          // V key groups (CH keys each)
    static_assert(CH >= 1 && CH * NT * VEC == BN * D, "tile/threads");
    static_assert(CH * (int)sizeof(T) >= 4, "V^T segments of at least 4 bytes");
    static_assert(NKG * (D / VEC) == NT, "V transpose mapping");
    static_assert(D % KSTEP == 0 && BN % 32 == 0 && D % 32 == 0, "shape");
    static_assert(LDS_BYTES * WPE * 4 / NW <= 160 * 1024, "LDS budget");
};


// Slot of key k (0..31) inside a 32-row block of the K tile in LDS.  MFMA
// A-operand row r is read by lane r; its accumulator row r sits in lane
// half (r>>2)&1 at index 4*(r>>3)+(r&3).  Storing key
// 16*((r>>2)&1) + 4*(r>>3) + (r&3) in slot r makes accumulator index i of
// lane half h hold key 16*h + i.  This is the inverse of that map.
__device__ inline int k_slot(int k) {
    return 8 * ((k >> 2) & 3) + 4 * (k >> 4) + (k & 3);
}

template <class E, int D, bool CAUSAL>
__global__ __launch_bounds__((Geom<E, D>::NT))
__attribute__((amdgpu_waves_per_eu(Geom<E, D>::WPE, Geom<E, D>::WPE)))
void fa_fwd_kernel(const typename E::T* __restrict__ Q,
                   const typename E::T* __restrict__ K,
                   const typename E::T* __restrict__ V,
                   typename E::T* __restrict__ O, float* __restrict__ LSE,
                   int BH, int Lq, int Lk, int nqb, float c)
{
    using G = Geom<E, D>;
    using T = typename G::T;
    using Frag = typename E::Frag;
    constexpr int NBQ = G::NBQ, BN = G::BN, BM = G::BM, KPL = G::KPL;
    constexpr int KSTEP = G::KSTEP, NS = G::NS, NMB = G::NMB, NDB = G::NDB;
    constexpr int NPV = G::NPV, VEC = G::VEC, KS = G::KS, VS = G::VS;
    constexpr int CH = G::CH, NKG = G::NKG, NT = G::NT;

    __shared__ __attribute__((aligned(16))) T smem[2 * G::STAGE_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;   // accumulator column = query
    const int half = lane >> 5;  // lane half

    // ---- work decode: XCD-grouped heads, heaviest causal blocks first ----
    int bh, lvl;
    xcd_decode(blockIdx.x, BH, bh, lvl);
    const int qb = CAUSAL ? (nqb - 1 - lvl) : lvl;
    const int q0 = qb * BM;
    const int q0w = q0 + wave * 32 * NBQ;          // first row of this wave
    const int qlast_w = q0w + 32 * NBQ - 1;        // last row of this wave

    const T* Qh = Q + (size_t)bh * Lq * D;
    const T* Kh = K + (size_t)bh * Lk * D;
    const T* Vh = V + (size_t)bh * Lk * D;

    // ---- Q fragments: resident for the whole key loop --------------------
    Frag qf[NBQ][NS];
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
        const int row = q0w + nb * 32 + col;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (row < Lq) {
                qf[nb][s] = E::load(Qh + (size_t)row * D + s * KSTEP + half * KPL);
            } else {
                qf[nb][s] = Frag{};
            }
        }
    }

    f32x16 oacc[NDB][NBQ];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) oacc[db][nb] = f32x16{};
    float m_run[NBQ], l_run[NBQ];
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
        m_run[nb] = -__builtin_inff();
        l_run[nb] = 0.f;
    }

    const int kv_end = CAUSAL ? min(Lk, q0 + BM) : Lk;
    const int nt = (kv_end + BN - 1) / BN;

    // ---- cooperative tile movement ---------------------------------------
    u32x4 kreg[CH], vreg[CH];
    auto load_tile = [&](int j) {
        const int kv0 = j * BN;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int cidx = tid + NT * i;
            const int row = cidx / (D / VEC);
            const int cc = cidx % (D / VEC);
            if (kv0 + row < Lk)
                kreg[i] = *reinterpret_cast<const u32x4*>(Kh + (size_t)(kv0 + row) * D + cc * VEC);
            else
                kreg[i] = u32x4{};
        }
        const int kg = tid % NKG, dc = tid / NKG;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int row = kg * CH + i;
            if (kv0 + row < Lk)
                vreg[i] = *reinterpret_cast<const u32x4*>(Vh + (size_t)(kv0 + row) * D + dc * VEC);
            else
                vreg[i] = u32x4{};
        }
    };
    auto store_tile = [&](int buf) {
        T* Ks = smem + buf * G::STAGE_ELEMS;
        T* Vt = Ks + G::K_ELEMS;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int cidx = tid + NT * i;
            const int row = cidx / (D / VEC);
            const int cc = cidx % (D / VEC);
            const int slot = (row & ~31) | k_slot(row & 31);
            *reinterpret_cast<u32x4*>(Ks + slot * KS + cc * VEC) = kreg[i];
        }
        // V^T: thread holds CH consecutive keys x VEC consecutive d; write
        // one row segment of CH keys per d (at most 16 bytes per store).
        const int kg = tid % NKG, dc = tid / NKG;
        using Chunk = typename VecOf<T, VEC>::type;
        constexpr int SEG = (CH * (int)sizeof(T) >= 16) ? VEC : CH;
        using Seg = typename VecOf<T, SEG>::type;
        Chunk rows[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) rows[i] = __builtin_bit_cast(Chunk, vreg[i]);
#pragma unroll
        for (int dd = 0; dd < VEC; ++dd) {
            T* dst = Vt + (dc * VEC + dd) * VS + kg * CH;
#pragma unroll
            for (int p0 = 0; p0 < CH; p0 += SEG) {
                Seg sv;
#pragma unroll
                for (int e = 0; e < SEG; ++e) sv[e] = rows[p0 + e][dd];
                *reinterpret_cast<Seg*>(dst + p0) = sv;
            }
        }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int j = 0; j < nt; ++j) {
        const int buf = j & 1;
        const int kv0 = j * BN;
        if (j + 1 < nt) load_tile(j + 1);

        // waves whose rows all precede this tile's first key skip it
        const bool active = !CAUSAL || kv0 <= qlast_w;
        if (active) {
            const T* Ks = smem + buf * G::STAGE_ELEMS;
            const T* Vt = Ks + G::K_ELEMS;

            // S^T = K Q^T: rows = keys (permuted slots), columns = queries
            f32x16 sacc[NMB][NBQ];
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NBQ; ++nb) sacc[mb][nb] = f32x16{};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
                    const Frag a = E::load(Ks + (mb * 32 + col) * KS + s * KSTEP + half * KPL);
#pragma unroll
                    for (int nb = 0; nb < NBQ; ++nb)
                        sacc[mb][nb] = E::mfma(a, qf[nb][s], sacc[mb][nb]);
                }
            }

            // mask: keys beyond Lk, and keys after the query (causal)
            const bool need_mask = (kv0 + BN > Lk) || (CAUSAL && kv0 + BN - 1 > q0w);
            if (need_mask) {
#pragma unroll
                for (int nb = 0; nb < NBQ; ++nb) {
                    const int qi = q0w + nb * 32 + col;
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int kj = kv0 + mb * 32 + 16 * half + i;
                            const bool dead = (kj >= Lk) || (CAUSAL && kj > qi);
                            if (dead) sacc[mb][nb][i] = -__builtin_inff();
                        }
                }
            }

            // online softmax (base 2), per query column
            Frag pf[NMB][NPV][NBQ];
#pragma unroll
            for (int nb = 0; nb < NBQ; ++nb) {
                float mx = -__builtin_inff();
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[mb][nb][i]);
                mx = half_max(mx);
                const float m_new = fmaxf(m_run[nb], mx * c);
                // a row with no visible key yet keeps alpha = 1, P = 0
                const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(m_run[nb] - m_use);
                float rs = 0.f;
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
                    float p[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mb][nb][i], c, -m_use));
                        rs += p[i];
                    }
#pragma unroll
                    for (int t = 0; t < NPV; ++t) pf[mb][t][nb] = E::from_f32(p + t * KPL);
                }
                l_run[nb] = l_run[nb] * alpha + rs;
                m_run[nb] = m_new;
                // alpha == 1 exactly when the row max did not move; skip the
                // multiply when that holds for every row of the wave
                if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db) oacc[db][nb] *= alpha;
                }
            }

            // O^T += V^T P^T: rows = d, columns = queries
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int t = 0; t < NPV; ++t)
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const Frag a = E::load(Vt + (db * 32 + col) * VS + mb * 32 + 16 * half + t * KPL);
#pragma unroll
                        for (int nb = 0; nb < NBQ; ++nb)
                            oacc[db][nb] = E::mfma(a, pf[mb][t][nb], oacc[db][nb]);
                    }
        }

        if (j + 1 < nt) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O / l, LSE = ln2 * (m + log2 l) -------------------------
    T* Oh = O + (size_t)bh * Lq * D;
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
        const float lt = half_sum(l_run[nb]);
        const float inv = 1.0f / lt;
        const int row = q0w + nb * 32 + col;
        if (row < Lq) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 v4 = {oacc[db][nb][4 * g + 0], oacc[db][nb][4 * g + 1],
                                oacc[db][nb][4 * g + 2], oacc[db][nb][4 * g + 3]};
                    v4 *= inv;
                    E::store4(Oh + (size_t)row * D + db * 32 + 8 * g + 4 * half, v4);
                }
            if (half == 0)
                LSE[(size_t)bh * Lq + row] = (m_run[nb] + __builtin_amdgcn_logf(lt)) * kLn2;
        }
    }
}

// ===========================================================================
// bf16 kernel with direct global->LDS tile loads (gfx950).
//
// K and V tiles are copied from HBM straight into LDS with
// buffer_load_dwordx4 ... lds (lane L of a wave instruction lands at byte
// 16*L of a 1 KB LDS block), so no registers or VALU instructions stage
// them; with the buffer form the compiler also counts the LDS fragment
// reads precisely (lgkmcnt(n) instead of lgkmcnt(0)), so they overlap the
// MFMAs.
// Both tiles keep their natural row layout [key][d] with the 16-byte chunks
// of each row XOR-swizzled by a function of the row index (a different one
// for K and V, chosen so that both fragment reads are free of LDS bank
// conflicts); each lane picks the global chunk that belongs at its LDS
// position.  The
// V^T operand of the PV product is read with ds_read_b64_tr_b16: in each
// 16-lane group, lane l receives element l%4 of the 8-byte rows supplied by
// lanes (l%16)/4 + 4i (i = 0..3), so rows "4 keys x 4 d-quads" give every
// lane 4 keys of its own d column; two such reads form one operand.
// Tile rows at or beyond Lk arrive as zeros from the buffer's range check
// (finite data that the mask turns into weight 0).  The key loop is
// unrolled by two, so each access names its buffer at a constant offset.
// ===========================================================================

// keys per tile, waves per workgroup, waves per SIMD the registers are
// sized for, 32-query blocks per wave (each K or V fragment read from LDS
// feeds that many MFMAs).  d = 64 runs 64-key tiles and 4-wave workgroups
// (128 query rows) at four waves per SIMD (126 VGPRs, 32 KB of LDS each):
// 3.5-6 % faster than 128-key tiles at two waves per SIMD on L = 4096 and
// 16384.  A d = 64 grid of at most two workgroups per CU instead runs two
// key halves per workgroup (8 waves on the same 128 rows, see
// launch_direct).
// d = 256 takes 32-key tiles so that two waves per SIMD fit the register
// file (O alone is 128 registers): 8 waves of 32 rows, one softmax beside
// the other wave's MFMAs, 16 % faster than 64-key tiles at one wave per
// SIMD on the B=1 H=8 Lq=8000 Lk=8192 workload.
//
// ONE: the four tile buffers live in one LDS object (each buffer address is
// then the object's base plus a constant, which spares address registers:
// the d = 256 kernel needs that to stay within 256 VGPRs, 9 % faster) or in
// four (the compiler can then tell a buffer that a tile copy is filling
// from the one being read, and does not wait for the copy before reading
// V; with one object it does).
template <int BN_, int NW_, int WPE_, int NBQ_, bool ONE_> struct DCfgT {
    static constexpr int BN = BN_, NW = NW_, WPE = WPE_, NBQ = NBQ_;
    static constexpr bool ONE = ONE_;
};
template <int D> struct DCfg;
template <> struct DCfg<64>  : DCfgT<64, 4, 4, 1, false> {};
template <> struct DCfg<128> : DCfgT<128, 8, 2, 1, false> {};
template <> struct DCfg<256> : DCfgT<32, 8, 2, 1, true> {};

// The four K/V tile buffers (N elements each): buf(i) for a constant i.
template <int N, bool ONE> struct TileBufs;
template <int N> struct TileBufs<N, true> {
    __device__ static uint16_t* buf(int i) {
        __shared__ __attribute__((aligned(1024))) uint16_t t[4 * N];
        return t + i * N;
    }
};
template <int N> struct TileBufs<N, false> {
    __device__ static uint16_t* buf(int i) {
        __shared__ __attribute__((aligned(1024))) uint16_t t0[N];
        __shared__ __attribute__((aligned(1024))) uint16_t t1[N];
        __shared__ __attribute__((aligned(1024))) uint16_t t2[N];
        __shared__ __attribute__((aligned(1024))) uint16_t t3[N];
        return i == 0 ? t0 : i == 1 ? t1 : i == 2 ? t2 : t3;
    }
};
// Instruction schedule (measured): K fragments read ahead of their S MFMAs;
// VALU instructions (the first exponentials) before the first PV MFMA; VALU
// instructions beside each later PV MFMA.
constexpr int kPreK = 4, kValuPv0 = 48, kValuPvN = 6;

template <int D> struct DGeom {
    static constexpr int NW = DCfg<D>::NW, NT = 64 * NW, WPE = DCfg<D>::WPE;
    static constexpr int BN = DCfg<D>::BN;
    static constexpr int NBQ = DCfg<D>::NBQ;       // 32-query blocks per wave
    static constexpr int BM = NW * 32 * NBQ;       // query rows per workgroup
    static constexpr int NS = D / 16;              // MFMA steps along d for S
    static constexpr int NMB = BN / 32;
    static constexpr int NDB = D / 32;
    static constexpr int CPR = D / 8;              // 16-byte chunks per row
    // Chunk swizzles: logical chunk lc of tile row r sits at physical chunk
    // lc ^ f(r).  LDS has 64 banks of 4 bytes, so the bank group (of 16)
    // of a chunk is its position in the tile modulo 16.
    //  * K is read with ds_read_b128, one slot row per lane: each pass of
    //    16 lanes reads one logical chunk of 16 consecutive rows, so f_k
    //    must give those rows 16 different bank groups.
    //  * V is read with ds_read_b64_tr_b16: each 32-lane pass reads 4
    //    logical chunks of 4 rows r0 + i (r0 a multiple of 4), so f_v must
    //    give the 4 x 4 (row, chunk) pairs 16 different bank groups.  f_v
    //    depends only on r & 3 (d >= 128) or bit 1 of r (d = 64), i.e. on
    //    the lane, so the read addresses stay lane offset + constant.
    __device__ static inline int f_k(int r) { return CPR >= 16 ? (r & 15) : ((r >> 1) & 7); }
    __device__ static inline int f_v(int r) { return CPR >= 16 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }
    static constexpr int NVL = NDB < 4 ? NDB : 4;   // V^T lane offsets (one per db & 3)
    static constexpr int TILE = BN * D;            // elements per K or V tile
    static constexpr int NBLK = BN * CPR / 64;     // 1 KB blocks per tile
    static constexpr int BPW = NBLK / NW;          // blocks per wave per tile
    static_assert(BPW * NW == NBLK && BPW >= 1, "tile / waves");
    static_assert(BN % 32 == 0 && BM % BN == 0, "tile shape");
    static_assert(BPW < 64, "vmcnt range");
    static_assert(4 * TILE * 2 * (WPE * 4 / NW > 0 ? WPE * 4 / NW : 1) <= 160 * 1024, "LDS budget");
};



// SPLIT: the key tiles a query block visits are divided among nsplit
// workgroups; each writes its partial result over its share, normalised,
// in fp32 (Opart [nsplit][BH][Lq][D], Lpart [nsplit][BH][Lq], natural-log
// LSE, O = 0 and LSE = -inf for a row that sees no key of the share), and
// fa_merge_kernel combines the shares.
//
// KS = 2 (key halves): the workgroup holds two sets of NW waves on the same
// query rows; set h takes the key tiles jlo + h, jlo + h + 2, ... through its
// own pair of LDS buffers, and at the end set 1 hands its (m, l, O) to set 0
// through LDS, which merges the two like two blocks of the online softmax
// and writes the result.  That doubles the waves of a small grid and halves
// the serial chain of tiles of each query block.
template <int D, int MASK, bool SPLIT, int KS>
__global__ __launch_bounds__((DGeom<D>::NT * KS))
__attribute__((amdgpu_waves_per_eu(DGeom<D>::WPE, DGeom<D>::WPE)))
void fa_fwd_direct_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                          const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                          float* __restrict__ LSE, int BH, int Lq, int Lk, int nqb, float c,
                          int wl, int wr, int nsplit, float* __restrict__ Opart,
                          float* __restrict__ Lpart, int serp)
{
    constexpr bool CAUSAL = MASK == kCausal;
    constexpr bool WINDOW = MASK == kWindow;
    using G = DGeom<D>;
    using E = BF16;
    using Frag = bf16x8;
    constexpr int BN = G::BN, BM = G::BM, NS = G::NS, NMB = G::NMB, NDB = G::NDB;
    constexpr int CPR = G::CPR, NW = G::NW, NBQ = G::NBQ;

    static_assert(KS == 1 || (KS == 2 && !SPLIT), "key halves");
    // K/V tile buffers, two per tensor; with key halves, half h's tiles sit
    // at h * TILE in each buffer
    using TB = TileBufs<KS * G::TILE, DCfg<D>::ONE>;
    uint16_t* const Kb0 = TB::buf(0);
    uint16_t* const Kb1 = TB::buf(1);
    uint16_t* const Vb0 = TB::buf(2);
    uint16_t* const Vb1 = TB::buf(3);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = KS == 1 ? tid >> 6 : (tid >> 6) % NW;   // query rows of this wave
    const int kh = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6) / NW;   // key half
    const int col = lane & 31;
    const int half = lane >> 5;

    // ---- work decode: XCD-grouped heads, heaviest causal blocks first ----
    // Workgroups are dispatched round-robin over the 8 XCDs, so block id p
    // runs on XCD p % 8; every query block of a head goes to one XCD (its L2
    // serves the K/V re-reads) and, causal, the longest rows start first.
    // With key splits, each (head, split) pair counts as one head here.
    int bh, lvl, split = 0;
    {
        xcd_decode(blockIdx.x, SPLIT ? BH * nsplit : BH, bh, lvl);
        if (SPLIT) {
            split = bh % nsplit;
            bh /= nsplit;
        }
    }
    // Causal: rank of the block's work among its head's blocks (0 = the
    // longest rows).  Plainly the dispatch order.  When the whole grid is
    // resident at once (serp > 0 levels per round), the blocks of a head
    // are dealt to the CUs of its XCD in rounds of serp levels, one block
    // per CU per round; alternate rounds run in reverse order (a serpentine
    // deal), so the CU that takes the heaviest block of one round takes the
    // lightest of the next and the work per CU evens out.
    int rank = lvl;
    if (CAUSAL && serp > 0) {
        const int r = lvl / serp, i = lvl - r * serp;
        const int m = min(serp, nqb - r * serp);   // levels in this round
        rank = r * serp + ((r & 1) ? m - 1 - i : i);
    }
    const int qb = CAUSAL ? (nqb - 1 - rank) : lvl;
    const int q0 = qb * BM;
    const int q0w = q0 + wave * 32 * NBQ;   // query block nb: rows q0w + 32 nb + col
    const int qlast_w = q0w + 32 * NBQ - 1;

    const uint16_t* Qh = Q + (size_t)bh * Lq * D;
    const uint16_t* Kh = K + (size_t)bh * Lk * D;
    const uint16_t* Vh = V + (size_t)bh * Lk * D;

    // ---- Q fragments: resident for the whole key loop --------------------
    Frag qf[NBQ][NS];
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
        const int row = q0w + 32 * nb + col;
#pragma unroll
        for (int s = 0; s < NS; ++s)
            qf[nb][s] = (row < Lq) ? E::load(Qh + (size_t)row * D + s * 16 + half * 8) : Frag{};
    }
    f32x16 oacc[NBQ][NDB];
    float m_run[NBQ], l_run[NBQ], c_run[NBQ];
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[nb][db] = f32x16{};
        m_run[nb] = -__builtin_inff();
        l_run[nb] = 0.f;
        c_run[nb] = 0.f;
    }

    // key tiles [jlo, nt) hold every key a row of this block may see
    const int kv_end = CAUSAL ? min(Lk, q0 + BM) : WINDOW ? min(Lk, q0 + BM + wr) : Lk;
    // (clamped to the last tile: a block whose rows all lie past Lk - 1 + wl
    // still visits one tile, fully masked, so its rows come out empty)
    int jlo = WINDOW ? min(max(0, q0 - wl), Lk - 1) / BN : 0;
    int nt = max((kv_end + BN - 1) / BN, jlo + 1);
    if (SPLIT) {
        // this split's share of the block's tiles; an empty share writes
        // empty partial rows and leaves before any copy or barrier (the
        // branch is the same for the whole workgroup)
        const int per = (nt - jlo + nsplit - 1) / nsplit;
        const int js = jlo + split * per;
        const int je = min(nt, js + per);
        if (js >= je) {
#pragma unroll
            for (int nb = 0; nb < NBQ; ++nb) {
                const int row = q0w + 32 * nb + col;
                if (row >= Lq) continue;
                float* Op = Opart + (((size_t)split * BH + bh) * Lq + row) * D;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *reinterpret_cast<f32x4*>(Op + db * 32 + 8 * g + 4 * half) = f32x4{};
                if (half == 0) Lpart[((size_t)split * BH + bh) * Lq + row] = -__builtin_inff();
            }
            return;
        }
        jlo = js;
        nt = je;
    }

    // ---- tile copy: HBM -> LDS, no registers ------------------------------
    // Per-lane parts of the copy addresses (element offsets inside a tile):
    // LDS block blk of 64 chunks, lane's physical chunk p -> tile row and
    // logical chunk.  K rows are stored in the permuted slot order of k_slot.
    unsigned kofs_g[G::BPW], vofs_g[G::BPW];   // byte offsets inside a tile
#pragma unroll
    for (int i = 0; i < G::BPW; ++i) {
        const int blk = wave + NW * i;
        const int p = blk * 64 + lane;
        const int row = p / CPR;
        const int kr = (row & ~31) | (16 * ((row >> 2) & 1) + 4 * ((row & 31) >> 3) + (row & 3));
        kofs_g[i] = (unsigned)(kr * D + ((p % CPR) ^ G::f_k(row)) * 8) * 2u;
        vofs_g[i] = (unsigned)(row * D + ((p % CPR) ^ G::f_v(row)) * 8) * 2u;
    }
    // Each wave copies BPW 1 KB blocks of a tile through a buffer resource
    // whose base is the tile's first row and whose size covers only its
    // rows below Lk (none for a tile index past the block's last one, the
    // prefetch after the final tile).  A lane whose row lies outside reads
    // zeros from the hardware's range check without touching memory: finite
    // values that the mask gives weight 0.  So every step issues the same
    // copies, the per-lane offsets never change, and the counted waits
    // below stay exact; the LDS destination comes from a scalar copy of the
    // wave index.
    const int swave = __builtin_amdgcn_readfirstlane(wave);
    const int hofs = kh * G::TILE;   // this key half's buffers
    auto issue = [&](const uint16_t* Xh, int j, uint16_t* Xd,
                     const unsigned (&ofs)[G::BPW]) FA_INLINE {
        const int jc = min(j, nt - 1);   // j >= jlo
        const int bytes = j < nt ? min(BN, Lk - jc * BN) * D * 2 : 0;
        const uint16_t* base = Xh + (size_t)jc * BN * D;
#pragma unroll
        for (int i = 0; i < G::BPW; ++i)
            buffer_copy<16>(base, bytes, ofs[i],
                            (FA_LDS void*)(Xd + hofs + (swave + NW * i) * 512));
    };
    auto issue_k = [&](int j, uint16_t* Kd) FA_INLINE { issue(Kh, j, Kd, kofs_g); };
    auto issue_v = [&](int j, uint16_t* Vd) FA_INLINE { issue(Vh, j, Vd, vofs_g); };
    // K fragment (A operand of S^T) for d-step s of key block mb: slot row
    // mb*32 + col, logical chunk 2s + half; f_k(mb*32 + col) = f_k(col), so
    // mb only adds a whole-row offset and one lane offset per s suffices.
    // The swizzle touches only the low 4 bits of the chunk index 2s + half,
    // so steps s and s + 8 differ by a constant 16 chunks: 8 lane offsets
    // serve every d.
    constexpr int NKF = NS < 8 ? NS : 8;
    int kfo[NKF];
#pragma unroll
    for (int st = 0; st < NKF; ++st)
        kfo[st] = hofs + col * D + (((2 * st + half) ^ G::f_k(col)) * 8);
    auto k_frag = [&](const uint16_t* Ks, int mb, int st) FA_INLINE {
        return E::load(Ks + mb * 32 * D + kfo[st % NKF] + (st / NKF) * 128);
    };
    // V^T fragment for PV MFMA (mb, t, db): two transposed 8-byte reads.
    // Lane l of 16-lane group g supplies row 16*(g>>1) + 8t + 4w + (l&15)/4
    // of key block mb and d-quad 4*((l&15)%4) of the 16-column half g&1 of
    // d-block db, i.e. logical chunk 4db + 2(g&1) + (l%4)/2.  The row's
    // swizzle f_v depends only on the lane, and XORs bits 2.. of the chunk
    // (the d-block bits) with a lane value, so the address is one of NVL
    // lane offsets (chosen by db & 3) plus a compile-time constant.
    const int g16 = lane >> 4, rr = lane & 15;
    const int vh = g16 >> 1, vdh = g16 & 1, vi = rr >> 2, vq = rr & 3;
    int vlane[G::NVL];
#pragma unroll
    for (int x = 0; x < G::NVL; ++x) {
        const int lc = 4 * x + 2 * vdh + (vq >> 1);
        vlane[x] = hofs + (16 * vh + vi) * D + (lc ^ G::f_v(vi)) * 8 + (vq & 1) * 4;
    }
    auto v_frag = [&](const uint16_t* Vs, int mb, int t, int db) FA_INLINE {
        s16x4 u[2];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const int cofs = (mb * 32 + 8 * t + 4 * w) * D + (db & ~3) * 32;
            const uint16_t* a = Vs + cofs + vlane[db & (G::NVL - 1)];
            u[w] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(FA_LDS void*)a);
        }
        const s16x8 v8 = __builtin_shufflevector(u[0], u[1], 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(Frag, v8);
    };

    // ---- per-tile pieces ---------------------------------------------------
    // S^T = K Q^T for the wave's NBQ query blocks; each K fragment feeds NBQ
    // MFMAs and is read kPreK fragments ahead
    auto s_tile = [&](const uint16_t* Kc, f32x16 (&sacc)[NBQ][NMB]) FA_INLINE {
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb)
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) sacc[nb][mb] = f32x16{};
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
                const Frag a = k_frag(Kc, mb, s);
#pragma unroll
                for (int nb = 0; nb < NBQ; ++nb) sacc[nb][mb] = E::mfma(a, qf[nb][s], sacc[nb][mb]);
            }
        constexpr int NK = NS * NMB, PRE = kPreK;
        __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);
#pragma unroll
        for (int i = 0; i < NK - PRE; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, NBQ, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PRE * NBQ, 0);
    };
    // mask, running max and O rescale for query block nb; returns the max
    // used by the exponentials and sets alpha
    auto row_max = [&](int kv0, int nb, f32x16 (&sacc)[NMB], float& alpha,
                       float& hmax) FA_INLINE {
        const int qb0 = q0w + 32 * nb;
        // some key of the tile lies past Lk, right of a row's last key, or
        // (window) left of a row's first key
        if ((kv0 + BN > Lk) || (CAUSAL && kv0 + BN - 1 > qb0) ||
            (WINDOW && (kv0 + BN - 1 > qb0 + wr || kv0 < qb0 + 31 - wl))) {
            // This lane's query sees keys kb + e for e in [lo, lo + span],
            // where element i of key block mb is e = mb*32 + i.  One
            // unsigned compare per element; an empty range gets lo past
            // the tile.  The scheduling barrier after each key block keeps
            // the compiler from hoisting all 64 compare masks into SGPRs.
            const int qi = qb0 + col;
            const int kb = kv0 + 16 * half;
            int hi = Lk - 1;
            if (CAUSAL) hi = min(hi, qi);
            if (WINDOW) hi = min(hi, qi + wr);
            hi = min(hi - kb, BN);
            int lo = WINDOW ? max(qi - wl - kb, 0) : 0;
            unsigned span = (unsigned)(hi - lo);
            if (hi < lo) { lo = BN + 1; span = 0u; }
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if ((unsigned)(mb * 32 + i - lo) > span) sacc[mb][i] = -__builtin_inff();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // NMB independent 3-input chains, then combined
        float pm[NMB];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
            float a = fmaxf(fmaxf(sacc[mb][0], sacc[mb][1]), sacc[mb][2]);
#pragma unroll
            for (int i = 3; i < 15; i += 2) a = fmaxf(fmaxf(a, sacc[mb][i]), sacc[mb][i + 1]);
            pm[mb] = fmaxf(a, sacc[mb][15]);
        }
#pragma unroll
        for (int w = 1; w < NMB; w *= 2)
#pragma unroll
            for (int mb = 0; mb + w < NMB; mb += 2 * w) pm[mb] = fmaxf(pm[mb], pm[mb + w]);
        // The reference max moves only when the tile's max exceeds it by
        // more than kLazy (base 2), so most tiles skip the O rescale.  P <= 2^8
        // stays exact in range; but the key at a row's maximum then gets a
        // rounded bf16 weight 2^delta instead of exp2(0) = 1, while l sums the
        // unrounded P.  That one mismatch is carried separately (c_run, the
        // rounding of each lane's tile maximum) and O is normalised by l plus
        // it, so the global maximum's weight is consistent between numerator
        // and denominator as with the exact max; LSE keeps the true l.
        hmax = pm[0];
        const float m_tile = half_max(pm[0]) * c;
        const float m_new = (m_tile > m_run[nb] + kLazy) ? m_tile : m_run[nb];
        const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
        alpha = __builtin_amdgcn_exp2f(m_run[nb] - m_use);
        // rescale O before the exponentials so that they and the PV MFMAs
        // can share one basic block (alpha == 1: skipped exactly)
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[nb][db] *= alpha;
        }
        m_run[nb] = m_new;
        return m_use;
    };
    // P = exp2(S c - m) as MFMA operands; returns this lane's partial sum
    auto exps = [&](const f32x16 (&sacc)[NMB], float m_use,
                    Frag (&pf)[NMB][2]) FA_INLINE {
        float rsum[NMB];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
            float p[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mb][i], c, -m_use));
            const float s0 = (p[0] + p[1]) + (p[2] + p[3]);
            const float s1 = (p[4] + p[5]) + (p[6] + p[7]);
            const float s2 = (p[8] + p[9]) + (p[10] + p[11]);
            const float s3 = (p[12] + p[13]) + (p[14] + p[15]);
            rsum[mb] = (s0 + s1) + (s2 + s3);
            pf[mb][0] = E::from_f32(p);
            pf[mb][1] = E::from_f32(p + 8);
        }
        float rs = 0.f;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) rs += rsum[mb];
        return rs;
    };
    // O^T += V^T P^T; each V^T fragment feeds NBQ MFMAs
    auto pv = [&](const uint16_t* Vc, const Frag (&pf)[NBQ][NMB][2]) FA_INLINE {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const Frag v = v_frag(Vc, mb, t, db);
#pragma unroll
                    for (int nb = 0; nb < NBQ; ++nb)
                        oacc[nb][db] = E::mfma(v, pf[nb][mb][t], oacc[nb][db]);
                }
    };
    // exponentials of key block 0 first, then each V^T fragment's MFMAs
    // with its two transposed reads and a share of the remaining VALU work
    auto sched_pv_valu = [&]() FA_INLINE {
        constexpr int NV = NMB * 2 * NDB;   // V^T fragments per tile
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPv0 * NBQ, 0);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, NBQ, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, kValuPvN * NBQ, 0);
        }
    };
    // Wait until at most N of this wave's tile copies are in flight and its
    // LDS reads are done, then the workgroup barrier.  A copy counts as done
    // once its data is in LDS, so after the barrier every wave sees the
    // tiles whose copies all waves waited for.  No memory fence: a
    // workgroup-scope fence would wait for every copy in flight (vmcnt(0)),
    // including the prefetch that is meant to overlap the next phase; the
    // empty asm statements keep the compiler from moving memory accesses
    // across the barrier.
    auto sync_after = [&](auto n_in_flight) {
        constexpr int N = decltype(n_in_flight)::value;
        constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4);   // lgkmcnt(0)
        __builtin_amdgcn_s_waitcnt(imm);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    using InFlight0 = std::integral_constant<int, 0>;

    // waves whose rows see no key of tile j skip its math (with key halves,
    // the last tile of half 1 may lie past the block's last one)
    auto sees = [&](int j) FA_INLINE {
        const int kv0 = j * BN;
        return (KS == 1 || j < nt) && (!CAUSAL || kv0 <= qlast_w) &&
               (!WINDOW || (kv0 <= qlast_w + wr && kv0 + BN - 1 >= q0w - wl));
    };
    // softmax of tile j from its scores, then O += P V_j
    auto soft_pv = [&](int j, f32x16 (&sacc)[NBQ][NMB], const uint16_t* Vc) FA_INLINE {
        const int kv0 = j * BN;
        float alpha[NBQ], rs[NBQ];
        Frag pf[NBQ][NMB][2];
        float dmax[NBQ];
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) {
            float hmax;
            const float m_use = row_max(kv0, nb, sacc[nb], alpha[nb], hmax);
            rs[nb] = exps(sacc[nb], m_use, pf[nb]);
            // bf16 rounding of P at this lane's tile maximum
            const float pmx = __builtin_amdgcn_exp2f(__builtin_fmaf(hmax, c, -m_use));
            dmax[nb] = (float)(__bf16)pmx - pmx;
        }
        pv(Vc, pf);
        sched_pv_valu();
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) {
            l_run[nb] = l_run[nb] * alpha[nb] + rs[nb];
            c_run[nb] = c_run[nb] * alpha[nb] + dmax[nb];
        }
    };
    // every wave: S_j, softmax_j, PV_j; the copies of its key half's next
    // tile j + KS overlap them
    auto step = [&](int j, const uint16_t* Kc, const uint16_t* Vc, uint16_t* Kn,
                    uint16_t* Vn) FA_INLINE {
        issue_k(j + KS, Kn);
        issue_v(j + KS, Vn);
        if (sees(j)) {
            f32x16 sacc[NBQ][NMB];
            s_tile(Kc, sacc);
            soft_pv(j, sacc, Vc);
        }
        sync_after(InFlight0{});   // this wave's copies of tile j+1 landed
    };
    // both key halves run the same steps (and barriers): half h takes tile
    // jj + h of each pair jj
    issue_k(jlo + kh, Kb0);
    issue_v(jlo + kh, Vb0);
    sync_after(InFlight0{});
    for (int jj = jlo; jj < nt; jj += 2 * KS) {
        step(jj + kh, Kb0, Vb0, Kb1, Vb1);
        if (jj + KS < nt) step(jj + KS + kh, Kb1, Vb1, Kb0, Vb0);
    }

    // ---- epilogue: O / l, LSE = ln2 * (m + log2 l) -------------------------
    __builtin_amdgcn_s_waitcnt(0x0F70);   // no copy left in flight
    if constexpr (KS == 2) {
        // Merge of the key halves (the block-merge step of the online
        // softmax): half 1 leaves (m, l, c, O) in LDS, lane by lane, and half
        // 0 rescales both to m = max(m0, m1).  Every wave's copies landed
        // (vmcnt(0) above) before the barrier, so the tile buffers are free:
        // query wave w's exchange goes through buffer w, quad q of lane l at
        // (q * 64 + l) * 16 bytes.
        constexpr int NF = NBQ * (NDB * 16 + 4);   // floats per lane
        static_assert(NW <= 4 && NF * 64 * 4 <= KS * G::TILE * 2, "merge fits the tile buffers");
        uint16_t* const xb = wave == 0 ? Kb0 : wave == 1 ? Kb1 : wave == 2 ? Vb0 : Vb1;
        FA_LDS float* xs = (FA_LDS float*)(FA_LDS void*)xb;
        auto xq = [&](int q) { return (FA_LDS f32x4*)(xs + (q * 64 + lane) * 4); };
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (kh == 1) {
#pragma unroll
            for (int nb = 0; nb < NBQ; ++nb) {
                const int q0q = nb * (NDB * 4 + 1);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *xq(q0q + db * 4 + g) =
                            f32x4{oacc[nb][db][4 * g], oacc[nb][db][4 * g + 1],
                                  oacc[nb][db][4 * g + 2], oacc[nb][db][4 * g + 3]};
                *xq(q0q + NDB * 4) = f32x4{m_run[nb], l_run[nb], c_run[nb], 0.f};
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): LDS writes done
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (kh == 1) return;
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) {
            const int q0q = nb * (NDB * 4 + 1);
            const f32x4 mlc = *xq(q0q + NDB * 4);
            const float m = fmaxf(m_run[nb], mlc[0]);
            const float mu = (m == -__builtin_inff()) ? 0.f : m;
            const float a0 = __builtin_amdgcn_exp2f(m_run[nb] - mu);
            const float a1 = __builtin_amdgcn_exp2f(mlc[0] - mu);
            l_run[nb] = l_run[nb] * a0 + mlc[1] * a1;
            c_run[nb] = c_run[nb] * a0 + mlc[2] * a1;
            m_run[nb] = m;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 o1 = *xq(q0q + db * 4 + g);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        oacc[nb][db][4 * g + e] = oacc[nb][db][4 * g + e] * a0 + o1[e] * a1;
                }
        }
    }
    uint16_t* Oh = O + (size_t)bh * Lq * D;
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
        const float lt = half_sum(l_run[nb]);
        // O is normalised by the sum of the weights its numerator used
        const float ln = lt + half_sum(c_run[nb]);
        // a window or a key split can leave a row with no key: O = 0 and
        // LSE = -inf (log of an empty sum)
        constexpr bool MAY_BE_EMPTY = WINDOW || SPLIT;
        const float inv = (!MAY_BE_EMPTY || lt > 0.f) ? 1.0f / ln : 0.f;
        const int row = q0w + 32 * nb + col;
        if (SPLIT && row < Lq) {
            float* Op = Opart + (((size_t)split * BH + bh) * Lq + row) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 v4 = {oacc[nb][db][4 * g + 0], oacc[nb][db][4 * g + 1],
                                oacc[nb][db][4 * g + 2], oacc[nb][db][4 * g + 3]};
                    *reinterpret_cast<f32x4*>(Op + db * 32 + 8 * g + 4 * half) = v4 * inv;
                }
            if (half == 0)
                Lpart[((size_t)split * BH + bh) * Lq + row] =
                    lt > 0.f ? (m_run[nb] + __builtin_amdgcn_logf(lt)) * kLn2 : -__builtin_inff();
        } else if (row < Lq) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 v4 = {oacc[nb][db][4 * g + 0], oacc[nb][db][4 * g + 1],
                                oacc[nb][db][4 * g + 2], oacc[nb][db][4 * g + 3]};
                    v4 *= inv;
                    E::store4(Oh + (size_t)row * D + db * 32 + 8 * g + 4 * half, v4);
                }
            if (half == 0)
                LSE[(size_t)bh * Lq + row] = (!MAY_BE_EMPTY || lt > 0.f)
                    ? (m_run[nb] + __builtin_amdgcn_logf(lt)) * kLn2 : -__builtin_inff();
        }
    }
}

template <int D, int MASK>
hipError_t launch_direct(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int Lq, int Lk, float scale, int wl, int wr,
                         hipStream_t stream)
{
    using G = DGeom<D>;
    const int BH = B * H;
    const int nqb = (Lq + G::BM - 1) / G::BM;
    const float c = exp2_factor(scale * (double)kLog2e);
    const int cus = cu_count();
    int serp = 0;
    auto go = [&](auto kern, int threads) {
        hipLaunchKernelGGL(kern, dim3((unsigned)(nqb * BH)), dim3(threads), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, BH,
                           Lq, Lk, nqb, c, wl, wr, 1, nullptr, nullptr, serp);
        return hipGetLastError();
    };
    // d = 64 on a grid of at most two workgroups per CU: key halves, twice
    // the waves per workgroup (two such workgroups fill a CU at four waves
    // per SIMD, in 2 x 64 KB of LDS)
    // The whole grid is then resident at once; causal, the blocks are dealt
    // in serpentine order when every XCD's CUs take whole levels of its
    // heads (heads per XCD dividing CUs per XCD).
    if constexpr (D == 64) {
        static_assert(4 * 2 * G::TILE * 2 * 2 <= 160 * 1024, "two workgroups per CU");
        if ((long long)nqb * BH <= 2LL * cus) {
            if (MASK == kCausal && BH % 8 == 0 && cus % 8 == 0 && (cus / 8) % (BH / 8) == 0)
                serp = (cus / 8) / (BH / 8);
            return go(fa_fwd_direct_kernel<D, MASK, false, 2>, 2 * G::NT);
        }
    }
    return go(fa_fwd_direct_kernel<D, MASK, false, 1>, G::NT);
}

// ---- merge of key-split partials ------------------------------------------
// Block-merge step of "Flash Attention 原理与实现详解" (tbr8.org), section 2.1
// "Tiling（分块计算）策略", applied to normalised partials (O_s, LSE_s):
// LSE = m + ln(sum_s e^(LSE_s - m)), O = sum_s e^(LSE_s - m) O_s / sum_s
// e^(LSE_s - m) with m = max_s LSE_s.  One thread per 4 elements of a row;
// rows with every partial empty stay empty (O = 0, LSE = -inf).
template <int D>
__global__ __launch_bounds__(256)
void fa_merge_kernel(const float* __restrict__ Opart, const float* __restrict__ Lpart,
                     uint16_t* __restrict__ O, float* __restrict__ LSE, int rows, int nsplit)
{
    constexpr int TPR = D / 4;              // threads per row
    const int row = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
    const int c4 = (threadIdx.x % TPR) * 4;
    if (row >= rows) return;
    const size_t stride_o = (size_t)rows * D;
    float m = -__builtin_inff();
    for (int s = 0; s < nsplit; ++s) m = fmaxf(m, Lpart[(size_t)s * rows + row]);
    const float m_use = (m == -__builtin_inff()) ? 0.f : m;
    f32x4 acc = {};
    float l = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const float w = __builtin_amdgcn_exp2f((Lpart[(size_t)s * rows + row] - m_use) * kLog2e);
        l += w;
        acc += w * *reinterpret_cast<const f32x4*>(Opart + s * stride_o + (size_t)row * D + c4);
    }
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    BF16::store4(O + (size_t)row * D + c4, acc * inv);
    if (c4 == 0) LSE[row] = l > 0.f ? m_use + __builtin_amdgcn_logf(l) * kLn2 : -__builtin_inff();
}

template <int D, int MASK>
hipError_t launch_split(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int Lq, int Lk, float scale, int nsplit, float* opart,
                        float* lpart, hipStream_t stream)
{
    using G = DGeom<D>;
    const int BH = B * H;
    const int nqb = (Lq + G::BM - 1) / G::BM;
    hipLaunchKernelGGL((fa_fwd_direct_kernel<D, MASK, true, 1>),
                       dim3((unsigned)(nqb * BH * nsplit)), dim3(G::NT), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, BH, Lq,
                       Lk, nqb, exp2_factor(scale * (double)kLog2e), 0, 0, nsplit, opart, lpart, 0);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int rows = BH * Lq;
    constexpr int RPB = 256 / (D / 4);     // rows per merge block
    hipLaunchKernelGGL((fa_merge_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256),
                       0, stream, opart, lpart, static_cast<uint16_t*>(o), lse, rows, nsplit);
    return hipGetLastError();
}

template <int MASK>
hipError_t launch_direct_d(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Lq, int Lk, int d, float scale, int wl, int wr,
                           hipStream_t stream)
{
    switch (d) {
    case 64:  return launch_direct<64, MASK>(q, k, v, o, lse, B, H, Lq, Lk, scale, wl, wr, stream);
    case 128: return launch_direct<128, MASK>(q, k, v, o, lse, B, H, Lq, Lk, scale, wl, wr, stream);
    case 256: return launch_direct<256, MASK>(q, k, v, o, lse, B, H, Lq, Lk, scale, wl, wr, stream);
    default:  return hipErrorInvalidValue;
    }
}

template <class E, int D, bool CAUSAL>
hipError_t launch_one(const void* q, const void* k, const void* v, void* o,
                      float* lse, int B, int H, int Lq, int Lk, float scale,
                      hipStream_t stream)
{
    using G = Geom<E, D>;
    using T = typename E::T;
    const int BH = B * H;
    const int nqb = (Lq + G::BM - 1) / G::BM;
    const long long nblocks = (long long)nqb * BH;
    const float c = exp2_factor(scale * (double)kLog2e);
    hipLaunchKernelGGL((fa_fwd_kernel<E, D, CAUSAL>), dim3((unsigned)nblocks),
                       dim3(G::NT), 0, stream,
                       static_cast<const T*>(q), static_cast<const T*>(k),
                       static_cast<const T*>(v), static_cast<T*>(o), lse,
                       BH, Lq, Lk, nqb, c);
    return hipGetLastError();
}

template <class E, int D>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o,
                    float* lse, int B, int H, int Lq, int Lk, bool causal,
                    float scale, hipStream_t stream)
{
    return causal ? launch_one<E, D, true>(q, k, v, o, lse, B, H, Lq, Lk, scale, stream)
                  : launch_one<E, D, false>(q, k, v, o, lse, B, H, Lq, Lk, scale, stream);
}

hipError_t launch_f32(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Lq, int Lk, int d, bool causal, float scale,
                      hipStream_t stream)
{
    switch (d) {
    case 64:  return launch_d<F32, 64>(q, k, v, o, lse, B, H, Lq, Lk, causal, scale, stream);
    case 128: return launch_d<F32, 128>(q, k, v, o, lse, B, H, Lq, Lk, causal, scale, stream);
    case 256: return launch_d<F32, 256>(q, k, v, o, lse, B, H, Lq, Lk, causal, scale, stream);
    default:  return hipErrorInvalidValue;
    }
}

template <class E, int D>
TileConfig cfg_of() {
    return TileConfig{Geom<E, D>::BM, Geom<E, D>::BN, Geom<E, D>::NT};
}

}  // namespace

bool tile_config(DType dt, int d, TileConfig* out)
{
    if (dt == DType::BF16) {
        switch (d) {
        case 64:  *out = TileConfig{DGeom<64>::BM, DGeom<64>::BN, DGeom<64>::NT}; return true;
        case 128: *out = TileConfig{DGeom<128>::BM, DGeom<128>::BN, DGeom<128>::NT}; return true;
        case 256: *out = TileConfig{DGeom<256>::BM, DGeom<256>::BN, DGeom<256>::NT}; return true;
        }
    } else if (dt == DType::F32) {
        switch (d) {
        case 64:  *out = cfg_of<F32, 64>();  return true;
        case 128: *out = cfg_of<F32, 128>(); return true;
        case 256: *out = cfg_of<F32, 256>(); return true;
        }
    }
    return false;
}

hipError_t launch_fwd(DType dt, const void* q, const void* k, const void* v,
                      void* o, float* lse, int B, int H, int Lq, int Lk,
                      int d, bool causal, float scale, hipStream_t stream)
{
    if (dt == DType::BF16)
        return causal ? launch_direct_d<kCausal>(q, k, v, o, lse, B, H, Lq, Lk, d, scale, 0, 0, stream)
                      : launch_direct_d<kFull>(q, k, v, o, lse, B, H, Lq, Lk, d, scale, 0, 0, stream);
    return launch_f32(q, k, v, o, lse, B, H, Lq, Lk, d, causal, scale, stream);
}

hipError_t launch_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int Lq, int Lk, int d, int wl, int wr, float scale,
                             hipStream_t stream)
{
    return launch_direct_d<kWindow>(q, k, v, o, lse, B, H, Lq, Lk, d, scale, wl, wr, stream);
}

hipError_t launch_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Lq, int Lk, int d, bool causal, float scale,
                            int nsplit, float* opart, float* lpart, hipStream_t stream)
{
    switch (d) {
    case 64:
        return causal ? launch_split<64, kCausal>(q, k, v, o, lse, B, H, Lq, Lk, scale, nsplit, opart, lpart, stream)
                      : launch_split<64, kFull>(q, k, v, o, lse, B, H, Lq, Lk, scale, nsplit, opart, lpart, stream);
    case 128:
        return causal ? launch_split<128, kCausal>(q, k, v, o, lse, B, H, Lq, Lk, scale, nsplit, opart, lpart, stream)
                      : launch_split<128, kFull>(q, k, v, o, lse, B, H, Lq, Lk, scale, nsplit, opart, lpart, stream);
    case 256:
        return causal ? launch_split<256, kCausal>(q, k, v, o, lse, B, H, Lq, Lk, scale, nsplit, opart, lpart, stream)
                      : launch_split<256, kFull>(q, k, v, o, lse, B, H, Lq, Lk, scale, nsplit, opart, lpart, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace fa
