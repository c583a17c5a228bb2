// Device helpers shared by the kernel sources (HIP only): vector types, the
// exchange between the two 32-lane halves of a wave, the HBM -> LDS tile
// copy and the XCD-aware work decode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define FA_LDS __attribute__((address_space(3)))
// on a kernel's lambdas: inline them at every call (an outlined lambda
// would take its array arguments through scratch memory)
#define FA_INLINE __attribute__((always_inline))

constexpr float kLog2e = 1.4426950408889634f;  // log2(e), base change of exp
constexpr float kLn2 = 0.69314718055994531f;   // ln(2), LSE back to base e

// Which keys a query sees: all of them, the causal prefix j <= i (top-left),
// or a sliding window i - wl <= j <= i + wr (the window-size pair of
// "Flash Attention 原理与实现详解" (tbr8.org), section 6.3 "滑动窗口注意力";
// (wl, 0) is a causal window).  Always also j < Lk.
enum Mask : int { kFull = 0, kCausal = 1, kWindow = 2 };

// Lane l and lane l ^ 32 hold the same query column of a 32x32 MFMA
// accumulator; combine their values.  v_permlane32_swap exchanges the two
// 32-lane halves without going through the LDS crossbar: each lane receives
// its partner's value.
__device__ inline float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x),
                                                    false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]),
                 __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ inline float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x),
                                                    false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) +
           __builtin_bit_cast(float, (unsigned)r[1]);
}

// One copy of BYTES (4 or 16) per lane HBM -> LDS through a raw buffer
// resource of `bytes` bytes at `base`: lane L's BYTES at base + vofs land at
// byte BYTES * L of the LDS block `dst` (buffer_load_dword / _dwordx4 ...
// lds); a lane whose BYTES end past `bytes` gets zeros from the range check
// and touches no memory.  Word 3 of the resource: 32-bit data format, no
// swizzle or stride (gfx9 family).  Both the copy and the buffer-resource
// type exist only for the device; the host pass sees an empty body.
template <int BYTES>
__device__ inline void buffer_copy(const void* base, int bytes, unsigned vofs,
                                   __attribute__((address_space(3))) void* dst) {
    static_assert(BYTES == 4 || BYTES == 16, "copy width");
#if defined(__HIP_DEVICE_COMPILE__)
    const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes,
                                                     0x00020000);
    if constexpr (BYTES == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, vofs, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, vofs, 0, 0, 0);
#endif
}

// Work decode shared by the kernels.  Workgroups are dispatched round-robin
// over the 8 XCDs, so block p runs on XCD p % 8.  With `units` (heads, or
// (head, split) pairs) a multiple of 8, every block of a unit goes to one
// XCD, whose L2 then serves the unit's K/V (or Q/dO) re-reads; `lvl` is
// the block's index among its unit's blocks in dispatch order.  Otherwise
// units interleave plainly.
__device__ inline void xcd_decode(int p, int units, int& unit, int& lvl) {
    if ((units & 7) == 0) {
        const int own = units >> 3;   // units per XCD
        const int slot = p >> 3;
        unit = (p & 7) + 8 * (slot % own);
        lvl = slot / own;
    } else {
        unit = p % units;
        lvl = p / units;
    }
}

}  // namespace fa
