// Device helpers shared by the kernel sources (HIP only): the HBM -> LDS
// tile copy and the XCD-aware work decode.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

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
