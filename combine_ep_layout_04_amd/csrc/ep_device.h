// ep_device.h -- device-side helpers shared by the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Cache-policy operand of a gfx950 vector memory instruction: bit 0 sc0,
// bit 1 nt, bit 4 sc1.  Rows written once and not read again by the kernel
// go out with sc1 | nt (device scope, non-temporal): they stream past the
// caches.  On the dispatch pattern this measured about 2% faster than nt
// alone with cold caches and 3% back to back.
constexpr int kCpolNT = 2;
constexpr int kCpolStream = 16 | 2;

// Raw buffer resource over `bytes` bytes at p (stride 0; the 32-bit data
// format word of the gfx9 resource descriptor).  Accesses past `bytes`
// read 0 and write nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

// 16 bytes at byte offset `off` of a write-once row.
__device__ __forceinline__ void store_row16(__amdgpu_buffer_rsrc_t rs, int off, const uint4& v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0, kCpolStream);
}

}  // namespace ep
