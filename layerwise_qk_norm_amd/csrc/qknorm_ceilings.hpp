// Measurement kernels: one-shot copies that give each byte mix of the fused
// kernels a bandwidth ceiling. Kept apart from the fused kernels' source, which
// they share nothing with but the helpers they include.
#pragma once
#include "qknorm_kernels.hpp"

namespace qkn {

// ================================================================ ceilings

// Both kernels run one pass of a one-shot grid in which each thread moves one
// vector: workgroups [0, wa) serve tensor a, the rest tensor b. Each tensor's
// whole vectors sit behind one buffer descriptor (na, nb bytes, below 2^31), so
// a workgroup's only arithmetic is its offset -- the prologue of a workgroup
// that lives for one load and one store is part of what such a grid pays per
// byte. Workgroup 0 also moves the ta, tb bytes after the whole vectors one at
// a time.

// Copy: one 16-byte nontemporal load and store per thread; a workgroup moves
// TPB * 16 contiguous bytes.
template <int TPB>
__global__ void __launch_bounds__(TPB)
copy_ceiling_kernel(const void* a, const void* b, void* oa, void* ob, uint32_t na, uint32_t nb,
                    uint32_t wa, uint32_t ta, uint32_t tb)
{
    const bool in_a = blockIdx.x < wa;
    const uint32_t n = in_a ? na : nb;
    const uint32_t off = ((in_a ? blockIdx.x : blockIdx.x - wa) * TPB + threadIdx.x) * 16;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(in_a ? a : b), (short)0, (int)n, 0x00020000);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(in_a ? oa : ob, (short)0, (int)n, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNT), rd, off, 0, kNT);
    if (blockIdx.x == 0) {
        for (uint32_t i = threadIdx.x; i < ta; i += TPB)
            static_cast<char*>(oa)[na + i] = static_cast<const char*>(a)[na + i];
        for (uint32_t i = threadIdx.x; i < tb; i += TPB)
            static_cast<char*>(ob)[nb + i] = static_cast<const char*>(b)[nb + i];
    }
}

// Each input byte zero-extended to one 16-bit word.
__device__ __forceinline__ u32x4 widen_bytes(uint32_t d0, uint32_t d1)
{
    u32x4 o;
    o[0] = (d0 & 0xffu) | ((d0 & 0xff00u) << 8);
    o[1] = ((d0 >> 16) & 0xffu) | ((d0 >> 8) & 0xff0000u);
    o[2] = (d1 & 0xffu) | ((d1 & 0xff00u) << 8);
    o[3] = ((d1 >> 16) & 0xffu) | ((d1 >> 8) & 0xff0000u);
    return o;
}

// Widening (the byte mix of E4M3 inputs with bf16 outputs, twice as many bytes
// written as read): each thread loads 8 input bytes and stores their 16 output
// bytes, so a wave's load covers 512 contiguous bytes and its store 1 KiB of
// whole lines. na, nb count the bytes of whole 8-byte chunks (outputs twice
// that, below 2^31).
template <int TPB>
__global__ void __launch_bounds__(TPB)
widen_ceiling_kernel(const void* a, const void* b, void* oa, void* ob, uint32_t na, uint32_t nb,
                     uint32_t wa, uint32_t ta, uint32_t tb)
{
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const bool in_a = blockIdx.x < wa;
    const uint32_t n = in_a ? na : nb;
    const uint32_t off = ((in_a ? blockIdx.x : blockIdx.x - wa) * TPB + threadIdx.x) * 8;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(in_a ? a : b), (short)0, (int)n, 0x00020000);
    const __amdgpu_buffer_rsrc_t rd =
        __builtin_amdgcn_make_buffer_rsrc(in_a ? oa : ob, (short)0, (int)(2 * n), 0x00020000);
    const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kNT));
    __builtin_amdgcn_raw_buffer_store_b128(widen_bytes(x[0], x[1]), rd, 2 * off, 0, kNT);
    if (blockIdx.x == 0) {
        for (uint32_t i = threadIdx.x; i < ta; i += TPB)
            static_cast<uint16_t*>(oa)[na + i] = static_cast<const uint8_t*>(a)[na + i];
        for (uint32_t i = threadIdx.x; i < tb; i += TPB)
            static_cast<uint16_t*>(ob)[nb + i] = static_cast<const uint8_t*>(b)[nb + i];
    }
}

}  // namespace qkn
