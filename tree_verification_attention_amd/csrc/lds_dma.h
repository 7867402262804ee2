// Device helpers shared by the bf16 attention kernels: operand vector types, direct-to-LDS
// loads and their completion waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ta {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

#define TA_INLINE __attribute__((always_inline))

// A 32-key block whose exponentials (relative to the row's reference maximum) sum past this
// sends the workgroup to its exact path; below it nothing can overflow fp32 or bf16.
constexpr float kSumGuard = 18446744073709551616.0f;  // 2^64

// Wait until at most N vector-memory operations of this wavefront are outstanding (the counter
// holds 63 at most; waiting for fewer is only more conservative).
template <int N>
__device__ TA_INLINE void wait_vmem() {
    constexpr int M = N > 63 ? 63 : N;
    static_assert(M >= 0, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (M & 15) | ((M >> 4) << 14));
}

// LDS byte address of a shared-memory pointer (the value a load-to-LDS instruction takes in M0).
__device__ TA_INLINE uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// 16 bytes per lane from saddr + voff into LDS at m0 + 16 * lane. The load is issued from inline
// assembly so that the compiler does not wait for it before unrelated LDS reads (it cannot tell
// which LDS bytes a direct-to-LDS load writes); completion is awaited with wait_vmem. The
// compiler does not insert wait states for what an inline-assembly load reads either, so the
// s_nop supplies them: five after a VALU write of an SGPR the load reads (saddr may come from
// v_readfirstlane), one after an SALU write of M0.
__device__ TA_INLINE void load_lds_saddr(const void *saddr, uint32_t voff, uint32_t m0) {
    const uint64_t p = (uint64_t)(uintptr_t)saddr;
    const uint64_t u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p) |
                       ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) << 32);
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(u), "{m0}"(m0) : "memory");
}

// Barrier that orders LDS only: direct-to-LDS loads in flight stay in flight across it (their
// completion is tracked with wait_vmem), unlike a full __syncthreads().
__device__ TA_INLINE void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Per-lane placement of a 64-key tile's direct-to-LDS loads (16-byte chunk = 8 bf16 of a key
// row; DCH chunks per row, CB = DCH / 4 column blocks):
//   K: instruction j fills 1 KB block j = 16 keys x 4 chunks, chunk-major: lane l takes key
//      16 (j / CB) + l % 16, chunk 4 (j % CB) + l / 16. The QK operand read of 16 lanes (16
//      consecutive keys, one chunk) is then 256 consecutive bytes.
//   V: instruction j fills four 256-byte blocks of 4 keys x 4 chunks, key-major: lane l takes
//      block 4 j + l / 16, i.e. key 4 (block / CB) + (l / 4) % 4, chunk 4 (block % CB) + l % 4.
// ``row`` is the key inside the tile, ``off`` the byte offset inside the key row.
template <int DCH>
__device__ TA_INLINE void tile_load_pos(bool is_v, int j, int lane, int &row, uint32_t &off) {
    constexpr int CB = DCH / 4;
    if (!is_v) {
        row = 16 * (j / CB) + (lane & 15);
        off = 16u * (uint32_t)(4 * (j % CB) + (lane >> 4));
    } else {
        const int blk = 4 * j + (lane >> 4);
        row = 4 * (blk / CB) + ((lane >> 2) & 3);
        off = 16u * (uint32_t)(4 * (blk % CB) + (lane & 3));
    }
}

// First key (inside the tile) of the aligned group of at most 16 keys that load instruction j
// reads: one page of a paged prefix always holds the whole group.
template <int DCH>
__device__ TA_INLINE int tile_load_group(bool is_v, int j) {
    constexpr int CB = DCH / 4;
    return is_v ? 4 * ((4 * j) / CB) : 16 * (j / CB);
}

}  // namespace ta
