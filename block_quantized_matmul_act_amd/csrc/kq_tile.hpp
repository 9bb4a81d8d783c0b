// kq_tile.hpp -- building blocks of the persistent tile kernels (gfx950):
// buffer resources and buffer -> LDS copies, explicit vector-memory and LDS
// waits, LDS reads written as instructions of our own, and the int8 / bf16
// matrix-core calls.
#pragma once

#include "kq_device.hpp"

namespace kq {
namespace tl {

constexpr int RSRC_FLAGS = 0x00020000;
// A store offset the buffer range check always drops: the host checks that
// every row offset, overhanging tile rows included, stays below 2^31, so
// adding this cannot wrap 2^32 and always lands past the output.
constexpr int OOB_VOFF = (int)0x80000000u;

typedef __attribute__((address_space(3))) void *lds_ptr_t;

__device__ __forceinline__ v16i mma_i8(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16f mma_bf16(v8bf a, v8bf b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4i mma16_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mma16_bf16(v8bf a, v8bf b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// s_waitcnt on the vector-memory counter only (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier without a memory fence (a fence would also wait for the
// copies in flight).  LDS filled by buffer->LDS copies is made visible by the
// vmcnt wait each wave performs before it.
__device__ __forceinline__ void barrier_nofence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t rs, void *lds, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void copy4(__amdgpu_buffer_rsrc_t rs, void *lds, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds, 4, voff, soff, 0, 0);
}
__device__ __forceinline__ v4i ld16(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0));
}
__device__ __forceinline__ v2u ld8(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
    return __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0));
}
__device__ __forceinline__ uint32_t ld4(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
}

// LDS reads of staged data, written as instructions of our own: the
// compiler's wait insertion tracks only a few buffer -> LDS copies at a time
// and, past that, makes every LDS read wait for the newest copy in flight.
// The caller orders these reads after the copies they need with an explicit
// vmcnt wait and makes each result usable with lds_wait.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
template <int OFF>
__device__ __forceinline__ v4i lds_read16(uint32_t addr) {
    v4i r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
template <int OFF>
__device__ __forceinline__ v2u lds_read8(uint32_t addr) {
    v2u r;
    asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
// lgkmcnt wait with a count known only after unrolling (folds to one case)
template <typename R>
__device__ __forceinline__ void lds_wait_n(int n, R &r);
// s_waitcnt lgkmcnt(N), tied to a register it guards so that no use of that
// register is scheduled above it
template <int N>
__device__ __forceinline__ void lds_wait(v4i &r) {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "i"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait(v4f &r) {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "i"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait(v2u &r) {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "i"(N));
}
template <typename R>
__device__ __forceinline__ void lds_wait_n(int n, R &r) {
    switch (n) {
        case 0: lds_wait<0>(r); break;
        case 1: lds_wait<1>(r); break;
        case 2: lds_wait<2>(r); break;
        case 3: lds_wait<3>(r); break;
        case 4: lds_wait<4>(r); break;
        case 5: lds_wait<5>(r); break;
        case 6: lds_wait<6>(r); break;
        case 7: lds_wait<7>(r); break;
        case 8: lds_wait<8>(r); break;
        case 9: lds_wait<9>(r); break;
        case 10: lds_wait<10>(r); break;
        case 11: lds_wait<11>(r); break;
        case 12: lds_wait<12>(r); break;
        case 13: lds_wait<13>(r); break;
        case 14: lds_wait<14>(r); break;
        default: lds_wait<15>(r); break;
    }
}

}  // namespace tl
}  // namespace kq
