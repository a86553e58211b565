// gdn_mfma.hpp -- matrix-core and staging helpers shared by the chunked kernels
// (gdn_chunked.hip, gdn_bwd_chunked.hip).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gdn_kernels.hpp"

namespace gdn {

typedef float f4 __attribute__((ext_vector_type(4)));

// D = C + A B on a 16 x 16 x 4 fp32 tile.  Lane l = x + 16 g supplies A[x][g] and
// B[g][x]; it receives D[4 g + r][x] in component r.
__device__ __forceinline__ f4 mfma_16x16x4(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f4 f4_zero() { return f4{0.f, 0.f, 0.f, 0.f}; }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not
// for its global loads (__syncthreads also fences global memory, which would make
// every chunk wait for the reads it has just sent out for the next one).  The
// memory clobber keeps the compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Four consecutive io elements as loaded (bf16: 8 bytes, fp32: 16 bytes), widened
// to fp32 only when used, so that prefetched rows take half the registers.
template <class IO>
struct Raw4 {
    using T = typename std::conditional<IO::ESZ == 2, uint2, uint4>::type;
    __device__ static T load(const void *base, size_t idx) {
        return *reinterpret_cast<const T *>(static_cast<const char *>(base) + idx * IO::ESZ);
    }
    // from a (uniform) base pointer and a 32-bit byte offset: one address add per load
    __device__ static T load_at(const char *base, uint32_t off) { return *reinterpret_cast<const T *>(base + off); }
    __device__ static T keep(const T &w, bool on) {
        T z = w;
        if constexpr (IO::ESZ == 2) {
            z.x = on ? w.x : 0u;
            z.y = on ? w.y : 0u;
        } else {
            z.x = on ? w.x : 0u;
            z.y = on ? w.y : 0u;
            z.z = on ? w.z : 0u;
            z.w = on ? w.w : 0u;
        }
        return z;
    }
    __device__ static float4 widen(const T &w) {
        if constexpr (IO::ESZ == 2)
            return make_float4(bf16_to_f32(w.x & 0xffffu), bf16_to_f32(w.x >> 16), bf16_to_f32(w.y & 0xffffu),
                               bf16_to_f32(w.y >> 16));
        else
            return make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w));
    }
    // one element's bits (bf16 in the low half), widened when used
    __device__ static uint32_t load1_at(const char *base, uint32_t off) {
        if constexpr (IO::ESZ == 2)
            return *reinterpret_cast<const uint16_t *>(base + off);
        else
            return *reinterpret_cast<const uint32_t *>(base + off);
    }
    __device__ static float widen1(uint32_t w) { return IO::ESZ == 2 ? bf16_to_f32(w & 0xffffu) : __uint_as_float(w); }
};

// Stores that every lane issues, whether or not it has something to write.  A wave
// counts its outstanding vector memory operations in one in-order counter; a store
// under a branch leaves the count unknown where the paths join, so the next wait for
// earlier loads must wait for the store's acknowledgement too.  A raw buffer store
// past the resource's range is discarded, so a lane with nothing to write passes
// kDropped instead of branching round the store, and the count stays exact.
constexpr uint32_t kDropped = 0x80000000u;

// A raw buffer resource over [base, base + bytes); bytes must be below kDropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// One io element (bf16 rounded to nearest even, as IO::store1) at byte offset off.
template <class IO>
__device__ __forceinline__ void buf_store1(__amdgpu_buffer_rsrc_t r, uint32_t off, float f) {
    if constexpr (IO::ESZ == 2)
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)), r, off, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f), r, off, 0, 0);
}

__device__ __forceinline__ void buf_store_f32(__amdgpu_buffer_rsrc_t r, uint32_t off, float f) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f), r, off, 0, 0);
}

// Four floats as one 16-byte buffer store at byte offset off, nontemporal (written
// once and read back once, by another kernel); kDropped drops it.
__device__ __forceinline__ void buf_store_f4_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, f4 v) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 2);
}

// Sum over the 16 lanes x of each lane group g (lanes 16 g .. 16 g + 15), in the
// fixed butterfly order 8, 4, 2, 1; every lane of the group gets the sum.
__device__ __forceinline__ float sum16(float v) {
    v = v + __shfl_xor(v, 8, 64);
    v = v + __shfl_xor(v, 4, 64);
    v = v + __shfl_xor(v, 2, 64);
    v = v + __shfl_xor(v, 1, 64);
    return v;
}

}  // namespace gdn
