// Shared device helpers for the gfx950 kernels: bf16 conversion, MFMA
// operand types, wave-level reductions and the status-word update.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pd.h"

namespace pd {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;   // 16 B MFMA operand (16x16x32)
typedef __attribute__((ext_vector_type(4))) short s16x4;     //  8 B MFMA operand (16x16x16)
typedef __attribute__((ext_vector_type(4))) float f32x4;     // 16x16 accumulator slice per lane

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16 bits, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f2bf(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    bf16x8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
    return z;
}

// D(16x16, fp32) += A(16x32) * B(32x16), bf16 inputs. Lane l holds
// A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16] and D[4*(l/16) .. +3][l%16].
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x16) * B(16x16), bf16 inputs. Lane l holds
// A[l%16][4*(l/16) .. +3], B[4*(l/16) .. +3][l%16] and D[4*(l/16) .. +3][l%16].
__device__ __forceinline__ f32x4 mfma_16x16x16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Sum over a 256-thread block; every thread gets the result. `red` holds >= 4 floats.
__device__ __forceinline__ float block_sum_256(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ void flag(int32_t* status, int bits) {
    if (status) atomicOr(status, bits);
}

// Loads and stores of data that another workgroup of the same launch wrote
// or will read (the persistent decode kernel hands activations from phase to
// phase inside one launch). Each XCD has its own L2, which keeps no coherence
// with the others: with CG these accesses carry the device-scope cache bit
// (sc1), so a store is written through to memory and a load is served from
// memory, not from a stale line of the reader's L2. They are relaxed atomic
// accesses of 4 or 8 bytes (16-byte values go as two 8-byte halves); without
// CG they are plain accesses.
template <bool CG, typename T>
__device__ __forceinline__ T ldc(const T* p) {
    if constexpr (!CG) {
        return *p;
    } else if constexpr (sizeof(T) == 4) {
        const uint32_t v = __hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        return __builtin_bit_cast(T, v);
    } else if constexpr (sizeof(T) == 8) {
        const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        return __builtin_bit_cast(T, v);
    } else {
        static_assert(sizeof(T) == 16, "4, 8 or 16 bytes");
        const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
        typedef __attribute__((ext_vector_type(2))) uint64_t u64x2;
        u64x2 v;
        v[0] = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v[1] = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return __builtin_bit_cast(T, v);
    }
}

template <bool CG, typename T>
__device__ __forceinline__ void stc(T* p, const T& v) {
    if constexpr (!CG) {
        *p = v;
    } else if constexpr (sizeof(T) == 2) {
        __hip_atomic_store(reinterpret_cast<uint16_t*>(p), __builtin_bit_cast(uint16_t, v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else if constexpr (sizeof(T) == 4) {
        __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else if constexpr (sizeof(T) == 8) {
        __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
        static_assert(sizeof(T) == 16, "2, 4, 8 or 16 bytes");
        typedef __attribute__((ext_vector_type(2))) uint64_t u64x2;
        const u64x2 w = __builtin_bit_cast(u64x2, v);
        uint64_t* q = reinterpret_cast<uint64_t*>(p);
        __hip_atomic_store(q, (uint64_t)w[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(q + 1, (uint64_t)w[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace pd
