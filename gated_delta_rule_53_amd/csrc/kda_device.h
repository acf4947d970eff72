// kda_device.h -- device-side helpers shared by the KDA kernels (gfx950, wave64).
//
// Matrix-core conventions.  Every tile product here is a 16x16 output tile
// C += A * B computed by one wave with the gfx950 MFMA instructions
//   v_mfma_f32_16x16x32_f16   (fp16 operands, fp32 accumulate, K step 32)
//   v_mfma_f32_16x16x4_f32    (fp32 operands, fp32 accumulate, K step 4)
// Operands are addressed as "K-contiguous rows": A row i (0..15) starts at
// A + i*lda and B column j (0..15) starts at Bt + j*ldb, i.e. B is passed
// transposed.  For lane l, with i = l & 15 and g = l >> 4, the fp16 form
// feeds A[i][k0+8g .. k0+8g+7] and B[k0+8g .. +7][i]; the fp32 form feeds
// A[i][k0+g] and B[k0+g][i].  The accumulator element acc[r] of lane l is
// C[4g + r][i].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;  // tokens per chunk

struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(uint32_t(x.bits) << 16); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    // round to nearest even; inputs here are finite
    uint32_t u = __float_as_uint(f);
    uint32_t r = ((u >> 16) & 1u) + 0x7FFFu;
    bf16_t b;
    b.bits = uint16_t((u + r) >> 16);
    return b;
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }
template <>
__device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }

// exp(x) through the hardware base-2 exponential
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// ---------------------------------------------------------------------------
// Tile products.  OT is the operand type held in memory (LDS or global).
// ---------------------------------------------------------------------------
template <typename OT>
struct Mma;

template <>
struct Mma<_Float16> {
    static constexpr int KSTEP = 32;
    __device__ __forceinline__ static void step(floatx4& acc, const _Float16* a, const _Float16* b, int g) {
        half8 av = *reinterpret_cast<const half8*>(a + 8 * g);
        half8 bv = *reinterpret_cast<const half8*>(b + 8 * g);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc, 0, 0, 0);
    }
};

template <>
struct Mma<float> {
    static constexpr int KSTEP = 4;
    __device__ __forceinline__ static void step(floatx4& acc, const float* a, const float* b, int g) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[g], b[g], acc, 0, 0, 0);
    }
};

// acc += A[16 x K] * B[K x 16]; A rows K-contiguous (lda), B given as B^T rows (ldb).
template <typename OT>
__device__ __forceinline__ void mma_tile(floatx4& acc, const OT* A, int lda, const OT* Bt, int ldb, int K,
                                         int lane) {
    const int i = lane & 15, g = lane >> 4;
    const OT* a = A + i * lda;
    const OT* b = Bt + i * ldb;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += Mma<OT>::KSTEP) Mma<OT>::step(acc, a + k0, b + k0, g);
}

// Workgroup barrier that orders LDS only: global loads issued before it stay in
// flight (a plain __syncthreads() also waits for every outstanding global access,
// which would drain any prefetch).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders the LDS accesses of one wave's lanes: writes before it are seen by
// reads after it from any lane of the same wave (LDS executes a wave's
// operations in order, so only compiler reordering has to be prevented).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

__device__ __forceinline__ floatx4 zero4() {
    floatx4 z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

}  // namespace kda
