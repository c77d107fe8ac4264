// Device helpers shared by the gfx950 kernels: bf16 storage conversions,
// 64-lane wavefront reductions and MFMA operand vector types.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;                                    // bfloat16 storage (top half of an fp32)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));  // MFMA A/B operand: 8 bf16 per lane
typedef float f32x16 __attribute__((ext_vector_type(16)));  // 32x32 MFMA accumulator per lane
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ bf16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
    return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + __expf(-x)); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Sum over the 32 lanes that share bit 5 of the lane id (one half-wave).
__device__ __forceinline__ float half_wave_sum(float v) {
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Residual-row geometry. The fp32 residual stream is stored stream-major:
// rows [0, B*Nt) are the text stream (registers then text tokens, sample-major),
// rows [B*Nt, B*(Nt+Ni)) the image stream (sample-major). Row-wise operators see
// one matrix; attention maps rows to (sample, sequence position).
struct RowGeom {
    int B;    // samples
    int Nt;   // text-stream tokens per sample (registers + text)
    int Ni;   // image tokens per sample
    __host__ __device__ int S() const { return Nt + Ni; }
    __host__ __device__ int batch_of(int r) const {
        int tr = B * Nt;
        return r < tr ? r / Nt : (r - tr) / Ni;
    }
    __host__ __device__ int seq_of(int r) const {
        int tr = B * Nt;
        return r < tr ? r % Nt : Nt + (r - tr) % Ni;
    }
    __host__ __device__ int row_of(int b, int s) const {
        return s < Nt ? b * Nt + s : B * Nt + b * Ni + (s - Nt);
    }
};
