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

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest, ties to even: gfx950's v_cvt_pk_bf16_f32 (one
// instruction for two values; for finite inputs it gives the same bits as adding
// 0x7FFF plus the kept lsb and truncating).
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// ---- MXFP8 (E4M3 elements with a power-of-two scale per 32 values)
// Scale exponent of a block whose largest magnitude is amax: floor(log2(amax)) - 8
// (8 = exponent of E4M3's largest normal, 448), at least -127; amax = 0 (or an
// fp32 denormal) gives -127. Read from the exponent field, so exact.
__device__ __forceinline__ int mx_scale_exp(float amax) {
    const int ef = (int)((__float_as_uint(amax) >> 23) & 255);
    return ef == 0 ? -127 : max(ef - 127 - 8, -127);
}
// 2^k for k in [-126, 127], exact.
__device__ __forceinline__ float pow2f(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }
// Four values -> four E4M3 bytes (round to nearest even; values clamped to
// +-448 first, since the conversion turns larger magnitudes into NaN).
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
    a = fminf(fmaxf(a, -448.f), 448.f);
    b = fminf(fmaxf(b, -448.f), 448.f);
    c = fminf(fmaxf(c, -448.f), 448.f);
    d = fminf(fmaxf(d, -448.f), 448.f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// x * sigmoid(x) with the hardware exponential and reciprocal (v_exp_f32,
// v_rcp_f32: about 1 ulp each; __fdividef compiles to the full IEEE division
// sequence here, about ten VALU instructions per element).
__device__ __forceinline__ float silu_f(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// GELU in its tanh form, 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), written
// as x * sigmoid(2 sqrt(2/pi) (x + 0.044715 x^3)) (the same function: 0.5 (1 + tanh z)
// = sigmoid(2 z)).
__device__ __forceinline__ float gelu_tanh_f(float x) {
    const float z = 1.5957691216057308f * (x + 0.044715f * x * x * x);
    return x * __builtin_amdgcn_rcpf(1.f + __expf(-z));
}

// Lane reductions through DPP (row-local VALU operand swizzles) rather than
// LDS-routed permutes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over each 16-lane DPP row; every lane receives its row's sum.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
    v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
    v += dpp_f<0x141>(v);   // row_half_mirror: the other quad of each 8
    v += dpp_f<0x140>(v);   // row_mirror: the other 8 of each 16
    return v;
}
// Sum over the 32 lanes that share bit 5 of the lane id (one half-wave).
__device__ __forceinline__ float half_wave_sum(float v) {
    v = row16_sum(v);
    return v + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));   // lane ^ 16 within 32
}
// Sum over all 64 lanes (uniform result).
__device__ __forceinline__ float wave_sum(float v) {
    v = half_wave_sum(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
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
