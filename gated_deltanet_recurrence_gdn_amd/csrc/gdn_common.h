// gdn_common.h -- small device helpers shared by the GDN kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// bf16 <-> fp32.  Widening is exact (bf16 is the top half of an fp32).
// Narrowing is the native conversion (v_cvt_pk_bf16_f32 on gfx950): round to
// nearest even, NaN stays NaN.
typedef __bf16 gdn_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float gdn_f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const gdn_f32x2_t v = {lo, hi};
    const gdn_bf16x2_t b = __builtin_convertvector(v, gdn_bf16x2_t);
    uint32_t u;
    __builtin_memcpy(&u, &b, 4);
    return u;
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    const __bf16 b = (__bf16)f;
    uint16_t u;
    __builtin_memcpy(&u, &b, 2);
    return u;
}

// OCP FP8 E4M3 -> bf16 / fp32 with gfx950's conversion instructions at scale 1.
// Every finite E4M3 value is exactly a bf16 (3 mantissa bits, exponents 2^-9 ..
// 2^8), so the widening is exact; NaN stays NaN.
// fp8x4_to_bf16x4: bytes 0-3 of w -> four bf16, two per returned word.
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
    const gdn_bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const gdn_bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    uint2 r;
    __builtin_memcpy(&r.x, &lo, 4);
    __builtin_memcpy(&r.y, &hi, 4);
    return r;
}
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float *f) {
    const gdn_f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const gdn_f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    f[0] = lo[0];
    f[1] = lo[1];
    f[2] = hi[0];
    f[3] = hi[1];
}

// Cross-lane data movement inside a row of 16 lanes (DPP).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of L consecutive lanes (L in {1, 2, 4, 8, 16}); every
// lane of the group receives the group sum.
template <int L>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(L == 1 || L == 2 || L == 4 || L == 8 || L == 16, "group size");
    if constexpr (L >= 2) x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (L >= 4) x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (L >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror: other quad of the 8
    if constexpr (L >= 16) x += dpp_mov<0x140>(x); // row_mirror: other half of the 16
    return x;
}

// ---- the fused prologue's activations (fp32) --------------------------------
// b = sigmoid(x); a = exp(-softplus(x)) = 1 / (1 + e^x); log2 a = -softplus(x) / ln 2,
// written as -(max(y, 0) + log2(1 + 2^-|y|)) with y = x log2 e so that nothing
// overflows for large |x|.
constexpr float LOG2E_F = 1.4426950408889634f;
__device__ __forceinline__ float sigmoid_f32(float x) { return 1.0f / (1.0f + exp2f(-x * LOG2E_F)); }
__device__ __forceinline__ float decay_from_logit(float x) { return 1.0f / (1.0f + exp2f(x * LOG2E_F)); }
__device__ __forceinline__ float log2_decay_from_logit(float x) {
    const float y = x * LOG2E_F;
    return -(fmaxf(y, 0.0f) + log2f(1.0f + exp2f(-fabsf(y))));
}
// 1 / max(||x||_2, 1e-12) from the sum of squares: a zero row stays zero.
__device__ __forceinline__ float inv_norm(float sumsq) { return 1.0f / fmaxf(sqrtf(sumsq), 1e-12f); }

}  // namespace gdn
