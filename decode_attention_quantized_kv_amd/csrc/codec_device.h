// Device-side quantizer of the k8v4 codec, shared by the append kernel and
// the decode kernel that appends the step's new token itself.  One wavefront
// quantizes one (token, kv head): lane i holds dimensions (D/64)*i ..
// (D/64)*i + D/64 - 1.  Rules (blog.123qwe.co.kr/?p=3927, section 5: 8-bit
// keys, 4-bit values in groups of 32 with fp16 scales): symmetric absmax --
// s = fp16_rne(max|x| / q), code = clamp(rint(x / s), -q, q) with q = 127
// (keys) or 7 (values), an fp16 overflow of s saturating to 65504 and s == 0
// giving zero codes -- or the affine variant (unsigned codes with a zero
// point over the range widened to include zero).  The divisions are IEEE
// fp32 divisions and rintf rounds half to even, so every caller produces the
// same bits.
#pragma once

#include "q8k4v_device.h"

namespace q8k4v {

template <int D, bool BF16>
Q8K4V_DEV void load_row(const void* base, size_t row, int lane, float (&x)[D / 64]) {
    constexpr int EPL = D / 64;
    if (BF16) {
        const uint16_t* p = (const uint16_t*)base + row * D + EPL * lane;
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = bf16_to_f32(p[e]);
    } else {
        const float* p = (const float*)base + row * D + EPL * lane;
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = p[e];
    }
}

Q8K4V_DEV float wave_max(float x, int lanes) {
    for (int m = 1; m < lanes; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}

Q8K4V_DEV float wave_min(float x, int lanes) {
    for (int m = 1; m < lanes; m <<= 1) x = fminf(x, __shfl_xor(x, m));
    return x;
}

// fp16 scale of an absmax: IEEE fp32 division, RNE into fp16, saturating.
Q8K4V_DEV _Float16 scale_of(float absmax, float qmax) {
    const float s32 = absmax / qmax;
    _Float16 s16 = (_Float16)s32;
    if (__builtin_isinf((float)s16)) s16 = (_Float16)65504.0f;
    return s16;
}

Q8K4V_DEV int code_of(float x, float s, float qmax) {
    if (s == 0.0f) return 0;
    float r = rintf(x / s);
    r = fminf(fmaxf(r, -qmax), qmax);
    return (int)r;
}

// Affine block parameters from the block's min and max (over the lanes that
// hold it): fp16 scale and zero point.
struct Affine {
    _Float16 s16;
    float s, z;
};

Q8K4V_DEV Affine affine_of(float mn, float mx, float qmax) {
    const float lo = fminf(mn, 0.0f), hi = fmaxf(mx, 0.0f);
    Affine a;
    a.s16 = scale_of(hi - lo, qmax);
    a.s = (float)a.s16;
    a.z = (a.s == 0.0f) ? 0.0f : fminf(fmaxf(rintf(-lo / a.s), 0.0f), qmax);
    return a;
}

Q8K4V_DEV int affine_code(float x, const Affine& a, float qmax) {
    if (a.s == 0.0f) return 0;
    return (int)fminf(fmaxf(rintf(x / a.s) + a.z, 0.0f), qmax);
}

// Value codes of one token for this lane's dimensions (nibble values: two's
// complement when symmetric, unsigned when affine), with its group's scale
// (and zero point) reduced over the LPG lanes of the group.
template <int EPL, int LPG, bool AFF>
Q8K4V_DEV void value_codes(const float (&x)[EPL], int (&c)[EPL], _Float16* s16, int* z) {
    if (AFF) {
        float mn = x[0], mx = x[0];
#pragma unroll
        for (int e = 1; e < EPL; ++e) { mn = fminf(mn, x[e]); mx = fmaxf(mx, x[e]); }
        const Affine a = affine_of(wave_min(mn, LPG), wave_max(mx, LPG), 15.0f);
#pragma unroll
        for (int e = 0; e < EPL; ++e) c[e] = affine_code(x[e], a, 15.0f);
        *s16 = a.s16;
        *z = (int)a.z;
    } else {
        float va = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) va = fmaxf(va, fabsf(x[e]));
        va = wave_max(va, LPG);
        *s16 = scale_of(va, 7.0f);
        const float vs = (float)*s16;
#pragma unroll
        for (int e = 0; e < EPL; ++e) c[e] = code_of(x[e], vs, 7.0f);
        *z = 0;
    }
}

}  // namespace q8k4v
