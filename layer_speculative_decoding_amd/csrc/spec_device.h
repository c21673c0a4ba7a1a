// Device-side helpers shared by the libspec kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spec {

constexpr int kWave = 64;

// ------------------------------------------------------------ bfloat16
// bfloat16 is carried as raw uint16_t bits; conversion to float is exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
// Round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Storage traits: T is either float or uint16_t (bfloat16 bits).
template <typename T> struct Store;
template <> struct Store<float> {
    static constexpr int kPer16 = 4;  // elements per 16-byte vector
    __device__ __forceinline__ static float round(float x) { return x; }
    __device__ __forceinline__ static float to_f32(float x) { return x; }
    __device__ __forceinline__ static float from_f32(float x) { return x; }
    __device__ __forceinline__ static void unpack(const uint4 &v, float *o) {
        o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
        o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
    }
};
template <> struct Store<uint16_t> {
    static constexpr int kPer16 = 8;
    __device__ __forceinline__ static float round(float x) { return bf16_to_f32(f32_to_bf16(x)); }
    __device__ __forceinline__ static float to_f32(uint16_t x) { return bf16_to_f32(x); }
    __device__ __forceinline__ static uint16_t from_f32(float x) { return f32_to_bf16(x); }
    __device__ __forceinline__ static void unpack(const uint4 &v, float *o) {
        o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
        o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
    }
};

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// Activation buffers are float32 on both paths.  A bfloat16 matrix-core
// product takes a float32 operand as two bfloat16 pieces hi + lo (hi the
// float32 value with its low 16 bits dropped, lo the remainder rounded to
// nearest): the pair carries the value to within 2^-16 of its magnitude, and
// each piece times a bfloat16 weight is exact in float32, so two products
// replace one float32 product at that precision.
__device__ __forceinline__ void split2_one(float x, uint16_t &hi, uint16_t &lo) {
    const uint32_t u = __float_as_uint(x);
    hi = (uint16_t)(u >> 16);
    lo = f32_to_bf16(x - __uint_as_float(u & 0xFFFF0000u));
}
__device__ __forceinline__ void split2_bf16(const uint4 &a, const uint4 &b, uint4 &hi, uint4 &lo) {
    const uint32_t x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x0 = x[2 * i] & 0xFFFF0000u, x1 = x[2 * i + 1] & 0xFFFF0000u;
        h[i] = (x0 >> 16) | x1;
        const uint16_t l0 = f32_to_bf16(__uint_as_float(x[2 * i]) - __uint_as_float(x0));
        const uint16_t l1 = f32_to_bf16(__uint_as_float(x[2 * i + 1]) - __uint_as_float(x1));
        l[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}
// Two floats to packed bfloat16, round to nearest even (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    const f32x2_t v = {a, b};
    const bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
    uint32_t u;
    __builtin_memcpy(&u, &r, 4);
    return u;
}
// split2_bf16 of x[0..7] with the hardware conversion for the lo pieces
__device__ __forceinline__ void split2_bf16_hw(const float *x, uint4 &hi, uint4 &lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x0 = __float_as_uint(x[2 * i]) & 0xFFFF0000u, x1 = __float_as_uint(x[2 * i + 1]) & 0xFFFF0000u;
        h[i] = (x0 >> 16) | x1;
        l[i] = cvt_pk_bf16(x[2 * i] - __uint_as_float(x0), x[2 * i + 1] - __uint_as_float(x1));
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// Streaming (non-temporal) 16-byte load for data read once per step.
__device__ __forceinline__ uint4 ld16_stream(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------------------ reductions
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
// (value, index) arg-max with ties to the lowest index.
__device__ __forceinline__ void argmax_merge(float &v, int &i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float v2 = __shfl_xor(v, o, kWave);
        int i2 = __shfl_xor(i, o, kWave);
        argmax_merge(v, i, v2, i2);
    }
}

// ------------------------------------------------------------ Philox4x64-10
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC'11): ten rounds of two 64x64->128 multiplies, word exchange and key xor,
// the key bumped by the Weyl constants between rounds.
struct Philox4 { uint64_t w[4]; };
__device__ __forceinline__ Philox4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                                 uint64_t k0, uint64_t k1) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += W0; k1 += W1; }
        const uint64_t lo0 = M0 * c0, hi0 = __umul64hi(M0, c0);
        const uint64_t lo1 = M1 * c2, hi1 = __umul64hi(M1, c2);
        const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    }
    Philox4 r; r.w[0] = c0; r.w[1] = c1; r.w[2] = c2; r.w[3] = c3;
    return r;
}
// (2m + 1) * 2^-24 with m the top 23 bits: exact in float32, in (0, 1).
__device__ __forceinline__ float word_to_uniform(uint64_t w) {
    return ((float)(uint32_t)(w >> 41) + 0.5f) * 1.1920928955078125e-07f;  // 2^-23
}
// Stream purposes.
enum : uint32_t { kDraft = 0, kAccept = 1, kTarget = 2 };
// Gumbel noise -log(-log u) for vocab entries v .. v+3 (v a multiple of 4).
__device__ __forceinline__ void gumbel4(uint64_t seed, uint32_t b, uint32_t pos, uint32_t purpose,
                                        uint32_t v4, float g[4]) {
    Philox4 r = philox4x64_10(v4, pos, 0, purpose, seed, b);
#pragma unroll
    for (int i = 0; i < 4; ++i) g[i] = -logf(-logf(word_to_uniform(r.w[i])));
}
__device__ __forceinline__ float pick_word(const Philox4 &r, uint32_t i) {
    const uint64_t w = i == 0 ? r.w[0] : (i == 1 ? r.w[1] : (i == 2 ? r.w[2] : r.w[3]));
    return -logf(-logf(word_to_uniform(w)));
}
// Gumbel noise of vocab entries v0 and v1 (one Philox block when they share it).
__device__ __forceinline__ void gumbel_pair(uint64_t seed, uint32_t b, uint32_t pos, uint32_t purpose,
                                            uint32_t v0, uint32_t v1, float &g0, float &g1) {
    const Philox4 r = philox4x64_10(v0 >> 2, pos, 0, purpose, seed, b);
    g0 = pick_word(r, v0 & 3);
    if ((v1 >> 2) == (v0 >> 2)) {
        g1 = pick_word(r, v1 & 3);
    } else {
        const Philox4 r1 = philox4x64_10(v1 >> 2, pos, 0, purpose, seed, b);
        g1 = pick_word(r1, v1 & 3);
    }
}
__device__ __forceinline__ float accept_uniform(uint64_t seed, uint32_t b, uint32_t pos) {
    Philox4 r = philox4x64_10(0, pos, 0, kAccept, seed, b);
    return word_to_uniform(r.w[0]);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

}  // namespace spec
