// hsw_device.h -- device-side helpers shared by the gfx950 kernels of libhsw.
//
// Vector types for MFMA operands, bf16 <-> fp32 conversions, 16-byte global
// loads/stores and wave-level reductions.  gfx950 only: wave64, MFMA
// v_mfma_f32_16x16x32_bf16 (8 bf16 per lane per operand) and
// v_mfma_f32_16x16x16_{bf16,f16} (4 per lane).
//
// Lane layout of the 16x16 MFMA family used throughout (wave64, lane l,
// quad q = l / 16, column c = l % 16):
//   A (16 x K):  lane l holds row c, K-slots of quad q;
//   B (K x 16):  lane l holds column c, K-slots of quad q;
//   D (16 x 16): lane l holds column c, rows 4q .. 4q+3.
// Which K index each (quad, slot) pair denotes only has to agree between A
// and B, since the product sums over K; every kernel loads A and B with the
// same (quad, slot) -> K mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hsw {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ u32x4 ld16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void st16(void *p, u32x4 v) {
    *reinterpret_cast<u32x4 *>(p) = v;
}

// Builds with HSW_CHECK_DEVICE=1 launch a check of the call's device-resident
// arguments before its kernels; each kernel then returns at once if the check
// recorded a violation (the flag is written by an earlier kernel on the same
// stream).  Release builds compile this to nothing.
#ifndef HSW_CHECK_DEVICE
#define HSW_CHECK_DEVICE 0
#endif
__device__ __forceinline__ bool checks_failed(const unsigned long long *flag) {
#if HSW_CHECK_DEVICE
    return flag != nullptr && *flag != 0ull;
#else
    (void)flag;
    return false;
#endif
}

__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x32_f16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x16_bf16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(u16x4, a),
                                                     __builtin_bit_cast(u16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x16_f16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed fp16, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, f16x2{(_Float16)a, (_Float16)b});
}

// Two bf16 (packed in one word) -> two fp16 (packed), round to nearest even:
// exact for |v| in the fp16 normal range; |v| >= 65536 becomes infinity.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
    return pack_f16x2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (a low, b high), round to nearest even: one
// v_cvt_pk_bf16_f32 (converting the halves one at a time costs three
// instructions per pair).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
}

// Split four fp32 values into bf16 hi = bf16(p) and lo = bf16(p - hi) so that
// hi + lo carries about 16 significant bits of p.  (Element by element: the
// packed-pair form needs more live registers where the prefill kernels sit at
// the 256-VGPR limit, and spilled there.)
__device__ __forceinline__ void split_hi_lo(const float p[4], u32x2 &hi, u32x2 &lo) {
    uint16_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = f2bf(p[i]);
        l[i] = f2bf(p[i] - bf2f(h[i]));
    }
    hi = u32x2{(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
    lo = u32x2{(uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16)};
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
    return fmaxf(v, __shfl_xor(v, mask, kWave));
}
__device__ __forceinline__ float wave_sum_xor(float v, int mask) {
    return v + __shfl_xor(v, mask, kWave);
}

// Reduce over the four quads (lanes c, c+16, c+32, c+48).
__device__ __forceinline__ float quad_max(float v) {
    v = wave_max_xor(v, 16);
    return wave_max_xor(v, 32);
}
__device__ __forceinline__ float quad_sum(float v) {
    v = wave_sum_xor(v, 16);
    return wave_sum_xor(v, 32);
}

// Rotate-half RoPE pieces shared by the RoPE kernel and the attention kernels
// that rotate q as they load it, so both produce the same bits.
// colibri "What the engine implements": pairs (i, i + rope_dim/2) of the
// first rope_dim dims turn by pos * theta^(-2i/rope_dim); gaudi-cookbook
// "The RoPE fix for large positions": that angle reaches 5e5 rad and must be
// formed and reduced in double precision.  The frequencies theta^(-2i/R) come
// from the host (libm pow in double).  Here a = pos * inv_freq in double, then
// Cody-Waite reduction by pi/2 in double: k = rint(a * 2/pi),
// r = (a - k * PIO2_HI) - k * PIO2_LO with PIO2_HI + PIO2_LO = pi/2 to 3.5e-27
// (each step one fma, whose product is exact), so |r| <= pi/4 carries the
// angle to about one double ulp of a.  cos r and sin r are then the Taylor
// polynomials through r^10 / r^9 in fp32 (truncation below 2e-9 on
// |r| <= pi/4) and the quadrant k mod 4 swaps / negates them.
__device__ __forceinline__ void rope_cos_sin(int64_t pos, double inv_freq, float &c, float &s) {
    constexpr double kTwoOverPi = 0.6366197723675814;
    constexpr double kPio2Hi = 1.5707963267341256;      // pi/2 to 33 bits
    constexpr double kPio2Lo = 6.077100506506192e-11;   // pi/2 - kPio2Hi
    const double a = (double)pos * inv_freq;
    const double k = rint(a * kTwoOverPi);
    const double r = fma(-k, kPio2Lo, fma(-k, kPio2Hi, a));
    const float x = (float)r, x2 = x * x;
    float sp = fmaf(x2, 1.0f / 362880.0f, -1.0f / 5040.0f);
    sp = fmaf(x2, sp, 1.0f / 120.0f);
    sp = fmaf(x2, sp, -1.0f / 6.0f);
    const float sr = fmaf(x * x2, sp, x);
    float cp = fmaf(x2, -1.0f / 3628800.0f, 1.0f / 40320.0f);
    cp = fmaf(x2, cp, -1.0f / 720.0f);
    cp = fmaf(x2, cp, 1.0f / 24.0f);
    cp = fmaf(x2, cp, -0.5f);
    const float cr = fmaf(x2, cp, 1.0f);
    const int q = (int)((long long)k & 3);
    c = q == 0 ? cr : q == 1 ? -sr : q == 2 ? -cr : sr;
    s = q == 0 ? sr : q == 1 ? cr : q == 2 ? -sr : -cr;
}
// (x_lo, x_hi) -> (x_lo c - x_hi s, x_hi c + x_lo s), with the fused
// multiply-adds spelled out so every kernel rounds identically.
__device__ __forceinline__ void rope_rotate(float xl, float xh, float c, float s, float &yl, float &yh) {
    yl = fmaf(xl, c, -(xh * s));
    yh = fmaf(xh, c, xl * s);
}
// The same on 8 packed bf16 pairs (16 bytes each), rounded to bf16.
__device__ __forceinline__ void rope_rotate_bf16x8(u32x4 &lo, u32x4 &hi, const float c[8], const float s[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float yl0, yh0, yl1, yh1;
        rope_rotate(__uint_as_float(lo[i] << 16), __uint_as_float(hi[i] << 16), c[2 * i], s[2 * i], yl0, yh0);
        rope_rotate(__uint_as_float(lo[i] & 0xffff0000u), __uint_as_float(hi[i] & 0xffff0000u), c[2 * i + 1],
                    s[2 * i + 1], yl1, yh1);
        lo[i] = pack_bf16x2(yl0, yl1);
        hi[i] = pack_bf16x2(yh0, yh1);
    }
}

// Wait until at most N vector-memory operations of the wave are outstanding
// and redefine the twelve q registers there: uses of q (filled by untracked
// loads) cannot be scheduled above the wait, which a bare s_waitcnt does not
// guarantee.
template <int N>
__device__ __forceinline__ void wait_vmcnt_q(u32x4 (&q)[2][6]) {
    asm volatile("s_waitcnt vmcnt(%12)"
                 : "+v"(q[0][0]), "+v"(q[0][1]), "+v"(q[0][2]), "+v"(q[0][3]), "+v"(q[0][4]), "+v"(q[0][5]),
                   "+v"(q[1][0]), "+v"(q[1][1]), "+v"(q[1][2]), "+v"(q[1][3]), "+v"(q[1][4]), "+v"(q[1][5])
                 : "n"(N)
                 : "memory");
}

// Redefine the twelve q registers here (no instruction).  After q was loaded
// by tracked loads, the compiler's waits for every one of them land before
// this point, once, rather than at each register's first use inside a loop,
// where, counting only its own loads, each would also wait for the untracked
// chunk loads in flight.
__device__ __forceinline__ void settle_q(u32x4 (&q)[2][6]) {
    asm volatile(""
                 : "+v"(q[0][0]), "+v"(q[0][1]), "+v"(q[0][2]), "+v"(q[0][3]), "+v"(q[0][4]), "+v"(q[0][5]),
                   "+v"(q[1][0]), "+v"(q[1][1]), "+v"(q[1][2]), "+v"(q[1][3]), "+v"(q[1][4]), "+v"(q[1][5]));
}

// A value loaded by an ordinary (tracked) load, forced to have arrived here:
// placed before a kernel's untracked loads, the compiler's wait for it cannot
// land after them (where, counting only its own loads, it would be vmcnt(0)).
__device__ __forceinline__ double pin_loaded(double x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t *p) { return bf2f(*p); }
    static __device__ __forceinline__ void store(uint16_t *p, float f) { *p = f2bf(f); }
};
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float *p) { return *p; }
    static __device__ __forceinline__ void store(float *p, float f) { *p = f; }
};

}  // namespace hsw
