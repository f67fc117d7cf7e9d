// rope_round.h -- RoPE angles and the exact fp64 -> bf16 rounding shared by the
// KV-append kernel and the decode kernel's fused append.
//
// RoPE (Qwen3 decoder, theta 1e6: audio.cpp "Fun-ASR-Nano Native Runtime
// Design", "Decoder And Prompt"), rotate-half pairing: dimension i pairs with
// i + 64, frequency f_i = theta^(-2i/128).  Rotations are evaluated in fp64
// from the exactly widened bf16 inputs and rounded once to bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace hipdecode {
namespace rope {

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kHalf = 64;   // rotation pairs of a 128-dimension head

// Frequency of pair i, theta^(-2i/128) = 2^(-(i/64) log2 theta), in fp64,
// from log2 theta computed once on the host: one exp2 per lane, which is
// much shorter than a pow, and within a few units in the last place of it.
__device__ inline double frequency(double log2_theta, int i) { return exp2(-((double)i / 64.0) * log2_theta); }

// (cos, sin) of the angle pos * freq, in fp64.
__device__ inline double2 angle_of(double freq, int pos)
{
    double sn, c;
    sincos((double)pos * freq, &sn, &c);
    return make_double2(c, sn);
}

// fp64 -> fp32 rounded to odd: the fp32 number next to x towards zero, with
// its last bit set when x is not exactly representable.  fp32 keeps 16 more
// significand bits than bf16 (normal or subnormal alike, the exponent ranges
// being the same), more than the two that rounding to odd needs for a second
// rounding, to bf16 nearest even, to equal the direct one (Boldo and
// Melquiond, "Emulation of FMA and correctly rounded sums: proved algorithms
// using rounding to odd", IEEE Trans. Computers, 2008).  The hardware
// conversion rounds to nearest; it is stepped back by one unit in the last
// place when that went away from zero.
__device__ inline float round_to_odd_f32(double x)
{
    const float t = (float)x;
    const double back = (double)t;
    const bool inexact = back != x;
    uint32_t b = __float_as_uint(t);
    b -= (inexact && fabs(back) > fabs(x)) ? 1u : 0u;
    b |= inexact ? 1u : 0u;
    return __uint_as_float(b);
}

// Nearest-even bf16 bits of x (low half) and y (high half); NaN gives 0x7FC0.
__device__ inline uint32_t pack_bf16(double x, double y)
{
    const f32x2_t v = {round_to_odd_f32(x), round_to_odd_f32(y)};
    uint32_t u = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    u = x != x ? (u & 0xFFFF0000u) | 0x7FC0u : u;
    u = y != y ? (u & 0x0000FFFFu) | 0x7FC00000u : u;
    return u;
}

// bf16 bits of the low (element 0) or high (element 1) half widened to fp64.
__device__ inline double lo_f64(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ inline double hi_f64(uint32_t w) { return (double)__uint_as_float(w & 0xFFFF0000u); }

// Rotates one word of a head: the two dimensions held in `own` (bf16, low
// half first), given the two partner dimensions `partner` (64 higher or
// lower) and their angles c0, c1.  The first half of a head takes
// x cos - partner sin, the second partner sin + x cos.
//
// Rounding: t = fp32 nearest of each fp64 value r, then the hardware's bf16
// nearest even of t.  Every bf16 rounding boundary (a midpoint between bf16
// neighbours) is an fp32 number and rounding is monotonic, so t lies on the
// same side of each boundary as r unless t is itself a boundary; the two
// roundings then agree with the direct one.  When a t is a boundary (low 16
// bits 0x8000, probability about 2^-16 per value) or NaN, the word takes the
// exact path of pack_bf16.
__device__ inline uint32_t rotate2(uint32_t own, uint32_t partner, bool second_half, double2 c0, double2 c1)
{
    const double x0 = lo_f64(own), x1 = hi_f64(own);
    const double y0 = lo_f64(partner), y1 = hi_f64(partner);
    const double r0 = second_half ? x0 * c0.x + y0 * c0.y : x0 * c0.x - y0 * c0.y;
    const double r1 = second_half ? x1 * c1.x + y1 * c1.y : x1 * c1.x - y1 * c1.y;
    const float t0 = (float)r0, t1 = (float)r1;
    const bool unsure = (__float_as_uint(t0) & 0xFFFFu) == 0x8000u || t0 != t0 ||
                        (__float_as_uint(t1) & 0xFFFFu) == 0x8000u || t1 != t1;
    if (__builtin_expect(unsure, 0))
        return pack_bf16(r0, r1);
    const f32x2_t v = {t0, t1};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

}  // namespace rope
}  // namespace hipdecode
