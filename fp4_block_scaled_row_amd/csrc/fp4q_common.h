// fp4q_common.h -- device helpers shared by the gfx950 kernels of libfp4q.
//
// Number formats follow "MXFP4 Quantization: Audit the 4.25-Bit Blocks"
// (E2M1 lattice, E8M0 scale) and "Sub-4-Bit Microscaling" section 2 (E4M3
// block scale, fp32 tensor scale).  Nothing here is shared with the CPU
// oracle used by the tests.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;   // 4 wave64 per workgroup
constexpr int kWaves = kThreads / 64;

enum InType { kF32 = 0, kBF16 = 1 };
enum Rot { kRotNone = 0, kRotFwhtRow = 1, kRotRht16 = 2, kRotFwht128 = 3 };

// ----------------------------------------------------------------------------
// bit casts and widening
__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return as_f(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return as_f(w & 0xFFFF0000u); }

// fp32 value whose exponent field encodes E8M0 byte b (the scale operand of the
// gfx950 scaled FP4 conversions reads only this field: 2^(b - 127)).
__device__ __forceinline__ float e8m0_operand(uint32_t b) { return as_f(b << 23); }

// ----------------------------------------------------------------------------
// cross-lane helpers (wave64)
// Every control used here reads a valid lane for every lane, so bound_ctrl
// changes nothing; with it set (and old = 0) the compiler folds the move into
// the consuming VALU instruction as its DPP operand.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kQuadEven = 0xA0;  // quad_perm [0,0,2,2]: each lane pair takes its even lane's value
constexpr int kQuadOdd = 0xF5;   // quad_perm [1,1,3,3]: each lane pair takes its odd lane's value
constexpr int kRowHalfMirror = 0x141;  // lane i of each 8-lane half-row <- lane 7 - i
constexpr int kRowRor8 = 0x128;        // row_ror:8: lane i of each 16-lane row <- lane (i + 8) mod 16 = i ^ 8

__device__ __forceinline__ float dpp_xor1_f(float v) { return as_f(dpp_u32<kQuadXor1>(as_u(v))); }
__device__ __forceinline__ float dpp_xor2_f(float v) { return as_f(dpp_u32<kQuadXor2>(as_u(v))); }
__device__ __forceinline__ float dpp_xor8_f(float v) { return as_f(dpp_u32<kRowRor8>(as_u(v))); }

// max(m, |a|, |b|) in one v_max3_f32 with absolute-value modifiers.  It
// passes over quiet NaNs as fmaxf does; callers give it arithmetic results,
// which are never signalling NaNs, so the canonicalising max the compiler
// puts before each fmaxf operand is not needed.
__device__ __forceinline__ float max3_abs(float m, float a, float b) {
  float r;
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(m), "v"(a), "v"(b));
  return r;
}

// Largest |v[i]| of 8 values as an fp32 bit pattern, the same value as the
// integer maximum of the magnitude bits (as_u(v) & 0x7FFFFFFF) for every
// input without a NaN; a NaN anywhere gives a NaN pattern, which like the
// integer maximum is at least 0x7F800000.  Four v_maximum3_f32 (the IEEE
// maximum, which propagates NaNs) with absolute-value modifiers, against
// eight masks and four integer maxima.
__device__ __forceinline__ uint32_t abs_max_bits8(const float v[8]) {
  float m;
  asm("v_maximum3_f32 %0, |%1|, |%2|, |%3|\n\t"
      "v_maximum3_f32 %0, %0, |%4|, |%5|\n\t"
      "v_maximum3_f32 %0, %0, |%6|, |%7|\n\t"
      "v_maximum3_f32 %0, %0, |%8|, |%8|"
      : "=&v"(m) : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
  return as_u(m);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t p = (uint32_t)__shfl_xor((int)v, o, 64);
    v = v > p ? v : p;
  }
  return v;
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ----------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11): counter (c0..c3), key (k0, k1).
struct U4 { uint32_t x, y, z, w; };
__host__ __device__ __forceinline__ U4 philox4x32_10(U4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    U4 n;
    n.x = (uint32_t)(p1 >> 32) ^ c.y ^ k0;
    n.y = (uint32_t)p1;
    n.z = (uint32_t)(p0 >> 32) ^ c.w ^ k1;
    n.w = (uint32_t)p0;
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// The same rounds in a kernel whose key is uniform across the wave (a kernel
// argument): each round's two three-way XORs (product high word, counter
// word, key) are one v_bitop3_b32 each (truth table 0x96, the parity of its
// three inputs) with the key in a scalar register, 4 instead of 6 vector
// instructions per round (the compiler keeps the key XOR apart).  Same
// outputs as philox4x32_10.
__device__ __forceinline__ uint32_t xor3_uniform(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}
__device__ __forceinline__ U4 philox4x32_10_uniform_key(U4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    U4 n;
    n.x = xor3_uniform((uint32_t)(p1 >> 32), c.y, k0);
    n.y = (uint32_t)p1;
    n.z = xor3_uniform((uint32_t)(p0 >> 32), c.w, k1);
    n.w = (uint32_t)p0;
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Sixteen-bit draw for element (8*g + f) of a Philox output block.
__device__ __forceinline__ uint32_t draw16(const U4& o, int f) {
  const uint32_t w = (f >> 1) == 0 ? o.x : (f >> 1) == 1 ? o.y : (f >> 1) == 2 ? o.z : o.w;
  return (f & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// Sign mask of a seeded +-1 diagonal for positions 0..31 of a Hadamard block
// (word 0 of Philox(key = seed, counter = (0, 0, 1, 0))); bit j set = negate.
__host__ __device__ __forceinline__ uint32_t rht_sign_word(uint64_t seed, uint32_t block128, int word) {
  U4 c = {block128, 0u, 1u, 0u};
  U4 o = philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  return word == 0 ? o.x : word == 1 ? o.y : word == 2 ? o.z : o.w;
}

// ----------------------------------------------------------------------------
// E2M1 decisions on an exactly known quotient (fp64), used by the exact path.
// Lattice {0, .5, 1, 1.5, 2, 3, 4, 6}; nearest, ties to the even code.
__device__ __forceinline__ uint32_t e2m1_rne_mag_f64(double a) {
  // decision points between neighbouring lattice points and which side a tie takes
  const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  uint32_t k = 0;
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    // code i -> i+1 when a > mid, or a == mid and code i is odd (i+1 even)
    k += (a > mid[i] || (a == mid[i] && (i & 1))) ? 1u : 0u;
  }
  return k;
}

// Stochastic decision (round |q| up iff it exceeds lo + u/65536 (hi-lo)).
__device__ __forceinline__ uint32_t e2m1_sr_mag_f64(double a, uint32_t u) {
  const double L[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  if (a >= 6.0) return 7u;
  uint32_t k = 0;
#pragma unroll
  for (int i = 1; i < 7; ++i) k += (a >= L[i]) ? 1u : 0u;
  const double lo = L[k], hi = L[k + 1];
  const double t = lo + (double)u * 0x1p-16 * (hi - lo);   // exact (<= 19 significant bits)
  return (a > t) ? k + 1 : k;
}

// Stochastic decision on an fp32 magnitude a that is itself the value to round
// (exact quotient).  `nonzero` tells whether the source element was nonzero,
// which decides the u == 0 case when a underflowed to zero in fp32.
__device__ __forceinline__ uint32_t e2m1_sr_mag_f32(float a, uint32_t u, bool nonzero) {
  const uint32_t b = as_u(a);
  if (!(a < 6.0f)) return 7u;                       // >= 6, inf, NaN
  if (a >= 1.0f) {                                  // lattice step 0.5 * 2^floor(log2 a)
    const uint32_t k = (b >> 22) - 252u;            // 2..6
    const uint32_t frac22 = b & 0x3FFFFFu;          // (a - lo) / (hi - lo) in 2^-22 units
    return k + (frac22 > (u << 6) ? 1u : 0u);
  }
  if (a >= 0.5f) {
    const uint32_t frac23 = b & 0x7FFFFFu;          // (a - 0.5) / 0.5 in 2^-23 units
    return 1u + (frac23 > (u << 7) ? 1u : 0u);
  }
  const bool up = (a > (float)u * 0x1p-17f) || (u == 0u && nonzero);
  return up ? 1u : 0u;
}

// ----------------------------------------------------------------------------
// E4M3 (FN flavour: bias 7, subnormals k 2^-9, max 448 = 0x7E, 0x7F NaN).
// Value of magnitude byte c (0..127) by the hardware conversion
// (v_cvt_f32_fp8, one instruction, no branch): e4m3_value_hw for bytes
// 0x00-0x7E (0x7F, the NaN code, gives NaN); e4m3_value gives 0x7F the 480
// of its bit pattern, with one select more.
__device__ __forceinline__ float e4m3_value_hw(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 0); }
__device__ __forceinline__ float e4m3_value(uint32_t c) { return c == 0x7Fu ? 480.0f : e4m3_value_hw(c); }

// Nearest E4M3 byte (ties to even, saturating at 448) to the exact real
// t = bamax / (mult * g).  t_est = bamax * (1 / (mult g)) in fp64 is within
// 2^-51 (relative) of t; the exact value is either a tie or at least 2^-31
// away from every decision point, so only a candidate tie needs the exact
// fp64 residual bamax - mid * mult * g (exact: 31-bit product).
__device__ __forceinline__ uint32_t e4m3_encode_exact(float bamax, double t_est, double mg) {
  if (t_est >= 448.0) return 0x7Eu;
  double s;       // position in units of the local quantum
  int base;       // code of the lower neighbour at s = 0
  double quantum;
  if (t_est < 0.015625) {          // below 2^-6: quantum 2^-9
    quantum = 0x1p-9;
    s = t_est * 512.0;
    base = 0;
  } else {
    int e;
    const double m = frexp(t_est, &e);   // t = m 2^e, m in [0.5, 1)
    // t = (1 + f) 2^(e-1); quantum = 2^(e-4)
    quantum = ldexp(1.0, e - 4);
    s = (m * 2.0 - 1.0) * 8.0;           // in [0, 8)
    base = (e - 1 + 7) << 3;
  }
  const double fl = floor(s);
  const double fr = s - fl;
  int k = (int)fl;
  if (fabs(fr - 0.5) < 0x1p-36) {        // candidate tie: decide exactly
    const double mid = ((double)(base == 0 ? 0 : 8) + fl + 0.5) * quantum;  // lower + half step
    const double r = fma(mid, mg, -(double)bamax);  // sign of t - mid, negated
    if (r < 0.0 || (r == 0.0 && (k & 1))) k += 1;
  } else if (fr > 0.5) {
    k += 1;
  }
  uint32_t c = (uint32_t)(base + k);
  return c > 0x7Eu ? 0x7Eu : c;
}

}  // namespace fp4q
