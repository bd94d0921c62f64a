// fp4q_nv_common.h -- NVFP4 encoding steps shared by the two-pass and the
// single-read kernels ("Sub-4-Bit Microscaling", section 2; Four Over Six and
// stochastic rounding, "Adaptive Block-Scaled Data Types" transcript cues 8
// and 10).
//
// Exactness without per-element division.  For a block with E4M3 byte c the
// exact quotient is q = x / (s_c g).  1/(s_c g) rounded down and up by 2^-22
// (a 128-entry table, one per code) gives two fp32 products that bracket q;
// the gfx950 scaled FP4 conversion (scale operand 1.0) rounds each to
// nearest-even.  That rounding is monotone, so equal codes from both brackets
// are the rounding of q itself.  An element whose brackets disagree is
// recomputed from the correctly rounded fp64 quotient, which decides every
// rounding exactly (x has <= 24 significant bits and s g <= 28, so a non-tie
// quotient is at least 2^-47 away, relatively, from any decision point).  The
// E4M3 block scale is bracketed the same way with the fp8 conversion, falling
// back to an fp64 encoding with an exact residual check of ties.  Tensors with
// g < 2^-100 take the fp64 path for every element.
#pragma once

#include "fp4q_flat.h"

namespace fp4q {

struct NvCtx {
  float g;
  double g64;
  double mg6, inv6;          // 6 g and 1 / (6 g)
  double mg4, inv4;          // 4 g and 1 / (4 g)
  float inv6_lo, inv6_hi;    // 1 / (6 g) bracketed by 2^-22
  float inv4_lo, inv4_hi;
  bool exact_all;
};

// g = RN32(amax / D) with D = 6*448 (max->6) or 4*448 (Four Over Six).  amax /
// D is evaluated in fp64 then rounded to fp32: the quotient of a 24-bit
// integer by 21 (or 7) times a power of two never lies within 2^-53 of an
// fp32 rounding boundary unless it is exact, so this is the correctly
// rounded fp32 division.  amax 0 -> g = 1; a nonzero amax whose g underflows
// -> g = 2^-149.
// Context of a given tensor scale g (the derived factors below).
__device__ __forceinline__ void nv_context_g(float g, NvCtx& cx) {
  cx.g = g;
  cx.g64 = (double)g;
  cx.mg6 = 6.0 * cx.g64;
  cx.inv6 = 1.0 / cx.mg6;
  cx.mg4 = 4.0 * cx.g64;
  cx.inv4 = 1.0 / cx.mg4;
  cx.inv6_lo = (float)(cx.inv6 * (1.0 - 0x1p-22));
  cx.inv6_hi = (float)(cx.inv6 * (1.0 + 0x1p-22));
  cx.inv4_lo = (float)(cx.inv4 * (1.0 - 0x1p-22));
  cx.inv4_hi = (float)(cx.inv4 * (1.0 + 0x1p-22));
  cx.exact_all = !(g >= 0x1p-100f);
}

__device__ __forceinline__ void nv_context(float amax, bool fos, NvCtx& cx) {
  float g = (amax == 0.0f) ? 1.0f : (float)((double)amax / (fos ? 1792.0 : 2688.0));
  if (g == 0.0f) g = 0x1p-149f;
  nv_context_g(g, cx);
}

// The context of round-to-nearest max->6 quantization (g and the bracket
// factors of 1 / (6 g)) in a short dependency chain: every workgroup computes
// it before its first encode.
//   g = RN32(amax / 2688): amax / 2688 = (M / 21) 2^k with M the 24-bit
//   significand of amax; that quotient is an fp32 value or lies at least
//   2^-30 (relative) from every fp32 rounding boundary (a boundary has 25
//   significant bits, so M / 21 on it would make M a multiple of 21 times a
//   25-bit odd number), and the fp64 product with RN64(1 / 2688) is within
//   2^-52 of it: both round to the same fp32 value.
//   1 / (6 g): the fp64 hardware reciprocal refined by one Newton step
//   (relative error near 2^-53, against 2^-53 for a division), far inside
//   the 2^-22 by which the brackets stand off: they remain strict brackets.
// The fields used here match nv_context(amax, false, ...): g exactly, the
// brackets up to an ulp.
__device__ __forceinline__ void nv_context_rne6(float amax, NvCtx& cx) {
  float g = (amax == 0.0f) ? 1.0f : (float)((double)amax * (1.0 / 2688.0));
  if (g == 0.0f) g = 0x1p-149f;
  cx.g = g;
  cx.g64 = (double)g;
  cx.mg6 = 6.0 * cx.g64;
  const double r0 = __builtin_amdgcn_rcp(cx.mg6);
  cx.inv6 = fma(r0, fma(-cx.mg6, r0, 1.0), r0);
  cx.inv6_lo = (float)(cx.inv6 * (1.0 - 0x1p-22));
  cx.inv6_hi = (float)(cx.inv6 * (1.0 + 0x1p-22));
  cx.mg4 = cx.inv4 = 0.0;   // (Four Over Six only)
  cx.inv4_lo = cx.inv4_hi = 0.0f;
  cx.exact_all = !(g >= 0x1p-100f);
}

// s_inv[c] = (1/(s_c g)) (1 -+ 2^-22) for every finite E4M3 code c > 0.
__device__ __forceinline__ void nv_fill_inverse_table(float2* s_inv, const NvCtx& cx, int tid, int nthreads) {
  for (int c = tid; c < 128; c += nthreads) {
    float2 e = make_float2(0.0f, 0.0f);
    if (c != 0 && c != 127) {
      const double inv = 1.0 / ((double)e4m3_value((uint32_t)c) * cx.g64);
      e.x = (float)(inv * (1.0 - 0x1p-22));
      e.y = (float)(inv * (1.0 + 0x1p-22));
    }
    s_inv[c] = e;
  }
}

// Single adjusted multipliers for bf16 inputs.  A bf16 magnitude a has 8
// significant bits, so within 2^-12 (relative) of a threshold T = p s g (p a
// decision point of the E2M1 rounding, or 6 for the saturation count) lies
// at most one bf16 value, at relative offset d = (a - T) / T, and every other
// bf16 value is at least 2^-12 away.  A multiplier m = (1 + e) / (s g) with
// |e| <= 2^-14 keeps RN32(a m) on the same side of p as the exact a / (s g)
// for all far values; for the near value it does so when (1 + d)(1 + e) is at
// least 1 + 2^-22 above (or below) 1 -- half an fp32 ulp of any p is at most
// 2^-24 relative, so the product rounds away from p.  An exact tie (d = 0)
// must fall on the side of the even code.  The constraints of the 8 points
// bound the intended e from both sides; the midpoint of the interval is
// taken, and a code whose interval is narrower than 2 * 2^-21 is flagged so
// that its blocks take the exact path.  The 2^-21 of slack covers the
// deviation of the stored multiplier from (1 + e) / (s g): the fp32 product
// s g and its correctly rounded reciprocal (2^-23 together), the rounding of
// 1 + e and of the final product (2^-24 each).  Decision points and the side
// of their even neighbour:
//   0.25 down, 0.75 up, 1.25 down, 1.75 up, 2.5 down, 3.5 up, 5 down, 6 down
// (6 itself is not saturated).
//
// The constraints depend on s only through its significand: scaling s by a
// power of two scales T and maps the bf16 grid onto itself (T stays inside
// the normal range: 2^-111 <= T <= 2688 g for g >= 2^-100), so e is computed
// once per significand class (8 classes: 1, 1.125, ..., 1.875 -- subnormal
// E4M3 scales fall into the same classes) and point: 64 work items.
//
// All in fp32: T = th + tl exactly (th = RN32(p s g) with p s exact, tl the
// FMA error term); the nearest bf16 value a to th is the nearest to T unless
// T is near a bf16 midpoint (then no value is within 2^-12); a - th is exact
// (Sterbenz).  d uses the hardware reciprocal of th and the bounds
// (+-2^-22 - d) / (1 + d) are taken as (+-2^-22 - d)(1 - d): relative errors
// near 2^-22 on quantities below 2^-12, i.e. below 2^-33 in absolute terms,
// far inside the slack.  The 8 points of a class are folded with DPP.
//
// s_adj[c] = (m_c, flag) and s_br[c] = 1/(s_c g) times (1 -+ 2^-22) -- still
// a strict bracket of the exact reciprocal with the fp32 reciprocal's 2^-23
// error -- for the exact path, for every E4M3 code; c = 0 gives (0, 0)
// (every code of such a block is a signed zero), c = 127 (NaN scale) is
// flagged.  The flag is in the sign bit of the second member (-0.0 flagged,
// +0.0 not), so that its bits test as an integer.
// NCODES = 256 adds flagged entries for the byte values 128..255 (a negative
// or NaN conversion result), so that a raw conversion byte can index the
// table; s_br always has 128 entries.  s_eps: 8 entries of scratch.  Every
// thread of the workgroup calls this (it synchronises); the workgroup has at
// least NCODES threads.  Requires g >= 2^-100 for meaningful entries.
template <int NCODES = 128>
__device__ __forceinline__ void nv_fill_adjusted_table(float2* s_adj, float2* s_br, float4* s_eps, const NvCtx& cx,
                                                       int tid) {
  static_assert(NCODES == 128 || NCODES == 256, "one entry per E4M3 code, or per byte value");
  const float flag = as_f(0x80000000u);
  const float g = cx.g;
  if (tid < 64) {
    // straight-line code: this runs between learning g and the first encode
    const int cls = tid >> 3, k = tid & 7;
    const float sd = 1.0f + 0.125f * (float)cls;
    // decision points 0.25 0.75 1.25 1.75 2.5 3.5 5 6, times 4 one per byte
    const float p = 0.25f * (float)(uint32_t)((0x18140E0A07050301ull >> (8 * k)) & 0xFFu);
    const bool tie_up = ((0x2Au >> k) & 1u) != 0u;    // 0.75, 1.75, 3.5: the even code is above
    const float ps = p * sd;                           // exact
    const float th = ps * g;
    const float tl = fmaf(ps, g, -th);                 // T = th + tl exactly
    const uint32_t tb = as_u(th);
    const float a = as_f(((tb + 0x7FFFu + ((tb >> 16) & 1u)) >> 16) << 16);   // nearest bf16
    const float diff = (a - th) - tl;
    const bool near = fabsf(diff) < 0x1p-12f * th;
    const float d = diff * __builtin_amdgcn_rcpf(th);
    const bool up = d > 0.0f || (d == 0.0f && tie_up);
    const float lc = (0x1p-22f - d) * (1.0f - d), hc = (-0x1p-22f - d) * (1.0f - d);
    float lo = -0x1p-14f, hi = 0x1p-14f;
    if (near && up && lc > lo) lo = lc;                // (selects: no NaN can occur)
    if (near && !up && hc < hi) hi = hc;
    // fold the 8 consecutive lanes of this class: quad exchanges, then the
    // mirror within each half-row pairs quad 0 with quad 1
    float t = dpp_xor1_f(lo), u = dpp_xor1_f(hi);
    lo = t > lo ? t : lo;
    hi = u < hi ? u : hi;
    t = dpp_xor2_f(lo), u = dpp_xor2_f(hi);
    lo = t > lo ? t : lo;
    hi = u < hi ? u : hi;
    t = as_f(dpp_u32<kRowHalfMirror>(as_u(lo))), u = as_f(dpp_u32<kRowHalfMirror>(as_u(hi)));
    lo = t > lo ? t : lo;
    hi = u < hi ? u : hi;
    if (k == 0) {
      // the class's reciprocal, computed beside the folds
      const float inv = 1.0f / (sd * g);
      s_eps[cls] = (lo + 0x1p-21f <= hi - 0x1p-21f) ? make_float4(0.5f * (lo + hi), 0.0f, inv, 0.0f)
                                                    : make_float4(0.0f, flag, inv, 0.0f);
    }
  }
  __syncthreads();
  if (tid < NCODES) {
    const uint32_t c = (uint32_t)tid;
    float2 adj = make_float2(0.0f, flag), br = make_float2(0.0f, 0.0f);
    if (c == 0u) {
      adj = make_float2(0.0f, 0.0f);
    } else if (c < 127u) {
      const float sd = e4m3_value(c);
      const float4 e = s_eps[(as_u(sd) >> 20) & 7u];   // significand class of s_c
      // s_c = 2^k sigma with sigma the class significand: RN(1 / RN(s_c g)) is
      // 2^-k RN(1 / RN(sigma g)) while no product or quotient leaves the
      // normal range (g >= 2^-100; the table is not used otherwise)
      const float inv = cx.exact_all ? 1.0f / (sd * g) : __builtin_ldexpf(e.z, 127 - (int)(as_u(sd) >> 23));
      br = make_float2(inv * (1.0f - 0x1p-22f), inv * (1.0f + 0x1p-22f));
      adj = make_float2(inv * (1.0f + e.x), e.y);
    }
    s_adj[c] = adj;
    if (c < 128u) s_br[c] = br;
  }
}

// Exact decisions for brackets that disagree.  When the two bracket products
// of one quotient q = a / (k g) round to adjacent codes lo < hi, exactly one
// decision point p (the midpoint of their values) lies between them, and q
// is above, below or on it as a - (p k) g is positive, negative or zero: p k
// is exact in fp32 (a few significant bits each) and one FMA evaluates the
// difference exactly before its single rounding, so the sign is exact (for
// g >= 2^-100 no product underflows).  A tie takes the code with the even
// mantissa.  This replaces an fp64 division in the common near-tie case
// (bf16 inputs make quotients within 2^-24 of a decision point frequent).

// E4M3 scale byte of bamax / (mult g) given the bracket bytes cl < ch.
__device__ __forceinline__ uint32_t resolve_e4m3(float bamax, uint32_t cl, uint32_t ch, float mult, float g) {
  const float p = 0.5f * (e4m3_value(cl) + e4m3_value(ch));
  const float r = fmaf(-(p * mult), g, bamax);
  return r > 0.0f ? ch : (r < 0.0f ? cl : ((cl & 1u) ? ch : cl));
}

// E2M1 magnitude of |x| / (s g) given bracket magnitudes ml < mh (E2M1
// magnitude codes, mh = ml + 1); sd = s as fp32.
__device__ __forceinline__ uint32_t resolve_e2m1(float xabs, uint32_t ml, uint32_t mh, float sd, float g) {
  const float one = e8m0_operand(127u);
  const float2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ml | (mh << 4), one, 0);
  const float p = 0.5f * (v.x + v.y);
  const float r = fmaf(-(p * sd), g, xabs);
  return r > 0.0f ? mh : (r < 0.0f ? ml : ((ml & 1u) ? mh : ml));
}

// Round-to-nearest E2M1 magnitude of |x| / (s g) when it is k or k + 1.
__device__ __forceinline__ uint32_t e2m1_rne_mag_exact(float xabs, uint32_t k, float sd, float g) {
  return k >= 7u ? 7u : resolve_e2m1(xabs, k, k + 1u, sd, g);
}

// Lattice value of E2M1 magnitude code k (0, 0.5, 1, 1.5, 2, 3, 4, 6).
__device__ __forceinline__ float e2m1_lattice(uint32_t k) {
  return k < 4u ? 0.5f * (float)k : (k == 4u ? 2.0f : (k == 5u ? 3.0f : (k == 6u ? 4.0f : 6.0f)));
}

// Stochastic-rounding magnitude (R-17: up iff |q| > lo + u 2^-16 (hi - lo)
// between the lattice neighbours lo <= |q| < hi, |q| >= 6 -> 6) of
// |q| = a / (s g), decided exactly: the interval is fixed by FMA residuals
// against L[k] s g starting from the hint k, and the threshold t = lo +
// u 2^-16 (hi - lo) has at most 18 significant bits, so t s is exact and one
// FMA residual a - (t s) g decides.  With g >= 2^-100 every (t s) g is a
// multiple of 2^-149 (t of 2^-17, s of 2^-9, g of 2^-123), and so is a, so
// a nonzero residual never rounds to zero.
__device__ __forceinline__ uint32_t e2m1_sr_mag_exact(float a, uint32_t u, uint32_t k, float sd, float g) {
  while (k < 7u && fmaf(-(e2m1_lattice(k + 1u) * sd), g, a) >= 0.0f) ++k;
  while (k > 0u && fmaf(-(e2m1_lattice(k) * sd), g, a) < 0.0f) --k;
  if (k == 7u) return 7u;
  const float lo = e2m1_lattice(k), hi = e2m1_lattice(k + 1u);
  const float t = fmaf((float)u * 0x1p-16f, hi - lo, lo);
  return fmaf(-(t * sd), g, a) > 0.0f ? k + 1u : k;
}

// E4M3 block-scale byte RNE_E4M3(bamax / (mult g)), saturating at 448.  With
// g < 2^-100 (exact_all) 1/(mult g) may not fit fp32, so the fp64 encoding
// decides directly.
__device__ __forceinline__ uint32_t nv_scale_code(float bamax, float inv_lo, float inv_hi, double inv64, double mg,
                                                  bool exact_all, float mult, float g) {
  if (exact_all) return e4m3_encode_exact(bamax, (double)bamax * inv64, mg);
  const float tl = fminf(bamax * inv_lo, 448.0f);
  const float th = fminf(bamax * inv_hi, 448.0f);
  const uint32_t b = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(tl, th, 0, false);
  const uint32_t cl = b & 0xFFu, ch = (b >> 8) & 0xFFu;
  return cl == ch ? cl : resolve_e4m3(bamax, cl, ch, mult, g);
}

// Stochastic rounding from one product a ~ |q| (relative error at most
// 1.5 * 2^-22).  Below 1 the sum a + 1 carries a's position in the step-0.5
// intervals [0, .5) and [.5, 1) in its mantissa; from 1 on a's own mantissa
// does, the step being half the power of two below a.  Either way the
// exponent with the top mantissa bit gives the interval and the low 22 bits
// the fraction fr of the step in 2^-22 units, off by at most 7 units.  R-17's
// rule (round up iff the step fraction exceeds u 2^-16) is fr > u << 6 here.
// Within 16 units of that threshold the product may decide wrongly, and so
// it may when a and q lie on either side of a lattice point, which changes
// the result only when u = 0; such lanes are decided exactly.

// Codes of the 8 elements of a lane for E4M3 scale byte c.  Round to nearest:
// the two bracket products of s_inv[c] rounded by the FP4 conversion; they
// agree except within 2^-22 of a decision point.  Stochastic rounding: one
// product (above).  Elements left undecided take exact FMA-residual
// decisions; a tensor with g < 2^-100 takes correctly rounded fp64 quotients.
template <bool SR, bool COUNT>
__device__ __forceinline__ uint32_t nv_encode(const float v[8], uint32_t c, const NvCtx& cx,
                                              const float2* s_inv, const U4& rnd, uint32_t& satmask) {
  const float2 iv = s_inv[c];
  uint32_t codes = 0u, sat = 0u, redo = 0u;
  if constexpr (!SR) {
    const float one = e8m0_operand(127u);
    float qa[8], qb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qa[i] = v[i] * iv.x;
      qb[i] = v[i] * iv.y;
    }
    uint32_t cb = 0u;
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, qa[0], qa[1], one, 0);
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, qa[2], qa[3], one, 1);
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, qa[4], qa[5], one, 2);
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, qa[6], qa[7], one, 3);
    cb = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cb, qb[0], qb[1], one, 0);
    cb = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cb, qb[2], qb[3], one, 1);
    cb = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cb, qb[4], qb[5], one, 2);
    cb = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cb, qb[6], qb[7], one, 3);
    const uint32_t d = codes ^ cb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t r = ((d >> (4 * i)) & 7u) != 0u ? 1u : 0u;
      if constexpr (COUNT) {
        const uint32_t sa = fabsf(qa[i]) > 6.0f ? 1u : 0u, sb = fabsf(qb[i]) > 6.0f ? 1u : 0u;
        sat |= sa << i;
        r |= sa ^ sb;
      }
      redo |= r << i;
    }
  } else {
    // The rule above in few steps.  t = med3(a, (a + 1) / 2, 6) has the bits
    // of a + 1 (halved) below 1, of a from 1 to 6, and is 6 above.  With
    // W = (u << 6) + 1 + (251 << 22), e = bits(t) - W borrows from bit 22
    // exactly when the step fraction fr is at most u << 6, so e >> 22 is the
    // magnitude code with its round-up; the low 22 bits of e + 17 are below
    // 32 exactly when fr - (u << 6) lies in [-16, 15] modulo 2^22, which
    // with u = 0 also takes in fr within 16 units under the next lattice
    // point (the one case where a and q in different intervals can round
    // differently).  The signs come from the RNE conversion of the signed
    // products (which keeps the sign of zero).
    const float one = e8m0_operand(127u);
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = v[i] * iv.x;
    uint32_t sg = 0u;
    sg = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(sg, p[0], p[1], one, 0);
    sg = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(sg, p[2], p[3], one, 1);
    sg = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(sg, p[4], p[5], one, 2);
    sg = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(sg, p[6], p[7], one, 3);
    uint32_t near = ~0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float a = fabsf(p[i]);
      const float t = __builtin_amdgcn_fmed3f(a, __builtin_fmaf(a, 0.5f, 0.5f), 6.0f);
      const uint32_t e = as_u(t) - ((draw16(rnd, i) << 6) + 0x3EC00001u);
      near = min(near, (e << 10) + (17u << 10));
      codes |= (e >> 22) << (4 * i);
      if constexpr (COUNT) {
        sat |= (a > 6.0f ? 1u : 0u) << i;
        redo |= (fabsf(a - 6.0f) <= 0x1p-17f ? 1u : 0u) << i;   // relative 2^-20 of 6
      }
    }
    codes |= sg & 0x88888888u;
    if (near < (32u << 10)) redo = 0xFFu;
  }
  if (cx.exact_all) {
    // g < 2^-100: correctly rounded fp64 quotients for every element
    const double den = (double)e4m3_value(c) * cx.g64;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t mag = 0u, st = 0u;
      if (c != 0u) {
        const double qd = fabs((double)v[i]) / den;
        mag = SR ? e2m1_sr_mag_f64(qd, draw16(rnd, i)) : e2m1_rne_mag_f64(qd);
        st = qd > 6.0 ? 1u : 0u;
      }
      const uint32_t sg = (as_u(v[i]) >> 31) << 3;
      codes = (codes & ~(0xFu << (4 * i))) | ((mag | sg) << (4 * i));
      sat = (sat & ~(1u << i)) | (st << i);
    }
  } else if (redo != 0u) {
    // undecided elements: exact FMA-residual decisions against s g
    const float sd = e4m3_value(c);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((redo >> i) & 1u) {
        const uint32_t k = (codes >> (4 * i)) & 7u;
        uint32_t mag = 0u, st = 0u;
        if (c != 0u) {
          const float a = fabsf(v[i]);
          if constexpr (SR) mag = e2m1_sr_mag_exact(a, draw16(rnd, i), k, sd, cx.g);
          else mag = e2m1_rne_mag_exact(a, k, sd, cx.g);
          st = fmaf(-(6.0f * sd), cx.g, a) > 0.0f ? 1u : 0u;
        }
        const uint32_t sg = (as_u(v[i]) >> 31) << 3;
        codes = (codes & ~(0xFu << (4 * i))) | ((mag | sg) << (4 * i));
        sat = (sat & ~(1u << i)) | (st << i);
      }
    }
  }
  satmask = sat;
  return codes;
}

// Round-to-nearest codes (and saturation flags) of the 8 bf16-valued elements
// of a lane for E4M3 scale byte c, by one product with the adjusted multiplier
// of c (nv_fill_adjusted_table): the common case.  A flagged code, or a
// tensor with g < 2^-100, takes the bracketed path of nv_encode.
template <bool COUNT>
__device__ __forceinline__ uint32_t nv_encode_adj(const float v[8], uint32_t c, const NvCtx& cx, const float2* s_adj,
                                                  const float2* s_br, uint32_t& satmask) {
  const float2 mf = s_adj[c];
  if (as_u(mf.y) != 0u || cx.exact_all) {
    const U4 none = {0u, 0u, 0u, 0u};
    return nv_encode<false, COUNT>(v, c, cx, s_br, none, satmask);
  }
  const float one = e8m0_operand(127u);
  float qv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qv[i] = v[i] * mf.x;
  uint32_t codes = 0u;
  codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, qv[0], qv[1], one, 0);
  codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, qv[2], qv[3], one, 1);
  codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, qv[4], qv[5], one, 2);
  codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, qv[6], qv[7], one, 3);
  uint32_t sat = 0u;
  if constexpr (COUNT) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sat |= (fabsf(qv[i]) > 6.0f ? 1u : 0u) << i;
  }
  satmask = sat;
  return codes;
}

// Half of a block's sum of squared reconstruction errors, in the fixed fp32
// order (no contraction): dq = (value * s) * g, d = x - dq, acc += d * d.
__device__ __forceinline__ float half_sse(const float v[8], uint32_t codes, uint32_t c, float g) {
#pragma clang fp contract(off)
  const float one = e8m0_operand(127u);
  const float sd = e4m3_value(c);
  float val[8];
  float2_t p;
  p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, one, 0); val[0] = p.x; val[1] = p.y;
  p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, one, 1); val[2] = p.x; val[3] = p.y;
  p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, one, 2); val[4] = p.x; val[5] = p.y;
  p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, one, 3); val[6] = p.x; val[7] = p.y;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float vs = val[i] * sd;
    const float dq = vs * g;
    const float d = v[i] - dq;
    const float sq = d * d;
    acc = acc + sq;
  }
  return acc;
}

// ---------------------------------------------------------------- IF4
// "Adaptive Block-Scaled Data Types" transcript, cues 14 and 17: besides its
// FP4 encoding every 16-block is also encoded as scaled INT4 under the same
// E4M3 scale s -- integers k in [-7, 7] standing for k * 6 s g / 7, the
// integer grid stretched by 7/6 so that 7 lands on FP4's 6 -- and keeps the
// one with the lower block SSE (ties keep FP4), flagged in bit 7 of the
// scale byte.  Nibbles are sign-magnitude like E2M1 codes.

// s_i4[c] = RN32(7 / (6 s_c g)) (0 for c = 0; unused when exact_all),
// if4_dq(k, c) = RN32(k * 6 s_c g / 7): k * 6 * s_c * g is exact
// in fp64 (at most 33 significant bits) and the fp64 quotient is never
// within 2^-33 (relatively) of an fp32 rounding boundary unless the exact
// value lies on it, so converting it gives the single rounding.
// s_h7[c] = if4_dq(1, c), the step of the INT4 grid, for every code; the
// other multiples are computed where the rare frozen-order SSE needs them.
//
// The fp64 quotient by 7 takes a product and two FMAs instead of a division:
// q0 = RN(x y) with y = RN(1/7), the remainder r = x - 7 q0 (exact), then
// RN(q0 + r y), which is Markstein's correction and gives RN(x / 7); checked
// against the division for every integer x of 33 significant bits, which
// covers every k * 6 s_c g here up to a power of two.  A non-finite x (an
// infinite g) is passed through as the division would.
__device__ __forceinline__ float if4_div7(double x) {
  constexpr double y = 1.0 / 7.0;
  const double q0 = x * y;
  const double q1 = __builtin_fma(__builtin_fma(-q0, 7.0, x), y, q0);
  return (float)(__builtin_isfinite(x) ? q1 : x);
}
// p6 = 6 s_c g (exact in fp64: at most 30 significant bits)
__device__ __forceinline__ double if4_p6(uint32_t c, double g64) { return 6.0 * (double)e4m3_value(c) * g64; }
__device__ __forceinline__ float if4_dq(uint32_t k, uint32_t c, double g64) {
  return if4_div7((double)k * if4_p6(c, g64));
}
__device__ __forceinline__ void if4_fill_tables(float* s_i4, float* s_h7, const NvCtx& cx, int tid, int nthreads) {
  for (int c = tid; c < 128; c += nthreads) {
    const double sd = (double)e4m3_value((uint32_t)c);
    s_h7[c] = if4_dq(1u, (uint32_t)c, cx.g64);
    s_i4[c] = (c != 0 && c != 127 && !cx.exact_all) ? (float)(7.0 / (6.0 * sd * cx.g64)) : 0.0f;
  }
}

// INT4 magnitudes (and |q| > 7 saturation flags) of a lane's 8 elements
// under scale byte c, q = 7 x / (6 s g) rounded to the nearest integer, ties
// to even, |k| <= 7, in nibble i without its sign bit: an INT4 nibble has the
// sign of its element, as the FP4 nibble of the same element has, so the
// caller takes the sign bits from the FP4 codes.  One product a = |x| * RN32(7 / (6 s g)) is within
// 2^-23 (relatively) of |q|, so rint(a) is the answer unless a lies within
// 2^-19 of a half-integer (or, when counting, of 7); such a lane is decided
// exactly: the sign of 7 |x| - (2k + 1) 3 s g is exact in one fp64 FMA
// (7 |x| and (2k + 1) 3 s have at most 27 and 10 significant bits), and
// q > 7 is |x| > 6 s g, an exact fp32 FMA sign.  g < 2^-100 takes
// correctly rounded fp64 quotients, which decide exactly.
// kf (optional): the magnitudes k as floats, for the caller's SSE.
template <bool COUNT>
__device__ __forceinline__ uint32_t if4_encode_int4(const float v[8], uint32_t c, const NvCtx& cx,
                                                   const float* s_i4, uint32_t& satmask, float* kf = nullptr) {
  uint32_t codes = 0u, sat = 0u;
  const float sd = e4m3_value(c);
  if (!cx.exact_all) {
    const float m = s_i4[c];
    // the largest |a - r| over the lane decides "unsure" once (a compare per
    // element would accumulate in scalar registers)
    float dmax = 0.0f;
    bool unsure = false;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float a0 = fabsf(v[i]) * m, a1 = fabsf(v[i + 1]) * m;
      const float r0 = rintf(a0), r1 = rintf(a1);
      dmax = max3_abs(dmax, a0 - r0, a1 - r1);
      const float k0 = fminf(r0, 7.0f), k1 = fminf(r1, 7.0f);
      if (kf) {
        kf[i] = k0;
        kf[i + 1] = k1;
      }
      // byte i/2 = k0 + 16 k1 (exact small integers), one conversion per pair;
      // the first one's old operand is a dead value (the others overwrite it)
      codes = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(k1, 16.0f, k0), i >> 1, i == 0 ? as_u(k0) : codes);
      if constexpr (COUNT) {
        sat |= ((a0 > 7.0f ? 1u : 0u) << i) | ((a1 > 7.0f ? 1u : 0u) << (i + 1));
        unsure |= fabsf(a0 - 7.0f) <= 0x1p-17f || fabsf(a1 - 7.0f) <= 0x1p-17f;
      }
    }
    unsure |= dmax > 0.5f - 0x1p-19f;
    if (unsure && c != 0u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float ax = fabsf(v[i]);
        const double x7 = 7.0 * (double)ax;
        const uint32_t k0 = (codes >> (4 * i)) & 7u;
        // the product's integer is off by at most one: step from k0 - 1
        uint32_t k = k0 > 0u ? k0 - 1u : 0u;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if (k < 7u) {
            const double r = fma(-((double)(2u * k + 1u) * 3.0 * (double)sd), cx.g64, x7);
            if (r > 0.0 || (r == 0.0 && (k & 1u))) ++k;
          }
        }
        const uint32_t st = fmaf(-(6.0f * sd), cx.g, ax) > 0.0f ? 1u : 0u;
        codes = (codes & ~(7u << (4 * i))) | (k << (4 * i));
        sat = (sat & ~(1u << i)) | (st << i);
        if (kf) kf[i] = (float)k;
      }
    }
  } else {
    if (c != 0u) {
      const double den = 6.0 * (double)sd * cx.g64;
#pragma unroll 1
      for (int i = 0; i < 8; ++i) {
        const double q = 7.0 * (double)fabsf(v[i]) / den;
        const uint32_t k = q > 7.0 ? 7u : (uint32_t)rint(q);
        codes |= k << (4 * i);
        sat |= (q > 7.0 ? 1u : 0u) << i;
      }
    }
    if (kf) {
#pragma unroll
      for (int i = 0; i < 8; ++i) kf[i] = (float)((codes >> (4 * i)) & 7u);
    }
  }
  satmask = COUNT ? sat : 0u;
  return codes;
}

// Half of the INT4 candidate's block SSE in the order of half_sse, with
// dq = +-if4_dq(k, c) of the element's sign, so that d = x - dq is
// +-(|x| - if4_dq(k, c)) and its square that of |x| - if4_dq(k, c) (mags: the
// magnitudes of if4_encode_int4).
__device__ __forceinline__ float half_sse_int4(const float v[8], uint32_t mags, uint32_t c, double g64) {
#pragma clang fp contract(off)
  const double p6 = if4_p6(c, g64);
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float d = fabsf(v[i]) - if4_div7((double)((mags >> (4 * i)) & 7u) * p6);
    const float sq = d * d;
    acc = acc + sq;
  }
  return acc;
}

// ---------------------------------------------------------------- SSE decisions
// Four Over Six and IF4 keep their alternative candidate iff its block SSE in
// the frozen fp32 order of half_sse (S_lo + S_hi over the lane pair) is
// lower; ties keep the default.  Most blocks are decided by cheaper sums:
// d' = fma(-value, h, x) with h = fl(s g) (INT4: h = RN32(6 s g / 7) and the
// integer k as the value), the squares accumulated by FMAs in element order,
// A = A_lo + A_hi.  Error analysis, u = 2^-24, t_i = x_i - value_i s g
// exactly, M = 6 s g (at least every |value_i s g|), no overflow: the frozen
// d_i and d'_i both lie within u |t_i| + u (1 + u) M of t_i, and every square
// reaches its sum through at most nine roundings, so
//   |S - A| <= 22.2 u A + 16.2 u M sqrt(A) + 100 u^2 M^2
//           <= 30.4 u A + 8.2 u M^2 + 100 u^2 M^2   (M sqrt(A) <= (M^2 + A) / 2).
// Results rounded into the subnormal range add at most 2^-144 in all.
// sse_bound gives more than twice that; sse_decide decides a block only when
// its two sums are further apart than their bounds together, and sends
// everything else (near ties, sums above 2^120, infinities, NaNs) to the
// frozen order.

// A_lo or A_hi of one candidate: codes as E2M1 nibbles (signs included),
// h = fl(s g).
__device__ __forceinline__ float half_sse_fma(const float v[8], uint32_t codes, float h) {
  const float one = e8m0_operand(127u);
  float val[8];
  float2_t p;
  p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, one, 0); val[0] = p.x; val[1] = p.y;
  p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, one, 1); val[2] = p.x; val[3] = p.y;
  p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, one, 2); val[4] = p.x; val[5] = p.y;
  p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, one, 3); val[6] = p.x; val[7] = p.y;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float d = fmaf(-val[i], h, v[i]);
    acc = fmaf(d, d, acc);
  }
  return acc;
}

// The same for the INT4 candidate from its magnitudes k as floats (kf of
// if4_encode_int4), h7 = RN32(6 s g / 7); d' = |x| - k h7.
__device__ __forceinline__ float half_sse_int4_fma(const float v[8], const float kf[8], float h7) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float d = fmaf(-kf[i], h7, fabsf(v[i]));
    acc = fmaf(d, d, acc);
  }
  return acc;
}

// Bound on |S - A| for a block sum A of a candidate with M = 6 s g:
// 2^-18 A + 2^-19 M^2 + 2^-129 (64 u A + 32 u M^2 against the 30.4 u A +
// 8.2 u M^2 + ... above).
__device__ __forceinline__ float sse_bound(float a, float m) {
  return fmaf(0x1p-18f, a, fmaf(0x1p-19f, m * m, 0x1p-129f));
}

// 1: keep the alternative (its frozen SSE is lower), 0: keep the default,
// -1: the sums cannot tell; the frozen order must decide.  Both lanes of a
// pair hold the same sums and get the same answer.
__device__ __forceinline__ int sse_decide(float a_def, float a_alt, float e_def, float e_alt) {
  if (!(fmaxf(a_def, a_alt) < 0x1p120f)) return -1;
  const float gap = a_def - a_alt, et = e_def + e_alt;
  if (gap > et) return 1;
  if (-gap >= et) return 0;
  return -1;
}

// Exact max->6 round-to-nearest encoding of flat slot s of a contiguous bf16
// tensor from its 16-block (a: first half, b: second half), by the brackets
// and the exact decisions above; a block holding a non-finite value gets
// codes 0 and scale 0x7F.  cx and s_br (brackets of 1 / (s g) per scale
// code, see nv_fill_adjusted_table) belong to the tensor scale times
// xscale (a power of two) and the inputs are scaled by xscale too, which
// leaves every quotient unchanged; cx.g must be at least 2^-100.
__device__ __forceinline__ void nv_fix_slot_fma(const QuantLaunch& q, const NvCtx& cx, const float2* s_br,
                                                float xscale, int64_t s, const u32x4_t& a, const u32x4_t& b) {
  uint32_t bm = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bm = max(bm, max(a[i] & 0x7FFFu, (a[i] >> 16) & 0x7FFFu));
    bm = max(bm, max(b[i] & 0x7FFFu, (b[i] >> 16) & 0x7FFFu));
  }
  uint32_t codes = 0u, scale = 0x7Fu;
  if (bm < 0x7F80u) {
    const float bamax = as_f(bm << 16) * xscale;
    const float tl = fminf(bamax * cx.inv6_lo, 448.0f);
    const float th = fminf(bamax * cx.inv6_hi, 448.0f);
    const uint32_t sb2 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(tl, th, 0, false);
    const uint32_t cl = sb2 & 0xFFu, ch = (sb2 >> 8) & 0xFFu;
    const uint32_t c = cl == ch ? cl : resolve_e4m3(bamax, cl, ch, 6.0f, cx.g);
    const float2 iv = s_br[c];
    const float sd = e4m3_value(c);
    const u32x4_t own = (s & 1) ? b : a;
    const float one = e8m0_operand(127u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t word = own[i >> 1];
      const float v = ((i & 1) ? bf_hi(word) : bf_lo(word)) * xscale;
      const uint32_t ka = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v * iv.x, 0.0f, one, 0) & 0xFu;
      const uint32_t kb = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v * iv.y, 0.0f, one, 0) & 0xFu;
      uint32_t k = ka;
      if (ka != kb) k = (ka & 8u) | resolve_e2m1(fabsf(v), ka & 7u, kb & 7u, sd, cx.g);
      codes |= k << (4 * i);
    }
    scale = c;
  }
  __builtin_nontemporal_store(codes, reinterpret_cast<uint32_t*>(q.codes + (s << 2)));   // as the fast path
  __builtin_nontemporal_store((uint8_t)scale, q.scales + (s >> 1));   // as the fast paths
}

// Largest bf16 magnitude bit pattern of the 8 values of a raw slot (sign
// bits cleared, non-finite patterns included), from packed 16-bit maxima.
__device__ __forceinline__ uint32_t slot_max16(const uint4& w) {
  ushort2_t m = __builtin_bit_cast(ushort2_t, w.x & 0x7FFF7FFFu);
  m = __builtin_elementwise_max(m, __builtin_bit_cast(ushort2_t, w.y & 0x7FFF7FFFu));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(ushort2_t, w.z & 0x7FFF7FFFu));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(ushort2_t, w.w & 0x7FFF7FFFu));
  return m.x > m.y ? m.x : m.y;
}

// Lean max->6 round-to-nearest encoding of two raw bf16 slots of one lane
// (no rotation, no counters), free of branches.  The lane pair 2k, 2k+1 holds
// 16-block A in its first slots (w0) and 16-block B in its second slots (w1);
// the even lane works out the scale of A, the odd lane that of B (bamax: the
// largest magnitude of that block, non-finite values included), and each
// passes the other the multiplier it needs, so that the per-block work is done
// once per block instead of once per lane.
// The scale byte comes from its two brackets, the codes from one product with
// the adjusted multiplier of that byte (nv_fill_adjusted_table with 256
// entries).  Returns the codes of w0 and w1 and, in *scale, the raw conversion
// byte of the block this lane worked out (its scale byte unless the block is
// redone); bit 31 of *need is set when that block must be recomputed exactly
// (nv_fix_slot_fma): its scale brackets disagree or its byte is flagged (the
// other bits are unspecified).  A block holding a non-finite value needs no
// test of its own: its products are inf or NaN, which convert to a NaN byte
// (flagged); a finite block never gets one, since its quotient stays below
// 448 (1 + 2^-21), far from the overflow point 464.
__device__ __forceinline__ void nv_fast_pair(const NvCtx& cx, const float2* s_adj, const uint4& w0, const uint4& w1,
                                             float bamax, uint32_t& codes0, uint32_t& codes1,
                                             uint32_t& scale, uint32_t& need) {
  // (the old operand of a packing conversion only fills bytes that are
  // overwritten or ignored: a dead value avoids a register copy)
  const float tl = bamax * cx.inv6_lo, th = bamax * cx.inv6_hi;
  const uint32_t sb2 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(tl, th, (int)as_u(th), false);
  const float2 mf = s_adj[sb2 & 0xFFu];   // adjusted multiplier of this byte, flag (sign bit)
  // the upper bracket's byte is the lower one's or the next: their low bits
  // tell them apart (bit 8 and bit 0 of sb2, both moved to bit 31)
  need = (__builtin_amdgcn_alignbit(sb2, sb2, 9) ^ (sb2 << 31)) | as_u(mf.y);
  scale = sb2;
  // the multiplier of block A (worked out by the even lane) and of block B
  const float ma = as_f(dpp_u32<kQuadEven>(as_u(mf.x))), mb = as_f(dpp_u32<kQuadOdd>(as_u(mf.x)));
  const float one = e8m0_operand(127u);
  uint32_t ca = 0u, cb = 0u;
#define FP4Q_PAIR(C, M, K, WK)                                                                    \
  {                                                                                               \
    const float al = bf_lo(WK) * M, ah = bf_hi(WK) * M;                                           \
    C = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(K == 0 ? as_u(al) : C, al, ah, one, K);          \
  }
  FP4Q_PAIR(ca, ma, 0, w0.x)
  FP4Q_PAIR(ca, ma, 1, w0.y)
  FP4Q_PAIR(ca, ma, 2, w0.z)
  FP4Q_PAIR(ca, ma, 3, w0.w)
  FP4Q_PAIR(cb, mb, 0, w1.x)
  FP4Q_PAIR(cb, mb, 1, w1.y)
  FP4Q_PAIR(cb, mb, 2, w1.z)
  FP4Q_PAIR(cb, mb, 3, w1.w)
#undef FP4Q_PAIR
  codes0 = ca;
  codes1 = cb;
}

}  // namespace fp4q
