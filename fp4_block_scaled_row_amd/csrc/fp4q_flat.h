// fp4q_flat.h -- slot loading and the 16-point random Hadamard transform for
// the flat (elementwise) kernels.  A slot is 8 consecutive elements of one
// row; slot s covers flat elements 8s .. 8s+7 (flat index r*cols + c).  Lane
// l of a wave works on slot 64*t + l of wave-tile t, so a 16-block spans a
// lane pair and a 32-block a lane quad.
#pragma once

#include "fp4q_common.h"
#include "fp4q_internal.h"

namespace fp4q {

template <int IN>
struct SlotRaw {
  uint32_t w[IN == kF32 ? 8 : 4];
};

template <bool CONTIG>
__device__ __forceinline__ int64_t slot_in_offset(int64_t s, int64_t cols, int64_t stride) {
  const int64_t f = s << 3;
  if (CONTIG) return f;
  const int64_t r = f / cols;
  return r * stride + (f - r * cols);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte global load; NT marks it non-temporal (streamed once, not kept in
// the caches), used when no later pass re-reads the data.
template <bool NT>
__device__ __forceinline__ u32x4_t load16(const void* p) {
  const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
  if constexpr (NT) return __builtin_nontemporal_load(q);
  else return *q;
}

template <int IN, bool CONTIG, bool NT = false>
__device__ __forceinline__ void load_slot(const QuantLaunch& q, int64_t s, bool active, SlotRaw<IN>& r) {
  if (!active) {
#pragma unroll
    for (int i = 0; i < (IN == kF32 ? 8 : 4); ++i) r.w[i] = 0u;
    return;
  }
  const int64_t off = slot_in_offset<CONTIG>(s, q.cols, q.stride);
  if constexpr (IN == kF32) {
    const float* p = static_cast<const float*>(q.x) + off;
    const u32x4_t a = load16<NT>(p), b = load16<NT>(p + 4);
    r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
    r.w[4] = b.x; r.w[5] = b.y; r.w[6] = b.z; r.w[7] = b.w;
  } else {
    const u32x4_t a = load16<NT>(static_cast<const uint16_t*>(q.x) + off);
    r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
  }
}

template <int IN>
__device__ __forceinline__ void widen_slot(const SlotRaw<IN>& r, float v[8]) {
  if constexpr (IN == kF32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = as_f(r.w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf_lo(r.w[i]);
      v[2 * i + 1] = bf_hi(r.w[i]);
    }
  }
}

// Cross-lane butterfly stages in one instruction per element.  A stage over
// lane bit k pairs lane l (bit k clear, the lower member) with l ^ 2^k; the
// butterfly gives the lower member a + b and the upper one a - b.  The form
// used here is v <- p * s + v (v_fmac_f32_dpp: p is the partner's value read
// through the DPP control, s = +1 on the lower lane and -1 on the upper), so
// the upper lane gets b - a, the exact negative of a - b: the same rounded
// magnitude, sign flipped.  Partners always carry the same accumulated sign
// (it depends only on lane bits already processed), so the stages compose and
// the caller applies the product of the signs once, with its final scale.
// Only an output that is an exact zero can come out with the other sign.
// A DPP read of a register needs two wait states after the VALU write of
// it: each block opens with s_nop 1, and within a block every source was
// written at least eight instructions earlier.
#define FP4Q_FMAC_DPP(D, S, CTRL) "v_fmac_f32_dpp %" #D ", %" #D ", %" #S " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
#define FP4Q_QX1 "quad_perm:[1,0,3,2]"
#define FP4Q_QX2 "quad_perm:[2,3,0,1]"
#define FP4Q_RX8 "row_ror:8"

// v[i] <- p[i] * s + v[i] across the lane pair (lane bit 0), 8 registers.
__device__ __forceinline__ void fmac_dpp_xor1_8(float v[8], float s) {
  asm("s_nop 1\n\t"
      FP4Q_FMAC_DPP(0, 8, FP4Q_QX1) FP4Q_FMAC_DPP(1, 8, FP4Q_QX1) FP4Q_FMAC_DPP(2, 8, FP4Q_QX1)
      FP4Q_FMAC_DPP(3, 8, FP4Q_QX1) FP4Q_FMAC_DPP(4, 8, FP4Q_QX1) FP4Q_FMAC_DPP(5, 8, FP4Q_QX1)
      FP4Q_FMAC_DPP(6, 8, FP4Q_QX1) FP4Q_FMAC_DPP(7, 8, FP4Q_QX1)
      : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
      : "v"(s));
}

// 16-point random Hadamard transform of the 16-block held by a lane pair:
// y = (sigma * x) H16 / 4, natural order.  Butterfly stages h = 1, 2, 4 run in
// registers, h = 8 between the two lanes (the even lane holds positions 0..7).
// Sign flips and the final x0.25 are exact.  rht16_butterflies is the part
// after the signs; SCALED = false leaves out the final x0.25 and the odd
// lane's sign (the tensor amax takes the magnitudes, scaled once on the
// maximum).
template <bool SCALED = true>
__device__ __forceinline__ void rht16_butterflies(float v[8], bool odd_lane) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i & h) continue;
      const float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
  // the odd lane holds the negated difference until the final scale
  const float sg1 = odd_lane ? -1.0f : 1.0f;
  fmac_dpp_xor1_8(v, sg1);
  if constexpr (SCALED) {
    const float q = odd_lane ? -0.25f : 0.25f;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= q;
  }
}

__device__ __forceinline__ void rht16_pair(float v[8], uint32_t signs16, bool odd_lane) {
  const uint32_t sg = odd_lane ? (signs16 >> 8) : signs16;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = as_f(as_u(v[i]) ^ (((sg >> i) & 1u) << 31));
  rht16_butterflies(v, odd_lane);
}

// Widening and RHT16 of a raw slot, the signs flipped in the raw words (a
// bf16 word holds two positions, sign bits 15 and 31): the same values as
// widen_slot then rht16_pair.
template <int IN, bool SCALED = true>
__device__ __forceinline__ void widen_rht16(SlotRaw<IN> r, float v[8], uint32_t signs16, bool odd_lane) {
  const uint32_t sg = odd_lane ? (signs16 >> 8) : signs16;
  if constexpr (IN == kF32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) r.w[i] ^= ((sg >> i) & 1u) << 31;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.w[i] ^= (((sg >> (2 * i)) & 1u) << 15) | (((sg >> (2 * i + 1)) & 1u) << 31);
  }
  widen_slot<IN>(r, v);
  rht16_butterflies<SCALED>(v, odd_lane);
}

// Normalised FWHT of each 128-element chunk held by 16 consecutive lanes, 8
// consecutive elements each: the three butterfly stages of the element bits
// run in registers, the four of the lane bits across lanes in one block of
// DPP instructions (fmac_dpp_xor1_8 above for the sign convention): lane bits
// 0, 1 and 3 by v_fmac_f32_dpp (quad permutations, a row rotation by 8), lane
// bit 2 by a bank-masked add (lanes 0-3 and 8-11 of each row, partner + 4)
// and subtract (lanes 4-7 and 12-15, partner - 4) into fresh registers,
// which keep the sign.  The accumulated sign is s0 s1 s3; scaled once by
// c = fl32(1/sqrt(128)) with that sign folded in (SCALED = false leaves both
// out, for the tensor amax, which takes magnitudes).
#define FP4Q_ADD_X4(D, S) "v_add_f32_dpp %" #D ", %" #S ", %" #S " row_shl:4 row_mask:0xf bank_mask:0x5\n\t" \
                          "v_sub_f32_dpp %" #D ", %" #S ", %" #S " row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
template <bool SCALED = true>
__device__ __forceinline__ void fwht128_lanes(float v[8], int lane, float c) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i & h) continue;
      const float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
  const float s0 = (lane & 1) ? -1.0f : 1.0f, s1 = (lane & 2) ? -1.0f : 1.0f, s3 = (lane & 8) ? -1.0f : 1.0f;
  float t[8];
  // t: operands 0-7, v: 8-15, s0, s1, s3: 16-18
  asm("s_nop 1\n\t"
      FP4Q_FMAC_DPP(8, 16, FP4Q_QX1) FP4Q_FMAC_DPP(9, 16, FP4Q_QX1) FP4Q_FMAC_DPP(10, 16, FP4Q_QX1)
      FP4Q_FMAC_DPP(11, 16, FP4Q_QX1) FP4Q_FMAC_DPP(12, 16, FP4Q_QX1) FP4Q_FMAC_DPP(13, 16, FP4Q_QX1)
      FP4Q_FMAC_DPP(14, 16, FP4Q_QX1) FP4Q_FMAC_DPP(15, 16, FP4Q_QX1)
      FP4Q_FMAC_DPP(8, 17, FP4Q_QX2) FP4Q_FMAC_DPP(9, 17, FP4Q_QX2) FP4Q_FMAC_DPP(10, 17, FP4Q_QX2)
      FP4Q_FMAC_DPP(11, 17, FP4Q_QX2) FP4Q_FMAC_DPP(12, 17, FP4Q_QX2) FP4Q_FMAC_DPP(13, 17, FP4Q_QX2)
      FP4Q_FMAC_DPP(14, 17, FP4Q_QX2) FP4Q_FMAC_DPP(15, 17, FP4Q_QX2)
      FP4Q_ADD_X4(0, 8) FP4Q_ADD_X4(1, 9) FP4Q_ADD_X4(2, 10) FP4Q_ADD_X4(3, 11)
      FP4Q_ADD_X4(4, 12) FP4Q_ADD_X4(5, 13) FP4Q_ADD_X4(6, 14) FP4Q_ADD_X4(7, 15)
      FP4Q_FMAC_DPP(0, 18, FP4Q_RX8) FP4Q_FMAC_DPP(1, 18, FP4Q_RX8) FP4Q_FMAC_DPP(2, 18, FP4Q_RX8)
      FP4Q_FMAC_DPP(3, 18, FP4Q_RX8) FP4Q_FMAC_DPP(4, 18, FP4Q_RX8) FP4Q_FMAC_DPP(5, 18, FP4Q_RX8)
      FP4Q_FMAC_DPP(6, 18, FP4Q_RX8) FP4Q_FMAC_DPP(7, 18, FP4Q_RX8)
      : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7]),
        "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
      : "v"(s0), "v"(s1), "v"(s3));
  if constexpr (SCALED) {
    const float cs = c * (s0 * s1 * s3);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = t[i] * cs;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = t[i];
  }
}

__device__ __forceinline__ void store_rotated(float* rot, int64_t s, const float v[8]) {
  float4* p = reinterpret_cast<float4*>(rot + (s << 3));
  p[0] = make_float4(v[0], v[1], v[2], v[3]);
  p[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// Adds a thread's saturated, underflowed and non-finite counts to the
// counters: wave sums, then the workgroup's sums in LDS, then one atomic add
// per nonzero count per workgroup -- into the workgroup's counter slot
// (slots[3 (b % kCountSlots) + k], summed afterwards by count_reduce_kernel)
// when slots is given, else straight into the three counters.  Every thread
// of the workgroup calls it (it synchronises).
__device__ __forceinline__ void flush_counters(unsigned long long* c, unsigned long long* slots, uint32_t sat,
                                               uint32_t und, uint32_t nf) {
  __shared__ unsigned long long s_cnt[3];
  const unsigned long long a = wave_sum_u64(sat), b = wave_sum_u64(und), d = wave_sum_u64(nf);
  if (threadIdx.x < 3) s_cnt[threadIdx.x] = 0ull;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    if (a) atomicAdd(s_cnt + 0, a);
    if (b) atomicAdd(s_cnt + 1, b);
    if (d) atomicAdd(s_cnt + 2, d);
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    const unsigned long long v = s_cnt[threadIdx.x];
    unsigned long long* dst = slots ? slots + 3 * (blockIdx.x % kCountSlots) + threadIdx.x : c + threadIdx.x;
    if (v) atomicAdd(dst, v);
  }
}

}  // namespace fp4q

namespace fp4q {

// MXFP4 encoding of one slot of fp32 values v[8] at flat slot index s; the
// lane quad (lanes 4k..4k+3, slots 4k..4k+3 of a 32-block) must be executing
// together.  Writes the code word, the scale byte (first lane of the quad)
// and accumulates counters.  Audit page, "Encode one MXFP4 block step by step".
template <bool SR, bool COUNT, bool MANUAL>
__device__ __forceinline__ void mx_encode_slot(const float v[8], int64_t s, bool active, int lane,
                                               int manual_e, uint64_t seed, uint8_t* codes_out,
                                               uint8_t* scales_out, uint32_t& n_sat, uint32_t& n_und,
                                               uint32_t& n_nf) {
  uint32_t amax = abs_max_bits8(v);
  amax = max(amax, dpp_u32<kQuadXor1>(amax));
  amax = max(amax, dpp_u32<kQuadXor2>(amax));
  const bool nonfinite = amax >= 0x7F800000u;
  int e;
  if constexpr (MANUAL) {
    e = manual_e;
  } else {
    e = (amax == 0u) ? 0 : max((int)(amax >> 23) - 129, -127);
  }
  uint32_t codes = 0u;
  if constexpr (!SR) {
    const float sc = e8m0_operand((uint32_t)(e + 127));
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, v[0], v[1], sc, 0);
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, v[2], v[3], sc, 1);
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, v[4], v[5], sc, 2);
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, v[6], v[7], sc, 3);
  } else {
    const U4 ctr = {(uint32_t)s, (uint32_t)((uint64_t)s >> 32), 0u, 0u};
    const U4 rnd = philox4x32_10_uniform_key(ctr, (uint32_t)seed, (uint32_t)(seed >> 32));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float qv = ldexpf(v[i], -e);
      const uint32_t mag = e2m1_sr_mag_f32(fabsf(qv), draw16(rnd, i), v[i] != 0.0f);
      codes |= (mag | ((as_u(v[i]) >> 31) << 3)) << (4 * i);
    }
  }
  if (nonfinite) codes = 0u;
  if constexpr (COUNT) {
    if (active) {
      if (nonfinite) {
#pragma unroll
        for (int i = 0; i < 8; ++i) n_nf += ((as_u(v[i]) & 0x7FFFFFFFu) >= 0x7F800000u) ? 1u : 0u;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          n_sat += (fabsf(ldexpf(v[i], -e)) > 6.0f) ? 1u : 0u;
          n_und += (v[i] != 0.0f && ((codes >> (4 * i)) & 7u) == 0u) ? 1u : 0u;
        }
      }
    }
  }
  if (active) {
    *reinterpret_cast<uint32_t*>(codes_out + (s << 2)) = codes;
    if ((lane & 3) == 0) scales_out[s >> 2] = (uint8_t)(nonfinite ? 0xFFu : (uint32_t)(e + 127));
  }
}

}  // namespace fp4q
