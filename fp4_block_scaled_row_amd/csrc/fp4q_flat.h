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

// 16-point random Hadamard transform of the 16-block held by a lane pair:
// y = (sigma * x) H16 / 4, natural order.  Butterfly stages h = 1, 2, 4 run in
// registers, h = 8 between the two lanes (the even lane holds positions 0..7).
// Sign flips and the final x0.25 are exact.  rht16_butterflies is the part
// after the signs; SCALED = false leaves out the final x0.25 (the tensor
// amax takes it once, on the maximum).
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
  // (the even lane takes v + p, the odd lane p - v: one FMA with a sign)
  const float sg1 = odd_lane ? -1.0f : 1.0f;
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = dpp_xor1_f(v[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = SCALED ? fmaf(sg1, v[i], p[i]) * 0.25f : fmaf(sg1, v[i], p[i]);
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

// Partner value across lane bit 2 (xor 4) within a row of 16 lanes: lanes
// 4-7 and 12-15 read lane - 4 (row_shr:4, written to those banks only),
// lanes 0-3 and 8-11 lane + 4 (row_shl:4).  (Bit 3 is one row rotation.)
__device__ __forceinline__ float dpp_xor4_f(float v) {
  const int up = __builtin_amdgcn_update_dpp(0, (int)as_u(v), 0x114, 0xF, 0xA, false);
  return as_f((uint32_t)__builtin_amdgcn_update_dpp(up, (int)as_u(v), 0x104, 0xF, 0x5, false));
}

// Normalised FWHT of each 128-element chunk held by 16 consecutive lanes, 8
// consecutive elements each: the three butterfly stages of the element bits
// run in registers, the four of the lane bits across lanes (quad
// permutations for bits 0 and 1, bank-masked row shifts for bit 2, a row
// rotation by 8 for bit 3);
// the upper member of a pair keeps a - b.  Scaled once by c = fl32(1/sqrt(128))
// (SCALED = false leaves the scaling out, for the tensor amax).
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
  // the lower member of a pair takes v + p, the upper p - v: one FMA with a
  // per-lane sign (s v is exact, so it rounds as the sum or difference);
  // stage by stage over the 8 elements, so that no exchange waits on the
  // element it follows
  const float s0 = (lane & 1) ? -1.0f : 1.0f, s1 = (lane & 2) ? -1.0f : 1.0f;
  const float s2 = (lane & 4) ? -1.0f : 1.0f, s3 = (lane & 8) ? -1.0f : 1.0f;
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = dpp_xor1_f(v[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = fmaf(s0, v[i], p[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = dpp_xor2_f(v[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = fmaf(s1, v[i], p[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = dpp_xor4_f(v[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = fmaf(s2, v[i], p[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = dpp_xor8_f(v[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = SCALED ? fmaf(s3, v[i], p[i]) * c : fmaf(s3, v[i], p[i]);
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
  uint32_t amax = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = max(amax, as_u(v[i]) & 0x7FFFFFFFu);
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
    const U4 rnd = philox4x32_10(ctr, (uint32_t)seed, (uint32_t)(seed >> 32));
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
