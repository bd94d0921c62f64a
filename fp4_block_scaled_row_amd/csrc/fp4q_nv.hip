// fp4q_nv.hip -- NVFP4 and Four-Over-Six quantization kernels for gfx950.
//
// "Sub-4-Bit Microscaling (NVFP4, MXFP4 & Walsh-Hadamard Rotation)", section
// 2: E2M1 elements in 16-blocks, an unsigned E4M3 scale per block and one
// fp32 scale per tensor, g = amax / (6 * 448), s = RNE_E4M3(bamax / (6 g)),
// code = RNE_E2M1(x / (s g)).  "Adaptive Block-Scaled Data Types" transcript,
// cue 10 (Four Over Six): g = amax / (4 * 448) and each block also tries
// s4 = RNE_E4M3(bamax / (4 g)), keeping the scaling with the lower block SSE
// (ties keep max->6).  Cue 8: optional random Hadamard transform before
// quantization and stochastic rounding.
//
// Two passes because every block scale depends on the tensor amax:
//  1. nv_amax_kernel: max of the finite |x| (after rotation) per workgroup
//     into the workspace (no atomics, no memset needed).
//  2. nv_quant_kernel: every workgroup reduces those partials to the same g,
//     then streams the tensor again (mostly served by the Infinity Cache).
//
// Exactness.  The quotient x / (s g) is decided exactly without a division
// per element: with 1/(s g) rounded down and up by 2^-22 (a per-code table in
// LDS), the two fp32 products bracket the exact quotient, and the gfx950
// scaled FP4 conversion (scale operand 1.0) rounds each to nearest-even.  The
// rounding is monotone, so when both brackets give the same code that code is
// the rounding of the exact quotient.  The rare element whose brackets
// disagree is recomputed from the correctly rounded fp64 quotient, which is
// decision-exact (x has <= 24 significant bits and s g <= 28, so a non-tie
// quotient is at least 2^-47 away, relatively, from any decision point).
// E4M3 scales are encoded in fp64 with an exact residual check of ties.  For
// tensors with g < 2^-100 every element takes the fp64 path.
#include "fp4q_flat.h"
#include "fp4q_nv_common.h"

namespace fp4q {
namespace {

constexpr int kUnroll = 4;
constexpr int kPolMax6 = 0, kPolFos = 1, kPolIf4 = 2;   // block scaling policies

template <int IN, int ROT, bool CONTIG>
__device__ __forceinline__ void load_values(const QuantLaunch& q, const SlotRaw<IN>& r, int lane, float v[8]) {
  if constexpr (ROT == kRotRht16) {
    widen_rht16<IN>(r, v, q.rht_signs, (lane & 1) != 0);
  } else {
    widen_slot<IN>(r, v);
    if constexpr (ROT == kRotFwht128) fwht128_lanes(v, lane, q.rot_scale);
  }
}

// Rotated values without the rotation's final scale c.
template <int IN, int ROT>
__device__ __forceinline__ void load_unscaled(const QuantLaunch& q, const SlotRaw<IN>& r, int lane, float v[8]) {
  if constexpr (ROT == kRotRht16) {
    widen_rht16<IN, false>(r, v, q.rht_signs, (lane & 1) != 0);
  } else {
    widen_slot<IN>(r, v);
    fwht128_lanes<false>(v, lane, q.rot_scale);
  }
}

// ---------------------------------------------------------------- pass 1
//
// Rotated values: the largest |y| is taken before the rotation's final scale
// c (1/4 for RHT16, fl32(1/sqrt(128)) for FWHT-128; both below 1).  x ->
// fl(c x) is monotone, finite for finite x, and keeps infinities and NaNs, so
// the largest finite scaled value is fl(c * the largest finite unscaled one).
// The maxima are float maxima of absolute values (two values per
// instruction), which pass over NaNs; a wave whose maximum comes out infinite
// scans its slots again with the scaled values, filtering each one.
// stream: non-temporal loads, for tensors too large to stay in the Infinity
// Cache until pass 2 (otherwise the loads keep them there for pass 2).
template <int IN, int ROT, bool CONTIG>
__global__ __launch_bounds__(kThreads) void nv_amax_kernel(QuantLaunch q, bool stream) {
  __shared__ uint32_t s_red[kWaves];
  constexpr bool kRot = ROT != kRotNone;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  const int64_t ntiles = (q.nslots + 63) >> 6;
  uint32_t acc = 0u;  // fp32 abs bit pattern of the running finite max
  float mrot = 0.0f;  // rotated: the running max of |y| before the scale
  for (int64_t g = wave; g * kUnroll < ntiles; g += nwaves) {
    SlotRaw<IN> raw[kUnroll];
    if (stream) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t s = ((g * kUnroll + u) << 6) + lane;
        load_slot<IN, CONTIG, true>(q, s, s < q.nslots, raw[u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t s = ((g * kUnroll + u) << 6) + lane;
        load_slot<IN, CONTIG, false>(q, s, s < q.nslots, raw[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (g * kUnroll + u >= ntiles) break;
      if constexpr (IN == kBF16 && ROT == kRotNone) {
        ushort2_t m = __builtin_bit_cast(ushort2_t, raw[u].w[0] & 0x7FFF7FFFu);
#pragma unroll
        for (int i = 1; i < 4; ++i)
          m = __builtin_elementwise_max(m, __builtin_bit_cast(ushort2_t, raw[u].w[i] & 0x7FFF7FFFu));
        uint32_t mx = m.x > m.y ? m.x : m.y;
        if (mx >= 0x7F80u) {   // a non-finite value is present: take the finite max only
          mx = 0u;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t lo = raw[u].w[i] & 0x7FFFu, hi = (raw[u].w[i] >> 16) & 0x7FFFu;
            if (lo < 0x7F80u) mx = max(mx, lo);
            if (hi < 0x7F80u) mx = max(mx, hi);
          }
        }
        acc = max(acc, mx << 16);
      } else if constexpr (kRot) {
        float v[8];
        load_unscaled<IN, ROT>(q, raw[u], lane, v);
#pragma unroll
        for (int i = 0; i < 8; i += 2) mrot = max3_abs(mrot, v[i], v[i + 1]);
      } else {
        float v[8];
        load_values<IN, ROT, CONTIG>(q, raw[u], lane, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t a = as_u(v[i]) & 0x7FFFFFFFu;
          acc = max(acc, a < 0x7F800000u ? a : 0u);
        }
      }
    }
  }
  if constexpr (kRot) {
    if (__ballot(mrot == __builtin_inff()) == 0ull) {
      acc = as_u(mrot * (ROT == kRotRht16 ? 0.25f : q.rot_scale));
    } else {
      // (the whole wave: the rotation exchanges values between lanes)
      for (int64_t g = wave; g * kUnroll < ntiles; g += nwaves) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          if (g * kUnroll + u >= ntiles) break;
          const int64_t s = ((g * kUnroll + u) << 6) + lane;
          SlotRaw<IN> raw;
          load_slot<IN, CONTIG, false>(q, s, s < q.nslots, raw);
          float v[8];
          load_values<IN, ROT, CONTIG>(q, raw, lane, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t a = as_u(v[i]) & 0x7FFFFFFFu;
            acc = max(acc, a < 0x7F800000u ? a : 0u);
          }
        }
      }
    }
  }
  acc = wave_max_u32(acc);
  if (lane == 0) s_red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = s_red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = max(m, s_red[w]);
    q.partials[blockIdx.x] = m;
  }
}

template <int IN, int ROT, bool SR, int POL, bool COUNT, bool CONTIG>
__global__ __launch_bounds__(kThreads) void nv_quant_kernel(QuantLaunch q, int npartials) {
  constexpr bool FOS = POL == kPolFos;
  // bf16 values rounded to nearest: one product per element with the adjusted
  // multiplier of the block's scale code; otherwise (fp32 or rotated values,
  // stochastic rounding) the bracketed products
  constexpr bool kAdj = IN == kBF16 && ROT == kRotNone && !SR;
  __shared__ float2 s_inv[128];
  __shared__ float2 s_adj[kAdj ? 128 : 1];
  __shared__ float4 s_eps[8];
  __shared__ float s_i4[POL == kPolIf4 ? 128 : 1];
  __shared__ float s_h7[POL == kPolIf4 ? 128 : 1];
  __shared__ uint32_t s_red[kWaves];
  const int lane = threadIdx.x & 63;

  // ---- tensor scale (identical in every workgroup)
  uint32_t amax_bits;
  if (q.global_amax) {
    amax_bits = as_u(fabsf(*q.global_amax));
  } else {
    uint32_t m = 0u;
    for (int i = threadIdx.x; i < npartials; i += kThreads) m = max(m, q.partials[i]);
    m = wave_max_u32(m);
    if (lane == 0) s_red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = s_red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = max(m, s_red[w]);
    amax_bits = m;
  }
  NvCtx cx;
  nv_context(as_f(amax_bits), FOS, cx);
  if constexpr (kAdj) nv_fill_adjusted_table(s_adj, s_inv, s_eps, cx, threadIdx.x);
  else nv_fill_inverse_table(s_inv, cx, threadIdx.x, kThreads);
  if constexpr (POL == kPolIf4) if4_fill_tables(s_i4, s_h7, cx, threadIdx.x, kThreads);
  if (blockIdx.x == 0 && threadIdx.x == 0 && q.global_scale) *q.global_scale = cx.g;
  __syncthreads();

  // ---- stream the tensor
  const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  const int64_t ntiles = (q.nslots + 63) >> 6;
  uint32_t n_sat = 0, n_und = 0, n_nf = 0;
  const bool odd = (lane & 1) != 0;
  // wave-tile = 64 slots (512 elements); a wave owns kUnroll consecutive
  // tiles per iteration so its loads and its code/scale stores are contiguous
  for (int64_t grp = wave; grp * kUnroll < ntiles; grp += nwaves) {
    SlotRaw<IN> raw[kUnroll];
    // (every slot of the group present, the common case: loads without a
    // branch, so that the first tile waits for its own load only)
    if (((grp + 1) * kUnroll << 6) <= q.nslots) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) load_slot<IN, CONTIG, true>(q, ((grp * kUnroll + u) << 6) + lane, true, raw[u]);
    } else {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t s = ((grp * kUnroll + u) << 6) + lane;
        load_slot<IN, CONTIG, true>(q, s, s < q.nslots, raw[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t t = grp * kUnroll + u;
      if (t >= ntiles) break;
      const int64_t s = (t << 6) + lane;
      const bool active = s < q.nslots;
      const int64_t f = s << 3;
      float v[8];
      load_values<IN, ROT, CONTIG>(q, raw[u], lane, v);

      uint32_t bm = abs_max_bits8(v);
      bm = max(bm, dpp_u32<kQuadXor1>(bm));
      const bool nonfinite = bm >= 0x7F800000u;
      const float bamax = as_f(bm);

      U4 rnd = {0u, 0u, 0u, 0u};
      if constexpr (SR) {
        const U4 ctr = {(uint32_t)s, (uint32_t)((uint64_t)s >> 32), 0u, 0u};
        rnd = philox4x32_10_uniform_key(ctr, (uint32_t)q.seed, (uint32_t)(q.seed >> 32));
      }
      const uint32_t c6 = nonfinite ? 0u : nv_scale_code(bamax, cx.inv6_lo, cx.inv6_hi, cx.inv6, cx.mg6, cx.exact_all, 6.0f, cx.g);
      uint32_t sat6;
      uint32_t codes;
      if constexpr (kAdj) codes = nv_encode_adj<COUNT>(v, c6, cx, s_adj, s_inv, sat6);
      else codes = nv_encode<SR, COUNT>(v, c6, cx, s_inv, rnd, sat6);
      uint32_t sbyte = c6, satm = sat6;
      bool pick4 = false;
      if constexpr (FOS) {
        const uint32_t c4 = nonfinite ? 0u : nv_scale_code(bamax, cx.inv4_lo, cx.inv4_hi, cx.inv4, cx.mg4, cx.exact_all, 4.0f, cx.g);
        uint32_t sat4;
        uint32_t codes4;
        if constexpr (kAdj) codes4 = nv_encode_adj<COUNT>(v, c4, cx, s_adj, s_inv, sat4);
        else codes4 = nv_encode<SR, COUNT>(v, c4, cx, s_inv, rnd, sat4);
        // the FMA sums decide the block where they can (sse_decide), the
        // frozen order where they cannot; S_lo (even lane, elements 0..7) +
        // S_hi (odd lane, 8..15) either way, the same sum on both lanes (fp32
        // addition is commutative)
        const float h6 = e4m3_value(c6) * cx.g, h4 = e4m3_value(c4) * cx.g;
        float f6 = half_sse_fma(v, codes, h6), f4 = half_sse_fma(v, codes4, h4);
        {
          const float p6 = dpp_xor1_f(f6), p4 = dpp_xor1_f(f4);
          f6 = odd ? (p6 + f6) : (f6 + p6);
          f4 = odd ? (p4 + f4) : (f4 + p4);
        }
        int dec = sse_decide(f6, f4, sse_bound(f6, 6.0f * h6), sse_bound(f4, 6.0f * h4));
        if (dec < 0 && !nonfinite) {
          float e6 = half_sse(v, codes, c6, cx.g);
          float e4 = half_sse(v, codes4, c4, cx.g);
          const float p6 = dpp_xor1_f(e6), p4 = dpp_xor1_f(e4);
          e6 = odd ? (p6 + e6) : (e6 + p6);
          e4 = odd ? (p4 + e4) : (e4 + p4);
          dec = e4 < e6 ? 1 : 0;
        }
        pick4 = dec > 0 && !nonfinite;
        if (pick4) {
          codes = codes4;
          sbyte = c4;
          satm = sat4;
        }
        // choice bits: block k of this wave-tile is lane pair (2k, 2k+1)
        uint64_t bal = __ballot(pick4 && !odd && active);
        bal &= 0x5555555555555555ull;
        bal = (bal | (bal >> 1)) & 0x3333333333333333ull;
        bal = (bal | (bal >> 2)) & 0x0F0F0F0F0F0F0F0Full;
        bal = (bal | (bal >> 4)) & 0x00FF00FF00FF00FFull;
        bal = (bal | (bal >> 8)) & 0x0000FFFF0000FFFFull;
        bal = (bal | (bal >> 16)) & 0x00000000FFFFFFFFull;
        if (lane == 0) {
          const int64_t nblk = q.nslots >> 1;           // 16-blocks in the tensor
          const int64_t b0 = t << 5;                    // first block of this tile
          const int64_t nb = (nblk - b0) < 32 ? (nblk - b0) : 32;
          uint8_t* dst = q.choice_bits + (b0 >> 3);
          if (nb == 32) {
            *reinterpret_cast<uint32_t*>(dst) = (uint32_t)bal;
          } else {
            for (int k = 0; k < (int)((nb + 7) >> 3); ++k) dst[k] = (uint8_t)(bal >> (8 * k));
          }
        }
      }
      if constexpr (POL == kPolIf4) {
        uint32_t sati;
        float kf[8];
        const uint32_t mi = if4_encode_int4<COUNT>(v, c6, cx, s_i4, sati, kf);
        const uint32_t ci = mi | (codes & 0x88888888u);   // the signs of the FP4 codes
        // (as for Four Over Six: the FMA sums where they can decide)
        const float hf = e4m3_value(c6) * cx.g, h7 = s_h7[c6];
        float ff = half_sse_fma(v, codes, hf), fi = half_sse_int4_fma(v, kf, h7);
        {
          const float pf = dpp_xor1_f(ff), pi = dpp_xor1_f(fi);
          ff = odd ? (pf + ff) : (ff + pf);
          fi = odd ? (pi + fi) : (fi + pi);
        }
        int dec = sse_decide(ff, fi, sse_bound(ff, 6.0f * hf), sse_bound(fi, 7.0f * h7));
        if (dec < 0 && !nonfinite) {
          float ef = half_sse(v, codes, c6, cx.g);
          float ei = half_sse_int4(v, mi, c6, cx.g64);
          const float pf = dpp_xor1_f(ef), pi = dpp_xor1_f(ei);
          ef = odd ? (pf + ef) : (ef + pf);   // S_lo + S_hi on both lanes
          ei = odd ? (pi + ei) : (ei + pi);
          dec = ei < ef ? 1 : 0;
        }
        if (dec > 0) {
          codes = ci;
          sbyte = c6 | 0x80u;
          satm = sati;
        }
      }
      if (nonfinite) {
        codes = 0u;
        sbyte = 0x7Fu;
        satm = 0u;
      }
      if constexpr (COUNT) {
        if (active) {
          if (nonfinite) {
#pragma unroll
            for (int i = 0; i < 8; ++i) n_nf += ((as_u(v[i]) & 0x7FFFFFFFu) >= 0x7F800000u) ? 1u : 0u;
          } else {
            n_sat += __popc(satm);
#pragma unroll
            for (int i = 0; i < 8; ++i) n_und += (v[i] != 0.0f && ((codes >> (4 * i)) & 7u) == 0u) ? 1u : 0u;
          }
        }
      }
      if (active) {
        __builtin_nontemporal_store(codes, reinterpret_cast<uint32_t*>(q.codes + (f >> 1)));
        if (!odd) __builtin_nontemporal_store((uint8_t)sbyte, q.scales + (f >> 4));
        if constexpr (ROT != kRotNone) {
          if (q.rotated) store_rotated(q.rotated, s, v);
        }
      }
    }
  }
  if constexpr (COUNT) flush_counters(q.counters, q.count_slots, n_sat, n_und, n_nf);
}

// Streaming max->6 round-to-nearest encode of contiguous bf16 (no rotation,
// no counters): the paired encode of the single-read kernel without its
// on-chip phase.  A wave takes four 64-slot tiles per iteration, two pairs
// of tiles; lanes 2k and 2k+1 hold block k of both tiles of a pair, the even
// lane works out the first tile's block scale and the odd lane the second's
// (nv_fast_pair).  Blocks that need the exact path are redone at the end of
// each iteration (program order per address keeps the exact values last);
// with g < 2^-100 every block is, on inputs and g scaled by 2^100.
__global__ __launch_bounds__(kThreads) void nv_fast_kernel(QuantLaunch q, int npartials) {
  __shared__ float2 s_adj[256];
  __shared__ float2 s_br[128];
  __shared__ float4 s_eps[8];
  __shared__ uint32_t s_red[kWaves];
  const int lane = threadIdx.x & 63;
  uint32_t amax_bits;
  if (q.global_amax) {
    amax_bits = as_u(fabsf(*q.global_amax));
  } else {
    uint32_t m = 0u;
    for (int i = threadIdx.x; i < npartials; i += kThreads) m = max(m, q.partials[i]);
    m = wave_max_u32(m);
    if (lane == 0) s_red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = s_red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = max(m, s_red[w]);
    amax_bits = m;
  }
  NvCtx cx;
  nv_context(as_f(amax_bits), false, cx);
  if (blockIdx.x == 0 && threadIdx.x == 0 && q.global_scale) *q.global_scale = cx.g;
  const bool exact_all = cx.exact_all;
  float xscale = 1.0f;
  if (exact_all) {
    xscale = 0x1p100f;
    nv_context_g(cx.g * xscale, cx);
  }
  nv_fill_adjusted_table<256>(s_adj, s_br, s_eps, cx, threadIdx.x);
  __syncthreads();

  const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  const int64_t ntiles = (q.nslots + 63) >> 6;
  const bool odd = (lane & 1) != 0;
  const uint16_t* xs = static_cast<const uint16_t*>(q.x);
  for (int64_t grp = wave; grp * 4 < ntiles; grp += nwaves) {
    const int64_t t0 = grp * 4;
    uint4 w[4];
    // (every slot of the four tiles present, the common case: loads without a
    // branch, so that the first pair waits for its own loads only)
    if (((t0 + 4) << 6) <= q.nslots) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const u32x4_t a = load16<true>(xs + ((((t0 + r) << 6) + lane) << 3));
        w[r] = make_uint4(a.x, a.y, a.z, a.w);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t s = ((t0 + r) << 6) + lane;
        if (s < q.nslots) {
          const u32x4_t a = load16<true>(xs + (s << 3));
          w[r] = make_uint4(a.x, a.y, a.z, a.w);
        } else {
          w[r] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
    uint32_t redo = 0u;   // bit r: this lane's slot in tile t0 + r is redone
    if (exact_all) {
#pragma unroll
      for (int r = 0; r < 4; ++r) redo |= ((((t0 + r) << 6) + lane) < q.nslots ? 1u : 0u) << r;
    } else {
      uint32_t mine = 0u;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint4 w0 = w[2 * p], w1 = w[2 * p + 1];
        const uint32_t m0 = slot_max16(w0), m1 = slot_max16(w1);
        const uint32_t own = odd ? m1 : m0, give = odd ? m0 : m1;
        const uint32_t bm = max(own, dpp_u32<kQuadXor1>(give));
        uint32_t c0, c1, sc, nd;
        nv_fast_pair(cx, s_adj, w0, w1, as_f(bm << 16), c0, c1, sc, nd);
        const int64_t s0 = ((t0 + 2 * p) << 6) + lane, s1 = s0 + 64;
        if (s0 < q.nslots) __builtin_nontemporal_store(c0, reinterpret_cast<uint32_t*>(q.codes) + s0);
        if (s1 < q.nslots) __builtin_nontemporal_store(c1, reinterpret_cast<uint32_t*>(q.codes) + s1);
        // the block this lane worked out: tile t0 + 2p + odd, block lane / 2
        const int64_t tb = t0 + 2 * p + (odd ? 1 : 0);
        if ((tb << 6) + (lane & ~1) < q.nslots) __builtin_nontemporal_store((uint8_t)sc, q.scales + (tb << 5) + (lane >> 1));
        mine |= (nd >> 31) << (2 * p);
      }
      // slot r of a lane belongs to the block its pair worked out in the even
      // lane (r even) or the odd lane (r odd)
      const uint32_t other = dpp_u32<kQuadXor1>(mine);
      redo = odd ? (other | (mine << 1)) : (mine | (other << 1));
    }
    while (redo != 0u) {
      const int r = __builtin_ctz(redo);
      redo &= redo - 1u;
      const int64_t s = ((t0 + r) << 6) + lane;
      const u32x4_t a = load16<false>(xs + ((s & ~(int64_t)1) << 3)), b = load16<false>(xs + ((s | 1) << 3));
      nv_fix_slot_fma(q, cx, s_br, xscale, s, a, b);
    }
  }
}

// Half of a block's SSE (half_sse's frozen fp32 order) with the scale value
// sd given instead of its code.
__device__ __forceinline__ float half_sse_sd(const float v[8], uint32_t codes, float sd, float g) {
#pragma clang fp contract(off)
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
    const float vs = val[i] * sd;
    const float dq = vs * g;
    const float d = v[i] - dq;
    const float sq = d * d;
    acc = acc + sq;
  }
  return acc;
}

// Four Over Six of one 16-block held by a lane pair (8 values v per lane,
// the even lane elements 0..7), by the exact general steps: both scale
// bytes, both candidates by bracketed products with exact decisions, the
// frozen-order SSEs summed over the pair (S_lo + S_hi), max->4 kept iff its
// SSE is lower; a block holding a non-finite value gets codes 0, scale 0x7F,
// max->6.  Both lanes of the pair must run it together.
__device__ __forceinline__ void fos_block_exact(const float v[8], bool odd, const NvCtx& cx, const float2* s_br,
                                                uint32_t& codes, uint32_t& sbyte, bool& pick4) {
  uint32_t bm = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) bm = max(bm, as_u(v[i]) & 0x7FFFFFFFu);
  bm = max(bm, dpp_u32<kQuadXor1>(bm));
  const bool nonfinite = bm >= 0x7F800000u;
  const float bamax = as_f(bm);
  const U4 none = {0u, 0u, 0u, 0u};
  uint32_t sat;
  const uint32_t c6 = nonfinite ? 0u : nv_scale_code(bamax, cx.inv6_lo, cx.inv6_hi, cx.inv6, cx.mg6, cx.exact_all, 6.0f, cx.g);
  const uint32_t c4 = nonfinite ? 0u : nv_scale_code(bamax, cx.inv4_lo, cx.inv4_hi, cx.inv4, cx.mg4, cx.exact_all, 4.0f, cx.g);
  const uint32_t k6 = nv_encode<false, false>(v, c6, cx, s_br, none, sat);
  const uint32_t k4 = nv_encode<false, false>(v, c4, cx, s_br, none, sat);
  float e6 = half_sse(v, k6, c6, cx.g), e4 = half_sse(v, k4, c4, cx.g);
  const float p6 = dpp_xor1_f(e6), p4 = dpp_xor1_f(e4);
  e6 = odd ? (p6 + e6) : (e6 + p6);
  e4 = odd ? (p4 + e4) : (e4 + p4);
  pick4 = (e4 < e6) && !nonfinite;
  codes = nonfinite ? 0u : (pick4 ? k4 : k6);
  sbyte = nonfinite ? 0x7Fu : (pick4 ? c4 : c6);
}

// 32 choice bits of a 64-lane ballot taken on the even (SEL = 0) or odd
// (SEL = 1) lanes: bit k = lane 2k + SEL.
template <int SEL>
__device__ __forceinline__ uint32_t pair_bits(uint64_t bal) {
  bal = (bal >> SEL) & 0x5555555555555555ull;
  bal = (bal | (bal >> 1)) & 0x3333333333333333ull;
  bal = (bal | (bal >> 2)) & 0x0F0F0F0F0F0F0F0Full;
  bal = (bal | (bal >> 4)) & 0x00FF00FF00FF00FFull;
  bal = (bal | (bal >> 8)) & 0x0000FFFF0000FFFFull;
  bal = (bal | (bal >> 16)) & 0x00000000FFFFFFFFull;
  return (uint32_t)bal;
}

// Streaming Four Over Six of contiguous bf16 rounded to nearest, without
// counters: the straight-line paired layout of nv_fast_kernel (lanes 2k and
// 2k+1 hold block k of two tiles; the even lane works out the first tile's
// block scales, the odd lane the second's, and they pass each other the
// multipliers and scale values).  Per element: one product per candidate
// with the adjusted multiplier of its scale byte (one table serves both, it
// depends on s g only), the FP4 conversion, and the frozen-order SSE of each
// candidate.  A block whose scale brackets disagree or whose byte is flagged
// (in either candidate; non-finite blocks convert to a flagged NaN byte) is
// redone by fos_block_exact, both lanes of its pair together; with
// g < 2^-100 every block is.  Same bytes as nv_quant_kernel's Four Over Six.
__global__ __launch_bounds__(kThreads) void nv_fos_fast_kernel(QuantLaunch q, int npartials) {
  __shared__ float2 s_adj[256];
  __shared__ float2 s_br[128];
  __shared__ float4 s_eps[8];
  __shared__ uint32_t s_red[kWaves];
  const int lane = threadIdx.x & 63;
  uint32_t amax_bits;
  if (q.global_amax) {
    amax_bits = as_u(fabsf(*q.global_amax));
  } else {
    uint32_t m = 0u;
    for (int i = threadIdx.x; i < npartials; i += kThreads) m = max(m, q.partials[i]);
    m = wave_max_u32(m);
    if (lane == 0) s_red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = s_red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = max(m, s_red[w]);
    amax_bits = m;
  }
  NvCtx cx;
  nv_context(as_f(amax_bits), true, cx);
  if (blockIdx.x == 0 && threadIdx.x == 0 && q.global_scale) *q.global_scale = cx.g;
  const bool exact_all = cx.exact_all;
  nv_fill_adjusted_table<256>(s_adj, s_br, s_eps, cx, threadIdx.x);
  __syncthreads();

  const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  const int64_t ntiles = (q.nslots + 63) >> 6;
  const int64_t nblk = q.nslots >> 1;
  const bool odd = (lane & 1) != 0;
  const uint16_t* xs = static_cast<const uint16_t*>(q.x);
  const float one = e8m0_operand(127u);
  for (int64_t grp = wave; grp * 4 < ntiles; grp += nwaves) {
    const int64_t t0 = grp * 4;
    uint4 w[4];
    // (as nv_fast_kernel: unconditional loads of a group of full tiles)
    if (((t0 + 4) << 6) <= q.nslots) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const u32x4_t a = load16<true>(xs + ((((t0 + r) << 6) + lane) << 3));
        w[r] = make_uint4(a.x, a.y, a.z, a.w);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t s = ((t0 + r) << 6) + lane;
        if (s < q.nslots) {
          const u32x4_t a = load16<true>(xs + (s << 3));
          w[r] = make_uint4(a.x, a.y, a.z, a.w);
        } else {
          w[r] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint4 w0 = w[2 * p], w1 = w[2 * p + 1];
      const int64_t ta = t0 + 2 * p;              // tiles ta (this lane's w0) and ta + 1 (w1)
      const int64_t s0 = (ta << 6) + lane, s1 = s0 + 64;
      float xa[8] = {bf_lo(w0.x), bf_hi(w0.x), bf_lo(w0.y), bf_hi(w0.y), bf_lo(w0.z), bf_hi(w0.z), bf_lo(w0.w), bf_hi(w0.w)};
      float xb[8] = {bf_lo(w1.x), bf_hi(w1.x), bf_lo(w1.y), bf_hi(w1.y), bf_lo(w1.z), bf_hi(w1.z), bf_lo(w1.w), bf_hi(w1.w)};
      uint32_t ca = 0u, cb = 0u, sbyte = 0u;
      bool pa = false, pb = false, need_a = true, need_b = true;
      if (!exact_all) {
        const uint32_t m0 = slot_max16(w0), m1 = slot_max16(w1);
        const uint32_t own = odd ? m1 : m0, give = odd ? m0 : m1;
        const float bamax = as_f(max(own, dpp_u32<kQuadXor1>(give)) << 16);
        // both scale bytes of the block this lane works out, from their brackets
        const uint32_t b6 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(bamax * cx.inv6_lo, bamax * cx.inv6_hi, 0, false);
        const uint32_t b4 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(bamax * cx.inv4_lo, bamax * cx.inv4_hi, 0, false);
        const float2 e6 = s_adj[b6 & 0xFFu], e4 = s_adj[b4 & 0xFFu];
        const uint32_t need = (__builtin_amdgcn_alignbit(b6, b6, 9) ^ (b6 << 31)) | as_u(e6.y) |
                              (__builtin_amdgcn_alignbit(b4, b4, 9) ^ (b4 << 31)) | as_u(e4.y);
        // (a NaN for byte 0x7F: such a block is flagged and redone exactly)
        const float sd6 = e4m3_value_hw(b6 & 0x7Fu), sd4 = e4m3_value_hw(b4 & 0x7Fu);
        // block A (tile ta) was worked out by the even lane, block B by the odd one
        const float ma6 = as_f(dpp_u32<kQuadEven>(as_u(e6.x))), mb6 = as_f(dpp_u32<kQuadOdd>(as_u(e6.x)));
        const float ma4 = as_f(dpp_u32<kQuadEven>(as_u(e4.x))), mb4 = as_f(dpp_u32<kQuadOdd>(as_u(e4.x)));
        const float sa6 = as_f(dpp_u32<kQuadEven>(as_u(sd6))), sb6 = as_f(dpp_u32<kQuadOdd>(as_u(sd6)));
        const float sa4 = as_f(dpp_u32<kQuadEven>(as_u(sd4))), sb4 = as_f(dpp_u32<kQuadOdd>(as_u(sd4)));
        need_a = (dpp_u32<kQuadEven>(need) >> 31) != 0u;
        need_b = (dpp_u32<kQuadOdd>(need) >> 31) != 0u;
        uint32_t a6 = 0u, a4 = 0u, c6 = 0u, c4 = 0u;
        // (the old operand of the first conversion of each word only fills
        // bytes that the next three overwrite: a dead value, no zeroing move)
#define FP4Q_FOS_CVT(C, X, M, K)                                                                    \
  {                                                                                                 \
    const float lo = X[2 * K] * M, hi = X[2 * K + 1] * M;                                           \
    C = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(K == 0 ? as_u(lo) : C, lo, hi, one, K);            \
  }
#define FP4Q_FOS_WORD(K)                                                                            \
  FP4Q_FOS_CVT(a6, xa, ma6, K) FP4Q_FOS_CVT(a4, xa, ma4, K) FP4Q_FOS_CVT(c6, xb, mb6, K)            \
  FP4Q_FOS_CVT(c4, xb, mb4, K)
        FP4Q_FOS_WORD(0)
        FP4Q_FOS_WORD(1)
        FP4Q_FOS_WORD(2)
        FP4Q_FOS_WORD(3)
#undef FP4Q_FOS_WORD
#undef FP4Q_FOS_CVT
        // the FMA sums decide each block where they can (sse_decide), the
        // frozen order where they cannot; S_lo (even lane) + S_hi (odd lane),
        // the same sum on both lanes
        const float ha6 = sa6 * cx.g, ha4 = sa4 * cx.g, hb6 = sb6 * cx.g, hb4 = sb4 * cx.g;
        float fa6 = half_sse_fma(xa, a6, ha6), fa4 = half_sse_fma(xa, a4, ha4);
        float fb6 = half_sse_fma(xb, c6, hb6), fb4 = half_sse_fma(xb, c4, hb4);
        {
          const float q1 = dpp_xor1_f(fa6), q2 = dpp_xor1_f(fa4), q3 = dpp_xor1_f(fb6), q4 = dpp_xor1_f(fb4);
          fa6 = odd ? (q1 + fa6) : (fa6 + q1);
          fa4 = odd ? (q2 + fa4) : (fa4 + q2);
          fb6 = odd ? (q3 + fb6) : (fb6 + q3);
          fb4 = odd ? (q4 + fb4) : (fb4 + q4);
        }
        int da = sse_decide(fa6, fa4, sse_bound(fa6, 6.0f * ha6), sse_bound(fa4, 6.0f * ha4));
        int db = sse_decide(fb6, fb4, sse_bound(fb6, 6.0f * hb6), sse_bound(fb4, 6.0f * hb4));
        if (da < 0) {
          float ea6 = half_sse_sd(xa, a6, sa6, cx.g), ea4 = half_sse_sd(xa, a4, sa4, cx.g);
          const float q1 = dpp_xor1_f(ea6), q2 = dpp_xor1_f(ea4);
          ea6 = odd ? (q1 + ea6) : (ea6 + q1);
          ea4 = odd ? (q2 + ea4) : (ea4 + q2);
          da = ea4 < ea6 ? 1 : 0;
        }
        if (db < 0) {
          float eb6 = half_sse_sd(xb, c6, sb6, cx.g), eb4 = half_sse_sd(xb, c4, sb4, cx.g);
          const float q3 = dpp_xor1_f(eb6), q4 = dpp_xor1_f(eb4);
          eb6 = odd ? (q3 + eb6) : (eb6 + q3);
          eb4 = odd ? (q4 + eb4) : (eb4 + q4);
          db = eb4 < eb6 ? 1 : 0;
        }
        pa = da > 0;
        pb = db > 0;
        ca = pa ? a4 : a6;
        cb = pb ? c4 : c6;
        const bool pw = odd ? pb : pa;                       // the block this lane worked out
        sbyte = pw ? (b4 & 0xFFu) : (b6 & 0xFFu);
      }
      if (need_a) {
        uint32_t sba = 0u;
        fos_block_exact(xa, odd, cx, s_br, ca, sba, pa);
        if (!odd) sbyte = sba;
      }
      if (need_b) {
        uint32_t sbb = 0u;
        fos_block_exact(xb, odd, cx, s_br, cb, sbb, pb);
        if (odd) sbyte = sbb;
      }
      if (s0 < q.nslots) __builtin_nontemporal_store(ca, reinterpret_cast<uint32_t*>(q.codes) + s0);
      if (s1 < q.nslots) __builtin_nontemporal_store(cb, reinterpret_cast<uint32_t*>(q.codes) + s1);
      const int64_t tb = ta + (odd ? 1 : 0);             // the block this lane worked out: tile tb, block lane / 2
      if ((tb << 6) + (lane & ~1) < q.nslots) __builtin_nontemporal_store((uint8_t)sbyte, q.scales + (tb << 5) + (lane >> 1));
      // choice bits of tiles ta and ta + 1: block k of a tile is bit k of its 32-bit word
      const uint64_t bal = __ballot(odd ? pb : pa);
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int64_t b0 = (ta + h) << 5;              // first block of the tile
          if (b0 >= nblk) break;
          const uint32_t bits = h ? pair_bits<1>(bal) : pair_bits<0>(bal);
          const int64_t nb = (nblk - b0) < 32 ? (nblk - b0) : 32;
          uint8_t* dst = q.choice_bits + (b0 >> 3);
          if (nb == 32) {
            *reinterpret_cast<uint32_t*>(dst) = bits;
          } else {
            for (int k = 0; k < (int)((nb + 7) >> 3); ++k) dst[k] = (uint8_t)(bits >> (8 * k));
          }
        }
      }
    }
  }
}

int amax_grid(int64_t nslots) {
  const int64_t ntiles = (nslots + 63) >> 6;
  int64_t want = (ntiles + kWaves * kUnroll - 1) / (kWaves * kUnroll);
  int64_t cap = (int64_t)device_cu_count() * 4;
  if (cap > kAmaxPartialsMax) cap = kAmaxPartialsMax;
  return (int)(want < 1 ? 1 : (want > cap ? cap : want));
}

template <int IN, int ROT, bool SR, int POL, bool COUNT, bool CONTIG>
hipError_t launch_t(const QuantLaunch& q, hipStream_t st) {
  int np = 0;
  if (!q.global_amax) {
    np = amax_grid(q.nslots);
    // (measured: cached loads for the 134 MB 8192^2 bf16 tensors, whose pass 2
    // then finds them in the 256 MB Infinity Cache; non-temporal for the 470 MB
    // 8192 x 28672 weight, C4 ~210 -> ~205 us)
    const int64_t in_bytes = q.nslots * (IN == kF32 ? 32 : 16);
    const bool stream = in_bytes > ((int64_t)192 << 20);
    hipLaunchKernelGGL((nv_amax_kernel<IN, ROT, CONTIG>), dim3(np), dim3(kThreads), 0, st, q, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (q.counters && !q.count_slots) {
    hipError_t e = launch_zero_counters(q.counters, st);
    if (e != hipSuccess) return e;
  }
  const int64_t ntiles = (q.nslots + 63) >> 6;
  const int64_t want = (ntiles + kWaves * kUnroll - 1) / (kWaves * kUnroll);
  const int64_t cap = (int64_t)device_cu_count() * 16;   // (measured: 16 per CU against 4, 8, 32, 64)
  const int grid = (int)(want < 1 ? 1 : (want > cap ? cap : want));
  if constexpr (IN == kBF16 && ROT == kRotNone && !SR && POL == kPolMax6 && !COUNT && CONTIG) {
    static_assert(kUnroll == 4, "nv_fast_kernel takes four tiles per wave iteration");
    hipLaunchKernelGGL(nv_fast_kernel, dim3(grid), dim3(kThreads), 0, st, q, np);
  } else if constexpr (IN == kBF16 && ROT == kRotNone && !SR && POL == kPolFos && !COUNT && CONTIG) {
    hipLaunchKernelGGL(nv_fos_fast_kernel, dim3(grid), dim3(kThreads), 0, st, q, np);
  } else {
    hipLaunchKernelGGL((nv_quant_kernel<IN, ROT, SR, POL, COUNT, CONTIG>), dim3(grid), dim3(kThreads), 0, st, q, np);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !COUNT || !q.count_slots) return e;
  return launch_count_reduce(q.count_slots, q.counters, st);
}

template <int IN, int ROT, bool SR, int POL, bool COUNT>
hipError_t d_contig(const QuantLaunch& q, hipStream_t st) {
  return q.stride == q.cols ? launch_t<IN, ROT, SR, POL, COUNT, true>(q, st)
                            : launch_t<IN, ROT, SR, POL, COUNT, false>(q, st);
}
template <int IN, int ROT, bool SR, int POL>
hipError_t d_count(const QuantLaunch& q, hipStream_t st) {
  return q.counters ? d_contig<IN, ROT, SR, POL, true>(q, st) : d_contig<IN, ROT, SR, POL, false>(q, st);
}
template <int IN, int ROT, bool SR>
hipError_t d_fos(const QuantLaunch& q, hipStream_t st) {
  // (combinations the entry point rejects are not instantiated)
  if (q.four_over_six) {
    if constexpr (ROT == kRotFwht128) return hipErrorInvalidValue;
    else return d_count<IN, ROT, SR, kPolFos>(q, st);
  }
  if (q.if4) {
    if constexpr (SR) return hipErrorInvalidValue;
    else return d_count<IN, ROT, SR, kPolIf4>(q, st);
  }
  return d_count<IN, ROT, SR, kPolMax6>(q, st);
}
template <int IN, int ROT>
hipError_t d_sr(const QuantLaunch& q, hipStream_t st) {
  return q.stochastic ? d_fos<IN, ROT, true>(q, st) : d_fos<IN, ROT, false>(q, st);
}
template <int IN>
hipError_t d_rot(const QuantLaunch& q, hipStream_t st) {
  if (q.rotation == kRotFwht128) {
    if (q.stochastic) return hipErrorInvalidValue;
    return d_fos<IN, kRotFwht128, false>(q, st);
  }
  return q.rotation == kRotRht16 ? d_sr<IN, kRotRht16>(q, st) : d_sr<IN, kRotNone>(q, st);
}

}  // namespace

hipError_t launch_nv_quant(const QuantLaunch& q0, hipStream_t st) {
  // q0.partials is the workspace base (layout in fp4q_internal.h)
  QuantLaunch q = q0;
  int grid = 0, nres = 0;
  if (q.partials && nv_resident_shape(q, &grid, &nres)) return launch_nv_resident(q, grid, nres, st);
  if (q.partials) {
    unsigned char* ws = reinterpret_cast<unsigned char*>(q.partials);
    if (q.counters) q.count_slots = reinterpret_cast<unsigned long long*>(ws + kWsCountOffsetBytes);
    q.partials = reinterpret_cast<uint32_t*>(ws + kWsPartialsOffsetBytes);
  }
  // (an empty tensor still runs both passes: g = 1 is reported, counters zeroed)
  return q.in_dtype == kF32 ? d_rot<kF32>(q, st) : d_rot<kBF16>(q, st);
}

}  // namespace fp4q
