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
  widen_slot<IN>(r, v);
  if constexpr (ROT == kRotRht16) rht16_pair(v, q.rht_signs, (lane & 1) != 0);
  if constexpr (ROT == kRotFwht128) fwht128_lanes(v, lane, q.rot_scale);
}

// ---------------------------------------------------------------- pass 1
template <int IN, int ROT, bool CONTIG>
__global__ __launch_bounds__(kThreads) void nv_amax_kernel(QuantLaunch q) {
  __shared__ uint32_t s_red[kWaves];
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  const int64_t ntiles = (q.nslots + 63) >> 6;
  uint32_t acc = 0u;  // fp32 abs bit pattern of the running finite max
  for (int64_t g = wave; g * kUnroll < ntiles; g += nwaves) {
    SlotRaw<IN> raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t s = ((g * kUnroll + u) << 6) + lane;
      load_slot<IN, CONTIG, false>(q, s, s < q.nslots, raw[u]);   // kept in the caches for pass 2
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
  acc = wave_max_u32(acc);
  if (lane == 0) s_red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = s_red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = max(m, s_red[w]);
    q.partials[blockIdx.x] = m;
  }
  if (blockIdx.x == 0 && threadIdx.x < 3 && q.counters) q.counters[threadIdx.x] = 0ull;
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
  __shared__ float s_dq[POL == kPolIf4 ? 1024 : 1];
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
  if constexpr (POL == kPolIf4) if4_fill_tables(s_i4, s_dq, cx, threadIdx.x, kThreads);
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
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t s = ((grp * kUnroll + u) << 6) + lane;
      load_slot<IN, CONTIG, true>(q, s, s < q.nslots, raw[u]);
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

      uint32_t bm = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) bm = max(bm, as_u(v[i]) & 0x7FFFFFFFu);
      bm = max(bm, dpp_u32<kQuadXor1>(bm));
      const bool nonfinite = bm >= 0x7F800000u;
      const float bamax = as_f(bm);

      U4 rnd = {0u, 0u, 0u, 0u};
      if constexpr (SR) {
        const U4 ctr = {(uint32_t)s, (uint32_t)((uint64_t)s >> 32), 0u, 0u};
        rnd = philox4x32_10(ctr, (uint32_t)q.seed, (uint32_t)(q.seed >> 32));
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
        float e6 = half_sse(v, codes, c6, cx.g);
        float e4 = half_sse(v, codes4, c4, cx.g);
        const float p6 = dpp_xor1_f(e6), p4 = dpp_xor1_f(e4);
        // S_lo (even lane, elements 0..7) + S_hi (odd lane, 8..15); fp32
        // addition is commutative so both lanes get the same sum.
        e6 = odd ? (p6 + e6) : (e6 + p6);
        e4 = odd ? (p4 + e4) : (e4 + p4);
        pick4 = (e4 < e6) && !nonfinite;
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
        const uint32_t ci = if4_encode_int4<COUNT>(v, c6, cx, s_i4, sati);
        float ef = half_sse(v, codes, c6, cx.g);
        float ei = half_sse_int4(v, ci, s_dq + 8 * c6);
        const float pf = dpp_xor1_f(ef), pi = dpp_xor1_f(ei);
        ef = odd ? (pf + ef) : (ef + pf);   // S_lo + S_hi on both lanes
        ei = odd ? (pi + ei) : (ei + pi);
        if (ei < ef) {
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
        if (!odd) q.scales[f >> 4] = (uint8_t)sbyte;
        if constexpr (ROT != kRotNone) {
          if (q.rotated) store_rotated(q.rotated, s, v);
        }
      }
    }
  }
  if constexpr (COUNT) flush_counters(q.counters, n_sat, n_und, n_nf);
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
        if ((tb << 6) + (lane & ~1) < q.nslots) q.scales[(tb << 5) + (lane >> 1)] = (uint8_t)sc;
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
    hipLaunchKernelGGL((nv_amax_kernel<IN, ROT, CONTIG>), dim3(np), dim3(kThreads), 0, st, q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (q.counters) {
    hipError_t e = launch_zero_counters(q.counters, st);
    if (e != hipSuccess) return e;
  }
  const int64_t ntiles = (q.nslots + 63) >> 6;
  const int64_t want = (ntiles + kWaves * kUnroll - 1) / (kWaves * kUnroll);
  const int64_t cap = (int64_t)device_cu_count() * 8;
  const int grid = (int)(want < 1 ? 1 : (want > cap ? cap : want));
  if constexpr (IN == kBF16 && ROT == kRotNone && !SR && POL == kPolMax6 && !COUNT && CONTIG) {
    static_assert(kUnroll == 4, "nv_fast_kernel takes four tiles per wave iteration");
    hipLaunchKernelGGL(nv_fast_kernel, dim3(grid), dim3(kThreads), 0, st, q, np);
  } else {
    hipLaunchKernelGGL((nv_quant_kernel<IN, ROT, SR, POL, COUNT, CONTIG>), dim3(grid), dim3(kThreads), 0, st, q, np);
  }
  return hipGetLastError();
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
  if (q.partials) q.partials += kWsPartialsOffsetBytes / sizeof(uint32_t);
  // (an empty tensor still runs both passes: g = 1 is reported, counters zeroed)
  return q.in_dtype == kF32 ? d_rot<kF32>(q, st) : d_rot<kBF16>(q, st);
}

}  // namespace fp4q
