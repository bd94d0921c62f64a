// fp4q_mx.hip -- MXFP4 quantization kernel for gfx950.
//
// "MXFP4 Quantization: Audit the 4.25-Bit Blocks", sections "Read the shared
// E8M0 scale" and "Encode one MXFP4 block step by step": per 32-block of a
// row, e = floor(log2(amax/4)) clamped to [-127, 127] (all-zero block: 0),
// scale byte e + 127, every element divided by 2^e and rounded onto the E2M1
// lattice with ties to the even code, |v| > 6 clamped to 6; two nibbles per
// byte, element 2k low.
//
// One pass, HBM-bound.  A lane owns 8 elements (one 16-byte bf16 load), a lane
// quad owns a 32-block; the block amax is an integer max of the abs bit
// patterns reduced across the quad with DPP.  Element rounding uses the
// gfx950 scaled FP4 conversion (v_cvt_scalef32_pk_fp4_*), which divides by
// 2^(b-127) for the E8M0 byte b held in the exponent field of its scale
// operand and rounds to nearest-even with saturation at +-6 -- exactly the
// rule above, so the power-of-two division is exact and nothing else rounds.
#include "fp4q_flat.h"

namespace fp4q {
namespace {

// Tiles per wave step: 8 (measured ~2 % faster than 4 on bf16; 2 slower), or
// 1 for tensors too small to give every SIMD a wave with 8 (1024 x 1024 is
// 2048 tiles: 64 workgroups with 8, 512 with 1).
constexpr int kUnroll = 8;

template <int IN, int ROT, bool SR, bool COUNT, bool CONTIG, bool MANUAL, int UNROLL>
__global__ __launch_bounds__(kThreads) void mx_quant_kernel(QuantLaunch q) {
  constexpr int kUnroll = UNROLL;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  const int64_t ntiles = (q.nslots + 63) >> 6;
  uint32_t n_sat = 0, n_und = 0, n_nf = 0;

  // wave-tile = 64 slots (512 elements); a wave owns kUnroll consecutive
  // tiles per iteration so its loads and its code/scale stores are contiguous
  for (int64_t g = wave; g * kUnroll < ntiles; g += nwaves) {
    SlotRaw<IN> raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t s = ((g * kUnroll + u) << 6) + lane;
      load_slot<IN, CONTIG, true>(q, s, s < q.nslots, raw[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t t = g * kUnroll + u;
      if (t >= ntiles) break;                       // wave-uniform
      const int64_t s = (t << 6) + lane;
      const bool active = s < q.nslots;
      const int64_t f = s << 3;

      constexpr bool kPackedBf16 = (IN == kBF16 && ROT == kRotNone && !SR && !COUNT);
      if constexpr (!kPackedBf16) {
        float v[8];
        if constexpr (ROT == kRotRht16) widen_rht16<IN>(raw[u], v, q.rht_signs, (lane & 1) != 0);
        else widen_slot<IN>(raw[u], v);
        mx_encode_slot<SR, COUNT, MANUAL>(v, s, active, lane, q.manual_e, q.seed, q.codes, q.scales,
                                          n_sat, n_und, n_nf);
        if constexpr (ROT != kRotNone) {
          if (active && q.rotated) store_rotated(q.rotated, s, v);
        }
      } else {
        // bf16 fast path: packed 16-bit max of |x|, conversion straight from bf16
        ushort2_t m = __builtin_bit_cast(ushort2_t, raw[u].w[0] & 0x7FFF7FFFu);
#pragma unroll
        for (int i = 1; i < 4; ++i)
          m = __builtin_elementwise_max(m, __builtin_bit_cast(ushort2_t, raw[u].w[i] & 0x7FFF7FFFu));
        uint32_t amax = m.x > m.y ? m.x : m.y;
        amax = max(amax, dpp_u32<kQuadXor1>(amax));
        amax = max(amax, dpp_u32<kQuadXor2>(amax));
        const bool nonfinite = amax >= 0x7F80u;
        int e;
        if constexpr (MANUAL) {
          e = q.manual_e;
        } else {
          e = (amax == 0u) ? 0 : max((int)(amax >> 7) - 129, -127);
        }
        const float sc = e8m0_operand((uint32_t)(e + 127));
        uint32_t codes = 0u;
        codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2_t, raw[u].w[0]), sc, 0);
        codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2_t, raw[u].w[1]), sc, 1);
        codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2_t, raw[u].w[2]), sc, 2);
        codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2_t, raw[u].w[3]), sc, 3);
        if (nonfinite) codes = 0u;
        if (active) {
          *reinterpret_cast<uint32_t*>(q.codes + (f >> 1)) = codes;
          if ((lane & 3) == 0) q.scales[f >> 5] = (uint8_t)(nonfinite ? 0xFFu : (uint32_t)(e + 127));
        }
      }
    }
  }
  if constexpr (COUNT) flush_counters(q.counters, q.count_slots, n_sat, n_und, n_nf);
}

__global__ void zero_counters_kernel(unsigned long long* c) {
  if (threadIdx.x < 3) c[threadIdx.x] = 0ull;
}

// counters[k] = sum of the slots' count k, by one wave: lane l reads slots
// 2l and 2l+1 (six 8-byte words: the workspace is only 8-byte aligned), the
// wave sums, lane 0 writes the counters; the slots are zeroed for the next
// call.
static_assert(kCountSlots == 128, "one wave, two slots per lane");
__global__ __launch_bounds__(64) void count_reduce_kernel(unsigned long long* slots, unsigned long long* c) {
  const int l = threadIdx.x;
  unsigned long long* p = slots + 6 * l;
  unsigned long long v[6];
#pragma unroll
  for (int i = 0; i < 6; ++i) v[i] = p[i];
#pragma unroll
  for (int i = 0; i < 6; ++i) p[i] = 0ull;
  const unsigned long long k0 = wave_sum_u64(v[0] + v[3]), k1 = wave_sum_u64(v[1] + v[4]),
                           k2 = wave_sum_u64(v[2] + v[5]);
  if (l == 0) {
    c[0] = k0;
    c[1] = k1;
    c[2] = k2;
  }
}

template <int IN, int ROT, bool SR, bool COUNT, bool CONTIG, bool MANUAL>
hipError_t launch_t(const QuantLaunch& q, hipStream_t st) {
  const int64_t ntiles = (q.nslots + 63) >> 6;
  const int64_t cus = device_cu_count();
  const bool small = ntiles < cus * kWaves * kUnroll;   // fewer than one workgroup per CU with 8
  const int unroll = small ? 1 : kUnroll;
  const int64_t want = (ntiles + kWaves * unroll - 1) / (kWaves * unroll);
  const int64_t cap = cus * 8;
  const int grid = (int)(want < 1 ? 1 : (want > cap ? cap : want));
  if (small)
    hipLaunchKernelGGL((mx_quant_kernel<IN, ROT, SR, COUNT, CONTIG, MANUAL, 1>), dim3(grid), dim3(kThreads), 0, st, q);
  else
    hipLaunchKernelGGL((mx_quant_kernel<IN, ROT, SR, COUNT, CONTIG, MANUAL, kUnroll>), dim3(grid), dim3(kThreads), 0,
                       st, q);
  return hipGetLastError();
}

template <int IN, int ROT, bool SR, bool COUNT, bool CONTIG>
hipError_t dispatch_manual(const QuantLaunch& q, hipStream_t st) {
  return q.manual ? launch_t<IN, ROT, SR, COUNT, CONTIG, true>(q, st)
                  : launch_t<IN, ROT, SR, COUNT, CONTIG, false>(q, st);
}
template <int IN, int ROT, bool SR, bool COUNT>
hipError_t dispatch_contig(const QuantLaunch& q, hipStream_t st) {
  return (q.stride == q.cols) ? dispatch_manual<IN, ROT, SR, COUNT, true>(q, st)
                              : dispatch_manual<IN, ROT, SR, COUNT, false>(q, st);
}
template <int IN, int ROT, bool SR>
hipError_t dispatch_count(const QuantLaunch& q, hipStream_t st) {
  return q.counters ? dispatch_contig<IN, ROT, SR, true>(q, st) : dispatch_contig<IN, ROT, SR, false>(q, st);
}
template <int IN, int ROT>
hipError_t dispatch_sr(const QuantLaunch& q, hipStream_t st) {
  return q.stochastic ? dispatch_count<IN, ROT, true>(q, st) : dispatch_count<IN, ROT, false>(q, st);
}
template <int IN>
hipError_t dispatch_rot(const QuantLaunch& q, hipStream_t st) {
  return q.rotation == kRotRht16 ? dispatch_sr<IN, kRotRht16>(q, st) : dispatch_sr<IN, kRotNone>(q, st);
}

}  // namespace

hipError_t launch_zero_counters(unsigned long long* counters, hipStream_t st) {
  hipLaunchKernelGGL(zero_counters_kernel, dim3(1), dim3(64), 0, st, counters);
  return hipGetLastError();
}

hipError_t launch_count_reduce(unsigned long long* slots, unsigned long long* counters, hipStream_t st) {
  hipLaunchKernelGGL(count_reduce_kernel, dim3(1), dim3(64), 0, st, slots, counters);
  return hipGetLastError();
}

hipError_t launch_mx_quant(const QuantLaunch& q, hipStream_t st) {
  if (q.nslots == 0) return hipSuccess;
  const hipError_t e = q.in_dtype == kF32 ? dispatch_rot<kF32>(q, st) : dispatch_rot<kBF16>(q, st);
  if (e != hipSuccess || !q.counters || !q.count_slots) return e;
  return launch_count_reduce(q.count_slots, q.counters, st);
}

}  // namespace fp4q
