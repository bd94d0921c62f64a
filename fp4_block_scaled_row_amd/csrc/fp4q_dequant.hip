// fp4q_dequant.hip -- reconstruction of MXFP4 / NVFP4 tensors on gfx950.
//
// "MXFP4 Quantization: Audit the 4.25-Bit Blocks", "Encode one MXFP4 block
// step by step": a code reconstructs as its lattice value times the block
// scale.  MX: value * 2^(b-127), exact in fp32 and bf16 -- done by the gfx950
// scaled FP4 -> fp32/bf16 conversions, whose scale operand is the E8M0 byte.
// NV ("Sub-4-Bit Microscaling", section 2): value * s * g.  value * s is exact
// in fp32; the product with g is rounded once: for fp32 output by the fp32
// multiply, for bf16 output by rounding the fp32 product to nearest-even and,
// when that product sits exactly on a bf16 rounding boundary, deciding with
// the sign of its exact rounding error: fma(v s, g, -p) is that error exactly
// (the error of an fp32 product is an fp32 number), so the side of the
// boundary the exact product lies on is known without wider arithmetic; products
// below 2^-100, where the error could underflow, use the fp64 product
// (value * s * g has <= 31 significant bits).  bf16 outputs are stored
// non-temporally: they are written once and not read back by this kernel.
// IF4 ("Adaptive Block-Scaled Data Types" transcript, cues 14 and 17): a
// block whose scale byte has bit 7 set holds sign-magnitude INT4 nibbles k
// worth k * 6 s g / 7, looked up in a per-workgroup table of the 8
// magnitudes of each scale code rounded once to the output type; the other
// blocks decode as NV.
#include "fp4q_flat.h"

namespace fp4q {
namespace {

constexpr int kUnroll = 8;

__device__ __forceinline__ uint32_t bf16_of_product(float vs, float g) {
  const float av = fabsf(vs);
  const float a = av * g;
  const uint32_t b = as_u(a);
  const uint32_t hi = b >> 16;
  uint32_t r = (b + 0x7FFFu + (hi & 1u)) >> 16;
  if ((b & 0xFFFFu) == 0x8000u) {   // on a bf16 midpoint: which side is the exact product?
    int side;
    if (a >= 0x1p-100f) {
      const float e = fmaf(av, g, -a);
      side = e > 0.0f ? 1 : (e < 0.0f ? -1 : 0);
    } else {
      const double ex = (double)av * (double)g;
      side = ex > (double)a ? 1 : (ex < (double)a ? -1 : 0);
    }
    r = side > 0 ? hi + 1u : (side < 0 ? hi : hi + (hi & 1u));
  }
  return r | ((as_u(vs) >> 31) << 15);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Output bits (fp32, or bf16 in the low half) of k * 6 * s_c * g / 7 rounded
// once: the numerator is exact in fp64 and the fp64 quotient is never within
// 2^-33 (relatively) of an fp32 or bf16 rounding boundary unless the exact
// value lies on it.  Its fp32 rounding can still land exactly on a bf16
// midpoint; the fp64 value then says on which side the exact value is.
template <int OUT>
__device__ __forceinline__ uint32_t int4_magnitude_bits(int c, int k, float g) {
  const double q = (double)k * 6.0 * (double)e4m3_value((uint32_t)c) * (double)g / 7.0;
  const float f = (float)q;
  const uint32_t b = as_u(f);
  if constexpr (OUT == kF32) return b;
  const uint32_t hi = b >> 16;
  if ((b & 0xFFFFu) != 0x8000u) return (b + 0x7FFFu + (hi & 1u)) >> 16;
  return q > (double)f ? hi + 1u : (q < (double)f ? hi : hi + (hi & 1u));
}

template <int FMT, int OUT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(DequantLaunch d, int64_t nslots) {
  __shared__ uint32_t s_i4[FMT == 2 ? 1024 : 1];
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  const int64_t ntiles = (nslots + 63) >> 6;
  float g = 1.0f;
  if constexpr (FMT != 0) g = *d.global_scale;
  if constexpr (FMT == 2) {
    for (int e = threadIdx.x; e < 1024; e += kThreads) s_i4[e] = int4_magnitude_bits<OUT>(e >> 3, e & 7, g);
    __syncthreads();
  }
  const float one = e8m0_operand(127u);
  for (int64_t g0 = wave; g0 * kUnroll < ntiles; g0 += nwaves) {
    uint32_t cw[kUnroll], sb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t s = ((g0 * kUnroll + u) << 6) + lane;
      const bool act = s < nslots;
      cw[u] = act ? *reinterpret_cast<const uint32_t*>(d.codes + (s << 2)) : 0u;
      sb[u] = act ? (uint32_t)d.scales[FMT == 0 ? (s >> 2) : (s >> 1)] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t t = g0 * kUnroll + u;
      if (t >= ntiles) break;
      const int64_t s = (t << 6) + lane;
      if (s >= nslots) continue;
      if constexpr (FMT == 0) {
        const bool nan = sb[u] == 255u;
        const float sc = e8m0_operand(sb[u]);
        if constexpr (OUT == kF32) {
          float o[8];
          float2_t p;
          p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u], sc, 0); o[0] = p.x; o[1] = p.y;
          p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u], sc, 1); o[2] = p.x; o[3] = p.y;
          p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u], sc, 2); o[4] = p.x; o[5] = p.y;
          p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u], sc, 3); o[6] = p.x; o[7] = p.y;
          if (nan) {
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = as_f(0x7FC00000u);
          }
          store_rotated(static_cast<float*>(d.out), s, o);
        } else {
          uint4 o;
          o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[u], sc, 0));
          o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[u], sc, 1));
          o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[u], sc, 2));
          o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[u], sc, 3));
          if (nan) o = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
          __builtin_nontemporal_store(u32x4_t{o.x, o.y, o.z, o.w},
                                      reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(d.out) + (s << 3)));
        }
      } else {
        const bool nan = sb[u] == 0x7Fu || sb[u] == 0xFFu;
        if constexpr (FMT == 2) {
          if (sb[u] & 0x80u) {   // INT4 block
            const uint32_t* row = s_i4 + 8 * (sb[u] & 0x7Fu);
            if constexpr (OUT == kF32) {
              float o[8];
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                const uint32_t nib = (cw[u] >> (4 * i)) & 15u;
                o[i] = nan ? as_f(0x7FC00000u) : as_f(row[nib & 7u] | ((nib & 8u) << 28));
              }
              store_rotated(static_cast<float*>(d.out), s, o);
            } else {
              uint32_t h[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint32_t n0 = (cw[u] >> (8 * i)) & 15u, n1 = (cw[u] >> (8 * i + 4)) & 15u;
                h[i] = (row[n0 & 7u] | ((n0 & 8u) << 12)) | ((row[n1 & 7u] | ((n1 & 8u) << 12)) << 16);
              }
              if (nan) h[0] = h[1] = h[2] = h[3] = 0x7FC07FC0u;
              const u32x4_t o = {h[0], h[1], h[2], h[3]};
              __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(d.out) + (s << 3)));
            }
            continue;
          }
        }
        const float sd = e4m3_value(sb[u] & 0x7Fu);
        float val[8];
        float2_t p;
        p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u], one, 0); val[0] = p.x; val[1] = p.y;
        p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u], one, 1); val[2] = p.x; val[3] = p.y;
        p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u], one, 2); val[4] = p.x; val[5] = p.y;
        p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u], one, 3); val[6] = p.x; val[7] = p.y;
        if constexpr (OUT == kF32) {
          float o[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] = nan ? as_f(0x7FC00000u) : (val[i] * sd) * g;
          store_rotated(static_cast<float*>(d.out), s, o);
        } else {
          // fp32 products rounded to bf16 by the hardware conversion (nearest-even);
          // a product sitting exactly on a bf16 midpoint is redone exactly
          float pr[8];
          uint32_t tie = 0u;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            pr[i] = (val[i] * sd) * g;
            tie |= ((as_u(pr[i]) & 0xFFFFu) == 0x8000u) ? (1u << i) : 0u;
          }
          uint32_t h[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bf16x2_t pk = {(__bf16)pr[2 * i], (__bf16)pr[2 * i + 1]};
            h[i] = __builtin_bit_cast(uint32_t, pk);
          }
          if (tie != 0u) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              if ((tie >> i) & 1u) {
                const uint32_t r = bf16_of_product(val[i] * sd, g);
                h[i >> 1] = (i & 1) ? ((h[i >> 1] & 0xFFFFu) | (r << 16)) : ((h[i >> 1] & 0xFFFF0000u) | r);
              }
            }
          }
          if (nan) h[0] = h[1] = h[2] = h[3] = 0x7FC07FC0u;
          const u32x4_t o = {h[0], h[1], h[2], h[3]};
          __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(d.out) + (s << 3)));
        }
      }
    }
  }
}

template <int FMT, int OUT>
hipError_t launch_t(const DequantLaunch& d, hipStream_t st) {
  const int64_t nslots = d.rows * d.cols / 8;
  const int64_t ntiles = (nslots + 63) >> 6;
  const int64_t want = (ntiles + kWaves * kUnroll - 1) / (kWaves * kUnroll);
  const int64_t cap = (int64_t)device_cu_count() * 16;   // (measured: 16 per CU against 8)
  const int grid = (int)(want < 1 ? 1 : (want > cap ? cap : want));
  hipLaunchKernelGGL((dequant_kernel<FMT, OUT>), dim3(grid), dim3(kThreads), 0, st, d, nslots);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(const DequantLaunch& d, hipStream_t st) {
  if (d.rows == 0 || d.cols == 0) return hipSuccess;
  if (d.format == 0) return d.out_dtype == kF32 ? launch_t<0, kF32>(d, st) : launch_t<0, kBF16>(d, st);
  if (d.format == 2) return d.out_dtype == kF32 ? launch_t<2, kF32>(d, st) : launch_t<2, kBF16>(d, st);
  return d.out_dtype == kF32 ? launch_t<1, kF32>(d, st) : launch_t<1, kBF16>(d, st);
}

}  // namespace fp4q
