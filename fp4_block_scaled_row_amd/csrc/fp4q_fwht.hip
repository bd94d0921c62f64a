// fp4q_fwht.hip -- normalised Walsh-Hadamard transforms for gfx950, alone or
// fused with MXFP4 quantization of the rotated row.
//
// "Sub-4-Bit Microscaling (NVFP4, MXFP4 & Walsh-Hadamard Rotation)", section
// 3: y = x H_d / sqrt(d) with H_d the +-1 Sylvester Hadamard matrix, computed
// by the multiplier-free O(d log2 d) butterfly (a, b) -> (a + b, a - b), one
// stage per index bit, scaled once by fl32(1/sqrt(d)).  Stages over different
// bits commute, so each kernel runs them in whatever order keeps data in
// registers; the fp32 sums are then rounded in that order.
//
// Kernels:
//  * fwht8192_kernel: one 128-thread workgroup per row of 8192.  Layout L
//    (thread holds elements w*4096 + j*512 + l*8 + m): coalesced 16-byte loads,
//    6 butterfly stages in registers (bits 0-2 and 9-11).  An LDS transpose to
//    layout M (registers hold bits 3-8, lane bit 0 holds bit 12) runs 6
//    register stages plus one DPP stage; a second transpose returns to L,
//    where a lane quad holds a 32-block for the fused MXFP4 encoder.  The LDS
//    index is XOR-swizzled so both layouts access distinct banks.
//  * fwht_lds_kernel: any power of two 32 <= t <= 16384, one 256-thread
//    workgroup per t-chunk, all stages in LDS (also does the seeded signs).
//  * fwht_small_kernel: t in {2, 4, 8, 16}, per lane / lane pair in registers.
//
// The fused SwiGLU epilogue ("Sub-4-Bit Microscaling", section 3: the online
// rotation inside the SiLU_and_Mul kernel before down_proj) runs the first two
// kernels on h = SiLU(gate) * up, formed in fp32 as the two inputs are loaded
// (IN carries kSwiGlu); the activation never goes to memory.
#include <math.h>

#include "fp4q_flat.h"

namespace fp4q {
namespace {

constexpr int kSwiGlu = 2;   // IN flag: the input is SiLU_and_Mul(x, up)

// SiLU(g) * u = g / (1 + e^-g) * u in fp32 with the hardware exponential and
// reciprocal (about an ulp each); e^-g = inf gives -0 for finite g.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

__device__ __forceinline__ void load8_plain_f32(const void* base, int64_t off, float v[8]) {
  const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + off);
  const uint4 a = p[0], b = p[1];
  v[0] = as_f(a.x); v[1] = as_f(a.y); v[2] = as_f(a.z); v[3] = as_f(a.w);
  v[4] = as_f(b.x); v[5] = as_f(b.y); v[6] = as_f(b.z); v[7] = as_f(b.w);
}

__device__ __forceinline__ void load8_plain_bf16(const void* base, int64_t off, float v[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
  v[0] = bf_lo(a.x); v[1] = bf_hi(a.x); v[2] = bf_lo(a.y); v[3] = bf_hi(a.y);
  v[4] = bf_lo(a.z); v[5] = bf_hi(a.z); v[6] = bf_lo(a.w); v[7] = bf_hi(a.w);
}

// 8 consecutive fp32 input values at element offset `off` (IN & 1: the
// element type; IN & kSwiGlu: SiLU_and_Mul of f.x and f.up)
template <int IN>
__device__ __forceinline__ void load8(const FwhtLaunch& f, int64_t off, float v[8]) {
  if constexpr ((IN & 1) == kF32) load8_plain_f32(f.x, off, v);
  else load8_plain_bf16(f.x, off, v);
  if constexpr ((IN & kSwiGlu) != 0) {
    float u[8];
    if constexpr ((IN & 1) == kF32) load8_plain_f32(f.up, off, u);
    else load8_plain_bf16(f.up, off, u);
#pragma unroll
    for (int m = 0; m < 8; ++m) v[m] = silu_mul(v[m], u[m]);
  }
}

// ---------------------------------------------------------------- d = 8192
// LDS word index of element i.  gfx950 serves 4-byte accesses half a wave at
// a time over 32 banks (word bits 0-4) and 16-byte accesses 16 lanes at a
// time over 64 banks.  Layout M reads and writes 4 bytes per lane with lane
// bits 1-3 on word bits 0-2 and lane bits 0 and 4 on element bits 12 and 9,
// which the XOR moves onto word bits 4 and 3: 32 banks per half wave.
// Layout L moves 16 bytes per lane with lane bits on word bits 3-8 (the XOR
// is uniform there) and bit 2 flipped by lane bit 3: 64 banks per 16 lanes.
__device__ __forceinline__ int swz8192(int i) {
  const int k = ((i >> 9) & 1) | (((i >> 12) & 1) << 1) | (((i >> 10) & 1) << 2);
  return i ^ (k << 3) ^ (((i >> 6) & 1) << 2);
}

template <int IN, bool QUANT, bool SR, bool COUNT, bool MANUAL>
__global__ __launch_bounds__(128) void fwht8192_kernel(FwhtLaunch f, float c) {
  __shared__ float lds[8192];
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  uint32_t n_sat = 0, n_und = 0, n_nf = 0;
  const int iM = ((l & 1) << 12) | ((l >> 1) & 7) | (((l >> 4) & 3) << 9) | (w << 11);
  for (int64_t row = blockIdx.x; row < f.rows; row += gridDim.x) {
    float v[8][8];
    // ---- load (layout L) and widen
#pragma unroll
    for (int j = 0; j < 8; ++j) load8<IN>(f, row * f.stride + w * 4096 + j * 512 + l * 8, v[j]);
    // ---- stages on bits 0-2 (m) and 9-11 (j)
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int m = 0; m < 8; ++m)
          if (!(m & h)) {
            const float a = v[j][m], b = v[j][m + h];
            v[j][m] = a + b;
            v[j][m + h] = a - b;
          }
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (!(j & h))
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const float a = v[j][m], b = v[j + h][m];
            v[j][m] = a + b;
            v[j + h][m] = a - b;
          }
    // ---- transpose L -> M
    __syncthreads();  // previous row's reads are done
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int i = w * 4096 + j * 512 + l * 8 + 4 * k;
        *reinterpret_cast<float4*>(&lds[swz8192(i)]) =
            make_float4(v[j][4 * k], v[j][4 * k + 1], v[j][4 * k + 2], v[j][4 * k + 3]);
      }
    __syncthreads();
    float u[64];
#pragma unroll
    for (int r = 0; r < 64; ++r) u[r] = lds[swz8192(iM | (r << 3))];
    // ---- stages on bits 3-8 (r), then bit 12 across the lane pair
#pragma unroll
    for (int h = 1; h < 64; h <<= 1)
#pragma unroll
      for (int r = 0; r < 64; ++r)
        if (!(r & h)) {
          const float a = u[r], b = u[r + h];
          u[r] = a + b;
          u[r + h] = a - b;
        }
    const float sg = (l & 1) ? -1.0f : 1.0f;
    if constexpr ((IN & kSwiGlu) == 0) {
      // one v_fmac_f32_dpp per element: the odd lane holds u - p, the
      // negative of its p - u, until the scale by c, which takes the sign
      const float cs = c * sg;
#pragma unroll
      for (int r = 0; r < 64; r += 8) fmac_dpp_xor1_8(u + r, sg);
#pragma unroll
      for (int r = 0; r < 64; ++r) u[r] *= cs;
    } else {
      // (the even lane takes u + p, the odd lane p - u: a move and an FMA;
      // with the SwiGLU loads the DPP blocks above measured much slower, the
      // compiler then placing the next barrier before the butterflies)
#pragma unroll
      for (int r = 0; r < 64; ++r) {
        const float p = dpp_xor1_f(u[r]);
        u[r] = fmaf(sg, u[r], p) * c;
      }
    }
    // ---- transpose M -> L
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 64; ++r) lds[swz8192(iM | (r << 3))] = u[r];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int i = w * 4096 + j * 512 + l * 8 + 4 * k;
        const float4 q4 = *reinterpret_cast<const float4*>(&lds[swz8192(i)]);
        v[j][4 * k] = q4.x; v[j][4 * k + 1] = q4.y; v[j][4 * k + 2] = q4.z; v[j][4 * k + 3] = q4.w;
      }
    // ---- outputs
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t s = (row * 8192 + w * 4096 + j * 512 + l * 8) >> 3;
      if (f.y) store_rotated(f.y, s, v[j]);
      if constexpr (QUANT)
        mx_encode_slot<SR, COUNT, MANUAL>(v[j], s, true, l, f.manual_e, f.seed, f.codes, f.scales,
                                          n_sat, n_und, n_nf);
    }
  }
  if constexpr (COUNT) flush_counters(f.counters, f.count_slots, n_sat, n_und, n_nf);
}

// ---------------------------------------------------------------- generic LDS
template <int IN, bool QUANT, bool SR, bool COUNT, bool MANUAL>
__global__ __launch_bounds__(kThreads) void fwht_lds_kernel(FwhtLaunch f, int log2t, float c) {
  extern __shared__ float lds[];
  const int t = 1 << log2t;
  uint32_t* sgn = reinterpret_cast<uint32_t*>(lds + t);
  const int tid = threadIdx.x;
  uint32_t n_sat = 0, n_und = 0, n_nf = 0;
  if (f.random_signs) {
    for (int k = tid; k < (t + 127) / 128; k += kThreads) {
      const U4 ctr = {(uint32_t)k, 0u, 1u, 0u};
      const U4 o = philox4x32_10_uniform_key(ctr, (uint32_t)f.seed, (uint32_t)(f.seed >> 32));
      sgn[4 * k] = o.x; sgn[4 * k + 1] = o.y; sgn[4 * k + 2] = o.z; sgn[4 * k + 3] = o.w;
    }
  }
  const int64_t cpr = f.d / t;
  const int64_t total = f.rows * cpr;
  for (int64_t ch = blockIdx.x; ch < total; ch += gridDim.x) {
    const int64_t row = ch / cpr;
    const int64_t c0 = (ch - row * cpr) * t;
    __syncthreads();
    for (int sl = tid; sl < (t >> 3); sl += kThreads) {
      const int64_t off = row * f.stride + c0 + sl * 8;
      float v[8];
      load8<IN>(f, off, v);
      if (f.random_signs) {
        const uint32_t word = sgn[(sl * 8) >> 5] >> ((sl * 8) & 31);
#pragma unroll
        for (int m = 0; m < 8; ++m) v[m] = as_f(as_u(v[m]) ^ (((word >> m) & 1u) << 31));
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) lds[sl * 8 + m] = v[m];
    }
    __syncthreads();
    for (int h = 1; h < t; h <<= 1) {
      for (int p = tid; p < (t >> 1); p += kThreads) {
        const int i = ((p & ~(h - 1)) << 1) | (p & (h - 1));
        const float a = lds[i], b = lds[i + h];
        lds[i] = a + b;
        lds[i + h] = a - b;
      }
      __syncthreads();
    }
    for (int sl = tid; sl < (t >> 3); sl += kThreads) {
      float v[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) v[m] = lds[sl * 8 + m] * c;
      const int64_t s = (row * f.d + c0) / 8 + sl;
      if (f.y) store_rotated(f.y, s, v);
      if constexpr (QUANT)
        mx_encode_slot<SR, COUNT, MANUAL>(v, s, true, tid & 63, f.manual_e, f.seed, f.codes, f.scales,
                                          n_sat, n_und, n_nf);
    }
  }
  if constexpr (COUNT) flush_counters(f.counters, f.count_slots, n_sat, n_und, n_nf);
}

// ---------------------------------------------------------------- t <= 16
template <int IN, int T>
__global__ __launch_bounds__(kThreads) void fwht_small_kernel(FwhtLaunch f, float c, uint32_t signs) {
  const int lane = threadIdx.x & 63;
  const int64_t nslots = f.rows * f.d / 8;
  const int64_t ntiles = (nslots + 63) >> 6;
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  for (int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); t < ntiles; t += nwaves) {
    const int64_t s = (t << 6) + lane;
    const bool active = s < nslots;
    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (active) {
      const int64_t fl = s << 3;
      const int64_t row = fl / f.d;
      const int64_t off = row * f.stride + (fl - row * f.d);
      if constexpr (IN == kF32) {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(f.x) + off);
        const uint4 a = p[0], b = p[1];
        v[0] = as_f(a.x); v[1] = as_f(a.y); v[2] = as_f(a.z); v[3] = as_f(a.w);
        v[4] = as_f(b.x); v[5] = as_f(b.y); v[6] = as_f(b.z); v[7] = as_f(b.w);
      } else {
        const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(f.x) + off);
        v[0] = bf_lo(a.x); v[1] = bf_hi(a.x); v[2] = bf_lo(a.y); v[3] = bf_hi(a.y);
        v[4] = bf_lo(a.z); v[5] = bf_hi(a.z); v[6] = bf_lo(a.w); v[7] = bf_hi(a.w);
      }
    }
    if constexpr (T == 16) {
      rht16_pair(v, signs, (lane & 1) != 0);   // includes the exact x 1/4
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) v[m] = as_f(as_u(v[m]) ^ (((signs >> (m % T)) & 1u) << 31));
#pragma unroll
      for (int h = 1; h < T; h <<= 1)
#pragma unroll
        for (int m = 0; m < 8; ++m)
          if (!(m & h)) {
            const float a = v[m], b = v[m + h];
            v[m] = a + b;
            v[m + h] = a - b;
          }
#pragma unroll
      for (int m = 0; m < 8; ++m) v[m] *= c;
    }
    if (active) store_rotated(f.y, s, v);
  }
}

// ---------------------------------------------------------------- launchers
template <int IN, bool QUANT, bool SR, bool COUNT, bool MANUAL>
hipError_t launch_rows(const FwhtLaunch& f, hipStream_t st, float c, int log2t) {
  if (f.t == 8192 && f.d == 8192 && !f.random_signs) {
    const int64_t cap = (int64_t)device_cu_count() * 40;
    const int grid = (int)(f.rows < cap ? f.rows : cap);
    hipLaunchKernelGGL((fwht8192_kernel<IN, QUANT, SR, COUNT, MANUAL>), dim3(grid), dim3(128), 0, st, f, c);
    return hipGetLastError();
  }
  const int64_t total = f.rows * (f.d / f.t);
  const int64_t cap = (int64_t)device_cu_count() * 8;
  const int grid = (int)(total < cap ? total : cap);
  const size_t shmem = (size_t)f.t * 4 + (size_t)((f.t + 127) / 128) * 16;
  hipLaunchKernelGGL((fwht_lds_kernel<IN, QUANT, SR, COUNT, MANUAL>), dim3(grid), dim3(kThreads), shmem, st, f,
                     log2t, c);
  return hipGetLastError();
}

template <int IN, bool QUANT>
hipError_t d_quant_opts(const FwhtLaunch& f, hipStream_t st, float c, int log2t) {
  if constexpr (!QUANT) {
    return launch_rows<IN, false, false, false, false>(f, st, c, log2t);
  } else {
    if (f.stochastic) {
      if (f.counters) return f.manual ? launch_rows<IN, true, true, true, true>(f, st, c, log2t)
                                      : launch_rows<IN, true, true, true, false>(f, st, c, log2t);
      return f.manual ? launch_rows<IN, true, true, false, true>(f, st, c, log2t)
                      : launch_rows<IN, true, true, false, false>(f, st, c, log2t);
    }
    if (f.counters) return f.manual ? launch_rows<IN, true, false, true, true>(f, st, c, log2t)
                                    : launch_rows<IN, true, false, true, false>(f, st, c, log2t);
    return f.manual ? launch_rows<IN, true, false, false, true>(f, st, c, log2t)
                    : launch_rows<IN, true, false, false, false>(f, st, c, log2t);
  }
}

template <int IN>
hipError_t launch_small(const FwhtLaunch& f, hipStream_t st, float c) {
  uint32_t signs = 0u;
  if (f.random_signs) signs = rht_sign_word(f.seed, 0u, 0) & ((f.t >= 32) ? 0xFFFFFFFFu : ((1u << f.t) - 1u));
  const int64_t nslots = f.rows * f.d / 8;
  const int64_t ntiles = (nslots + 63) >> 6;
  const int64_t want = (ntiles + kWaves - 1) / kWaves;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  const int grid = (int)(want < 1 ? 1 : (want > cap ? cap : want));
  switch (f.t) {
    case 2: hipLaunchKernelGGL((fwht_small_kernel<IN, 2>), dim3(grid), dim3(kThreads), 0, st, f, c, signs); break;
    case 4: hipLaunchKernelGGL((fwht_small_kernel<IN, 4>), dim3(grid), dim3(kThreads), 0, st, f, c, signs); break;
    case 8: hipLaunchKernelGGL((fwht_small_kernel<IN, 8>), dim3(grid), dim3(kThreads), 0, st, f, c, signs); break;
    default: hipLaunchKernelGGL((fwht_small_kernel<IN, 16>), dim3(grid), dim3(kThreads), 0, st, f, c, signs); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwht_rows(const FwhtLaunch& f, hipStream_t st);

hipError_t launch_fwht(const FwhtLaunch& f, hipStream_t st) {
  const hipError_t e = launch_fwht_rows(f, st);
  if (e != hipSuccess || !f.quantize || !f.counters || !f.count_slots || f.rows == 0 || f.d == 0) return e;
  return launch_count_reduce(f.count_slots, f.counters, st);
}

hipError_t launch_fwht_rows(const FwhtLaunch& f, hipStream_t st) {
  if (f.rows == 0 || f.d == 0) return hipSuccess;
  const float c = (float)(1.0 / sqrt((double)f.t));
  int log2t = 0;
  while ((1 << log2t) < f.t) ++log2t;
  if (f.up) {   // fused SiLU_and_Mul: full-row transforms with quantization only
    if (f.t <= 16 || !f.quantize) return hipErrorInvalidValue;
    return f.in_dtype == kF32 ? d_quant_opts<kF32 | kSwiGlu, true>(f, st, c, log2t)
                              : d_quant_opts<kBF16 | kSwiGlu, true>(f, st, c, log2t);
  }
  if (f.t <= 16) return f.in_dtype == kF32 ? launch_small<kF32>(f, st, c) : launch_small<kBF16>(f, st, c);
  if (f.quantize)
    return f.in_dtype == kF32 ? d_quant_opts<kF32, true>(f, st, c, log2t) : d_quant_opts<kBF16, true>(f, st, c, log2t);
  return f.in_dtype == kF32 ? d_quant_opts<kF32, false>(f, st, c, log2t) : d_quant_opts<kBF16, false>(f, st, c, log2t);
}

}  // namespace fp4q
