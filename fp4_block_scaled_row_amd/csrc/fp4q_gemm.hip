// fp4q_gemm.hip -- MXFP4 x MXFP4 GEMM on gfx950's block-scaled FP4 matrix
// instructions: C[m][n] = sum_k A[m][k] B[n][k] over the reconstructed MXFP4
// values of two tensors in the quantizer's layout (codes [rows][K/2], element
// 2t in the low nibble of byte t; E8M0 scales [rows][K/32]), fp32
// accumulation, fp32 or bf16 output.  "Sub-4-Bit Microscaling", section 3:
// Y = X W^T with both operands 4-bit block-scaled; section 2: the E8M0 block
// scales are applied inside the matrix instruction.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E2M1: one instruction
// multiplies a 32x64 A tile by a 64x32 B tile.  Lane l supplies row (l mod 32)
// of A and column (l mod 32) of B for the K positions 32 (l / 32) .. +31
// (16 bytes of nibbles) together with the E8M0 byte of that 32-block; the
// 32x32 fp32 result of lane l, register r, is element (8 (r / 4) + 4 (l / 32)
// + r mod 4, l mod 32).
//
// Tiling: a 256-thread workgroup computes a 256x256 tile of C, each of its
// four waves (one per SIMD) a 128x128 quarter: 4x4 instructions per 64-K
// step on 256 accumulator registers, so every operand fetched from LDS feeds
// four instructions.  K advances 128 per stage: the A and B tiles (256 rows x
// 64 bytes, rows padded to 80 bytes in LDS to spread the 16-byte reads over
// the banks) and their scale bytes go through LDS, double-buffered, with the
// next stage's global loads
// in flight during the current stage's matrix instructions.  Workgroups are
// numbered so that each XCD walks a contiguous range of C tiles, in groups of
// 8 tile rows traversed column by column, so that the workgroups resident on
// one XCD at a time share both A row tiles and B column tiles in its L2.
#include "fp4q_common.h"
#include "fp4q_internal.h"

namespace fp4q {
namespace {

constexpr int kTile = 256;
constexpr int kWaveTile = kTile / 2;   // 128: a 2x2 arrangement of waves
constexpr int kSub = kWaveTile / 32;   // 4x4 instructions per wave
constexpr int kKStep = 128;
constexpr int kRowBytes = kKStep / 2;     // 64 bytes of nibbles per row and stage
constexpr int kLdsStride = kRowBytes + 16;
constexpr int kXcds = 8;
constexpr int kGroupRows = 8;

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

template <bool BF16OUT>
__global__ __launch_bounds__(256) void mx_gemm_kernel(GemmLaunch g, int tiles_m, int tiles_n, int ntiles) {
  __shared__ __align__(16) uint8_t s_a[2][kTile * kLdsStride];
  __shared__ __align__(16) uint8_t s_b[2][kTile * kLdsStride];
  __shared__ uint32_t s_sa[2][kTile];   // the 4 scale bytes of a row for the stage's 4 K-blocks
  __shared__ uint32_t s_sb[2][kTile];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  // XCD-contiguous tile order: workgroup w runs on XCD w mod 8
  const int w = blockIdx.x;
  const int per = (ntiles + kXcds - 1) / kXcds;
  const int t = (w % kXcds) * per + w / kXcds;
  if (t >= ntiles) return;
  const int group = t / (kGroupRows * tiles_n);
  const int first_m = group * kGroupRows;
  const int gsize = min(tiles_m - first_m, kGroupRows);
  const int in_g = t - group * kGroupRows * tiles_n;
  const int64_t m0 = (int64_t)(first_m + in_g % gsize) * kTile, n0 = (int64_t)(in_g / gsize) * kTile;

  const int64_t kb = g.K / 2, ksb = g.K / 32;
  const int nstage = (int)(g.K / kKStep);
  constexpr int kChunks = kTile * 4 / 256;   // 16-byte chunks per thread and operand
  uint4 ra[kChunks], rb[kChunks];
  uint32_t rsa = 0u, rsb = 0u;
  auto gload = [&](int st) {
    const int64_t kbyte = (int64_t)st * kRowBytes;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + 256 * i;   // row c / 4, part c mod 4
      const int row = c >> 2, part = c & 3;
      const int64_t ma = m0 + row, nb = n0 + row;
      ra[i] = ma < g.M ? *reinterpret_cast<const uint4*>(g.a_codes + ma * kb + kbyte + part * 16) : make_uint4(0, 0, 0, 0);
      rb[i] = nb < g.N ? *reinterpret_cast<const uint4*>(g.b_codes + nb * kb + kbyte + part * 16) : make_uint4(0, 0, 0, 0);
    }
    const int64_t ra_ = m0 + tid, rb_ = n0 + tid;   // one A row and one B row of scale bytes per thread
    rsa = ra_ < g.M ? *reinterpret_cast<const uint32_t*>(g.a_scales + ra_ * ksb + (int64_t)st * 4) : 0x7F7F7F7Fu;
    rsb = rb_ < g.N ? *reinterpret_cast<const uint32_t*>(g.b_scales + rb_ * ksb + (int64_t)st * 4) : 0x7F7F7F7Fu;
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 2, part = c & 3;
      *reinterpret_cast<uint4*>(&s_a[buf][row * kLdsStride + part * 16]) = ra[i];
      *reinterpret_cast<uint4*>(&s_b[buf][row * kLdsStride + part * 16]) = rb[i];
    }
    s_sa[buf][tid] = rsa;
    s_sb[buf][tid] = rsb;
  };

  const int wr = wv >> 1, wc = wv & 1;
  v16f_t acc[kSub][kSub];
#pragma unroll
  for (int i = 0; i < kSub; ++i)
#pragma unroll
    for (int j = 0; j < kSub; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (nstage > 0) {
    gload(0);
    lstore(0);
    __syncthreads();
  }
  for (int st = 0; st < nstage; ++st) {
    const int buf = st & 1;
    if (st + 1 < nstage) gload(st + 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int part = 2 * kk + (lane >> 5);   // this lane's 32 K positions of the 64-K step
      v8i_t a[kSub], b[kSub];
      int sa[kSub], sb[kSub];
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        const int arow = kWaveTile * wr + 32 * u + (lane & 31);
        const uint4 va = *reinterpret_cast<const uint4*>(&s_a[buf][arow * kLdsStride + part * 16]);
        a[u] = v8i_t{(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
        sa[u] = (int)((s_sa[buf][arow] >> (8 * part)) & 0xFFu);
        const int brow = kWaveTile * wc + 32 * u + (lane & 31);
        const uint4 vb = *reinterpret_cast<const uint4*>(&s_b[buf][brow * kLdsStride + part * 16]);
        b[u] = v8i_t{(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
        sb[u] = (int)((s_sb[buf][brow] >> (8 * part)) & 0xFFu);
      }
#pragma unroll
      for (int i = 0; i < kSub; ++i)
#pragma unroll
        for (int j = 0; j < kSub; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
    }
    if (st + 1 < nstage) {
      lstore(buf ^ 1);
      __syncthreads();
    }
  }

#pragma unroll
  for (int i = 0; i < kSub; ++i)
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      const int64_t col = n0 + kWaveTile * wc + 32 * j + (lane & 31);
      if (col >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + kWaveTile * wr + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= g.M) continue;
        if constexpr (BF16OUT) {
          static_cast<__bf16*>(g.c)[row * g.N + col] = (__bf16)acc[i][j][r];
        } else {
          static_cast<float*>(g.c)[row * g.N + col] = acc[i][j][r];
        }
      }
    }
}

}  // namespace

hipError_t launch_mx_gemm(const GemmLaunch& g, hipStream_t st) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  const int64_t tm = (g.M + kTile - 1) / kTile, tn = (g.N + kTile - 1) / kTile;
  const int64_t nt = tm * tn;
  if (nt > 0x7FFFFFFF / 2) return hipErrorInvalidValue;
  const int per = (int)((nt + kXcds - 1) / kXcds);
  const int grid = per * kXcds;
  if (g.out_bf16)
    hipLaunchKernelGGL((mx_gemm_kernel<true>), dim3(grid), dim3(256), 0, st, g, (int)tm, (int)tn, (int)nt);
  else
    hipLaunchKernelGGL((mx_gemm_kernel<false>), dim3(grid), dim3(256), 0, st, g, (int)tm, (int)tn, (int)nt);
  return hipGetLastError();
}

}  // namespace fp4q
