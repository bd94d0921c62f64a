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
// 64 bytes) are loaded straight into LDS (buffer loads with the LDS
// destination: in that form, unlike the flat one, the compiler lets an LDS
// read wait only for the loads it depends on), into a ring of four stage
// buffers kept three stages ahead of the one being multiplied; one fence-free
// barrier per stage, the loads being waited for explicitly.  The scale bytes
// go straight into registers, 16 bytes of a row (four stages) per load, one
// group of four stages ahead: the load unit moves about one cache line a
// clock per CU, and a 4-byte load per row and stage would cost a line for
// every 4 bytes.
// Buffer offsets are 32-bit: K is at most 2^23.  A tile wholly inside C
// (with 16-byte aligned rows) leaves through LDS as 16-byte row chunks; other
// tiles store element by element.  Workgroups are
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
constexpr int kXcds = 8;
constexpr int kGroupRows = 8;

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

typedef __attribute__((address_space(3))) void lds_void_t;

// LDS stage buffer: A codes (256 rows x 64 bytes, the four 16-byte chunks of
// a row permuted by (row >> 1) mod 4 to spread reads over the banks), then B
// codes.
constexpr int kCodeBytes = kTile * kRowBytes;               // 16 KiB
constexpr int kStageBytes = 2 * kCodeBytes;
constexpr int kLoadsPerStage = 2 * (kCodeBytes / 1024 / 4);   // per lane: 4 + 4 codes
constexpr int kGroup = 4;                                     // stages per 16 scale bytes of a row
typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int chunk_of(int row, int part) { return part ^ ((row >> 1) & 3); }

// Direct-to-LDS loads through a buffer descriptor at base (bytes long), of 16
// bytes per lane: lane l writes lds + 16 l; off is this lane's byte offset
// from base.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const uint8_t* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0,
                                           (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF), 0x00020000);
}
__device__ __forceinline__ void buf_lds16(const uint8_t* base, int64_t bytes, lds_void_t* lds, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(buf_rsrc(base, bytes), lds, 16, off, 0, 0, 0);
}

// s_waitcnt with vmcnt <= n (expcnt and lgkmcnt not waited for)
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <bool BF16OUT>
__global__ __launch_bounds__(256) void mx_gemm_kernel(GemmLaunch g, int tiles_m, int tiles_n, int ntiles) {
  // four stage buffers as separate objects, so that reads of one are not
  // ordered after the direct-to-LDS loads still in flight into the others
  __shared__ __align__(16) uint8_t s_st0[kStageBytes];
  __shared__ __align__(16) uint8_t s_st1[kStageBytes];
  __shared__ __align__(16) uint8_t s_st2[kStageBytes];
  __shared__ __align__(16) uint8_t s_st3[kStageBytes];
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
  // rows past M or N read a valid row instead; their results are not stored
  // buffer bases at the tile's first row; offsets below 256 kb + kb < 2^31
  const uint8_t* a_c = g.a_codes + m0 * kb;
  const uint8_t* b_c = g.b_codes + n0 * kb;
  const uint8_t* a_s = g.a_scales + m0 * ksb;
  const uint8_t* b_s = g.b_scales + n0 * ksb;
  const int64_t na_c = (g.M - m0) * kb, nb_c = (g.N - n0) * kb, na_s = (g.M - m0) * ksb, nb_s = (g.N - n0) * ksb;
  auto issue = [&](int st, uint8_t* buf) {
    const int64_t kbyte = (int64_t)st * kRowBytes;
#pragma unroll
    for (int i = 0; i < kCodeBytes / 1024 / 4; ++i) {
      const int region = wv * (kCodeBytes / 1024 / 4) + i;   // 16 rows x 64 bytes
      const int row = region * 16 + (lane >> 2);
      const int part = chunk_of(row, lane & 3);
      const int64_t ra = min(m0 + row, g.M - 1) - m0, rb = min(n0 + row, g.N - 1) - n0;
      buf_lds16(a_c, na_c, (lds_void_t*)(buf + region * 1024), (int)(ra * kb + kbyte + part * 16));
      buf_lds16(b_c, nb_c, (lds_void_t*)(buf + kCodeBytes + region * 1024), (int)(rb * kb + kbyte + part * 16));
    }
  };
  // scale bytes of the four stages of group gi for this lane's 4 A rows and 4 B
  // rows: 16 bytes a row, straight into registers (lanes l and l + 32 read the
  // same row; bytes past a row's end, read for a last group of fewer than four
  // stages, are never used)
  const int wr = wv >> 1, wc = wv & 1;
  int a_soff[kSub], b_soff[kSub];
#pragma unroll
  for (int u = 0; u < kSub; ++u) {
    const int r = kWaveTile * wr + 32 * u + (lane & 31), c = kWaveTile * wc + 32 * u + (lane & 31);
    a_soff[u] = (int)((min(m0 + r, g.M - 1) - m0) * ksb);
    b_soff[u] = (int)((min(n0 + c, g.N - 1) - n0) * ksb);
  }
  const __amdgpu_buffer_rsrc_t a_srs = buf_rsrc(a_s, na_s), b_srs = buf_rsrc(b_s, nb_s);
  v4u_t sA[2][kSub], sB[2][kSub];
  auto load_scales = [&](int gi, v4u_t (&da)[kSub], v4u_t (&db)[kSub]) {
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
      da[u] = __builtin_amdgcn_raw_buffer_load_b128(a_srs, a_soff[u] + 16 * gi, 0, 0);
      db[u] = __builtin_amdgcn_raw_buffer_load_b128(b_srs, b_soff[u] + 16 * gi, 0, 0);
    }
  };

  v16f_t acc[kSub][kSub];
#pragma unroll
  for (int i = 0; i < kSub; ++i)
#pragma unroll
    for (int j = 0; j < kSub; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // a stage's operands, both 64-K steps
  v8i_t a[2][kSub], b[2][kSub];
  int sa[2][kSub], sb[2][kSub];
  auto read = [&](const uint8_t* buf, const v4u_t (&ra_)[kSub], const v4u_t (&rb_)[kSub], int sg) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int part = 2 * kk + (lane >> 5);   // this lane's 32 K positions of the 64-K step
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        const int arow = kWaveTile * wr + 32 * u + (lane & 31);
        const uint4 va = *reinterpret_cast<const uint4*>(buf + arow * kRowBytes + chunk_of(arow, part) * 16);
        a[kk][u] = v8i_t{(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
        sa[kk][u] = (int)((ra_[u][sg] >> (8 * part)) & 0xFFu);
        const int brow = kWaveTile * wc + 32 * u + (lane & 31);
        const uint4 vb = *reinterpret_cast<const uint4*>(buf + kCodeBytes + brow * kRowBytes + chunk_of(brow, part) * 16);
        b[kk][u] = v8i_t{(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
        sb[kk][u] = (int)((rb_[u][sg] >> (8 * part)) & 0xFFu);
      }
    }
  };
  auto mma = [&](int kk) {
#pragma unroll
    for (int i = 0; i < kSub; ++i)
#pragma unroll
      for (int j = 0; j < kSub; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[kk][i], b[kk][j], acc[i][j], 4, 4, 0,
                                                                    sa[kk][i], 0, sb[kk][j]);
  };
  // one pipeline step: wait for this thread's loads of stage st (stages
  // st + 1 and st + 2, and the next scale group, stay in flight), one barrier -- after it every wave's
  // loads of stage st are in LDS and every wave is done with stage st - 1 --
  // then read stage st's operands, multiply the first 64-K step (its operands
  // arrive first), refill stage st - 1's buffer with stage st + 3 and
  // multiply the second step (the first step of a scale group also loads the
  // next group's scales after the refill).  Every LDS read of the step is
  // issued before the refill, so none of them waits for it.  The barrier
  // carries no memory fence: the loads are waited for explicitly.  The wait
  // counts the vm loads issued after stage st's refill, the moment step st
  // begins: the
  // refills of st + 1 and st + 2, and the scale group loaded by the first step
  // of st's group when that step came after st's refill was issued (st not
  // the first of its group)
  auto step = [&](int st, uint8_t* cur, uint8_t* fill, const v4u_t (&ra_)[kSub], const v4u_t (&rb_)[kSub],
                  v4u_t (&na_)[kSub], v4u_t (&nb_)[kSub]) {
    const int sg = st % kGroup;
    const int after = (st + 1 < nstage ? 1 : 0) + (st + 2 < nstage ? 1 : 0) +
                      ((sg != 0 && st - sg + kGroup < nstage) ? 1 : 0);
    if (after == 3) wait_vm<3 * kLoadsPerStage>();
    else if (after == 2) wait_vm<2 * kLoadsPerStage>();
    else if (after == 1) wait_vm<kLoadsPerStage>();
    else wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    read(cur, ra_, rb_, sg);
    __builtin_amdgcn_sched_barrier(0);
    mma(0);
    __builtin_amdgcn_sched_barrier(0);
    if (st + 3 < nstage) issue(st + 3, fill);
    if (sg == 0 && st + kGroup < nstage) load_scales(st / kGroup + 1, na_, nb_);
    __builtin_amdgcn_sched_barrier(0);
    mma(1);
  };

  if (nstage > 0) load_scales(0, sA[0], sB[0]);
  if (nstage > 0) issue(0, s_st0);
  if (nstage > 1) issue(1, s_st1);
  if (nstage > 2) issue(2, s_st2);
  // (unrolled over two rotations of the ring, two scale groups)
  for (int st = 0; st < nstage; st += 8) {
    step(st, s_st0, s_st3, sA[0], sB[0], sA[1], sB[1]);
    if (st + 1 < nstage) step(st + 1, s_st1, s_st0, sA[0], sB[0], sA[1], sB[1]);
    if (st + 2 < nstage) step(st + 2, s_st2, s_st1, sA[0], sB[0], sA[1], sB[1]);
    if (st + 3 < nstage) step(st + 3, s_st3, s_st2, sA[0], sB[0], sA[1], sB[1]);
    if (st + 4 < nstage) step(st + 4, s_st0, s_st3, sA[1], sB[1], sA[0], sB[0]);
    if (st + 5 < nstage) step(st + 5, s_st1, s_st0, sA[1], sB[1], sA[0], sB[0]);
    if (st + 6 < nstage) step(st + 6, s_st2, s_st1, sA[1], sB[1], sA[0], sB[0]);
    if (st + 7 < nstage) step(st + 7, s_st3, s_st2, sA[1], sB[1], sA[0], sB[0]);
  }

  // A tile wholly inside C, with 16-byte aligned rows: each wave writes its
  // quarter 32 rows at a time into its own stage buffer, in the accumulator
  // layout, and stores it back as 16-byte row chunks.
  const bool whole = m0 + kTile <= g.M && n0 + kTile <= g.N && g.N % 8 == 0 &&
                     (reinterpret_cast<uintptr_t>(g.c) & 15) == 0;
  if (whole) {
    __syncthreads();   // every wave is done with the stage buffers
    uint8_t* band = wv == 0 ? s_st0 : wv == 1 ? s_st1 : wv == 2 ? s_st2 : s_st3;
    const int64_t row0 = m0 + kWaveTile * wr, col0 = n0 + kWaveTile * wc;
#pragma unroll
    for (int i = 0; i < kSub; ++i) {
      if constexpr (BF16OUT) {
        constexpr int kStride = kWaveTile + 8;   // bf16 elements per band row (272 bytes)
        __bf16* t = reinterpret_cast<__bf16*>(band);
#pragma unroll
        for (int j = 0; j < kSub; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            t[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * kStride + 32 * j + (lane & 31)] = (__bf16)acc[i][j][r];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int rr = 4 * k + (lane >> 4), cc = (lane & 15) * 8;
          const uint4 v = *reinterpret_cast<const uint4*>(t + rr * kStride + cc);
          *reinterpret_cast<uint4*>(static_cast<__bf16*>(g.c) + (row0 + 32 * i + rr) * g.N + col0 + cc) = v;
        }
      } else {
        constexpr int kStride = kWaveTile + 4;   // floats per band row (528 bytes)
        float* t = reinterpret_cast<float*>(band);
#pragma unroll
        for (int j = 0; j < kSub; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            t[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * kStride + 32 * j + (lane & 31)] = acc[i][j][r];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int rr = 2 * k + (lane >> 5), cc = (lane & 31) * 4;
          const float4 v = *reinterpret_cast<const float4*>(t + rr * kStride + cc);
          *reinterpret_cast<float4*>(static_cast<float*>(g.c) + (row0 + 32 * i + rr) * g.N + col0 + cc) = v;
        }
      }
    }
    return;
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
