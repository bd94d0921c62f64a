// fp4q_internal.h -- launch interface between the C ABI (fp4q_api.hip) and
// the kernel translation units.  Host-side only declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

// Flat elementwise quantizers: a "slot" is 8 consecutive elements of a row.
struct QuantLaunch {
  const void* x;
  int64_t rows, cols, stride;
  int64_t nslots;            // rows * cols / 8
  int in_dtype;              // kF32 / kBF16
  int rotation;              // kRotNone / kRotRht16
  int stochastic;            // 0 / 1
  int manual;                // MX: manual exponent policy
  int manual_e;
  int four_over_six;         // NV
  int if4;                   // NV: per block FP4 or scaled INT4
  uint64_t seed;
  uint32_t rht_signs;        // 16-bit sign mask of the RHT diagonal
  float rot_scale;           // FWHT-128: fl32(1 / sqrt(128))
  uint8_t* codes;
  uint8_t* scales;
  float* global_scale;
  uint8_t* choice_bits;
  float* rotated;
  unsigned long long* counters;
  const float* global_amax;  // NV: caller-supplied amax (device) or null
  uint32_t* partials;        // NV: per-workgroup amax partials (workspace)
  unsigned long long* count_slots;  // counter slots in the workspace, or null (atomics into counters)
};

constexpr int kAmaxPartialsMax = 1024;  // workgroups of the NV amax pass
// NVFP4 workspace layout (bytes): [0, 64) header of the single-launch kernel
// (u64 word 2: wait limit override, word 3: epoch word of captured launches), [64,
// 64 + 8 * 1024) its per-workgroup flags, [8256, 8256 + 4 * 1024) the amax partials of the
// two-pass kernels, [16384, 16384 + 4096 * 16) sixteen copies of the result
// word of the single-launch kernel, 4 KiB apart.
constexpr size_t kWsFlagsOffsetBytes = 64;
constexpr size_t kWsPartialsOffsetBytes = kWsFlagsOffsetBytes + 8 * kAmaxPartialsMax;
constexpr size_t kWsResultsOffsetBytes = 16384;
constexpr size_t kWsResultStrideBytes = 4096;
constexpr int kWsResultCopies = 16;
constexpr size_t kNvWorkspaceBytes = kWsResultsOffsetBytes + kWsResultStrideBytes * kWsResultCopies;

// Counter slots: a counting kernel's workgroup b adds its three counts into
// slot b % kCountSlots (few workgroups per address, unlike one set of three
// global words), and a one-workgroup kernel sums the slots into the counters
// and zeroes them again.  NV: at [12352, 15424) of the NV workspace; MX: at
// the start of its own kMxWorkspaceBytes workspace.
constexpr int kCountSlots = 128;
constexpr size_t kCountSlotBytes = (size_t)kCountSlots * 3 * 8;
constexpr size_t kWsCountOffsetBytes = kWsPartialsOffsetBytes + 4 * kAmaxPartialsMax;
static_assert(kWsCountOffsetBytes + kCountSlotBytes <= kWsResultsOffsetBytes, "NV workspace layout");
constexpr size_t kMxWorkspaceBytes = 4096;
static_assert(kCountSlotBytes <= kMxWorkspaceBytes, "MX workspace layout");

hipError_t launch_zero_counters(unsigned long long* counters, hipStream_t s);
hipError_t launch_count_reduce(unsigned long long* slots, unsigned long long* counters, hipStream_t s);
hipError_t launch_mx_quant(const QuantLaunch& q, hipStream_t s);
hipError_t launch_nv_quant(const QuantLaunch& q, hipStream_t s);
bool nv_resident_shape(const QuantLaunch& q, int* grid, int* nres);
hipError_t launch_nv_resident(const QuantLaunch& q, int grid, int nres, hipStream_t s);

// Row Walsh-Hadamard transform of rows of length d (fp32 out), optionally
// fused with MXFP4 quantization of the rotated row.
struct FwhtLaunch {
  const void* x;             // input, or the gate of SiLU_and_Mul when `up` is set
  const void* up;            // SiLU_and_Mul: the up input (same shape and stride as x) or null
  int64_t rows, d, stride;
  int in_dtype;
  int t;                     // transform size (power of two, divides d)
  int random_signs;
  uint64_t seed;
  float* y;                  // fp32 output (may be null when quantizing)
  // fused MXFP4 quantization (quantize != 0)
  int quantize;
  int stochastic;
  int manual;
  int manual_e;
  uint8_t* codes;
  uint8_t* scales;
  unsigned long long* counters;
  unsigned long long* count_slots;   // counter slots in the workspace, or null
};
hipError_t launch_fwht(const FwhtLaunch& f, hipStream_t s);

struct DequantLaunch {
  int format;                // 0 MX, 1 NV, 2 IF4
  int64_t rows, cols;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* global_scale;
  int out_dtype;             // kF32 / kBF16
  void* out;
};
hipError_t launch_dequant(const DequantLaunch& d, hipStream_t s);

// MXFP4 x MXFP4 GEMM: C[M][N] = A[M][K] B[N][K]^T (K a multiple of 128).
struct GemmLaunch {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  int64_t M, N, K;
  void* c;
  int out_bf16;
};
hipError_t launch_mx_gemm(const GemmLaunch& g, hipStream_t s);

int device_cu_count();

}  // namespace fp4q
