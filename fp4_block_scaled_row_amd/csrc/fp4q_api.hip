// fp4q_api.hip -- the C ABI of libfp4q (see include/fp4q.h): host-side
// validation, workspace sizing and kernel dispatch.  Every check runs before
// anything is enqueued; an unsupported combination is refused, never
// substituted ("no silent fallback").
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "fp4q.h"
#include "fp4q_common.h"
#include "fp4q_internal.h"

namespace fp4q {

int device_cu_count() {
  // cached per device; several host threads may fill an entry at once, with
  // the same value
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace fp4q

using namespace fp4q;

// Scratch of fp4q_quantize_nvfp4_noalloc, for callers that cannot allocate:
// the NVFP4 workspace as a file-scope device array, one copy on every GPU the
// library runs on, held until the process ends.  It starts zeroed and needs
// no clearing between calls (each single-read launch carries a fresh epoch;
// the two-pass kernels write the partials they read).  In host code `scratch`
// names a host-side stand-in: kernels get its device address from
// hipGetSymbolAddress, kept per device (scratch_address).
__device__ __align__(256) unsigned char scratch[kNvWorkspaceBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_dev[64] = {};

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current.
fp4q_status scratch_address(void** p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FP4Q_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return FP4Q_ERR_HIP;
    g_scratch_dev[dev] = a;
  }
  *p = g_scratch_dev[dev];
  return FP4Q_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

fp4q_status hip_status(hipError_t e) { return e == hipSuccess ? FP4Q_OK : FP4Q_ERR_HIP; }

// Common checks of the quantize arguments.  Returns FP4Q_OK or the error.
fp4q_status check_quant(const fp4q_quant_args* a, const void* x, const fp4q_outputs* o, int format) {
  if (!a || !o) return FP4Q_ERR_INVALID_ARG;
  if (a->rows < 0 || a->cols < 0 || a->in_row_stride < a->cols) return FP4Q_ERR_INVALID_ARG;
  if (a->in_dtype != FP4Q_F32 && a->in_dtype != FP4Q_BF16) return FP4Q_ERR_INVALID_ARG;
  if (a->rounding != FP4Q_ROUND_RNE && a->rounding != FP4Q_ROUND_STOCHASTIC) return FP4Q_ERR_INVALID_ARG;
  if (a->rotation < FP4Q_ROT_NONE || a->rotation > FP4Q_ROT_FWHT128) return FP4Q_ERR_INVALID_ARG;
  if (a->scale_policy < FP4Q_SCALE_OCP_MAX || a->scale_policy > FP4Q_SCALE_IF4) return FP4Q_ERR_INVALID_ARG;
  const int want_block = format == FP4Q_MXFP4 ? 32 : 16;
  if (a->block_size != want_block) return FP4Q_ERR_UNSUPPORTED;
  if (format == FP4Q_MXFP4 && a->scale_policy != FP4Q_SCALE_OCP_MAX && a->scale_policy != FP4Q_SCALE_MANUAL)
    return FP4Q_ERR_UNSUPPORTED;
  if (format == FP4Q_NVFP4 && a->scale_policy != FP4Q_SCALE_NV_MAX6 && a->scale_policy != FP4Q_SCALE_FOUR_OVER_SIX &&
      a->scale_policy != FP4Q_SCALE_IF4)
    return FP4Q_ERR_UNSUPPORTED;
  if (a->scale_policy == FP4Q_SCALE_IF4 && a->rounding != FP4Q_ROUND_RNE) return FP4Q_ERR_UNSUPPORTED;
  if (a->scale_policy == FP4Q_SCALE_MANUAL && (a->manual_exponent < -127 || a->manual_exponent > 127))
    return FP4Q_ERR_INVALID_ARG;
  if (a->cols % want_block != 0) return FP4Q_ERR_INVALID_ARG;      // incomplete blocks
  const int64_t n = a->rows * a->cols;
  if (a->rows != 0 && n / a->rows != a->cols) return FP4Q_ERR_INVALID_ARG;  // overflow
  if (n > 0) {
    if (!x || !o->codes || !o->scales) return FP4Q_ERR_INVALID_ARG;
    const size_t esz = a->in_dtype == FP4Q_F32 ? 4 : 2;
    // 16-byte vector loads: base and row pitch must keep 8-element slots aligned
    if (!aligned(x, 16) || ((size_t)a->in_row_stride * esz) % 16 != 0) return FP4Q_ERR_UNSUPPORTED;
    if (!aligned(o->codes, 4)) return FP4Q_ERR_UNSUPPORTED;
    if (o->rotated && !aligned(o->rotated, 16)) return FP4Q_ERR_UNSUPPORTED;
  }
  if (o->counters && !aligned(o->counters, 8)) return FP4Q_ERR_INVALID_ARG;
  return FP4Q_OK;
}

QuantLaunch make_launch(const fp4q_quant_args* a, const void* x, const fp4q_outputs* o) {
  QuantLaunch q;
  memset(&q, 0, sizeof(q));
  q.x = x;
  q.rows = a->rows;
  q.cols = a->cols;
  q.stride = a->in_row_stride;
  q.nslots = a->rows * a->cols / 8;
  q.in_dtype = a->in_dtype == FP4Q_F32 ? kF32 : kBF16;
  q.rotation = a->rotation == FP4Q_ROT_RHT16 ? kRotRht16 : (a->rotation == FP4Q_ROT_FWHT128 ? kRotFwht128 : kRotNone);
  q.rot_scale = (float)(1.0 / sqrt(128.0));
  q.stochastic = a->rounding == FP4Q_ROUND_STOCHASTIC;
  q.manual = a->scale_policy == FP4Q_SCALE_MANUAL;
  q.manual_e = a->manual_exponent;
  q.four_over_six = a->scale_policy == FP4Q_SCALE_FOUR_OVER_SIX;
  q.if4 = a->scale_policy == FP4Q_SCALE_IF4;
  q.seed = a->seed;
  q.rht_signs = a->rotation == FP4Q_ROT_RHT16 ? (rht_sign_word(a->seed, 0u, 0) & 0xFFFFu) : 0u;
  q.codes = o->codes;
  q.scales = o->scales;
  q.global_scale = o->global_scale;
  q.choice_bits = o->choice_bits;
  q.rotated = o->rotated;
  q.counters = reinterpret_cast<unsigned long long*>(o->counters);
  return q;
}

}  // namespace

extern "C" {

size_t fp4q_workspace_bytes(const fp4q_quant_args* args) {
  if (!args) return 0;
  if (args->block_size == 16) return kNvWorkspaceBytes;
  if (args->block_size == 32) return kMxWorkspaceBytes;
  return 0;
}

fp4q_status fp4q_quantize_mxfp4(const fp4q_quant_args* args, const void* x, const fp4q_outputs* out,
                                void* workspace, size_t workspace_bytes, void* hip_stream) {
  fp4q_status st = check_quant(args, x, out, FP4Q_MXFP4);
  if (st != FP4Q_OK) return st;
  if (args->rotation == FP4Q_ROT_FWHT128) return FP4Q_ERR_UNSUPPORTED;
  // the workspace (optional) holds the counter slots of a counting call
  if (workspace && (workspace_bytes < kMxWorkspaceBytes || !aligned(workspace, 8))) return FP4Q_ERR_WORKSPACE;
  unsigned long long* slots = (workspace && out->counters) ? static_cast<unsigned long long*>(workspace) : nullptr;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const int64_t n = args->rows * args->cols;
  if (args->rotation == FP4Q_ROT_FWHT_ROW) {
    if (!is_pow2(args->cols) || args->cols < 32 || args->cols > 16384) return FP4Q_ERR_UNSUPPORTED;
    if (n == 0) return out->counters ? hip_status(launch_zero_counters(reinterpret_cast<unsigned long long*>(out->counters), s)) : FP4Q_OK;
    FwhtLaunch f;
    memset(&f, 0, sizeof(f));
    f.x = x;
    f.rows = args->rows;
    f.d = args->cols;
    f.stride = args->in_row_stride;
    f.in_dtype = args->in_dtype == FP4Q_F32 ? kF32 : kBF16;
    f.t = (int)args->cols;
    f.random_signs = 0;
    f.seed = args->seed;
    f.y = out->rotated;
    f.quantize = 1;
    f.stochastic = args->rounding == FP4Q_ROUND_STOCHASTIC;
    f.manual = args->scale_policy == FP4Q_SCALE_MANUAL;
    f.manual_e = args->manual_exponent;
    f.codes = out->codes;
    f.scales = out->scales;
    f.counters = reinterpret_cast<unsigned long long*>(out->counters);
    f.count_slots = slots;
    if (f.counters && !slots) {
      hipError_t e = launch_zero_counters(f.counters, s);
      if (e != hipSuccess) return FP4Q_ERR_HIP;
    }
    return hip_status(launch_fwht(f, s));
  }
  QuantLaunch q = make_launch(args, x, out);
  q.count_slots = slots;
  if (q.counters && (!slots || n == 0)) {
    hipError_t e = launch_zero_counters(q.counters, s);
    if (e != hipSuccess) return FP4Q_ERR_HIP;
  }
  return hip_status(launch_mx_quant(q, s));
}

fp4q_status fp4q_silu_mul_fwht_mxfp4(const fp4q_quant_args* args, const void* gate, const void* up,
                                     const fp4q_outputs* out, void* hip_stream) {
  fp4q_status st = check_quant(args, gate, out, FP4Q_MXFP4);
  if (st != FP4Q_OK) return st;
  if (args->rotation != FP4Q_ROT_FWHT_ROW) return FP4Q_ERR_UNSUPPORTED;
  if (!is_pow2(args->cols) || args->cols < 32 || args->cols > 16384) return FP4Q_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const int64_t n = args->rows * args->cols;
  if (n > 0) {
    if (!up) return FP4Q_ERR_INVALID_ARG;
    if (!aligned(up, 16)) return FP4Q_ERR_UNSUPPORTED;
  }
  if (out->counters) {
    hipError_t e = launch_zero_counters(reinterpret_cast<unsigned long long*>(out->counters), s);
    if (e != hipSuccess) return FP4Q_ERR_HIP;
  }
  if (n == 0) return FP4Q_OK;
  FwhtLaunch f;
  memset(&f, 0, sizeof(f));
  f.x = gate;
  f.up = up;
  f.rows = args->rows;
  f.d = args->cols;
  f.stride = args->in_row_stride;
  f.in_dtype = args->in_dtype == FP4Q_F32 ? kF32 : kBF16;
  f.t = (int)args->cols;
  f.seed = args->seed;
  f.y = out->rotated;
  f.quantize = 1;
  f.stochastic = args->rounding == FP4Q_ROUND_STOCHASTIC;
  f.manual = args->scale_policy == FP4Q_SCALE_MANUAL;
  f.manual_e = args->manual_exponent;
  f.codes = out->codes;
  f.scales = out->scales;
  f.counters = reinterpret_cast<unsigned long long*>(out->counters);
  return hip_status(launch_fwht(f, s));
}

fp4q_status fp4q_quantize_nvfp4(const fp4q_quant_args* args, const void* x, const float* global_amax,
                                const fp4q_outputs* out, void* workspace, size_t workspace_bytes,
                                void* hip_stream) {
  fp4q_status st = check_quant(args, x, out, FP4Q_NVFP4);
  if (st != FP4Q_OK) return st;
  if (args->rotation == FP4Q_ROT_FWHT_ROW) return FP4Q_ERR_UNSUPPORTED;
  if (args->rotation == FP4Q_ROT_FWHT128 &&
      (args->cols % 128 != 0 || args->rounding != FP4Q_ROUND_RNE || args->scale_policy == FP4Q_SCALE_FOUR_OVER_SIX))
    return FP4Q_ERR_UNSUPPORTED;
  if (!out->global_scale) return FP4Q_ERR_INVALID_ARG;
  const int64_t n = args->rows * args->cols;
  if (args->scale_policy == FP4Q_SCALE_FOUR_OVER_SIX && n > 0 && !out->choice_bits) return FP4Q_ERR_INVALID_ARG;
  if (!global_amax) {
    // (8-byte aligned: the single-read kernel keeps 64-bit atomic words in it)
    if (!workspace || workspace_bytes < fp4q_workspace_bytes(args) || !aligned(workspace, 8))
      return FP4Q_ERR_WORKSPACE;
  }
  QuantLaunch q = make_launch(args, x, out);
  q.global_amax = global_amax;
  q.partials = static_cast<uint32_t*>(workspace);
  return hip_status(launch_nv_quant(q, static_cast<hipStream_t>(hip_stream)));
}

fp4q_status fp4q_quantize_nvfp4_noalloc(const fp4q_quant_args* args, const void* x, const float* global_amax,
                                        const fp4q_outputs* out, void* hip_stream) {
  if (!args) return FP4Q_ERR_INVALID_ARG;
  // (the workspace an NVFP4 call needs does not grow with the tensor: the
  // kernels cap their grids, so the scratch covers every size)
  if (fp4q_workspace_bytes(args) > sizeof(scratch)) return FP4Q_ERR_WORKSPACE;
  void* ws = nullptr;
  const fp4q_status st = scratch_address(&ws);
  if (st != FP4Q_OK) return st;
  return fp4q_quantize_nvfp4(args, x, global_amax, out, ws, sizeof(scratch), hip_stream);
}

fp4q_status fp4q_fwht(int64_t rows, int64_t d, int64_t in_row_stride, int32_t in_dtype, const void* x, float* y,
                      int32_t transform_size, int32_t random_signs, uint64_t seed, void* hip_stream) {
  if (rows < 0 || d < 0 || in_row_stride < d) return FP4Q_ERR_INVALID_ARG;
  if (in_dtype != FP4Q_F32 && in_dtype != FP4Q_BF16) return FP4Q_ERR_INVALID_ARG;
  if (!is_pow2(transform_size) || transform_size < 2 || transform_size > 16384) return FP4Q_ERR_UNSUPPORTED;
  if (d % transform_size != 0 || d % 8 != 0) return FP4Q_ERR_UNSUPPORTED;
  if (rows * d == 0) return FP4Q_OK;
  if (!x || !y) return FP4Q_ERR_INVALID_ARG;
  const size_t esz = in_dtype == FP4Q_F32 ? 4 : 2;
  if (!aligned(x, 16) || ((size_t)in_row_stride * esz) % 16 != 0 || !aligned(y, 16)) return FP4Q_ERR_UNSUPPORTED;
  FwhtLaunch f;
  memset(&f, 0, sizeof(f));
  f.x = x;
  f.rows = rows;
  f.d = d;
  f.stride = in_row_stride;
  f.in_dtype = in_dtype == FP4Q_F32 ? kF32 : kBF16;
  f.t = transform_size;
  f.random_signs = random_signs != 0;
  f.seed = seed;
  f.y = y;
  return hip_status(launch_fwht(f, static_cast<hipStream_t>(hip_stream)));
}

fp4q_status fp4q_dequantize(int32_t format, int64_t rows, int64_t cols, int32_t block_size, const uint8_t* codes,
                            const uint8_t* scales, const float* global_scale, int32_t out_dtype, void* out,
                            void* hip_stream) {
  if (format != FP4Q_MXFP4 && format != FP4Q_NVFP4 && format != FP4Q_IF4) return FP4Q_ERR_INVALID_ARG;
  if (rows < 0 || cols < 0) return FP4Q_ERR_INVALID_ARG;
  if (out_dtype != FP4Q_F32 && out_dtype != FP4Q_BF16) return FP4Q_ERR_INVALID_ARG;
  if (block_size != (format == FP4Q_MXFP4 ? 32 : 16)) return FP4Q_ERR_UNSUPPORTED;
  if (cols % block_size != 0) return FP4Q_ERR_INVALID_ARG;
  if (rows * cols == 0) return FP4Q_OK;
  if (!codes || !scales || !out) return FP4Q_ERR_INVALID_ARG;
  if (format != FP4Q_MXFP4 && !global_scale) return FP4Q_ERR_INVALID_ARG;
  if (!aligned(codes, 4) || !aligned(out, 16)) return FP4Q_ERR_UNSUPPORTED;
  DequantLaunch dl;
  dl.format = format == FP4Q_MXFP4 ? 0 : (format == FP4Q_NVFP4 ? 1 : 2);
  dl.rows = rows;
  dl.cols = cols;
  dl.codes = codes;
  dl.scales = scales;
  dl.global_scale = global_scale;
  dl.out_dtype = out_dtype == FP4Q_F32 ? kF32 : kBF16;
  dl.out = out;
  return hip_status(launch_dequant(dl, static_cast<hipStream_t>(hip_stream)));
}

fp4q_status fp4q_mxfp4_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                            const uint8_t* b_codes, const uint8_t* b_scales, int32_t out_dtype, void* c,
                            void* hip_stream) {
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return FP4Q_ERR_INVALID_ARG;
  if (out_dtype != FP4Q_F32 && out_dtype != FP4Q_BF16) return FP4Q_ERR_INVALID_ARG;
  if (K % 128 != 0) return FP4Q_ERR_UNSUPPORTED;
  if (K > ((int64_t)1 << 23)) return FP4Q_ERR_UNSUPPORTED;   // 32-bit buffer offsets
  if (M == 0 || N == 0) return FP4Q_OK;
  if (!c || (K > 0 && (!a_codes || !a_scales || !b_codes || !b_scales))) return FP4Q_ERR_INVALID_ARG;
  if (M > (int64_t)1 << 31 || N > (int64_t)1 << 31) return FP4Q_ERR_UNSUPPORTED;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 4) || !aligned(b_scales, 4) ||
      !aligned(c, 4))
    return FP4Q_ERR_UNSUPPORTED;
  GemmLaunch g;
  g.a_codes = a_codes;
  g.a_scales = a_scales;
  g.b_codes = b_codes;
  g.b_scales = b_scales;
  g.M = M;
  g.N = N;
  g.K = K;
  g.c = c;
  g.out_bf16 = out_dtype == FP4Q_BF16;
  return hip_status(launch_mx_gemm(g, static_cast<hipStream_t>(hip_stream)));
}

fp4q_status fp4q_check_counters(const uint64_t* host_counters) {
  if (!host_counters) return FP4Q_ERR_INVALID_ARG;
  return host_counters[2] != 0 ? FP4Q_ERR_NONFINITE : FP4Q_OK;
}

const char* fp4q_status_string(fp4q_status s) {
  switch (s) {
    case FP4Q_OK: return "ok";
    case FP4Q_ERR_INVALID_ARG: return "invalid argument";
    case FP4Q_ERR_UNSUPPORTED: return "unsupported combination";
    case FP4Q_ERR_WORKSPACE: return "workspace missing or too small";
    case FP4Q_ERR_NONFINITE: return "non-finite input values";
    case FP4Q_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

const char* fp4q_version(void) { return "fp4q 0.1.0 (gfx950)"; }

}  // extern "C"
