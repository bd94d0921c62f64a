// fp4q_nv_resident.hip -- single-launch NVFP4 quantization that reads most of
// the tensor from HBM once (gfx950: four 256-thread workgroups per CU).
//
// Same computation as fp4q_nv.hip ("Sub-4-Bit Microscaling", section 2:
// g = amax / (6 * 448), s = RNE_E4M3(bamax / (6 g)), code = RNE_E2M1(x /
// (s g))), restricted to round-to-nearest without rotation on contiguous bf16:
//
//  phase 1  each workgroup owns a contiguous chunk of up to 32 sixteen-byte
//           slots per thread, each wave a contiguous run of them.  The first
//           reg_slots() stay in VGPRs, the next kLdsSlots go to LDS (both
//           non-temporal loads into VGPRs; the LDS-bound ones are issued first
//           and written to LDS once their maxima are taken), the rest are
//           loaded only for their maxima (cached loads, so that phase 2 finds
//           them closer).  Each lane folds the block maxima phase 2 will need
//           as its loads land (block_maxima);
//  barrier  every workgroup publishes (epoch, chunk max) in a 64-bit flag of
//           its own; the last workgroup polls all flags in parallel, folds the
//           maxima and writes (epoch, tensor max) into sixteen copies of a
//           result word, 4 KiB apart, each polled by a sixteenth of the
//           workgroups -- no contended counter and no single hot word,
//           relaxed atomics only (each word carries its own payload);
//  phase 2  codes and scales, two slot rows at a time (nv_fast_pair: a lane
//           pair works out one block scale per lane), from the on-chip slots,
//           then from the re-read slots (prefetched ahead), in straight-line
//           code; slots that need the exact path are recomputed at the end.
//
// The launch is an ordinary one with at most kResPerCu workgroups per CU.
// Results never depend on the workgroups being resident together: every wait
// is bounded in time (1 ms), and a workgroup whose wait runs out takes the
// tensor maximum from the flags already published, scanning itself only the
// chunks whose flags are missing and publishing their maxima for the others
// (same value, only slower: at worst one extra read of the tensor per
// workgroup that times out).
//
// Every launch carries a fresh epoch, so that flags and result words left by
// an earlier launch never pass for its own.  An ordinary launch takes it from
// a host counter (1 .. 2^31 - 1) as a kernel argument.  A launch captured in
// a HIP graph cannot (its arguments are frozen at capture), so it is preceded
// by a one-thread kernel that advances an epoch word kept in the workspace
// (2^31 .. 2^32 - 1, disjoint from the host's), and the kernel reads that word
// as it starts: every replay gets a fresh epoch too.  (One atomic ticket per
// workgroup on a shared word was measured instead: the 1024 atomics on one
// address serialise, about 20 us per launch.)  The workspace must be
// zero-filled before its first use.
//
// The 8192 x 8192 bf16 activation is 1024 x 256 x 32 slots on 256 CUs: 26 of
// every 32 slots stay on chip.
#include <atomic>
#include <utility>

#include "fp4q_flat.h"
#include "fp4q_nv_common.h"

namespace fp4q {
namespace {

constexpr int kResThreads = 256;
constexpr int kResPerCu = 4;               // workgroups resident per CU
// slots held in VGPRs within 128 registers (the bounds-tested variant needs a
// few more registers of its own; one more slot fits the full variant but
// measured no faster)
template <bool GUARD>
constexpr int reg_slots() { return GUARD ? 15 : 17; }
constexpr int kLdsSlots = 9;
constexpr int kMaxSlots = 32;
template <bool GUARD>
constexpr int reread_slots() { return kMaxSlots - reg_slots<GUARD>() - kLdsSlots; }
constexpr int kAhead = 2;   // re-read prefetch depth (2 measured faster than 1, 3, 4 or 6)
constexpr uint64_t kWaitTicks = 100000;    // 1 ms of the 100 MHz real-time counter (default)
constexpr int kSpinLimit = 1 << 24;        // backstop on the number of polls


// Largest finite bf16 magnitude bit pattern of a raw slot whose raw 16-bit
// maximum (slot_max16) is mx.
__device__ __forceinline__ uint32_t finite_max16(const uint4& w, uint32_t mx) {
  if (mx >= 0x7F80u) {   // a non-finite value is present: take the finite max only
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    mx = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = ws[i] & 0x7FFFu, hi = (ws[i] >> 16) & 0x7FFFu;
      if (lo < 0x7F80u) mx = max(mx, lo);
      if (hi < 0x7F80u) mx = max(mx, hi);
    }
  }
  return mx;
}

__device__ __forceinline__ uint32_t raw_finite_absmax(const uint4& w) {
  return finite_max16(w, slot_max16(w)) << 16;   // fp32 bit pattern of the max
}

// Slot j of a lane is workgroup slot wbase + 64 j + lane, with wbase = 64 nres
// times the wave's index: every wave streams one contiguous run of 64 nres
// sixteen-byte slots (1 KiB per slot row), which HBM serves far better than
// rows strided across the workgroup.
__device__ __forceinline__ uint32_t slot_of(int wbase, int j, int lane) { return (uint32_t)(wbase + j * 64 + lane); }

__device__ __forceinline__ const uint16_t* slot_ptr(const uint16_t* wg_x, uint32_t ls) { return wg_x + (size_t)ls * 8u; }

// Non-temporal loads of slots FIRST .. FIRST + N - 1 into r (zeros past the end).
template <bool GUARD, int FIRST, int N, int... J>
__device__ __forceinline__ void load_slots(uint4 (&r)[N], const uint16_t* wg_x, int wbase, int lane,
                                           int nres, uint32_t n_valid, std::integer_sequence<int, J...>) {
  auto one = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const uint32_t ls = slot_of(wbase, FIRST + j, lane);
    if (!GUARD || (FIRST + j < nres && ls < n_valid)) {
      const u32x4_t a = load16<true>(slot_ptr(wg_x, ls));
      r[j] = make_uint4(a.x, a.y, a.z, a.w);
    } else {
      r[j] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  (one(std::integral_constant<int, J>{}), ...);
}


__device__ __forceinline__ uint4 load_cached(const uint16_t* wg_x, uint32_t ls, bool valid) {
  if (valid) {
    const u32x4_t a = load16<false>(slot_ptr(wg_x, ls));
    return make_uint4(a.x, a.y, a.z, a.w);
  }
  return make_uint4(0u, 0u, 0u, 0u);
}

// Phase-2 state of one thread.  GUARD is false when every workgroup holds
// exactly kMaxSlots full slot rows: then no slot needs a bounds test and the
// encoding is straight-line code.  Slot rows are taken two at a time (rows j
// and j + 1, j even): the lane pair 2k, 2k+1 holds block k of row j and block
// k of row j + 1, the even lane works out the first block's scale, the odd
// lane the second's (nv_fast_pair).  need: a shift register, one bit per
// pair of rows shifted in at the bottom, set when the block this lane worked
// out for those rows must be recomputed exactly (about one element in 2000 on
// Student-t data: bf16 inputs put many quotients within 2^-22 of a rounding
// boundary); exact_slots() turns it into per-slot bits.
template <bool GUARD>
struct Phase2 {
  const NvCtx& cx;
  const float2* s_adj;
  uint32_t* codes_lane;   // code word of this lane's slot in row 0 (row j: + 64 j)
  uint8_t* scale_lane;    // scale byte of the block this lane works out for rows 0, 1 (rows j, j+1: + 32 j)
  int wbase, lane, nres;
  uint32_t n_valid;
  bool odd;
  uint32_t need;

  // bamax: the largest magnitude of the block this lane works out (0 for a
  // block past the end, which then needs no redo; its codes are not stored)
  __device__ __forceinline__ void pair(int j, const uint4& w0, const uint4& w1, float bamax) {
    bool v0 = true, v1 = true;
    if constexpr (GUARD) {
      // both lanes of a block agree (valid slot counts are even)
      v0 = j < nres && slot_of(wbase, j, lane) < n_valid;
      v1 = j + 1 < nres && slot_of(wbase, j + 1, lane) < n_valid;
    }
    uint32_t c0, c1, sc, nd;
    nv_fast_pair(cx, s_adj, w0, w1, bamax, c0, c1, sc, nd);
    // codes and scale bytes non-temporal: they stream out during the encode
    // instead of piling up as dirty L2 lines that drain after it (measured:
    // cached code stores make the launch ~2 us longer, cached scale bytes
    // ~0.3 us)
    if (!GUARD || v0) __builtin_nontemporal_store(c0, codes_lane + 64 * j);
    if (!GUARD || v1) __builtin_nontemporal_store(c1, codes_lane + 64 * (j + 1));
    if (!GUARD || (odd ? v1 : v0)) __builtin_nontemporal_store((uint8_t)sc, scale_lane + 32 * j);
    need = __builtin_amdgcn_alignbit(need, nd, 31);   // (need << 1) | bit 31 of nd
  }

  // Per-slot redo bits after all kMaxSlots / 2 pairs: slot j of a lane belongs
  // to the block its pair worked out in the even lane (j even) or in the odd
  // lane (j odd).
  __device__ __forceinline__ uint32_t exact_slots() const {
    static_assert(kMaxSlots == 32, "16 pairs: one 16-bit shift register");
    // pair p sits at bit 15 - p: reverse, then spread bit p to bit 2p
    uint32_t m = __builtin_bitreverse32(need) >> 16;
    m = (m | (m << 8)) & 0x00FF00FFu;
    m = (m | (m << 4)) & 0x0F0F0F0Fu;
    m = (m | (m << 2)) & 0x33333333u;
    m = (m | (m << 1)) & 0x55555555u;
    const uint32_t other = dpp_u32<kQuadXor1>(m);
    return odd ? (other | (m << 1)) : (m | (other << 1));
  }
};

// Phase-2 slot sources: slot j of a lane comes from its registers (j <
// reg_slots), from LDS (the next kLdsSlots), or from the re-read ring (the
// rest, prefetched kAhead slots ahead; compile-time indices throughout).
template <bool GUARD>
struct SlotSource {
  static constexpr int kRs = reg_slots<GUARD>();
  static constexpr int kRe = reread_slots<GUARD>();
  const uint4 (&r)[kRs];
  const uint4* s_data;
  uint4 (&pre)[kAhead];
  const uint16_t* wg_x;
  int wbase, lane, tid, nres;
  uint32_t n_valid;

  template <int J>
  __device__ __forceinline__ uint4 get() {
    if constexpr (J < kRs) {
      return r[J];
    } else if constexpr (J < kRs + kLdsSlots) {
      return s_data[(J - kRs) * kResThreads + tid];
    } else {
      constexpr int k = J - kRs - kLdsSlots;
      const uint4 w = pre[k % kAhead];
      if constexpr (k + kAhead < kRe) {
        const int jn = J + kAhead;
        const uint32_t ls = slot_of(wbase, jn, lane);
        if constexpr (GUARD) {
          pre[k % kAhead] = load_cached(wg_x, ls, jn < nres && ls < n_valid);
        } else {
          const u32x4_t a = load16<false>(slot_ptr(wg_x, ls));
          pre[k % kAhead] = make_uint4(a.x, a.y, a.z, a.w);
        }
      }
      return w;
    }
  }
};

template <bool GUARD, int... P>
__device__ __forceinline__ void encode_pairs(Phase2<GUARD>& p2, SlotSource<GUARD>& src, const uint32_t (&bmp)[kMaxSlots / 4],
                                             std::integer_sequence<int, P...>) {
  auto one = [&](auto pc) {
    constexpr int p = decltype(pc)::value;
    const uint4 w0 = src.template get<2 * p>();
    const uint4 w1 = src.template get<2 * p + 1>();
    const uint32_t h = bmp[p >> 1];
    p2.pair(2 * p, w0, w1, as_f((p & 1) ? (h & 0xFFFF0000u) : (h << 16)));
  };
  (one(std::integral_constant<int, P>{}), ...);
}

// Phase-1 view of a lane's slot j: its registers, the registers that stage
// its LDS entries, or its re-read slots; a slot past the end reads as zeros.
template <int RS, int SC>
struct Phase1Slots {
  const uint4 (&r)[RS];
  const uint4 (&st)[kLdsSlots];
  const uint4 (&sc)[SC];

  template <int J>
  __device__ __forceinline__ uint4 get() const {
    if constexpr (J < RS) {
      return r[J];
    } else if constexpr (J < RS + kLdsSlots) {
      return st[J - RS];
    } else {
      return sc[J - RS - kLdsSlots];
    }
  }
};

// The block maxima phase 2 needs: for every pair of rows, the largest
// magnitude (raw 16-bit pattern, non-finite included) of the block this lane
// works out, packed two pairs per word (pair p in the upper half of bmp[p / 2]
// when p is odd; bmp starts at zero).  acc collects the largest magnitude over
// the lane's slots, non-finite included (the caller takes the finite maximum
// apart when that is non-finite).  STAGED visits the pairs held wholly in the
// LDS-bound registers; otherwise the rest, in the order their loads land:
// register pairs, pairs that straddle registers and LDS, re-read pairs.
// Straight-line code; the compiler waits for each load at its first use.
template <int RS, bool STAGED, class S, int... P>
__device__ __forceinline__ void block_maxima(const S& slots, bool odd, uint32_t (&bmp)[kMaxSlots / 4], uint32_t& acc,
                                             std::integer_sequence<int, P...>) {
  auto one = [&](auto pc) {
    constexpr int p = decltype(pc)::value;
    const uint32_t m0 = slot_max16(slots.template get<2 * p>());
    const uint32_t m1 = slot_max16(slots.template get<2 * p + 1>());
    acc = max(acc, max(m0, m1));
    const uint32_t own = odd ? m1 : m0, give = odd ? m0 : m1;
    const uint32_t bm = max(own, dpp_u32<kQuadXor1>(give));
    bmp[p >> 1] |= (p & 1) ? bm << 16 : bm;   // (pairs are visited out of order)
    // (one pair at a time: interleaving them only lengthens live ranges)
    __builtin_amdgcn_sched_barrier(0);
  };
  constexpr int kFirstReread = RS + kLdsSlots;
  auto cls = [](int p) { return 2 * p + 1 < RS ? 1 : 2 * p >= kFirstReread ? 3 : 2 * p >= RS ? 0 : 2; };
  auto visit = [&](auto pc, auto kc) { if constexpr (cls(decltype(pc)::value) == decltype(kc)::value) one(pc); };
  if constexpr (STAGED) {
    (visit(std::integral_constant<int, P>{}, std::integral_constant<int, 0>{}), ...);
  } else {
    (visit(std::integral_constant<int, P>{}, std::integral_constant<int, 1>{}), ...);
    (visit(std::integral_constant<int, P>{}, std::integral_constant<int, 2>{}), ...);
    (visit(std::integral_constant<int, P>{}, std::integral_constant<int, 3>{}), ...);
    // (the packed words are formed here: left to itself the compiler carries
    // the 32 halves into phase 2 and spills them)
#pragma unroll
    for (int k = 0; k < kMaxSlots / 4; ++k) asm volatile("" : "+v"(bmp[k]));
  }
}

// Largest finite magnitude (16-bit pattern) over a lane's slots, read again
// from the input: the rare case of a lane holding a non-finite value.
__device__ __forceinline__ uint32_t lane_finite_max16(const uint16_t* wg_x, int wbase, int lane, int nres,
                                                   uint32_t n_valid) {
  uint32_t acc = 0u;
  for (int j = 0; j < nres; ++j) {
    const uint32_t ls = slot_of(wbase, j, lane);
    if (ls < n_valid) {
      const u32x4_t a = load16<false>(slot_ptr(wg_x, ls));
      const uint4 w = make_uint4(a.x, a.y, a.z, a.w);
      acc = max(acc, finite_max16(w, slot_max16(w)));
    }
  }
  return acc;
}

// Tensor maximum (finite bf16 magnitudes, as an fp32 bit pattern) after a
// wait ran out: the chunk maxima already published in the flags, and a scan
// by this workgroup of every chunk whose flag is missing (its maximum is then
// published in that chunk's flag, the value its owner publishes too, so that
// other workgroups that time out need not scan it again).  Every thread of the
// workgroup calls this.
__device__ uint32_t fallback_tensor_amax(const QuantLaunch& q, uint64_t* flags, uint32_t epoch, int nres,
                                         uint32_t* s_red, uint32_t* s_missing) {
  const uint16_t* x = static_cast<const uint16_t*>(q.x);
  const int tid = threadIdx.x, G = gridDim.x;
  const int64_t chunk = (int64_t)kResThreads * nres;   // slots per workgroup
  __syncthreads();
  for (int w = tid; w < kAmaxPartialsMax / 32; w += kResThreads) s_missing[w] = 0u;
  __syncthreads();
  uint32_t m = 0u;
  for (int i = tid; i < G; i += kResThreads) {
    const uint64_t f = __hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(f >> 32) == epoch) m = max(m, (uint32_t)f);
    else atomicOr(s_missing + (i >> 5), 1u << (i & 31));
  }
  __syncthreads();
  for (int w = 0; w < (G + 31) / 32; ++w) {
    uint32_t bitsw = s_missing[w];   // (the same value in every thread)
    while (bitsw != 0u) {
      const int i = 32 * w + __builtin_ctz(bitsw);
      bitsw &= bitsw - 1u;
      const int64_t s0 = (int64_t)i * chunk;
      const int64_t s1 = s0 + chunk < q.nslots ? s0 + chunk : q.nslots;
      uint32_t c = 0u;
      for (int64_t sl = s0 + tid; sl < s1; sl += kResThreads) {
        const u32x4_t a = load16<false>(x + (sl << 3));
        c = max(c, raw_finite_absmax(make_uint4(a.x, a.y, a.z, a.w)));
      }
      c = wave_max_u32(c);
      if ((tid & 63) == 0) s_red[tid >> 6] = c;
      __syncthreads();
      c = 0u;
#pragma unroll
      for (int v = 0; v < kResThreads / 64; ++v) c = max(c, s_red[v]);
      if (tid == 0)
        __hip_atomic_store(flags + i, ((uint64_t)epoch << 32) | c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      m = max(m, c);
      __syncthreads();
    }
  }
  m = wave_max_u32(m);
  if ((tid & 63) == 0) s_red[tid >> 6] = m;
  __syncthreads();
  m = 0u;
#pragma unroll
  for (int v = 0; v < kResThreads / 64; ++v) m = max(m, s_red[v]);
  __syncthreads();
  return m;
}

// Poll *p until its high word equals epoch; false if the wait runs out.  The
// limit is 1 ms of the 100 MHz counter unless *limit_word is nonzero (tests
// set it to a few ticks to drive the fallback scan); it is read only once a
// wait has begun, so its latency hides inside the wait.  The pause between
// polls doubles up to MAXPAUSE sleeps of 64 cycles: every poll reaches the
// device-wide coherence point, and workgroups polling flat out would slow
// down the ones still streaming their input.
template <int MAXPAUSE>
__device__ __forceinline__ bool wait_epoch(const uint64_t* p, uint32_t epoch, const uint64_t* limit_word, uint64_t& f) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  f = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((uint32_t)(f >> 32) == epoch) return true;
  const uint64_t set = __hip_atomic_load(limit_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t limit = set ? set : kWaitTicks;
  int pause = 1;
  for (int it = 0; it < kSpinLimit; ++it) {
    for (int k = 0; k < pause; ++k) __builtin_amdgcn_s_sleep(1);
    pause = pause < MAXPAUSE ? 2 * pause : MAXPAUSE;
    f = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(f >> 32) == epoch) return true;
    if (__builtin_amdgcn_s_memrealtime() - t0 > limit) return false;
  }
  return false;
}

// epoch: this launch's epoch, or 0 to read it from the workspace's epoch word
// (a launch captured in a graph, after epoch_advance_kernel).
template <bool GUARD>
__global__ __launch_bounds__(kResThreads, kResPerCu) void nv_resident_kernel(QuantLaunch q, int nres, unsigned char* ws,
                                                                     uint32_t epoch_arg) {
  __shared__ uint4 s_data[kLdsSlots * kResThreads];   // 36,864 bytes (four workgroups per CU)
  __shared__ float2 s_adj[256];   // adjusted multiplier and flag per conversion byte
  __shared__ float2 s_br[128];    // brackets of 1 / (s g) per scale code
  __shared__ float4 s_eps[8];     // multiplier adjustment per significand class
  __shared__ uint32_t s_red[kResThreads / 64];
  __shared__ uint32_t s_timeout;
  __shared__ uint32_t s_amax;
  __shared__ uint32_t s_epoch;
  __shared__ uint32_t s_missing[kAmaxPartialsMax / 32];   // fallback: chunks without a flag
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept scalar
  const int G = gridDim.x;
  uint64_t* hdr = reinterpret_cast<uint64_t*>(ws);   // [2] wait limit override, [3] graph epoch word
  uint64_t* flags = reinterpret_cast<uint64_t*>(ws + kWsFlagsOffsetBytes);   // one per workgroup
  constexpr int kResultWords = (int)(kWsResultStrideBytes / 8);
  uint64_t* results = reinterpret_cast<uint64_t*>(ws + kWsResultsOffsetBytes);   // kWsResultCopies copies
  const int64_t chunk = (int64_t)kResThreads * nres;
  const int64_t base = (int64_t)blockIdx.x * chunk;
  const int64_t rem = q.nslots - base;
  const uint32_t n_valid = (uint32_t)(rem < chunk ? (rem > 0 ? rem : 0) : chunk);
  const uint16_t* wg_x = static_cast<const uint16_t*>(q.x) + (base << 3);
  const int wbase = wv * 64 * nres;                                   // this wave's first slot
  if (tid == 0) s_timeout = 0u;
  // (a captured launch reads its epoch as it starts; it is used after phase 1)
  uint32_t epoch_word = epoch_arg;
  if (epoch_arg == 0u && tid == 0)
    epoch_word = (uint32_t)__hip_atomic_load(hdr + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---------------- phase 1
  constexpr int kRegSlots = reg_slots<GUARD>();
  constexpr int kScan = reread_slots<GUARD>();
  uint4 r[kRegSlots];
  uint32_t acc = 0u;
  uint32_t bmp[kMaxSlots / 4];
#pragma unroll
  for (int k = 0; k < kMaxSlots / 4; ++k) bmp[k] = 0u;
  {
    // The LDS-bound slots first, through VGPRs (a direct global->LDS load in
    // flight would make the first use of any loaded register wait for every
    // load issued), then the register slots, all back to back.
    uint4 st[kLdsSlots];
    load_slots<GUARD, kRegSlots>(st, wg_x, wbase, lane, nres, n_valid, std::make_integer_sequence<int, kLdsSlots>{});
    load_slots<GUARD, 0>(r, wg_x, wbase, lane, nres, n_valid, std::make_integer_sequence<int, kRegSlots>{});
    __builtin_amdgcn_sched_barrier(0);
    uint4 sc[kScan];
    const Phase1Slots<kRegSlots, kScan> slots{r, st, sc};
    const bool odd = (lane & 1) != 0;
    block_maxima<kRegSlots, true>(slots, odd, bmp, acc, std::make_integer_sequence<int, kMaxSlots / 2>{});
    // each lane's LDS entries are its own: phase 2 reads them back in program
    // order, with no barrier
#pragma unroll
    for (int j = 0; j < kLdsSlots; ++j) s_data[j * kResThreads + tid] = st[j];
    __builtin_amdgcn_sched_barrier(0);
    // the re-read slots, into the registers the staged slots leave free
#pragma unroll
    for (int k = 0; k < kScan; ++k) {
      const int j = kRegSlots + kLdsSlots + k;
      const uint32_t ls = slot_of(wbase, j, lane);
      if constexpr (GUARD) {
        sc[k] = load_cached(wg_x, ls, j < nres && ls < n_valid);
      } else {
        // (unconditional: a load under a branch makes the compiler wait for
        // every load before it)
        const u32x4_t a = load16<false>(slot_ptr(wg_x, ls));
        sc[k] = make_uint4(a.x, a.y, a.z, a.w);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    block_maxima<kRegSlots, false>(slots, odd, bmp, acc, std::make_integer_sequence<int, kMaxSlots / 2>{});
  }
  if (acc >= 0x7F80u) acc = lane_finite_max16(wg_x, wbase, lane, nres, n_valid);
  acc <<= 16;   // fp32 bit pattern
  acc = wave_max_u32(acc);
  if (lane == 0) s_red[wv] = acc;
  if (tid == 0) s_epoch = epoch_word;
  __syncthreads();
  const uint32_t epoch = s_epoch;

  // ---------------- grid-wide exchange of the chunk maxima
  if (tid == 0) {
    uint32_t m = s_red[0];
#pragma unroll
    for (int w = 1; w < kResThreads / 64; ++w) m = max(m, s_red[w]);
    __hip_atomic_store(flags + blockIdx.x, ((uint64_t)epoch << 32) | m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the master is the last workgroup: it streams the highest addresses and
  // tends to finish phase 1 last, so it rarely waits long
  uint32_t amax_bits = 0u;
  if (blockIdx.x == (unsigned)G - 1u) {
    uint32_t m = 0u;
    for (int i = tid; i < G; i += kResThreads) {
      uint64_t f = 0;
      // (the master polls briskly: its wait is the critical path)
      if (!wait_epoch<1>(flags + i, epoch, hdr + 2, f)) s_timeout = 1u;
      m = max(m, (uint32_t)f);
    }
    m = wave_max_u32(m);
    __syncthreads();
    if (lane == 0) s_red[wv] = m;
    __syncthreads();
    m = 0u;
#pragma unroll
    for (int w = 0; w < kResThreads / 64; ++w) m = max(m, s_red[w]);
    if (s_timeout) m = fallback_tensor_amax(q, flags, epoch, nres, s_red, s_missing);
    const uint64_t word = ((uint64_t)epoch << 32) | m;
    if (tid < kWsResultCopies)
      __hip_atomic_store(results + (size_t)tid * kResultWords, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    amax_bits = m;
  } else {
    __syncthreads();   // s_red is reused below
    if (tid == 0) {
      uint64_t f = 0;
      const uint64_t* mine = results + (size_t)(blockIdx.x % kWsResultCopies) * kResultWords;
      if (wait_epoch<4>(mine, epoch, hdr + 2, f)) s_red[0] = (uint32_t)f;
      else s_timeout = 1u;
    }
    __syncthreads();
    amax_bits = s_timeout ? fallback_tensor_amax(q, flags, epoch, nres, s_red, s_missing) : s_red[0];
  }

  NvCtx cx;
  nv_context_rne6(as_f(amax_bits), cx);
  nv_fill_adjusted_table<256>(s_adj, s_br, s_eps, cx, tid);
  if (tid == 0) {
    s_amax = amax_bits;
    if (blockIdx.x == (unsigned)G - 1u && q.global_scale) *q.global_scale = cx.g;
  }
  __syncthreads();

  // ---------------- phase 2
  // (slot indices are recomputed from an opaque copy of the lane id: keeping
  // them alive from phase 1 would cost registers)
  int lane2 = lane;
  asm volatile("" : "+v"(lane2));
  uint4 pre[kAhead];
#pragma unroll
  for (int k = 0; k < kAhead; ++k) {
    const int j = kRegSlots + kLdsSlots + k;
    const uint32_t ls = slot_of(wbase, j, lane2);
    if constexpr (GUARD) {
      pre[k] = load_cached(wg_x, ls, j < nres && ls < n_valid);
    } else {
      const u32x4_t a = load16<false>(slot_ptr(wg_x, ls));
      pre[k] = make_uint4(a.x, a.y, a.z, a.w);
    }
  }
  const bool odd = (lane2 & 1) != 0;
  Phase2<GUARD> p2{cx, s_adj,
                   reinterpret_cast<uint32_t*>(q.codes + (base << 2)) + wbase + lane2,
                   q.scales + (base >> 1) + (wbase >> 1) + (lane2 >> 1) + (odd ? 32 : 0),
                   wbase, lane2, nres, n_valid, odd, 0u};
  SlotSource<GUARD> src{r, s_data, pre, wg_x, wbase, lane2, wv * 64 + lane2, nres, n_valid};
  static_assert(kMaxSlots % 2 == 0, "slot rows are encoded in pairs");
  encode_pairs(p2, src, bmp, std::make_integer_sequence<int, kMaxSlots / 2>{});
  // Exact recomputations, after this thread's fast stores (program order per
  // address keeps the exact values last).  The context is rebuilt from LDS so
  // that phase 2 keeps only the two bracket factors in registers.  With
  // g < 2^-100 every slot is redone on inputs and g scaled by 2^100 (exact
  // power-of-two scaling: the quotients are unchanged and nothing underflows).
  asm volatile("" ::: "memory");
  uint32_t redo = p2.exact_slots();
  NvCtx cf;
  nv_context_rne6(as_f(s_amax), cf);
  float xscale = 1.0f;
  if (cf.exact_all) {
    xscale = 0x1p100f;
    nv_context_g(cf.g * xscale, cf);
    __syncthreads();
    nv_fill_adjusted_table<256>(s_adj, s_br, s_eps, cf, tid);
    __syncthreads();
    redo = 0u;
    for (int j = 0; j < nres; ++j) redo |= (slot_of(wbase, j, lane2) < n_valid ? 1u : 0u) << j;
  }
  // two slots per round, both blocks in flight together
  const uint16_t* xs = static_cast<const uint16_t*>(q.x);
  while (redo != 0u) {
    const int j0 = __builtin_ctz(redo);
    redo &= redo - 1u;
    const bool two = redo != 0u;
    const int j1 = two ? __builtin_ctz(redo) : j0;
    if (two) redo &= redo - 1u;
    const int64_t s0 = base + (int64_t)slot_of(wbase, j0, lane2);
    const int64_t s1 = base + (int64_t)slot_of(wbase, j1, lane2);
    const u32x4_t a0 = load16<false>(xs + ((s0 & ~(int64_t)1) << 3)), b0 = load16<false>(xs + ((s0 | 1) << 3));
    const u32x4_t a1 = load16<false>(xs + ((s1 & ~(int64_t)1) << 3)), b1 = load16<false>(xs + ((s1 | 1) << 3));
    nv_fix_slot_fma(q, cf, s_br, xscale, s0, a0, b0);
    if (two) nv_fix_slot_fma(q, cf, s_br, xscale, s1, a1, b1);
  }
}

// Host epochs 1 .. 2^31 - 1 (0 never: it is the value of a zeroed workspace,
// and it tells the kernel to read the workspace's word).
uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{0u};
  for (;;) {
    const uint32_t e = (counter.fetch_add(1u, std::memory_order_relaxed) + 1u) & 0x7FFFFFFFu;
    if (e != 0u) return e;
  }
}

// Advances the workspace's epoch word within 2^31 .. 2^32 - 1 (graph launches).
__global__ void epoch_advance_kernel(unsigned char* ws) {
  uint64_t* w = reinterpret_cast<uint64_t*>(ws) + 3;
  const uint32_t e = (uint32_t)*w;
  *w = (uint64_t)((((e + 1u) & 0x7FFFFFFFu) | 0x80000000u));
}

hipError_t launch_resident(const QuantLaunch& q, int grid, int nres, hipStream_t st) {
  unsigned char* ws = reinterpret_cast<unsigned char*>(q.partials);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t ce = hipStreamIsCapturing(st, &cs);
  if (ce != hipSuccess) return ce;
  uint32_t epoch = 0u;
  if (cs == hipStreamCaptureStatusNone) {
    epoch = next_epoch();
  } else {
    hipLaunchKernelGGL(epoch_advance_kernel, dim3(1), dim3(1), 0, st, ws);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // every workgroup full: kMaxSlots slot rows each and nothing left over
  const bool full = nres == kMaxSlots && q.nslots == (int64_t)grid * kResThreads * kMaxSlots;
  if (full) {
    hipLaunchKernelGGL((nv_resident_kernel<false>), dim3(grid), dim3(kResThreads), 0, st, q, nres, ws, epoch);
  } else {
    hipLaunchKernelGGL((nv_resident_kernel<true>), dim3(grid), dim3(kResThreads), 0, st, q, nres, ws, epoch);
  }
  return hipGetLastError();
}

// Workgroups of the single-launch kernel that fit on the device at once
// (kResPerCu per CU when its registers and LDS allow it), cached per device.
int64_t resident_workgroups() {
  static std::atomic<int64_t> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int64_t v = cached[dev].load(std::memory_order_relaxed);
  if (v != 0) return v;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&nv_resident_kernel<false>),
                                                   kResThreads, 0) != hipSuccess)
    per_cu = 0;
  if (per_cu > kResPerCu) per_cu = kResPerCu;
  v = per_cu > 0 ? (int64_t)per_cu * device_cu_count() : -1;
  cached[dev].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace

// Whether the single-launch kernel takes this call, and its launch shape.
bool nv_resident_shape(const QuantLaunch& q, int* grid, int* nres) {
  if (q.in_dtype != kBF16 || q.four_over_six || q.if4 || q.global_amax || q.stride != q.cols || q.nslots == 0) return false;
  if (q.rotation != kRotNone || q.stochastic || q.counters) return false;   // those variants stream twice
  const int64_t cap = resident_workgroups();
  if (cap <= 0) return false;
  int64_t g = (q.nslots + kResThreads - 1) / kResThreads;
  if (g > cap) g = cap;
  if (g > kAmaxPartialsMax) return false;
  const int64_t n = (q.nslots + g * kResThreads - 1) / (g * kResThreads);
  if (n > kMaxSlots) return false;
  *grid = (int)g;
  *nres = (int)n;
  return true;
}

hipError_t launch_nv_resident(const QuantLaunch& q, int grid, int nres, hipStream_t st) {
  return launch_resident(q, grid, nres, st);
}

}  // namespace fp4q
