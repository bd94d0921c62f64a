/*
 * fp4q.h -- C ABI of the MI355X (gfx950) block-scaled FP4 quantization
 * library libfp4q.so.
 *
 * What it computes (pages cited by title and section):
 *  - E2M1 elements: 1 sign, 2 exponent, 1 mantissa bit, bias 1, magnitudes
 *    {0, 0.5, 1, 1.5, 2, 3, 4, 6}, signed zero, no Inf/NaN ("MXFP4
 *    Quantization: Audit the 4.25-Bit Blocks", "Read the FP4 E2M1 value
 *    lattice"; "Sub-4-Bit Microscaling", section 1).  Code = sign << 3 |
 *    exponent << 1 | mantissa (the bit layout fixed by the metrale_circuit
 *    "hardware::exec" E2M1 -> E4M3 identity).
 *  - MXFP4: 32-element blocks along a row with one E8M0 scale byte
 *    2^(b-127); OCP max rule e = floor(log2(amax/4)) clamped to [-127, 127],
 *    all-zero block e = 0, or a manual exponent; elements divided by 2^e,
 *    rounded to nearest with ties to the even code, |v| > 6 clamps to 6
 *    (audit page, "Read the shared E8M0 scale", "Encode one MXFP4 block step
 *    by step").  4.25 bits per value.
 *  - NVFP4: 16-element blocks, unsigned E4M3 block scale and one fp32
 *    per-tensor scale g = amax / (6 * 448); s = RNE_E4M3(bamax / (6 g));
 *    elements rounded after dividing by s * g ("Sub-4-Bit Microscaling",
 *    section 2).  The division and the E4M3 rounding are decided on the exact
 *    real quotients.
 *  - Four Over Six: g = amax / (4 * 448), each 16-block keeps whichever of
 *    the max->6 and max->4 scalings has the lower block sum of squared error
 *    (ties keep max->6) and records a choice bit ("Adaptive Block-Scaled Data
 *    Types" transcript, cue 10).
 *  - IF4: g and the block scale s as for NVFP4 max->6; each 16-block is
 *    encoded twice, as FP4 and as scaled INT4 (integers -7..7 standing for
 *    k * 6 s g / 7, i.e. the integer grid stretched by 7/6 so 7 lands on
 *    FP4's 6), and keeps the one with the lower block sum of squared error
 *    (ties keep FP4); bit 7 of the block's E4M3 scale byte, unused by
 *    NVFP4, is set for INT4 ("Adaptive Block-Scaled Data Types" transcript,
 *    cues 14 and 17).  INT4 nibbles are sign-magnitude like E2M1 codes.
 *  - Stochastic rounding: round |q| up iff it exceeds lo + (u/65536)(hi-lo)
 *    for its neighbouring lattice points, u a 16-bit draw of Philox4x32-10
 *    keyed by (seed, flat element index r*cols + c): field (i mod 8) of
 *    Philox(key = seed, counter = (i/8, 0, 0)), field f = bits 16(f&1)..+15
 *    of word f>>1 (transcript cue 8: stochastic rounding keeps estimates
 *    unbiased).
 *  - Rotation: normalised Walsh-Hadamard transform y = x H / sqrt(t) of each
 *    t-chunk of a row, natural (Sylvester) order, fp32 arithmetic, scaled
 *    once by fl32(1/sqrt(t)) ("Sub-4-Bit Microscaling", section 3); the
 *    random Hadamard transform first flips signs with a seeded +-1 diagonal:
 *    position j is negated iff bit (j mod 32) of word (j/32 mod 4) of
 *    Philox(key = seed, counter = (j/128, 0, 1, 0)) is set (transcript cue 8).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, allocated and owned by the
 *    caller.  The library allocates no device memory (the scratch array of
 *    fp4q_quantize_nvfp4_noalloc is part of its code object).  Between calls
 *    it keeps only a per-process epoch counter of the single-read NVFP4
 *    kernel and per-device caches (CU count, that kernel's co-resident
 *    workgroups, the scratch address), all safe to use from several host
 *    threads.  Tensors are row-major; blocks run along a row.
 *  - Calls are asynchronous on `hip_stream` (a hipStream_t; NULL = the
 *    default stream) and never synchronise.
 *  - Argument, shape and combination checks run on the host before anything
 *    is enqueued; on any error nothing is enqueued.  An unsupported
 *    combination returns FP4Q_ERR_UNSUPPORTED: nothing is ever substituted.
 *  - Non-finite inputs are data, not errors: the block holding one gets the
 *    NaN scale code (0xFF for E8M0, 0x7F for E4M3), zero codes and choice
 *    bit 0, and counters[2] counts them.  Check after synchronising with
 *    fp4q_check_counters().
 *  - Launch failures return FP4Q_ERR_HIP.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP4Q_OK = 0,
  FP4Q_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad stride, bad enum value */
  FP4Q_ERR_UNSUPPORTED = 2,  /* a valid but unsupported combination (e.g. MXFP4 with 16-blocks) */
  FP4Q_ERR_WORKSPACE = 3,    /* workspace missing or smaller than fp4q_workspace_bytes() */
  FP4Q_ERR_NONFINITE = 4,    /* reported by fp4q_check_counters only */
  FP4Q_ERR_HIP = 5           /* a HIP launch or runtime call failed */
} fp4q_status;

enum { FP4Q_F32 = 0, FP4Q_BF16 = 1 };                       /* element types */
enum { FP4Q_MXFP4 = 0, FP4Q_NVFP4 = 1, FP4Q_IF4 = 2 };      /* formats (IF4: dequantize only) */
enum {
  FP4Q_SCALE_OCP_MAX = 0,        /* MX: e = floor(log2(amax/4)), clamp [-127,127], amax 0 -> 0 */
  FP4Q_SCALE_MANUAL = 1,         /* MX: e = manual_exponent for every block, in [-127, 127]   */
  FP4Q_SCALE_NV_MAX6 = 2,        /* NV: g = amax/2688, s = RNE_E4M3(bamax/(6g))               */
  FP4Q_SCALE_FOUR_OVER_SIX = 3,  /* NV: g = amax/1792, per block max->6 or max->4 by lower SSE */
  FP4Q_SCALE_IF4 = 4             /* NV: g, s as NV_MAX6; per block FP4 or 7/6-scaled INT4      */
};
enum { FP4Q_ROUND_RNE = 0, FP4Q_ROUND_STOCHASTIC = 1 };
enum {
  FP4Q_ROT_NONE = 0,
  FP4Q_ROT_FWHT_ROW = 1,         /* full-row normalised FWHT, cols a power of two (MXFP4 only)  */
  FP4Q_ROT_RHT16 = 2,            /* seeded +-1 diagonal then 16-point normalised FWHT per block */
  FP4Q_ROT_FWHT128 = 3           /* NVFP4 only: normalised FWHT of every 128-element head chunk  */
};

typedef struct {
  int64_t rows;            /* >= 0                                                          */
  int64_t cols;            /* >= 0, multiple of block_size                                  */
  int64_t in_row_stride;   /* elements between row starts of x, >= cols                      */
  int32_t in_dtype;        /* FP4Q_F32 or FP4Q_BF16                                          */
  int32_t block_size;      /* 32 for MXFP4, 16 for NVFP4; anything else is UNSUPPORTED        */
  int32_t scale_policy;    /* FP4Q_SCALE_*; must belong to the entry point's format          */
  int32_t manual_exponent; /* used by FP4Q_SCALE_MANUAL only                                 */
  int32_t rounding;        /* FP4Q_ROUND_*                                                   */
  int32_t rotation;        /* FP4Q_ROT_*                                                     */
  uint64_t seed;           /* Philox key for stochastic rounding and the RHT signs           */
} fp4q_quant_args;

typedef struct {
  uint8_t *codes;          /* [rows][cols/2] bytes; element 2k in the low nibble of byte k   */
  uint8_t *scales;         /* [rows][cols/block_size]: E8M0 (MX) or E4M3 (NV) bytes          */
  float *global_scale;     /* NV only: 1 float, g in the decode direction; else ignored      */
  uint8_t *choice_bits;    /* Four Over Six only: ceil(rows*cols/16 / 8) bytes; bit b%8 of   */
                           /* byte b/8 is 1 iff flat block b = r*(cols/16)+j kept max->4      */
  float *rotated;          /* optional (NULL): [rows][cols] fp32 rotated values (test hook)   */
  uint64_t *counters;      /* optional (NULL): 3 x u64 zeroed by the call: [0] saturated      */
                           /* (|x/scale| > 6), [1] underflowed (nonzero -> zero code),        */
                           /* [2] non-finite inputs                                           */
} fp4q_outputs;

/* Bytes of device workspace a quantize call uses.  MXFP4 (block 32): 4 KiB,
 * optional, 8-byte aligned, zero-filled before its first use: a counting call
 * given one sums its counts through 128 slots in it (one atomic add per
 * count per workgroup into slot b mod 128, then a one-workgroup kernel that
 * writes the counters and clears the slots) instead of adding every
 * workgroup's counts into the three counters directly.  The NVFP4
 * workspace (80 KiB, 8-byte aligned) belongs to the caller, must be
 * zero-filled before its first use and is then kept consistent by the
 * library, also across launches captured in a HIP graph and replayed (a
 * captured single-read launch takes its epoch from a word in the workspace,
 * advanced by a one-thread kernel captured before it); calls that share one
 * workspace must be ordered (same stream, or synchronised).  Layout: bytes
 * [16, 24) an optional wait limit of that kernel's grid-wide exchange in
 * ticks of the 100 MHz GPU clock (0: 1 ms; a small value makes every wait
 * run out, which tests use), [24, 32) the epoch word of captured launches,
 * [64, 8256) per-workgroup flags, [8256,
 * 12352) the per-workgroup maxima of the two-pass kernels, [12352, 15424)
 * the 128 counter slots (three 64-bit counts each) of a counting call,
 * [16384, 81920) sixteen copies of the single-read kernel's result word,
 * 4 KiB apart. */
size_t fp4q_workspace_bytes(const fp4q_quant_args *args);

/* MXFP4 quantization of x ([rows][in_row_stride] of in_dtype).  block_size
 * 32, policy OCP_MAX or MANUAL, rotation NONE / FWHT_ROW (cols a power of two
 * between 32 and 16384) / RHT16, rounding RNE or STOCHASTIC.  The fp32
 * rotated values are what gets quantized; `rotated`, when given, receives
 * them.  workspace may be NULL; when given it must hold
 * fp4q_workspace_bytes() bytes, 8-byte aligned (else FP4Q_ERR_WORKSPACE).
 * Sources: audit page sections cited above. */
fp4q_status fp4q_quantize_mxfp4(const fp4q_quant_args *args, const void *x,
                                const fp4q_outputs *out, void *workspace,
                                size_t workspace_bytes, void *hip_stream);

/* NVFP4 quantization ("Sub-4-Bit Microscaling", section 2; Four Over Six,
 * transcript cue 10; IF4, transcript cues 14 and 17).  block_size 16, policy
 * NV_MAX6, FOUR_OVER_SIX or IF4, rotation NONE, RHT16 or FWHT128, rounding
 * RNE or STOCHASTIC (IF4: RNE only, STOCHASTIC is UNSUPPORTED).  FWHT128 is
 * the per-head rotation of a KV cache ("Sub-4-Bit Microscaling", section 3,
 * the online post-RoPE Q/K rotation): the normalised FWHT of each 128-element
 * chunk of a row (head dimension 128, no signs), then NVFP4 of the rotated
 * values; cols must be a multiple of 128, RNE only, policy NV_MAX6 or IF4.  IF4 writes no
 * choice bits (choice_bits may be NULL): an INT4 block has bit 7 of its
 * scale byte set; counters count the kept candidate (INT4 saturates at
 * |7x / (6 s g)| > 7).  The tensor amax is
 * computed in the call (a first pass over x, after rotation) unless
 * `global_amax` (device pointer to one finite non-negative float) is given.
 * amax 0 gives g = 1; a nonzero amax whose g underflows gives g = 2^-149.
 * Needs fp4q_workspace_bytes() of workspace (8-byte aligned, else
 * FP4Q_ERR_WORKSPACE) unless global_amax is given.
 * Contiguous bf16 input with policy NV_MAX6, RNE, no rotation, no counters,
 * no global_amax and at most 32768 eight-element slots per CU (64 Mi
 * elements on 256 CUs) runs as one launch that reads most of x once (four
 * 256-thread workgroups per CU, which exchange their chunk maxima through the
 * workspace); every other case runs an amax pass and an encode pass.  Both
 * give identical bytes.  The single launch assumes its workgroups run
 * together; when they cannot (another stream holding CUs, say), each
 * workgroup whose wait for the tensor maximum runs out (after 1 ms) reads the
 * chunk maxima already published and scans the chunks still missing itself:
 * still the same bytes, at a cost of up to 1 ms plus up to one read of x per
 * such workgroup. */
fp4q_status fp4q_quantize_nvfp4(const fp4q_quant_args *args, const void *x,
                                const float *global_amax, const fp4q_outputs *out,
                                void *workspace, size_t workspace_bytes, void *hip_stream);

/* fp4q_quantize_nvfp4 without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, checks, results and
 * errors as fp4q_quantize_nvfp4; the workspace is an 80 KiB scratch array
 * that the library holds in device memory on every GPU it runs on until the
 * process ends (its address is looked up on the first call made with that
 * device current: the calling thread's current device must be the GPU of
 * hip_stream).  It allocates nothing and frees nothing.  The scratch covers
 * every tensor size (the NVFP4 workspace does not grow with the tensor); a
 * workspace need above 80 KiB would be refused with FP4Q_ERR_WORKSPACE.
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents: calls that overlap on one GPU (unordered streams, several
 * host threads) race and must not be made; calls ordered on one stream, or
 * synchronised, are safe.  Lookup failures return FP4Q_ERR_HIP. */
fp4q_status fp4q_quantize_nvfp4_noalloc(const fp4q_quant_args *args, const void *x,
                                        const float *global_amax, const fp4q_outputs *out,
                                        void *hip_stream);

/* Fused SwiGLU epilogue ("Sub-4-Bit Microscaling", section 3: the online
 * rotation inside the SiLU_and_Mul kernel right before down_proj): the
 * activation h = SiLU(gate) * up, SiLU(g) = g / (1 + e^-g), is formed in fp32
 * as gate and up are read (hardware exponential and reciprocal, within a few
 * ulps), never stored, rotated by the normalised full-row FWHT and
 * MXFP4-quantized as fp4q_quantize_mxfp4 does.  gate and up are
 * [rows][in_row_stride] device arrays of in_dtype sharing the row stride
 * (e.g. the two halves of a [rows][2 * cols] tensor).  block_size 32, policy
 * OCP_MAX or MANUAL, rounding RNE or STOCHASTIC, rotation must be FWHT_ROW
 * and cols a power of two between 32 and 16384 (else UNSUPPORTED).
 * `rotated`, when given, receives the rotated fp32 values that were
 * quantized; no workspace. */
fp4q_status fp4q_silu_mul_fwht_mxfp4(const fp4q_quant_args *args, const void *gate, const void *up,
                                     const fp4q_outputs *out, void *hip_stream);

/* Normalised Walsh-Hadamard transform of each transform_size-chunk of each
 * row: y[r, c0:c0+t] = (x[r, c0:c0+t] * sigma) H_t * fl32(1/sqrt(t)), fp32
 * out ([rows][d], dense).  transform_size t: a power of two with 2 <= t <=
 * 16384 dividing d; random_signs applies the seeded diagonal sigma ("Sub-4-
 * Bit Microscaling", section 3; transcript cue 8). */
fp4q_status fp4q_fwht(int64_t rows, int64_t d, int64_t in_row_stride, int32_t in_dtype,
                      const void *x, float *y, int32_t transform_size, int32_t random_signs,
                      uint64_t seed, void *hip_stream);

/* Reconstruction ("Encode one MXFP4 block step by step": multiply back by
 * the scale).  MX: value * 2^(b-127), exact.  NV: value * s * g rounded once
 * to the output type.  IF4: a block whose scale byte has bit 7 set holds
 * INT4 nibbles, k * 6 * s * g / 7 rounded once, s from the low 7 bits; other
 * blocks as NV.  A NaN scale code (low 7 bits 0x7F for NV and IF4) gives NaN
 * for its block.  format FP4Q_MXFP4 (block 32), FP4Q_NVFP4 or FP4Q_IF4
 * (block 16, global_scale: device pointer to g); out_dtype FP4Q_F32 or
 * FP4Q_BF16; out is [rows][cols]. */
fp4q_status fp4q_dequantize(int32_t format, int64_t rows, int64_t cols, int32_t block_size,
                            const uint8_t *codes, const uint8_t *scales,
                            const float *global_scale, int32_t out_dtype, void *out,
                            void *hip_stream);

/* MXFP4 GEMM, the consumer of two quantized operands ("Sub-4-Bit
 * Microscaling", section 3: Y = X W^T with X and W both 4-bit block-scaled;
 * section 2: block scales applied inside the matrix instruction):
 * C[m][n] = sum_k A[m][k] B[n][k] over the reconstructed values of A
 * ([M][K]: a_codes [M][K/2], a_scales [M][K/32]) and B ([N][K]: b_codes,
 * b_scales), exactly the planes fp4q_quantize_mxfp4 writes (B is the
 * [N][K] weight, so C = A B^T).  Products are exact; the sum is fp32 in the
 * matrix instructions' order.  C is dense [M][N] fp32 or bf16 (out_dtype,
 * rounded to nearest-even).  K must be a multiple of 128 and at most 2^23
 * (else UNSUPPORTED; not a multiple of 32: INVALID_ARG); code planes 16-byte
 * aligned, scale planes and C 4-byte aligned.  A NaN scale (0xFF) makes its
 * terms NaN. */
fp4q_status fp4q_mxfp4_gemm(int64_t M, int64_t N, int64_t K, const uint8_t *a_codes, const uint8_t *a_scales,
                            const uint8_t *b_codes, const uint8_t *b_scales, int32_t out_dtype, void *c,
                            void *hip_stream);

/* Host-side check of counters copied back from the device: FP4Q_ERR_NONFINITE
 * when counters[2] != 0, else FP4Q_OK (NULL -> FP4Q_ERR_INVALID_ARG). */
fp4q_status fp4q_check_counters(const uint64_t *host_counters);

/* Static, human-readable name of a status code. */
const char *fp4q_status_string(fp4q_status status);

/* Library version string. */
const char *fp4q_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4Q_H */
