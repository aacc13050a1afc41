/*
 * qgemm.h -- C ABI of a weight-only quantized GEMM for AMD MI355X (gfx950).
 *
 *   out[M, N] = A[M, K] . dequant(W)[K, N]            (times alpha for FP8 / FP4)
 *
 * A holds 16-bit activations; W is stored packed at low precision and is dequantized
 * in registers inside the kernels -- no 16-bit copy of W is ever written to memory.
 *
 * Formats (all other combinations return QGEMM_ERR_UNSUPPORTED):
 *   a_dtype  w_dtype        scale_layout          out_dtype     source
 *   F16      INT4           GROUP_F16 (G=32..256) F16 or F32    Low Bit Triton Kernels (GPU MODE
 *                                                               lecture 034), core pattern and
 *                                                               gemlite snippet; Bitblas lecture 033,
 *                                                               API example (MatmulConfig)
 *   BF16     FP8_E4M3       TENSOR_F32            BF16 or F32   FlashInfer PR #7495 analysis
 *                                                               (mm_bf16_fp8), introduction and
 *                                                               section 2 (public API)
 *   F16      FP8_E4M3       TENSOR_F32            F16 or F32    the same analysis, section 2
 *                                                               (mm_fp16_fp8)
 *   BF16     FP4_E2M1       BLOCK16_E4M3          BF16 or F32   FlashInfer PR #4466 analysis
 *                                                               (BF16 x FP4 GEMM), sections 1-3
 *   F16      INT2           GROUP_F16 (G=32..256) F16 or F32    Bitblas lecture 033, exercises
 *                                                               (the W2A16 combination), with
 *                                                               the INT4 recipe at 2 bits
 *   F16      NF4            GROUP_F16_LUT16       F16 or F32    Low Bit Triton Kernels (GPU MODE
 *                           (G=32..256)                         lecture 034), 4-bit value choice:
 *                                                               a non-uniform 16-value grid read
 *                                                               through a register table
 *
 * Value semantics (what the kernels compute):
 *   INT4 : w[k][n] = RNE_fp16((nibble - 8) * s[k / G][n]) -- the 16-bit operand the
 *          gemlite snippet forms -- accumulated in fp32.  No alpha.
 *   FP8  : w = e4m3(code) (exact in bf16 and in fp16; the MFMA takes the activations'
 *          type); the fp32 per-tensor alpha multiplies the fp32 accumulator once, in the
 *          epilogue, as the PR #7495 analysis prescribes.
 *   FP4  : w = e2m1(code) * e4m3(s_b) (exact in bf16) with one scale per 16 consecutive
 *          K of a column; alpha multiplies the fp32 accumulator in the epilogue.
 *   INT2 : w[k][n] = (code - 2) * s[k / G][n] (exact in fp16), accumulated in fp32.
 *   NF4  : w[k][n] = RNE_fp16(T[code] * s[k / G][n]) with T the 16-entry fp16 code book
 *          that travels with the scales (qgemm_quantize writes the NormalFloat-4 book),
 *          accumulated in fp32.  No alpha.
 *   Bias (qgemm_run_bias): bias[n] is added in fp32 after alpha.
 *   The 16-bit output is the round-to-nearest-even cast of the fp32 result, so a call
 *   with out_dtype F32 yields exactly the values a 16-bit call rounds.
 *
 * Threading and ownership: the library allocates no device memory, frees nothing and keeps
 * no per-call state; every buffer belongs to the caller.  All entry points are thread-safe.
 * Errors are returned synchronously before anything is enqueued; a detail string naming
 * the offending argument is available from qgemm_last_error() on the calling thread.
 * No C++ exception ever crosses this interface.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qgemm_status {
  QGEMM_OK = 0,
  QGEMM_ERR_INVALID_ARGUMENT = 1,   /* bad shape, NULL pointer, bad enum value          */
  QGEMM_ERR_UNSUPPORTED = 2,        /* valid but unsupported dtype / layout combination  */
  QGEMM_ERR_MISALIGNED = 3,         /* a pointer violates its alignment requirement      */
  QGEMM_ERR_WORKSPACE_TOO_SMALL = 4,
  QGEMM_ERR_HIP = 5                 /* the HIP runtime reported an error at launch       */
} qgemm_status_t;

typedef enum qgemm_dtype {
  QGEMM_DT_F16 = 0,
  QGEMM_DT_BF16 = 1,
  QGEMM_DT_F32 = 2,
  QGEMM_DT_INT4 = 3,
  QGEMM_DT_FP8_E4M3 = 4,   /* OCP e4m3 ("fn"): max 448, code S.1111.111 is NaN        */
  QGEMM_DT_FP4_E2M1 = 5,   /* e2m1: +-{0, .5, 1, 1.5, 2, 3, 4, 6}                      */
  QGEMM_DT_INT2 = 6,       /* signed 2-bit integer in [-2, 1], stored + 2               */
  QGEMM_DT_NF4 = 7         /* 4-bit index into a 16-entry fp16 code book                */
} qgemm_dtype_t;

typedef enum qgemm_scale_layout {
  QGEMM_SCALE_GROUP_F16 = 0,     /* INT4: fp16 scale per (group of G consecutive K, column) */
  QGEMM_SCALE_TENSOR_F32 = 1,    /* FP8 : no weight scales; one fp32 alpha (device pointer) */
  QGEMM_SCALE_BLOCK16_E4M3 = 2,  /* FP4 : e4m3 scale per (16 consecutive K, column) + alpha */
  QGEMM_SCALE_GROUP_F16_LUT16 = 3 /* NF4: 16 fp16 code-book entries, then GROUP_F16 scales   */
} qgemm_scale_layout_t;

/* kernel_hint values (testing and tuning; 0 is the right choice for applications) */
#define QGEMM_KERNEL_AUTO 0
#define QGEMM_KERNEL_DECODE 1     /* memory-bound skinny kernel, M <= 16 only            */
#define QGEMM_KERNEL_PREFILL 2    /* MFMA tile kernel, any M                              */
#define QGEMM_KERNEL_PREFILL_STREAMK 3  /* the MFMA tile kernel on a persistent grid: whole
                                           tiles round-robin, the last rounds' tiles split
                                           evenly in K over the workgroups (stream-K tail);
                                           never chosen automatically                        */
#define QGEMM_KERNEL_PREFILL_TRANSFORM 4 /* the MFMA tile kernel with dedicated dequantization
                                           wavefronts (the transform warpgroup of FlashInfer
                                           PR #7495 analysis, section 1): 64 x 128 tiles only
                                           (tile_hint 0 or 64), any split; never chosen
                                           automatically                                      */

/*
 * The problem descriptor, after the BitBLAS MatmulConfig (Bitblas lecture 033, API
 * example): sizes, operand dtypes, group size and scale layout.  Fields are fixed-width
 * so the struct has the same layout from C, C++ and ctypes (56 bytes).
 *   M >= 0 (any value; M = 0 is an empty product: qgemm_run validates the descriptor and
 *   enqueues nothing, ignoring the pointers); N % 16 == 0; K % 128 == 0; for INT4 also
 *   K % group_size == 0.  Each of M, N, K is at most 2^24.
 *   group_size: INT4, INT2 and NF4, one of 32, 64, 128, 256; FP4 requires 16; FP8 requires 0.
 *   FP8 weights take a_dtype BF16 (mm_bf16_fp8) or F16 (mm_fp16_fp8); the packed weights
 *   are the same for both.
 *   kernel_hint: QGEMM_KERNEL_*; split_k_hint: 0 = automatic, else the number of K
 *   slices (1..64) the chosen kernel uses (not with QGEMM_KERNEL_PREFILL_STREAMK); tile_hint: 0 = automatic, else for the decode
 *   kernel the number of 16-column blocks per workgroup (1 to 4), for the prefill
 *   kernel the rows of its workgroup tile (64: 64 x 128, 128: 128 x 128, 256: 256 x 256;
 *   QGEMM_KERNEL_PREFILL_TRANSFORM: 64 only).
 *   Hints only change the work split and the reduction order of the fp32 accumulation,
 *   never the packed layout; the automatic choice depends only on M, N, K and the formats
 *   (never on out_dtype or pointers).
 */
typedef struct qgemm_problem {
  int64_t M, N, K;
  int32_t a_dtype, w_dtype, out_dtype;
  int32_t group_size;
  int32_t scale_layout;
  int32_t kernel_hint;
  int32_t split_k_hint;
  int32_t tile_hint;
} qgemm_problem_t;

/*
 * qgemm_quantize -- offline, host memory only, no GPU needed.
 * Quantizes fp32 weights W given in the "nt" orientation w_nk[N][K] (row n is output
 * column n; the BitBLAS "nt" layout) into the canonical form that qgemm_pack takes:
 *   INT4: codes_canonical uint8[N][K/2], byte j of row n = code(k=2j) | code(k=2j+1) << 4,
 *         code = clamp(rint(w / s), -8, 7) + 8; scales_canonical fp16 [K/G][N] with
 *         s = RNE_fp16(absmax_group / 7)   (Low Bit Triton Kernels, core pattern: one
 *         scale per 128-ish group along K; gemlite snippet: nibble - 8).
 *   FP8 : codes uint8[N][K] = e4m3(clamp(w / alpha, +-448)), alpha = absmax / 448 (fp32);
 *         scales_canonical unused (may be NULL).
 *   INT2: codes_canonical uint8[N][K/4], byte j of row n = code(4j) | code(4j+1) << 2 |
 *         code(4j+2) << 4 | code(4j+3) << 6, code = clamp(rint(w / s), -2, 1) + 2; scales
 *         as INT4 with s = RNE_fp16(absmax_group / 1) (the INT4 recipe at 2 bits).
 *   NF4 : codes uint8[N][K/2] (nibble order as INT4) = the index c of the code-book entry
 *         nearest to w / s (ties to the lower index; c = 7, the entry 0, when s = 0);
 *         scales_canonical fp16 [16 + (K/G) N]: first the code book T[0..15], the
 *         NormalFloat-4 values (QLoRA's construction: the 8 positive and 7 negative
 *         quantiles of N(0,1) at evenly spaced probabilities from 1/2 to
 *         delta = ((1 - 1/30) + (1 - 1/32)) / 2, plus 0, divided by the largest; rounded
 *         to fp16), then [K/G][N] scales s = RNE_fp16(absmax_group).
 *   FP4 : codes uint8[N][K/2] (nibble order as INT4) = e2m1(clamp(w / (s_b alpha), +-6)),
 *         scales_canonical e4m3 uint8[N][K/16] = e4m3(min(absmax_b / (6 alpha), 448)),
 *         alpha = absmax / (6 * 448) (fp32).
 * Rounding is round-half-even; divisions are done in double and rounded once.  An
 * all-zero group / block / tensor gets scale 0 and signed code 0 (NF4: code 7).  alpha_out
 * receives alpha (FP8, FP4) or 1.0 (INT4, INT2, NF4); it may be NULL for those three.
 */
qgemm_status_t qgemm_quantize(const qgemm_problem_t* problem, const float* w_nk,
                              void* codes_canonical, void* scales_canonical, float* alpha_out);

/*
 * qgemm_pack -- offline, host memory only, no GPU needed.
 * Reorders canonical weights and scales (the layout qgemm_quantize writes) into the
 * device layout whose 16-byte lane chunks are gfx950 16x16x32 MFMA operand fragments, so
 * that no layout conversion happens at run time (Bitblas lecture 033, layout section: a
 * mismatched fragment layout forces a re-layout through shared memory).  Byte map, with
 * lane l of a 64-lane wavefront owning bytes [16 l, 16 l + 16) of every 1 KiB block:
 *   INT4 / FP4 weights: block (nb, kb) = columns 16nb..16nb+15 x k 128kb..128kb+127, block
 *     index nb*(K/128) + kb; dword t (0..3) of lane l holds column 16nb + (l & 15) at
 *     k = 128kb + 32t + 8(l >> 4) + J[s] in nibble s (bits 4s..4s+3), with
 *     J = (0,2,4,6,1,3,5,7) for INT4 and J = (0,1,...,7) for FP4.
 *   NF4 weights: as INT4 with J = (0,4,1,5,2,6,3,7) (byte b of a dword holds k offsets b
 *     and b + 4, the order of the byte-table lookup).
 *   INT2 weights: block (nb, kb) = 16 columns x 128 k = 512 bytes, index nb*(K/128) + kb;
 *     lane l owns bytes [8 l, 8 l + 8); bits 16h + 8b + 2f (h, b = 0..1, f = 0..3) of its
 *     dword d hold column 16nb + (l & 15), k = 128kb + 32(2d + b) + 8(l >> 4) + 2f + h.
 *   FP8 weights: block (nb, kb) = 16 columns x 64 k, index nb*(K/64) + kb; byte 8t + j
 *     (t = 0..1, j = 0..7) of lane l is column 16nb + (l & 15), k = 64kb + 32t + 8(l>>4) + j.
 *   INT4 and INT2 scales (fp16): span = max(G, 128), T = max(1, 128/G); element
 *     ((nb*(K/span) + kb)*16 + c)*T + t = scale of column 16nb + c, group kb*(span/G) + t.
 *   NF4 scales: a 256-byte header, then the INT4 scale layout.  Header dword q (0..3) holds
 *     the low bytes of T[4q..4q+3] (T[4q] in bits 0..7), dword 4 + q their high bytes; the
 *     rest of the header is zero.
 *   FP4 scales (e4m3): byte ((nb*(K/128) + kb)*16 + c)*8 + 4h + t = scale of column
 *     16nb + c, 16-k block 8kb + 2t + h.
 * Size query: pass w_packed == NULL and/or s_packed == NULL to receive the sizes only.
 * w_packed_bytes / s_packed_bytes are in/out: on input the capacity of the buffer (when
 * the buffer is non-NULL), on output the bytes needed.  FP8 has no packed scales
 * (s_packed_bytes = 0).  problem->M is ignored.
 */
qgemm_status_t qgemm_pack(const qgemm_problem_t* problem, const void* w_canonical,
                          const void* scales_canonical, void* w_packed, size_t* w_packed_bytes,
                          void* s_packed, size_t* s_packed_bytes);

/*
 * qgemm_workspace_bytes -- bytes of device workspace qgemm_run needs for this problem
 * (0 when none).  Workspace contract (for split-K reductions, FlashInfer PR #7495
 * analysis, section 2 names a workspace argument and a size query): the caller allocates
 * it, ZERO-FILLED, once; every completed qgemm_run returns its counter words to zero, so
 * it can be reused by later calls on the same stream without clearing.  Calls that overlap
 * in time (different streams) must use different workspaces.
 */
qgemm_status_t qgemm_workspace_bytes(const qgemm_problem_t* problem, size_t* bytes);

/*
 * qgemm_run -- enqueue out = A . dequant(W) (* alpha) on `stream`.
 *   A        device, row-major [M][K] of a_dtype, 16-byte aligned.
 *   w_packed device, qgemm_pack output, 16-byte aligned.
 *   s_packed device, qgemm_pack scale output (INT4, INT2, NF4, FP4; NULL for FP8),
 *            16-byte aligned.
 *   alpha    device pointer to one fp32 (FP8, FP4; NULL for INT4, INT2, NF4); 4-byte alignment only
 *            (FlashInfer PR #7495 analysis, section 3(a): scalar pointers must not be
 *            assumed 16-byte aligned).
 *   out      device, row-major [M][N] of out_dtype, 16-byte aligned.
 *   workspace / workspace_bytes: see qgemm_workspace_bytes; 256-byte aligned; may be
 *            NULL when 0 bytes are needed.
 *   stream   a hipStream_t; NULL means the default stream.
 * Returns after enqueueing; kernel faults surface at the caller's next synchronisation.
 * The result is bitwise deterministic for a given problem (including its hints).
 */
qgemm_status_t qgemm_run(const qgemm_problem_t* problem, const void* A, const void* w_packed,
                         const void* s_packed, const float* alpha, void* out, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * qgemm_run_bias -- enqueue out[m][n] = A . dequant(W) (* alpha) + bias[n] on `stream`, the
 * bias argument of mm_bf16_fp8 / mm_fp16_fp8 (FlashInfer PR #7495 analysis, section 2),
 * available for every format.  Arguments as qgemm_run, plus:
 *   bias     device, N values of out_dtype (fp32 for out_dtype F32), 16-byte aligned (the
 *            alignment that analysis, section 3(a), requires of a bias), else
 *            QGEMM_ERR_MISALIGNED; NULL means no bias, and the call is then exactly qgemm_run.
 * The bias is converted to fp32 (exact) and added to the fp32 result after alpha, before the
 * one rounding to out_dtype.
 */
qgemm_status_t qgemm_run_bias(const qgemm_problem_t* problem, const void* A, const void* w_packed,
                              const void* s_packed, const float* alpha, const void* bias, void* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * qgemm_run_no_alloc -- qgemm_run_bias without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Arguments, results and errors as qgemm_run_bias (bias may be NULL);
 * the launch plan, and so the result, is bitwise that of qgemm_run_bias on the same problem.
 * The split-K workspace is a static device array of QGEMM_NO_ALLOC_SCRATCH_BYTES per GPU,
 * held from the library's first use on that GPU until the process ends; a problem whose plan
 * needs more returns QGEMM_ERR_WORKSPACE_TOO_SMALL (qgemm_workspace_bytes tells in advance).
 * The array holds a fixed region of split-K tickets (one per output tile, at most 16384) and
 * the fp32 partial tiles after it.  The call allocates nothing.  The first call on a device
 * that needs the array enqueues one clear of its ticket region on `stream` before its GEMM;
 * every completed call leaves the tickets at zero again.  All calls on one GPU share the
 * array: calls that may overlap in time on one GPU (different streams, different host
 * threads) race and must not be made; calls in one stream's order are safe.
 */
#define QGEMM_NO_ALLOC_SCRATCH_BYTES ((32u << 20) + (64u << 10))
qgemm_status_t qgemm_run_no_alloc(const qgemm_problem_t* problem, const void* A, const void* w_packed,
                                  const void* s_packed, const float* alpha, const void* bias, void* out,
                                  void* stream);

/*
 * qgemm_status_string -- static, NUL-terminated name of a status code ("QGEMM_OK",
 * "QGEMM_ERR_MISALIGNED", ...; "QGEMM_ERR_UNKNOWN_STATUS" for a value outside the enum).
 * The pointer is owned by the library and valid for the life of the process.  Status codes
 * follow the FlashInfer PR #4466 analysis, section 2 (preparation and dispatch): a dtype or
 * backend combination the kernels do not implement is refused explicitly
 * (QGEMM_ERR_UNSUPPORTED, the analogue of its NotImplementedError) instead of falling back
 * to another path, and section 1 (input validation): every shape, dtype and pointer check
 * happens on the host before launch.
 */
const char* qgemm_status_string(qgemm_status_t status);

/*
 * qgemm_last_error -- detail text of the last error an entry point returned on the calling
 * thread ("" after a call that succeeded).  The text names the offending argument, the
 * value received and the value expected (e.g. which a_dtype / out_dtype a weight format
 * needs), after the validation messages of the FlashInfer PR #4466 analysis, section 1,
 * which name the expected dtype and the call that produces a correctly laid-out operand.
 * The pointer is owned by the library (thread-local storage) and stays valid until the next
 * qgemm_* call on the same thread.
 */
const char* qgemm_last_error(void);

/*
 * qgemm_plan_describe -- one NUL-terminated line naming the launch qgemm_run would make for
 * this problem: the kernel ("decode", "prefill" or "empty" for M = 0), its grid, its K split
 * and, for decode, the column blocks per workgroup, the k blocks per wavefront run, the runs
 * per share and how A reaches the MFMA fragments ("a=direct", "a=staged" or "a=dma"); for
 * prefill, the tile and the persistent schedule.  The dispatch decision of the FlashInfer
 * PR #4466 analysis, section 2 (preparation and dispatch), made inspectable: the text is
 * for people and tests, its fields may grow.  `buf` is caller-owned host memory of `len`
 * bytes; a line that does not fit returns QGEMM_ERR_INVALID_ARGUMENT (buf then holds the
 * truncated line); an invalid problem returns the status qgemm_workspace_bytes would.
 */
qgemm_status_t qgemm_plan_describe(const qgemm_problem_t* problem, char* buf, size_t len);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t qgemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
