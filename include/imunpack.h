/*
 * imunpack.h -- C ABI of the IM-Unpack exact low bit-width integer GEMM path
 * for AMD Instinct MI355X (gfx950).
 *
 * Method source: the summary page "IM-Unpack: Training and Inference with
 * Arbitrarily Low Precision Integers".  A float GEMM C = A.B is quantized with
 * round-to-nearest (RTN) so that the p-percentile magnitude of each matrix maps
 * to the integer beta ("Measured effects" table: p = 95%, beta = 15 / 31);
 * heavy hitters stay as out-of-range integers instead of being clipped
 * (summary paragraph, "Problem").  Out-of-range integers are unpacked into
 * several in-range b-bit integers placed in extra rows or columns, chosen per
 * matrix from outlier counts (row, column or Mix unpacking; "Approach" and the
 * unpack-ratio rows of the table); products of the unpacked narrow-integer
 * matrices, multiplied by powers of two and summed, equal the original integer
 * product ("Approach").
 *
 * Conventions (all entry points)
 * ------------------------------
 * - Every data pointer is a DEVICE pointer unless marked "host".  The caller
 *   owns every buffer.  No entry point allocates or frees memory (device, pinned
 *   or host heap): imu_init allocates, once per device, the pinned host buffer
 *   the plan headers are read back through and two events, and imu_release
 *   frees them.  imu_plan_unpack, imu_unpacked_gemm and imu_imunpack_matmul
 *   need imu_init on the calling thread's current device first (else
 *   IMU_ERR_INVALID_ARG).
 * - All work is enqueued on `stream` (HIP stream; 0 = the null stream).  Only
 *   imu_plan_unpack and imu_imunpack_matmul wait for the device, once each, to
 *   read the plan header (the unpacked sizes are data dependent).  Calls on one
 *   device from several host threads take turns between the planner launch and
 *   that read (they share the device's header buffer).
 * - IMU_LOG=1 in the environment prints, at that read, one line per batch
 *   entry on stderr: the chosen candidates, M' K' N', the unpack ratio, k_pad
 *   and the exponent segments' lengths, the row and column bases and
 *   allocations, the digit format and the plan status.
 * - Argument errors are returned synchronously and nothing is enqueued.
 *   Conditions found on the device (non-finite input, |x.r| >= 2^31) are
 *   latched in the operand's statistics and returned at the next wait.
 * - The integer result C is defined modulo 2^32 (two's complement int32),
 *   which equals the exact product whenever it fits in int32.  There is no
 *   overflow status: the digit products (int8 -> int32 MFMA, or fp6 -> fp32
 *   MFMA whose integer sums stay within 2^24 and are added into C as int32
 *   when they could pass it) and the int32 shift-and-add fold never form the
 *   product in wider integers, so an exact
 *   overflow test would need a second, wider product.  A caller can bound
 *   |C| <= K * max|q_A| * max|q_B| from the statistics headers (maxkey and r).
 * - Batched operands (batch > 1) are independent problems: each batch entry
 *   has its own percentile scale, plan and unpacked sizes.
 * - Calls on one stream are ordered; calls that share a workspace must not
 *   overlap in time.
 */
#ifndef IMUNPACK_H
#define IMUNPACK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IMU_OK = 0,
  IMU_ERR_INVALID_ARG = 1, /* bad shape, stride, dtype, parameter or null pointer */
  IMU_ERR_NONFINITE = 2,   /* an input element is NaN or +-Inf */
  IMU_ERR_RANGE = 3,       /* |fl32(x * r)| >= 2^31: the code does not fit int32 */
  IMU_ERR_WORKSPACE = 4,   /* workspace too small; *ws_needed holds the size */
  IMU_ERR_HIP = 5,         /* a HIP runtime call failed (detail: imu_last_error) */
  IMU_ERR_UNSUPPORTED = 6  /* valid request beyond this build's limits (see imu_last_error) */
} imu_status;

typedef enum { IMU_F32 = 0, IMU_BF16 = 1 } imu_dtype;

/* IMU_NORMAL: element (r, c) of the logical matrix is stored at r*ld + c.
 * IMU_TRANSPOSED: the stored array is the transpose: element (r, c) is at c*ld + r
 * (a weight W of shape N x K used as B = W^T with layout TRANSPOSED). */
typedef enum { IMU_NORMAL = 0, IMU_TRANSPOSED = 1 } imu_layout;

/* Unpacking strategy of one operand ("Approach"; Mix in the unpack-ratio rows).
 * IMU_GREEDY: line-at-a-time unpacking (all depths start at 1; while a code is
 * not covered, the row or column holding the most uncovered codes gets one more
 * level, rows first and lower indices first on ties), for comparing plan
 * quality with Mix; the operand may have at most 28672 rows + columns. */
typedef enum { IMU_ROW = 0, IMU_COL = 1, IMU_MIX = 2, IMU_GREEDY = 3 } imu_strategy;

/* Candidate depth maps the planner chooses from (Mix allows the first four):
 * ROW: each row gets its largest digit count; COL: each column does;
 * CR: heavy columns first, then rows; RC: heavy rows first, then columns;
 * GREEDY: the line-at-a-time depths (strategy IMU_GREEDY only). */
typedef enum {
  IMU_CAND_ROW = 0, IMU_CAND_COL = 1, IMU_CAND_CR = 2, IMU_CAND_RC = 3, IMU_CAND_GREEDY = 4
} imu_candidate;

/* One operand as it enters C = A.B.  `rows` x `cols` is the LOGICAL shape
 * (A: M x K, B: K x N).  `ld` >= stored row length; `batch` >= 1 entries spaced
 * `batch_stride` elements apart.  `data` must be 16-byte aligned. */
typedef struct {
  const void* data;
  int32_t dtype;  /* imu_dtype */
  int32_t layout; /* imu_layout */
  int64_t rows, cols, ld;
  int64_t batch, batch_stride;
} imu_matrix;

/* Digit format of the unpacked operands.  INT8: one signed byte per digit,
 * products on the int8 MFMA.  FP6: each digit as its e2m3 code (every integer
 * |d| <= 7 is exact in e2m3: sign bit 5, magnitudes 0..7 as 0, 8, 16, 20, 24,
 * 26, 28, 30), six bits per position, products on the f8f6f4 MFMA with fp32
 * accumulation; every partial sum is an integer below 2^24 in magnitude, so
 * the result is the same integer product.  FP6 needs bits <= 4 and both
 * operands K-contiguous (A IMU_NORMAL, B IMU_TRANSPOSED).  AUTO: FP6 where it
 * applies, else INT8. */
typedef enum { IMU_DIGITS_AUTO = 0, IMU_DIGITS_INT8 = 1, IMU_DIGITS_FP6 = 2 } imu_digits;

/* beta >= 1: the integer the p-percentile magnitude maps to.
 * p = p_num / p_den in (0, 1], held as a ratio of integers.
 * bits in [2, 8]: an in-range code satisfies |q| <= 2^(bits-1) - 1; unpacked
 * digits are signed base-2^(bits-1) digits and fit in int8.
 * gamma >= 0: a line is heavy when its out-of-range count exceeds gamma times
 * the mean count of its dimension (2 by default).
 * strat_a / strat_b: imu_strategy of A and B. */
typedef struct {
  int32_t beta, p_num, p_den, bits, gamma;
  int32_t strat_a, strat_b;
  int32_t clip; /* 0: RTN codes are never clipped (IM-Unpack); 1: the clipping
                   quantizer of the page's ablation rows ("Measured effects":
                   clipping at the 99.5-percentile): q = clamp(rne(fl32(x r)),
                   -beta, beta), so no code exceeds beta and none is an error */
  int32_t digits; /* imu_digits: format of the unpacked operands (IMU_DIGITS_FP6
                     where it does not apply: IMU_ERR_UNSUPPORTED) */
} imu_params;

/* Statistics of one operand prepared ahead of a call by imu_prepare_operand
 * (a weight reused across inference calls, or a training tensor that enters
 * several GEMMs).  stats = NULL: the call computes them itself.
 * transposed = 1: they were prepared for the transpose of the operand's
 * logical matrix (W prepared once, used as W in one GEMM and as W^T in
 * another); the row and column statistics then swap roles. */
typedef struct {
  const void* stats;
  int32_t transposed;
  int32_t pad_;
} imu_prepared;

/* Host-side summary of one batch entry's plan, filled by imu_plan_unpack. */
typedef struct {
  int64_t m, k, n;           /* original sizes M, K, N of this problem */
  int64_t m_u, k_u, n_u;     /* unpacked sizes M', K', N' (no padding) */
  int64_t m_alloc, n_alloc;  /* rows of A' and of B'^T as laid out (padded) */
  int64_t k_pad;             /* row length in bytes of A' and B'^T (padded K') */
  int64_t m_base, n_base;    /* first extra row of A' / first extra row of B'^T */
  int64_t a_offset, b_offset;/* byte offsets of this entry in the unpacked buffers */
  int32_t n_seg;             /* number of exponent segments of K' */
  int32_t choice_a, choice_b;/* imu_candidate chosen for A and B */
  int32_t digits;            /* format of A' and B'^T: IMU_DIGITS_INT8 or IMU_DIGITS_FP6 */
  double unpack_ratio;       /* M'K'N' / (MKN) */
  int64_t pair_sizes[25][3]; /* (M',K',N') of every candidate pair, A-major (5 x 5); -1 if not allowed */
} imu_plan_info;

/* Byte offsets inside one batch entry of a statistics buffer (see imu_stats_layout).
 * Header words at offset 0: float alpha, r, s, kth; uint32 maxkey; int32 status;
 * uint32 sel_prefix, sel_rank; uint64 total (T, out-of-range codes). */
typedef struct {
  int64_t stride;                    /* bytes per batch entry */
  int64_t row_oob, col_oob;          /* int32[rows], int32[cols] */
  int64_t row_maxdig, col_maxdig;    /* int32[rows], int32[cols] */
  int64_t cr_rowdig, rc_coldig;      /* int32[rows], int32[cols]: residual maxima (Mix) */
  int64_t hist;                      /* uint32[32768] percentile histogram */
} imu_stats_view;

/* Byte offsets inside a plan buffer.  Headers of all batch entries come first
 * (`header_stride` bytes each); each entry's arrays follow at
 * headers_bytes + b * entry_stride. */
typedef struct {
  int64_t header_stride, headers_bytes, entry_stride;
  int64_t da_r, da_c, db_r, db_c;    /* int32 depth maps: [M], [K], [K], [N] */
  int64_t lvl_a, lvl_b;              /* int32 [levels][M] / [levels][N]: unpacked row of (line, level) */
  int64_t kpre;                      /* int32 [segments][K+1]: per-segment prefix over k */
  int64_t amap, bmap;                /* int32 [m_alloc_max] / [n_alloc_max]: line | level << 24, -1 = padding */
  int64_t levels, segments;          /* array extents used above */
  int64_t m_alloc_max, n_alloc_max;
} imu_plan_view;

/* ---- set-up ------------------------------------------------------------------ */

/* Set-up for the calling thread's current device: a pinned, coherent host
 * buffer that receives the plan headers of up to max_batch batch entries per
 * call (2 KB each), two events, and the device's compute-unit count.  Call once
 * per device before the entry points that need it; calling again is cheap and
 * grows the buffer if max_batch is larger (waiting for the device first).
 * A call with more batch entries than the buffer holds returns
 * IMU_ERR_UNSUPPORTED.  Thread-safe.  max_batch in [1, 65535]. */
imu_status imu_init(int64_t max_batch);
/* Frees what imu_init allocated for the current device, after waiting for the
 * device (no call of the library may be in flight on it).  A later entry point
 * on that device needs imu_init again.  A no-op when nothing was set up. */
imu_status imu_release(void);

/* ---- sizes and layouts (host only, no device work) ------------------------ */

/* Bytes of one operand's statistics buffer (all batch entries). 0 on bad input. */
size_t imu_stats_bytes(const imu_matrix* x);
imu_status imu_stats_layout(const imu_matrix* x, imu_stats_view* view /* host */);

/* Bytes of the device plan buffer for A, B and p (all batch entries). 0 on bad input. */
size_t imu_plan_bytes(const imu_matrix* a, const imu_matrix* b, const imu_params* p);
imu_status imu_plan_layout(const imu_matrix* a, const imu_matrix* b, const imu_params* p,
                           imu_plan_view* view /* host */);

/* ---- the five entry points ------------------------------------------------ */

/* RTN quantization of one operand: the percentile scale and the outlier counts.
 * (Page: "Measured effects" table, p and beta rows; summary: heavy hitters
 * kept as out-of-range integers; "Approach": outlier counts per line.)
 * For each batch entry: alpha = the ceil(p*N)-th smallest |x| (if 0, the
 * largest |x|; if that is 0 too, r = s = 0 and every code is 0);
 * r = fl32(beta/alpha), s = fl32(alpha/beta); q = round_half_even(fl32(x*r)),
 * never clipped.  A code is out of range when |q| >= 2^(bits-1).  Writes per
 * row and per column out-of-range counts and largest digit counts and the total
 * T into `stats` (imu_stats_bytes(x) bytes, contents replaced).
 * q_out: optional int32 codes, logical rows x cols row-major per batch entry,
 * entries rows*cols apart; NULL to skip.  Asynchronous: device-detected errors
 * are reported by the next imu_plan_unpack. */
imu_status imu_quantize_rtn(const imu_matrix* x, const imu_params* p, void* stats,
                            int32_t* q_out, hipStream_t stream);

/* Plan of the unpacking ("Approach": row/column unpacking chosen per matrix
 * from outlier counts; Mix rows of the table).  Needs the statistics of A and
 * B from imu_quantize_rtn; with a Mix strategy the operand is read once more to
 * find the residual digit counts outside heavy lines.  Chooses for each batch
 * entry the allowed candidate pair with the smallest M'.K'.N' (ties: A-major
 * order ROW < COL < CR < RC) and writes depth maps, index maps and exponent
 * segments into `plan` (imu_plan_bytes bytes).  Waits once for the device and
 * fills info[0..batch-1] (host).  Returns IMU_ERR_NONFINITE / IMU_ERR_RANGE if
 * quantization found such input (then the plan is not valid). */
imu_status imu_plan_unpack(const imu_matrix* a, const imu_matrix* b, const imu_params* p,
                           void* stats_a, void* stats_b, void* plan,
                           imu_plan_info* info /* host, batch entries */, hipStream_t stream);

/* Unpack one operand into its digits ("Approach": out-of-range integers
 * decomposed into several in-range low bit-width integers in extra rows or
 * columns; summary: "larger matrices").  operand 0 = A -> A' (m_alloc x k_pad
 * per entry), operand 1 = B -> B'^T (n_alloc x k_pad per entry), each entry at
 * info.a_offset / info.b_offset of x_u, in the plan's digit format
 * (info.digits; fp6 only for A IMU_NORMAL, B IMU_TRANSPOSED).
 * int8 digits: one byte per position.  B'^T is row-major.  A' is stored in
 * MFMA fragment order: 1 KB blocks of 32 rows x 32 K' bytes, ordered by row
 * block then K' block, block (rb, c) at byte (rb * k_pad/32 + c) * 1024;
 * inside a block, bytes [16h, 16h + 16) of the block's row r are at
 * 16 * (r + 32h) (h = 0, 1).
 * fp6 digits: the e2m3 code of each digit (imu_digits), six bits per position.
 * A row of B'^T is a bit stream of 3/4 k_pad bytes, position p at bits
 * [6p, 6p + 6) (little endian).  A' takes 1536-byte blocks of 32 rows x 64
 * positions, block (rb, c) at byte (rb * k_pad/64 + c) * 1536; inside a block,
 * the 24 bytes at 24 * (r + 32h) hold positions 32h .. 32h + 31 of the block's
 * row r as such a stream.
 * Rows are level-major (original lines
 * first, then level 1 lines, ...).  A's rows keep their index order inside a
 * level; B's columns (the rows of B'^T) are in depth order, descending depth
 * then index: row j < N of B'^T is the column at position j of that order, and
 * level w >= 1 of the column at position j is row n_base + (columns deeper than
 * 1, ..., w-1, summed) + j.  Columns are the exponent segments of K'
 * (e = v + v' ascending, then k, then v), each padded with zero digits to a
 * multiple of 128 positions.  Every byte of the valid rows is written. */
imu_status imu_unpack(const imu_matrix* x, int32_t operand, const imu_params* p,
                      const void* stats, const void* plan, const imu_plan_info* info,
                      int8_t* x_u, hipStream_t stream);

/* Low bit-width GEMMs on the unpacked operands with the shift-and-accumulate
 * fold and dequantization ("Approach": power-of-two scaling and summation
 * reproduce the integer GEMM exactly).  For each exponent segment e the digit
 * product P_e = A'[:,K'_e] . B'[K'_e,:] (int8 MFMA, or fp6 MFMA into fp32
 * sums that stay integers within 2^24: each wave bounds its sums and, before
 * they could pass 2^24, adds them into C as int32 shifted to their exponent
 * and starts again from zero) is accumulated as
 * acc = acc * 2^(bits-1) + P_e (from the highest e down); each unpacked
 * element (i,u),(n,w) then adds acc << ((bits-1)(u+w)) into C[i,n] (mod 2^32).
 * c: int32 M x N row-major per entry (ldc elements per row, entries
 * c_batch_stride apart).  out (optional): fl32(fl32(C) * fl32(s_A * s_B)),
 * same layout as c.  The caller's info must come from the same plan.
 * Extra columns of a plan without extra rows are folded inside the tiles of
 * their original columns when the call's output tiles (256 x 128) are at least
 * as many as the GPU's CUs, else in a pass of extra tiles with atomic adds (as
 * extra rows always are); the environment variable IMU_FOLD_COLUMNS=1 or 0
 * forces either way.  The result is the same. */
imu_status imu_unpacked_gemm(const int8_t* a_u, const int8_t* b_u, const imu_params* p,
                             const void* stats_a, const void* stats_b, const void* plan,
                             const imu_plan_info* info, int64_t batch, int32_t* c, int64_t ldc,
                             int64_t c_batch_stride, float* out, hipStream_t stream);

/* The whole path: quantize A and B, plan, unpack, GEMM, fold, dequantize.
 * c / out: M x N row-major per batch entry, entries M*N apart (out optional).
 * ws: device workspace of ws_bytes.  If it is too small the call returns
 * IMU_ERR_WORKSPACE with *ws_needed set (the plan is deterministic, so a retry
 * with a larger workspace is exact); ws_needed may be NULL.  info: optional
 * host array of batch entries. */
imu_status imu_imunpack_matmul(const imu_matrix* a, const imu_matrix* b, const imu_params* p,
                               int32_t* c, float* out, void* ws, size_t ws_bytes,
                               size_t* ws_needed, imu_plan_info* info, hipStream_t stream);

/* imu_imunpack_matmul without a workspace argument, for callers that cannot
 * allocate device memory (tight serving loops, harnesses that forbid
 * allocation).  Statistics, plan and unpacked operands live in a static device
 * array of the library, imu_noalloc_scratch_bytes() = 128 MiB per GPU, held
 * from module load until the process ends; its address on each device is
 * looked up by imu_init, which must have run on the current device.  The call
 * itself allocates nothing.  A problem that needs more than the array returns
 * IMU_ERR_WORKSPACE (*ws_needed, if not NULL, holds the size it needs; the
 * unpack kernels then write nothing).  Every call on a GPU uses that GPU's one
 * array and leaves the last call's contents in it: calls that overlap in time
 * on one GPU (other streams, other host threads) race on it.  Results equal
 * imu_imunpack_matmul's. */
imu_status imu_imunpack_matmul_noalloc(const imu_matrix* a, const imu_matrix* b, const imu_params* p,
                                       int32_t* c, float* out, size_t* ws_needed, imu_plan_info* info,
                                       hipStream_t stream);
/* Size in bytes of the static array imu_imunpack_matmul_noalloc works in. */
size_t imu_noalloc_scratch_bytes(void);

/* Statistics of one operand for later calls: the percentile scale, RTN
 * codes' out-of-range counts and largest digit counts (as imu_quantize_rtn)
 * and the Mix residuals of both line directions (what imu_plan_unpack adds for
 * a Mix operand), into `stats` (imu_stats_bytes(x) bytes, contents replaced).
 * The same quantization serves every GEMM the matrix enters with the same
 * beta, p, bits and gamma ("Key results": LLaMA inference with fixed weights;
 * training, where one tensor enters the forward and a gradient GEMM).
 * Asynchronous; device-detected errors surface at the call that uses them. */
imu_status imu_prepare_operand(const imu_matrix* x, const imu_params* p, void* stats, hipStream_t stream);

/* imu_imunpack_matmul with the statistics of A and/or B prepared by
 * imu_prepare_operand: the call skips those operands' quantization passes
 * (percentile, counts, residual) and only reads their statistics.  Each
 * prepared buffer must describe this operand's data (or its transpose, with
 * transposed = 1), with the same dtype and the same beta, p, bits and gamma;
 * results equal imu_imunpack_matmul's.  pre_a / pre_b may be NULL.  Calls may
 * share a prepared buffer, also concurrently. */
imu_status imu_imunpack_matmul_prepared(const imu_matrix* a, const imu_matrix* b, const imu_params* p,
                                        const imu_prepared* pre_a, const imu_prepared* pre_b, int32_t* c,
                                        float* out, void* ws, size_t ws_bytes, size_t* ws_needed,
                                        imu_plan_info* info, hipStream_t stream);

/* Attention probabilities P = row softmax of `logits`, quantized as the A
 * operand of the attention-output GEMM P.V ("Key results", third bullet: the
 * attention-output GEMMs; "Measured effects": RTN for all GEMMs).  Writes P
 * (bf16, into `p`) and P's statistics (as imu_prepare_operand(p) would, into
 * `stats`, imu_stats_bytes(p) bytes, contents replaced) for
 * imu_imunpack_matmul_prepared; P's percentile histogram is counted while P
 * is written, so P is not read for it.
 * The page fixes no softmax arithmetic; P is the binary32 softmax fixed step
 * by step: m = maxNum of the row, t = x - m, y = t * fl(log2 e); e = 0 when
 * y < -100, else 2^n * poly(f) with n = rint(y), f = y - n and poly the
 * degree-7 Taylor polynomial of 2^f (coefficients fl((ln 2)^k / k!), Horner,
 * no fused multiply-add); S = the row's e summed by 64 lanes, lane l adding
 * positions 256 j + 4 l + c (j = 0, 1, ..., c = 0..3) in order, then the 64
 * lane sums halved pairwise (l and l + 32, then l + 16, ... l + 1); P =
 * bf16 nearest-even of fl(e / S).  -Inf logits give P = 0; a row with a NaN
 * or +Inf gives NaN probabilities, reported as IMU_ERR_NONFINITE by the call
 * that uses the statistics.
 * logits: IMU_F32 or IMU_BF16, IMU_NORMAL (the softmax runs along stored
 * rows), rows x cols per batch entry.  p: IMU_BF16, IMU_NORMAL, the same rows,
 * cols and batch, sharing no bytes with the logits.  Asynchronous. */
imu_status imu_softmax_prepare(const imu_matrix* logits, const imu_matrix* p_out, const imu_params* p, void* stats,
                               hipStream_t stream);

/* Fixed part of the imu_imunpack_matmul workspace (statistics and plan); the
 * unpacked operands need sum over entries of (m_alloc + n_alloc) * k_pad more. */
size_t imu_workspace_fixed_bytes(const imu_matrix* a, const imu_matrix* b, const imu_params* p);

/* ---- diagnostics ----------------------------------------------------------- */

const char* imu_status_string(imu_status s);
/* Detail of the last error on the calling thread (empty string if none). */
const char* imu_last_error(void);
/* Library version string. */
const char* imu_version(void);
/* Measurement hook for harnesses that time the GEMM inside a larger run: when
 * `before` and `after` are non-NULL, every later imu_unpacked_gemm and
 * imu_imunpack_matmul call on the calling thread records `before` on its stream
 * right before its first GEMM launch and `after` right after its last one
 * (when the call makes a single GEMM launch, the two are attached to that
 * launch as its start and stop events, so they add no marker to the stream).
 * Both NULL switches it off.  The events stay owned by the caller and must
 * belong to the device the calls run on.  Returns IMU_ERR_INVALID_ARG if only
 * one of the two is NULL. */
imu_status imu_set_gemm_events(hipEvent_t before, hipEvent_t after);

#ifdef __cplusplus
}
#endif
#endif /* IMUNPACK_H */
