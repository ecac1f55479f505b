// Internal definitions shared by the HIP kernels and the C-ABI host code of
// the IM-Unpack integer GEMM library (gfx950).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "imunpack.h"

namespace imu {

// ---------------------------------------------------------------------------
// constants
// ---------------------------------------------------------------------------
constexpr int kHistBins = 32768;    // 15-bit magnitude key of bf16 (and the top of fp32)
constexpr int kHistCoarse = 256;    // coarse counts (128 keys each) kept after the key bins
constexpr int kKPad = 128;          // every exponent segment of K' is padded to this many positions
constexpr int kMaxSeg = 64;         // room for 2*max_digits(2)-1 = 61 segments
constexpr int kStatusNonfinite = 1; // device status bits
constexpr int kStatusRange = 2;
constexpr int kStatusGreedy = 4;    // the greedy planner did not finish (cannot happen for consistent counts)
constexpr int kNumCand = 5;         // candidate depth maps: row, col, cr, rc, greedy
constexpr int kNumPairs = kNumCand * kNumCand;
constexpr int kGreedyMaxLines = 28672;  // rows + columns of an operand the greedy planner holds in LDS

__host__ __device__ inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
__host__ __device__ inline int64_t ceil_div(int64_t x, int64_t m) { return (x + m - 1) / m; }
__host__ __device__ inline int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
__host__ __device__ inline int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

// Largest number of base-2^(bits-1) digits of a code with |q| < 2^31.
__host__ __device__ inline int max_digits(int bits) { return (31 + bits - 2) / (bits - 1); }

// ---------------------------------------------------------------------------
// statistics buffer of one operand (one slot per batch entry)
// ---------------------------------------------------------------------------
struct StatsHeader {
  float alpha, r, s, kth;
  uint32_t maxkey;      // largest |x| as an fp32 bit pattern without sign
  int32_t status;       // kStatus* bits
  uint32_t sel_prefix;  // radix-select state: key prefix found so far
  uint32_t sel_rank;    // rank still to find inside that prefix (1-based)
  unsigned long long total;  // T: out-of-range codes
  uint32_t arrive;           // workgroups that finished the current pass (last-workgroup election, barriers)
  int32_t pad1;
  int64_t rows, cols;
};
static_assert(sizeof(StatsHeader) == 64, "stats header");

struct StatsLayout {
  int64_t R = 0, C = 0;
  int64_t row_oob = 0, col_oob = 0, row_maxdig = 0, col_maxdig = 0, cr_rowdig = 0, rc_coldig = 0;
  int64_t hist = 0, stride = 0;
};

inline StatsLayout stats_layout(int64_t R, int64_t C) {
  StatsLayout L;
  L.R = R;
  L.C = C;
  int64_t o = 256;
  auto take = [&](int64_t bytes) {
    int64_t at = o;
    o += round_up(bytes, 256);
    return at;
  };
  L.row_oob = take(4 * R);
  L.col_oob = take(4 * C);
  L.row_maxdig = take(4 * R);
  L.col_maxdig = take(4 * C);
  L.cr_rowdig = take(4 * R);
  L.rc_coldig = take(4 * C);
  L.hist = take(4 * (int64_t)(kHistBins + kHistCoarse));
  L.stride = o;
  return L;
}

// ---------------------------------------------------------------------------
// plan buffer
// ---------------------------------------------------------------------------
struct PlanHeader {
  int32_t choice_a, choice_b, status, n_seg;
  int64_t m_u, k_u, n_u;
  int64_t m_base, n_base, m_alloc, n_alloc;
  int64_t k_pad;
  int32_t lev_a, lev_b, emax, fmt;  // fmt: digit format of A' and B'^T (kDigitsInt8 / kDigitsFp6)
  int64_t pair[kNumPairs][3];
  int64_t seg_off[kMaxSeg + 1];
  int32_t seg_len[kMaxSeg];
  int64_t reserved[8];  // [0]: tag closing the host copy; [1]: the planner's arrival counter
  // B's columns in depth order (descending depth, then column index): slot j
  // of level w holds the column at position j of that order, for
  // j < lvcnt_b[w] (the columns deeper than w; lvcnt_b[0] = N), as B'^T row
  // lvbase_b[w] + j (lvbase_b[0] = 0).  b_perm: the order is not the identity.
  int32_t lvcnt_b[32];
  int64_t lvbase_b[32];
  int32_t b_perm, pad1;
};
constexpr int64_t kPlanHeaderStride = 2048;
static_assert(sizeof(PlanHeader) <= kPlanHeaderStride, "plan header");
// byte offsets read by the Python binding
static_assert(offsetof(PlanHeader, n_seg) == 12, "plan header layout");
static_assert(offsetof(PlanHeader, pair) == 96, "plan header layout");
static_assert(offsetof(PlanHeader, seg_off) == 696, "plan header layout");
static_assert(offsetof(PlanHeader, seg_len) == 1216, "plan header layout");

// The planner splits the lines (rows of A, columns of B, then k) into chunks
// of kPlanLines, one workgroup each; every workgroup keeps a record.
constexpr int kPlanLines = 512;
constexpr int kPlanTasks = 64;  // >= max levels and >= max segments
constexpr int kPlanSums = 2 * kNumCand + kNumPairs;  // M'[5], N'[5], K'[5][5]
struct PlanWgRecord {
  long long sum[kPlanSums + 1];  // candidate sizes of this chunk: M'[5], N'[5], K'[5][5] (+1: 16-byte size)
  int32_t cnt[kPlanTasks]; // per task (level or segment): entries of this chunk
  int32_t off[kPlanTasks]; // per task: entries of earlier chunks of the same kind
  int32_t mx[4];           // chunk maxima: depth (rows/cols) or dA, dB, dA + dB - 2 (k)
};
static_assert(sizeof(PlanWgRecord) % 16 == 0, "plan record");

struct PlanLayout {
  int64_t M = 0, K = 0, N = 0, batch = 0;
  int64_t pad_m = 0, pad_n = 0;  // base/extra boundary and allocation granularity
  int64_t levels = 0, segments = 0, m_alloc_max = 0, n_alloc_max = 0;
  int64_t headers_bytes = 0, entry_stride = 0;
  int64_t da_r = 0, da_c = 0, db_r = 0, db_c = 0, lvl_a = 0, lvl_b = 0, kpre = 0, amap = 0, bmap = 0;
  int64_t kmap = 0, kmap_max = 0;
  int64_t wg_a = 0, wg_b = 0, wg_k = 0;  // planner workgroups over A's rows, B's columns, k
  int64_t cand = 0, rec = 0;             // packed candidate depths; workgroup records
  int64_t gdep = 0;                      // greedy depths: A rows [M], A cols [K], B rows [K], B cols [N]
  int64_t total = 0;
};

// One entry of the K' position table: k | v << 20 | v' << 25 | lastA << 30 |
// lastB << 31, where v / v' are A's / B's inner index and lastA / lastB mark the
// last inner index of k (dA-1 / dB-1), the only one that carries digits at the
// unpacked levels u > 0.  kKmapPad marks zero padding at the end of an exponent
// segment.
constexpr uint32_t kKmapPad = 0xFFFFFFFFu;
constexpr int64_t kMaxK = (1ll << 20) - 2;
__host__ __device__ inline uint32_t kmap_pack(int64_t k, int v, int vp, int dA, int dB) {
  return (uint32_t)k | ((uint32_t)v << 20) | ((uint32_t)vp << 25) | ((uint32_t)(v == dA - 1) << 30) |
         ((uint32_t)(vp == dB - 1) << 31);
}

// Byte offset of element (row, p) of A' in MFMA fragment order: 1 KB blocks of
// 32 rows x 32 K' bytes, ordered by row block then K' block; inside a block,
// 16-byte half h of row r is lane r + 32 h.  Split into a row part and a K'
// part that add up.
__host__ __device__ inline int64_t frag_row_offset(int64_t row, int64_t k_pad) {
  return (row >> 5) * (k_pad >> 5) * 1024 + (row & 31) * 16;
}
__host__ __device__ inline int64_t frag_pos_offset(int64_t p) {
  return (p >> 5) * 1024 + ((p >> 4) & 1) * 512 + (p & 15);
}

// Digit formats of the unpacked operands.  int8: one byte per position.  fp6:
// the e2m3 code of each digit (|d| <= 7 is exact; sign in bit 5, magnitudes
// 0..7 as 0, 8, 16, 20, 24, 26, 28, 30), six bits per position, for bits <= 4.
// B'^T rows are then bit streams (position p at bits [6p, 6p + 6) of the
// row, 3/4 k_pad bytes); A' keeps the MFMA fragment order of the 32 x 64
// operand of v_mfma_f32_32x32x64_f8f6f4: 1536-byte blocks of 32 rows x 64
// positions, ordered by row block then position block, where lane
// l = row % 32 + 32 ((p % 64) / 32) holds 24 bytes with position p % 32 at bits
// [6 (p % 32), 6 (p % 32) + 6).
constexpr int kDigitsInt8 = 0, kDigitsFp6 = 1;
constexpr uint64_t kFp6Mag = 0x1E1C1A1814100800ull;  // byte m: e2m3 magnitude code of m
__host__ __device__ inline int64_t unpacked_row_bytes(int64_t k_pad, int fmt) {
  return fmt == kDigitsFp6 ? k_pad / 4 * 3 : k_pad;
}
__host__ __device__ inline int64_t frag6_row_offset(int64_t row, int64_t k_pad) {
  return (row >> 5) * (k_pad >> 6) * 1536 + (row & 31) * 24;
}
// position p a multiple of 16: the 12 bytes of positions p .. p + 15 in a lane
__host__ __device__ inline int64_t frag6_pos_offset(int64_t p) {
  return (p >> 6) * 1536 + ((p >> 5) & 1) * 768 + ((p >> 4) & 1) * 12;
}

// GEMM macro tile (rows of A' x rows of B'^T) used for a problem of this shape;
// the plan pads the base region and the allocation to these multiples.
struct GemmTile {
  int bm, bn;
};
inline GemmTile gemm_tile_for(int64_t M, int64_t N) {
  (void)M;
  (void)N;
  return GemmTile{256, 128};
}

inline PlanLayout plan_layout(int64_t M, int64_t K, int64_t N, int64_t batch, int bits) {
  PlanLayout L;
  L.M = M;
  L.K = K;
  L.N = N;
  L.batch = batch;
  GemmTile t = gemm_tile_for(M, N);
  L.pad_m = t.bm;
  L.pad_n = t.bn;
  int D = max_digits(bits);
  L.levels = D;
  L.segments = 2 * D - 1;
  L.m_alloc_max = round_up(M, L.pad_m) + (int64_t)(D - 1) * M + L.pad_m;
  L.n_alloc_max = round_up(N, L.pad_n) + (int64_t)(D - 1) * N + L.pad_n;
  L.headers_bytes = round_up(batch * kPlanHeaderStride, 256);
  int64_t o = 0;
  auto take = [&](int64_t bytes) {
    int64_t at = o;
    o += round_up(bytes, 256);
    return at;
  };
  L.da_r = take(4 * M);
  L.da_c = take(4 * K);
  L.db_r = take(4 * K);
  L.db_c = take(4 * N);
  L.lvl_a = take(4 * M * L.levels);
  L.lvl_b = take(4 * N * L.levels);
  L.kpre = take(4 * (K + 1) * L.segments);
  L.amap = take(4 * L.m_alloc_max);
  L.bmap = take(4 * L.n_alloc_max);
  L.kmap_max = K * (int64_t)D * D + kKPad * L.segments;
  L.kmap = take(4 * L.kmap_max);
  L.wg_a = ceil_div(M, kPlanLines);
  L.wg_b = ceil_div(N, kPlanLines);
  L.wg_k = ceil_div(K, kPlanLines);
  L.cand = take(4 * (M + N + 2 * K));
  L.gdep = take(4 * (M + N + 2 * K));
  L.rec = take((int64_t)sizeof(PlanWgRecord) * (L.wg_a + L.wg_b + L.wg_k));
  L.entry_stride = o;
  L.total = L.headers_bytes + batch * L.entry_stride;
  return L;
}

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
template <int DT>
struct Elem;
template <>
struct Elem<IMU_F32> {
  using T = float;
  static constexpr int bytes = 4;
};
template <>
struct Elem<IMU_BF16> {
  using T = uint16_t;
  static constexpr int bytes = 2;
};

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Magnitude key of |x| as an fp32 bit pattern (sign dropped).
__device__ inline uint32_t mag_key(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// Number of base-2^(BITS-1) digits of |q| (1 for |q| < 2^(BITS-1)).
template <int BITS>
__device__ inline int digit_count(uint32_t m) {
  int bl = 32 - __clz((int)m);  // bit length; 0 for m == 0
  return bl == 0 ? 1 : 1 + (bl - 1) / (BITS - 1);
}

// Digit count of the largest code of a line whose largest |x r| is f (f >= 0):
// rne(f), clamped to beta when clipping; without clipping f >= 2^31 is a
// range error reported elsewhere (1 is returned).
template <int BITS>
__device__ inline int line_digits(float f, int clip, int beta) {
  if (clip) return digit_count<BITS>(f >= (float)beta ? (uint32_t)beta : (uint32_t)__builtin_rintf(f));
  return f < 2147483648.0f ? digit_count<BITS>((uint32_t)__builtin_rintf(f)) : 1;
}

// RTN code of x: one binary32 product, round half to even.  Sets *bad when the
// code does not fit int32 (|x r| >= 2^31, including Inf/NaN products).
__device__ inline int32_t rtn_code(float x, float r, bool* bad) {
  float y = x * r;
  if (!(__builtin_fabsf(y) < 2147483648.0f)) {
    *bad = true;
    return 0;
  }
  return (int32_t)__builtin_rintf(y);
}

// Signed digit t of q: sign(q) * ((|q| >> ((BITS-1) t)) mod 2^(BITS-1)).
template <int BITS>
__device__ inline int32_t digit_of(int32_t q, int t) {
  uint32_t m = q < 0 ? (uint32_t)(-(int64_t)q) : (uint32_t)q;
  int sh = (BITS - 1) * t;
  uint32_t d = sh >= 32 ? 0u : ((m >> sh) & ((1u << (BITS - 1)) - 1u));
  return q < 0 ? -(int32_t)d : (int32_t)d;
}

// Reduction over the wave, returned as a scalar: butterflies inside each row
// of 16 lanes (quad swaps, half-row and row mirrors), then the row broadcasts
// leave the total in lane 63.  Rows the broadcast does not write receive 0,
// the identity of the sums and maxima used here.
#define IMU_DPP(v, ctrl, rows) (uint32_t) __builtin_amdgcn_update_dpp(0, (int)(v), ctrl, rows, 0xF, false)
template <typename Op>
__device__ inline uint32_t wave_reduce(uint32_t v, Op op) {
  v = op(v, IMU_DPP(v, 0xB1, 0xF));   // lane ^ 1
  v = op(v, IMU_DPP(v, 0x4E, 0xF));   // lane ^ 2
  v = op(v, IMU_DPP(v, 0x141, 0xF));  // mirror inside 8 lanes
  v = op(v, IMU_DPP(v, 0x140, 0xF));  // mirror inside 16 lanes
  v = op(v, IMU_DPP(v, 0x142, 0xA));  // lane 15 of rows 0, 2 into rows 1, 3
  v = op(v, IMU_DPP(v, 0x143, 0xC));  // lane 31 into rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
#undef IMU_DPP
struct AddU32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};
struct MaxU32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};

__device__ inline int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ inline int wave_max_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ inline uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

// ---------------------------------------------------------------------------
// launch argument blocks
// ---------------------------------------------------------------------------
struct StreamArgs {       // one operand traversed in stored orientation
  const void* x;
  int64_t srows, scols, ld, bstride;  // stored shape and strides (elements)
  int vec_ok;                          // 8-element vector loads are safe
  uint8_t* stats;
  int64_t stats_stride;
  // stored-row / stored-column arrays (logical rows or cols depending on layout)
  int64_t srow_oob, scol_oob, srow_maxdig, scol_maxdig, srow_res, scol_res, hist;
  int transposed;  // logical = stored^T
  int beta, p_num, p_den, gamma;
  int clip;        // codes clamped to [-beta, beta] (clipping quantizer)
};

// Work split of the streaming kernels: operand o owns workgroups
// [wg_begin, wg_begin + wgs_per_entry * batch).
struct QuantOp {
  StreamArgs s;
  int batch;
  int wg_begin, wgs_per_entry, rows_per_wg;
};
struct QuantJobs {
  QuantOp op[2];
  int nops;
};

}  // namespace imu
