// Host-side launchers of the HIP kernels (internal).
#pragma once

#include "common.h"

namespace imu {

// Byte offset of batch entry b inside the unpacked buffer of an operand: the
// entries before it, each (rows x k_pad) rounded up to 256 bytes.
__host__ __device__ inline int64_t unpacked_entry_bytes(const PlanHeader* h, int operand) {
  return round_up((operand == 0 ? h->m_alloc : h->n_alloc) * unpacked_row_bytes(h->k_pad, h->fmt), 256);
}

// quantize.hip
hipError_t launch_fill_u32(void* p, uint32_t v, int64_t nwords, hipStream_t s);
hipError_t launch_fill_2d(int32_t* p, int64_t rows, int64_t cols, int64_t ld, int batch, int64_t bstride, hipStream_t s);
hipError_t launch_hist(int dtype, QuantJobs J, int pass, int final_pass, hipStream_t s);
hipError_t launch_round_count(int dtype, int bits, QuantJobs J, int32_t* q0, int32_t* q1, hipStream_t s);
hipError_t launch_residual(int dtype, int bits, QuantJobs J, hipStream_t s);
// Row softmax of logits into the bf16 operand of J.op[0] (its first
// histogram pass included); the other passes follow as for any operand.
struct SoftmaxIn {
  const void* z;        // logits, rows x cols per batch entry (row-major)
  int64_t ld, bstride;  // elements
  int vec_ok;           // groups of 4 logits and of 4 outputs are aligned loads and stores
};
hipError_t launch_softmax_hist(int zdtype, const SoftmaxIn& in, QuantJobs J, hipStream_t s);

// plan.hip
struct PlanArgs {  // the plan headers must be zero when the planner starts (arrival counter)
  const uint8_t* stats_a;
  const uint8_t* stats_b;
  int64_t stats_stride_a, stats_stride_b;
  StatsLayout sla, slb;
  uint8_t* plan;
  PlanLayout pl;
  int gamma, strat_a, strat_b, bits;
  int fmt;                 // digit format the unpack and the GEMM will use (kDigitsInt8 / kDigitsFp6)
  uint8_t* host_hdr;       // pinned host copy of the headers (kPlanHeaderStride per entry), or null
  int64_t host_tag;        // written last into reserved[0] of each host copy
};
hipError_t launch_plan(const PlanArgs& a, hipEvent_t done, hipStream_t s);  // done: completes with the last launch, or null

// Greedy depths of the operands whose strategy is IMU_GREEDY (before the plan
// launches, after the headers are cleared).
struct GreedyOp {
  const void* x;
  int dtype, transposed;        // element (i, k) of the logical operand at transposed ? k*ld+i : i*ld+k
  int64_t ld, bstride;          // elements
  int64_t R, C;                 // logical shape (rows + cols <= kGreedyMaxLines)
  const uint8_t* stats;
  int64_t stats_stride, row_oob, col_oob;  // out-of-range counts of the logical rows / columns
  int64_t rows_off, cols_off;   // int32 offsets of its row / column depths in the plan's greedy area
};
struct GreedyArgs {
  GreedyOp op[2];
  int nops;
  uint8_t* plan;
  PlanLayout pl;
  int bits, clip, beta;
};
hipError_t launch_greedy(const GreedyArgs& g, int batch, hipStream_t s);

// unpack.hip
struct UnpackArgs {
  const void* x;
  int64_t bstride;
  int64_t so, sk;          // element strides of the outer line index and of k
  int64_t n_outer, K;      // outer lines (A: M rows, B: N cols) and inner length K
  int operand;             // 0 = A, 1 = B
  int vec_ok;              // 16-byte loads of 8 consecutive k are aligned (inner-contiguous only)
  const uint8_t* stats;
  int64_t stats_stride;
  const uint8_t* plan;
  PlanLayout pl;
  int8_t* out;                  // start of the unpacked buffer (all batch entries)
  int after_a;                  // 1: B' entries follow all A' entries of the buffer
  int beta, clip;               // clipping quantizer: codes clamped to [-beta, beta]
  int fmt;                      // digit format (kDigitsInt8 / kDigitsFp6): must match the plan's
  int64_t cap;                  // bytes available at out; entries that would not fit are skipped
};
// Operands of one dtype share a launch: launch_unpack takes one or two
// UnpackArgs (A then B) and launches them together when their staging shape
// matches (both inner-contiguous or both outer-contiguous), else one each.
hipError_t launch_unpack(int dtype, int bits, const UnpackArgs* ops, int nops, int batch, hipStream_t s);

// gemm.hip
struct GemmArgs {
  // one launch serves every batch entry (blockIdx.y); an entry's sizes come
  // from its plan header, its A' / B'^T from the sum of the earlier entries'
  // sizes (entries consecutive in a_u and in b_u)
  const int8_t* a_u;
  const int8_t* b_u;
  const uint8_t* plan;        // plan buffer (headers, then per-entry arrays)
  int64_t headers_bytes, entry_stride, amap_off, bmap_off;  // PlanLayout of the plan
  const uint8_t* stats_a;
  const uint8_t* stats_b;
  int64_t stats_stride_a, stats_stride_b;
  int32_t* c;
  float* out;
  int64_t ldc, cbs;           // C / out row stride and batch stride
  int64_t M, N;
  int bits;
  int mode;                   // 2: extra tiles of the entries folded by atomics; else base tiles (per
                              // entry: add to C after that pass, or store C, folding extra columns)
  int fold_cols;              // entries with extra columns only fold them in the base pass
  int group_m;                // tile rows per group of the workgroup -> tile order (power of two)
  int fmt;                    // digit format of every entry (kDigitsInt8 / kDigitsFp6)
  int tile_rows;              // rows of a tile (columns: 128): 256, or 128 for int8 digits
};
// tiles_x: the largest tile count of an entry for this mode; batch entries on
// blockIdx.y.  start / stop: events recorded as the launch starts / ends
// (attached to it), or null
// fold: the base pass also folds the extra columns of entries with extra
// columns only (required whenever such an entry is present)
hipError_t launch_gemm(const GemmArgs& a, int64_t tiles_x, int batch, bool fold, hipStream_t s,
                       hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

}  // namespace imu
