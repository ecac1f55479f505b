// Unpacking planner (gfx950): three short kernels over chunks of lines.
//
// Method: summary page "IM-Unpack: Training and Inference with Arbitrarily Low
// Precision Integers", "Approach" (row/column unpacking chosen per matrix from
// outlier counts) and the unpack-ratio rows of the "Measured effects" table
// (Mix beats every fixed row/column pairing).  The page gives no rule for Mix;
// the rule here keeps every candidate covering (d_r[i] + d_c[k] - 1 >= digits
// of every code) and picks the allowed pair with the smallest M'K'N', ties in
// A-major order ROW < COL < CR < RC.  All work is integer; the plan is a pure
// function of the per-line statistics, so it is deterministic.
//
// The lines (rows of A, columns of B, then k) are cut into chunks of
// kPlanLines, one workgroup per chunk and batch entry, in three launches:
// (1) plan_sums: the depth of every line under each of the 4 candidates (packed
//     bytes, kept for (2)) and the chunk's share of M'[4], N'[4], K'[4][4]; the
//     last workgroup to finish adds the shares up and picks the pair.
// (2) plan_counts: the chosen depth maps and, per chunk, the entries of every
//     task (each level of A's rows or B's columns: lines deeper than the level;
//     each exponent segment e of K': triples (k, v, v') with v + v' = e).
// (3) plan_write: from all chunks' counts, each workgroup derives the level
//     bases or padded segment offsets and its own offset in every task
//     (workgroup 0 also writes the header sizes), then scans its lines (a
//     thread owns 2 consecutive lines, one block-wide scan per batch of tasks)
//     and writes the level-major line maps, the per-segment prefixes over k and
//     the K' position table used by the unpack kernels.  B's columns are laid
//     out in depth order (descending depth, then index; a counting sort whose
//     classes are the depths), so the GEMM's tiles hold columns of one depth.
//     The header records the columns deeper than each level and each level's
//     first row.
// Records exchanged inside one launch are written with device-scope atomic
// stores (through the XCD-local L2) and read after a device-scope acquire; the
// counter that elects the last workgroup is a word of the plan header, which
// the caller clears before the first launch.
#include <hip/hip_ext.h>

#include "common.h"
#include "kernels.h"

namespace imu {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = kPlanLines / kThreads;  // lines per thread
constexpr int kMaxD = 32;                    // depths are clamped here (>= max_digits(2) + 1)
constexpr int kTaskBatch = 8;                // scan tasks per block-wide scan
static_assert(kPlanLines % kThreads == 0, "chunk split");
static_assert(kMaxSeg <= kPlanTasks && kMaxD <= kPlanTasks, "task slots");

__device__ inline void st_dev(long long* p, long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Elects the workgroup that finishes last.  Every thread's earlier stores have
// completed before the count is taken; the elected workgroup resets the
// counter for the next kernel (stream ordered).
__device__ inline bool last_to_arrive(uint32_t* counter, uint32_t total, int* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) *s_flag = atomicAdd(counter, 1u) == total - 1;
  __syncthreads();
  const bool last = *s_flag != 0;
  if (last && threadIdx.x == 0) *counter = 0;
  return last;
}

// Inclusive scan of a 64-bit value over the 64 lanes of a wave.
__device__ inline long long wave_incl_scan_i64(long long v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// Block-wide exclusive scans of kTaskBatch counters per thread at once.
__device__ inline void block_excl_scan_multi(const int* cnt, int* ex, int* tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl[kTaskBatch];
#pragma unroll
  for (int j = 0; j < kTaskBatch; ++j) incl[j] = cnt[j];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1)
#pragma unroll
    for (int j = 0; j < kTaskBatch; ++j) {
      const int v = __shfl_up(incl[j], o, 64);
      if (lane >= o) incl[j] += v;
    }
  __syncthreads();  // the previous call's readers are done with `tot`
  if (lane == 63)
#pragma unroll
    for (int j = 0; j < kTaskBatch; ++j) tot[wave * kTaskBatch + j] = incl[j];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kTaskBatch; ++j) {
    int base = 0;
    for (int w = 0; w < wave; ++w) base += tot[w * kTaskBatch + j];
    ex[j] = base + incl[j] - cnt[j];
  }
}

struct Src {
  const int32_t *row_oob, *col_oob, *row_max, *col_max, *cr_rowdig, *rc_coldig;
  long long T;
  int64_t R, C;
};

__device__ inline Src src_of(const uint8_t* st, const StatsLayout& L) {
  Src s;
  s.row_oob = reinterpret_cast<const int32_t*>(st + L.row_oob);
  s.col_oob = reinterpret_cast<const int32_t*>(st + L.col_oob);
  s.row_max = reinterpret_cast<const int32_t*>(st + L.row_maxdig);
  s.col_max = reinterpret_cast<const int32_t*>(st + L.col_maxdig);
  s.cr_rowdig = reinterpret_cast<const int32_t*>(st + L.cr_rowdig);
  s.rc_coldig = reinterpret_cast<const int32_t*>(st + L.rc_coldig);
  s.T = (long long)reinterpret_cast<const StatsHeader*>(st)->total;
  s.R = L.R;
  s.C = L.C;
  return s;
}

// Row depths of the 4 candidates (row, col, cr, rc) for row i, packed in bytes:
// ROW unpacks rows to their digit count, COL leaves rows whole, CR unpacks
// rows to the digit count of their residual after the heavy columns, RC
// unpacks only heavy rows (out-of-range count x C above gamma T).
__device__ inline uint32_t row_depths(const Src& s, int64_t i, int gamma) {
  const int mx = min(max(1, s.row_max[i]), kMaxD);
  const int cr = min(max(1, s.cr_rowdig[i]), kMaxD);
  const int rc = (long long)s.row_oob[i] * s.R > gamma * s.T ? mx : 1;
  return (uint32_t)mx | 1u << 8 | (uint32_t)cr << 16 | (uint32_t)rc << 24;
}
// Column depths of the 4 candidates for column k, packed in bytes (mirror image).
__device__ inline uint32_t col_depths(const Src& s, int64_t k, int gamma) {
  const int mx = min(max(1, s.col_max[k]), kMaxD);
  const int cr = (long long)s.col_oob[k] * s.C > gamma * s.T ? mx : 1;
  const int rc = min(max(1, s.rc_coldig[k]), kMaxD);
  return 1u | (uint32_t)mx << 8 | (uint32_t)cr << 16 | (uint32_t)rc << 24;
}
__device__ inline int pick(uint32_t packed, int c) { return (packed >> (8 * c)) & 0xFF; }

__device__ inline bool allowed(int strat, int c) {
  return (strat == IMU_MIX && c < 4) || (strat == IMU_ROW && c == 0) || (strat == IMU_COL && c == 1) ||
         (strat == IMU_GREEDY && c == 4);
}
// Depth of candidate c of a line: packed bytes for row..rc, the greedy depth g for c = 4.
__device__ inline int dep(uint32_t packed, int g, int c) { return c == 4 ? g : pick(packed, c); }

// number of triples (k, v, v') with v + v' = e, v < dA, v' < dB
__device__ inline int seg_count(int dA, int dB, int e) {
  const int lo = max(0, e - (dB - 1)), hi = min(dA - 1, e);
  return max(0, hi - lo + 1);
}

// Chunk of workgroup w: kind 0 = rows of A, 1 = columns of B, 2 = k.
struct Chunk {
  int kind;
  int64_t first, n;  // first line and number of lines of this kind
  int64_t rank;      // chunk index within its kind
};
__device__ inline Chunk chunk_of(const PlanLayout& L, int64_t w) {
  Chunk c;
  if (w < L.wg_a) {
    c.kind = 0;
    c.rank = w;
    c.n = L.M;
  } else if (w < L.wg_a + L.wg_b) {
    c.kind = 1;
    c.rank = w - L.wg_a;
    c.n = L.N;
  } else {
    c.kind = 2;
    c.rank = w - L.wg_a - L.wg_b;
    c.n = L.K;
  }
  c.first = c.rank * kPlanLines;
  return c;
}

struct Entry {  // one batch entry's plan buffers
  PlanHeader* ph;
  int32_t *da_r, *da_c, *db_r, *db_c, *lvl_a, *lvl_b, *amap, *bmap, *kpre;
  uint32_t *kmap, *cand;
  int32_t* gdep;  // greedy depths: A rows [M], A cols [K], B rows [K], B cols [N]
  PlanWgRecord* rec;
};
__device__ inline Entry entry_of(const PlanArgs& a, int b) {
  const PlanLayout& L = a.pl;
  uint8_t* e = a.plan + L.headers_bytes + b * L.entry_stride;
  Entry x;
  x.ph = reinterpret_cast<PlanHeader*>(a.plan + b * kPlanHeaderStride);
  x.da_r = reinterpret_cast<int32_t*>(e + L.da_r);
  x.da_c = reinterpret_cast<int32_t*>(e + L.da_c);
  x.db_r = reinterpret_cast<int32_t*>(e + L.db_r);
  x.db_c = reinterpret_cast<int32_t*>(e + L.db_c);
  x.lvl_a = reinterpret_cast<int32_t*>(e + L.lvl_a);
  x.lvl_b = reinterpret_cast<int32_t*>(e + L.lvl_b);
  x.amap = reinterpret_cast<int32_t*>(e + L.amap);
  x.bmap = reinterpret_cast<int32_t*>(e + L.bmap);
  x.kpre = reinterpret_cast<int32_t*>(e + L.kpre);
  x.kmap = reinterpret_cast<uint32_t*>(e + L.kmap);
  x.cand = reinterpret_cast<uint32_t*>(e + L.cand);  // [M] A rows, [N] B cols, [K] A cols, [K] B rows
  x.rec = reinterpret_cast<PlanWgRecord*>(e + L.rec);
  x.gdep = reinterpret_cast<int32_t*>(e + L.gdep);
  return x;
}

// Arrival counter of the planner's first launch: a word of the entry's own
// plan header (the statistics may be shared, read-only, between calls).  The
// caller clears the headers before the planner runs.
__device__ inline uint32_t* arrive_counter(const PlanArgs& a, int b) {
  return reinterpret_cast<uint32_t*>(&reinterpret_cast<PlanHeader*>(a.plan + b * kPlanHeaderStride)->reserved[1]);
}

// Shared memory of a planner workgroup, all phases.
struct PlanShared {
  long long red[kThreads / kPlanSums][kPlanSums];
  int red32[kWaves][kNumPairs];
  long long tot[kPlanSums];
  int choice[2];
  int flag;
  int hist[(kMaxD + 1) * (kMaxD + 1)];  // depth histogram (rows/cols) or (dA, dB) pairs (k)
  int smax[kWaves][4];
  long long task_tot[3][kPlanTasks];    // per kind and task: entries of all chunks
  int off[kPlanTasks];                  // this chunk's offset in every task of its kind
  long long base[kPlanTasks];           // level bases (rows/cols) or segment offsets (k)
  long long segoff[kMaxSeg + 1];        // padded segment offsets
  long long end_rows[2];                // first row past the last level: A rows, B columns
  long long m_base, n_base, m_alloc, n_alloc;
  int lev[2], nseg;
  int scan_tot[kWaves * kTaskBatch];
};

// --- (1) candidate depths of a chunk's lines and its share of the sizes -----
__device__ void phase_sums(const PlanArgs& a, int b, int64_t w, PlanShared& S) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const PlanLayout& L = a.pl;
  const Entry E = entry_of(a, b);
  const Src A = src_of(a.stats_a + b * a.stats_stride_a, a.sla);
  const Src B = src_of(a.stats_b + b * a.stats_stride_b, a.slb);
  const Chunk c = chunk_of(L, w);
  const int gamma = a.gamma;
  if (w == 0 && t == 0)  // status of this plan (and of the greedy planner); later failures are OR-ed in
    E.ph->status = (int32_t)(reinterpret_cast<const StatsHeader*>(a.stats_a + b * a.stats_stride_a)->status |
                             reinterpret_cast<const StatsHeader*>(a.stats_b + b * a.stats_stride_b)->status |
                             (int32_t)E.ph->reserved[2]);
  // a chunk's shares fit 32 bits (kPlanLines lines, depths <= 32); only its kind's
  // 5 (rows, columns) or 25 (k) sums are non-zero
  int acc[kNumPairs];
#pragma unroll
  for (int j = 0; j < kNumPairs; ++j) acc[j] = 0;
  uint32_t dx[kPer], dy[kPer];
  int gx[kPer], gy[kPer];  // greedy depths (1 when that operand's strategy is not greedy)
  const bool ga = a.strat_a == IMU_GREEDY, gb = a.strat_b == IMU_GREEDY;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {  // clamped indices: all loads issued before use
    const int64_t i = min64(c.first + t + (int64_t)j * kThreads, c.n - 1);
    gx[j] = gy[j] = 1;
    if (c.kind == 0) {
      dx[j] = row_depths(A, i, gamma);
      if (ga) gx[j] = E.gdep[i];
    } else if (c.kind == 1) {
      dx[j] = col_depths(B, i, gamma);
      if (gb) gx[j] = E.gdep[L.M + 2 * L.K + i];
    } else {
      dx[j] = col_depths(A, i, gamma);
      dy[j] = row_depths(B, i, gamma);
      if (ga) gx[j] = E.gdep[L.M + i];
      if (gb) gy[j] = E.gdep[L.M + L.K + i];
    }
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t i = c.first + t + (int64_t)j * kThreads;
    if (i >= c.n) continue;
    if (c.kind == 0) {
      E.cand[i] = dx[j];
#pragma unroll
      for (int q = 0; q < kNumCand; ++q) acc[q] += dep(dx[j], gx[j], q);
    } else if (c.kind == 1) {
      E.cand[L.M + i] = dx[j];
#pragma unroll
      for (int q = 0; q < kNumCand; ++q) acc[q] += dep(dx[j], gx[j], q);
    } else {
      E.cand[L.M + L.N + i] = dx[j];
      E.cand[L.M + L.N + L.K + i] = dy[j];
#pragma unroll
      for (int ca = 0; ca < kNumCand; ++ca)
#pragma unroll
        for (int cb = 0; cb < kNumCand; ++cb)
          acc[ca * kNumCand + cb] += dep(dx[j], gx[j], ca) * dep(dy[j], gy[j], cb);
    }
  }
  const int nsum = c.kind == 2 ? kNumPairs : kNumCand;  // uniform over the workgroup
#pragma unroll
  for (int j = 0; j < kNumPairs; ++j) {
    if (j < nsum) {
      const int v = wave_sum_i32(acc[j]);
      if (lane == 0) S.red32[wave][j] = v;
    }
  }
  __syncthreads();
  if (t < kPlanSums) {  // record slots: [0,5) A rows, [5,10) B columns, [10,35) k pairs
    const int first = c.kind == 0 ? 0 : c.kind == 1 ? kNumCand : 2 * kNumCand;
    long long v = 0;
    if (t >= first && t < first + nsum)
      for (int q = 0; q < kWaves; ++q) v += S.red32[q][t - first];
    st_dev(&E.rec[w].sum[t], v);
  }
}

// Totals of all chunks' shares and the joint choice (S.choice).  With
// write_header the workgroup also writes the choice and every pair's sizes.
__device__ void choose(const PlanArgs& a, int b, int64_t G, bool write_header, PlanShared& S) {
  const int t = threadIdx.x;
  const Entry E = entry_of(a, b);
  // the records were written through to memory before the election; after an
  // acquire at device scope (drops stale cached lines) plain loads see them
  // and can all be in flight at once
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  constexpr int kGroups = kThreads / kPlanSums;  // thread t adds value t % 35 of records t / 35 (mod kGroups)
  constexpr int kLoads = 8;                      // loads in flight per thread: 56 records a round
  if (t < kGroups * kPlanSums) {
    const int j = t % kPlanSums, g = t / kPlanSums;
    long long v = 0;
    for (int64_t q0 = g; q0 < G; q0 += kLoads * kGroups) {
      long long w[kLoads];
#pragma unroll
      for (int i = 0; i < kLoads; ++i) w[i] = E.rec[min64(q0 + i * kGroups, G - 1)].sum[j];  // unconditional
#pragma unroll
      for (int i = 0; i < kLoads; ++i) v += q0 + i * kGroups < G ? w[i] : 0;
    }
    S.red[g][j] = v;
  }
  __syncthreads();
  if (t < kPlanSums) {
    long long v = 0;
    for (int g = 0; g < kGroups; ++g) v += S.red[g][t];
    S.tot[t] = v;
  }
  __syncthreads();
  // cost of pair (ca, cb) = M'[ca] K'[ca][cb] N'[cb] < 2^88: M'K' < 2^59 is
  // exact in 64 bits (M' < 2^29, K' < 2^30), its product with N' < 2^29 is
  // kept as (high, low) 64-bit words
  if (t < 64) {  // wave 0: lane q < 25 is pair (q / 5, q % 5)
    const int q = t, ca = q / kNumCand, cb = q % kNumCand;
    const bool ok = q < kNumPairs && allowed(a.strat_a, ca) && allowed(a.strat_b, cb);
    unsigned long long hi = ~0ull, lo = ~0ull;
    if (ok) {
      const unsigned long long mk = (unsigned long long)S.tot[ca] * (unsigned long long)S.tot[2 * kNumCand + q];
      const unsigned long long nu = (unsigned long long)S.tot[kNumCand + cb];
      hi = __umul64hi(mk, nu);
      lo = mk * nu;
    }
    if (write_header && q < kNumPairs) {
      E.ph->pair[q][0] = ok ? S.tot[ca] : -1;
      E.ph->pair[q][1] = ok ? S.tot[2 * kNumCand + q] : -1;
      E.ph->pair[q][2] = ok ? S.tot[kNumCand + cb] : -1;
    }
    // smallest cost over lanes 0..31 (the 25 pairs), ties to the first pair in
    // A-major order: butterflies on (not allowed, high, low, index)
    int best = ok ? q : 64 + q;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      const unsigned long long ohi = __shfl_xor(hi, o, 64), olo = __shfl_xor(lo, o, 64);
      const int obest = __shfl_xor(best, o, 64);
      const bool take = ohi < hi || (ohi == hi && (olo < lo || (olo == lo && obest < best)));
      if (take) {
        hi = ohi;
        lo = olo;
        best = obest;
      }
    }
    if (q == 0) {
      const int best_a = (best & 63) / kNumCand, best_b = (best & 63) % kNumCand;
      S.choice[0] = best_a;
      S.choice[1] = best_b;
      if (write_header) {
        PlanHeader* ph = E.ph;
        ph->choice_a = best_a;
        ph->choice_b = best_b;
        ph->m_u = S.tot[best_a];
        ph->k_u = S.tot[2 * kNumCand + (best & 63)];
        ph->n_u = S.tot[kNumCand + best_b];
      }
    }
  }
  __syncthreads();
}

// --- (2) chosen depth maps and a chunk's entries per task -------------------
__device__ void phase_counts(const PlanArgs& a, int b, int64_t w, int ca, int cb, PlanShared& S) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const PlanLayout& L = a.pl;
  const Entry E = entry_of(a, b);
  const Chunk c = chunk_of(L, w);
  for (int i = t; i < (kMaxD + 1) * (kMaxD + 1); i += kThreads) S.hist[i] = 0;
  __syncthreads();
  uint32_t dx[kPer], dy[kPer];
  int gx[kPer], gy[kPer];  // greedy depths when the chosen candidate is the greedy one
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t i = min64(c.first + t + (int64_t)j * kThreads, c.n - 1);
    gx[j] = gy[j] = 1;
    if (c.kind == 0) {
      dx[j] = E.cand[i];
      if (ca == 4) gx[j] = E.gdep[i];
    } else if (c.kind == 1) {
      dx[j] = E.cand[L.M + i];
      if (cb == 4) gx[j] = E.gdep[L.M + 2 * L.K + i];
    } else {
      dx[j] = E.cand[L.M + L.N + i];
      dy[j] = E.cand[L.M + L.N + L.K + i];
      if (ca == 4) gx[j] = E.gdep[L.M + i];
      if (cb == 4) gy[j] = E.gdep[L.M + L.K + i];
    }
  }
  int m0 = 1, m1 = 1, m2 = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t i = c.first + t + (int64_t)j * kThreads;
    if (i >= c.n) continue;
    if (c.kind < 2) {
      const int d = dep(dx[j], gx[j], c.kind == 0 ? ca : cb);
      (c.kind == 0 ? E.da_r : E.db_c)[i] = d;
      m0 = max(m0, d);
      atomicAdd(&S.hist[d], 1);
    } else {
      const int x = dep(dx[j], gx[j], ca), y = dep(dy[j], gy[j], cb);
      E.da_c[i] = x;
      E.db_r[i] = y;
      m0 = max(m0, x);
      m1 = max(m1, y);
      m2 = max(m2, x + y - 2);
      atomicAdd(&S.hist[x * (kMaxD + 1) + y], 1);
    }
  }
  m0 = wave_max_i32(m0);
  m1 = wave_max_i32(m1);
  m2 = wave_max_i32(m2);
  if (lane == 0) {
    S.smax[wave][0] = m0;
    S.smax[wave][1] = m1;
    S.smax[wave][2] = m2;
  }
  __syncthreads();
  int x_hi = 1, y_hi = 1;
  for (int q = 0; q < kWaves; ++q) {
    x_hi = max(x_hi, S.smax[q][0]);
    y_hi = max(y_hi, S.smax[q][1]);
  }
  PlanWgRecord* my = E.rec + w;
  if (t < kPlanTasks) {  // task counts of this chunk
    int v = 0;
    if (c.kind < 2) {
      for (int d = t + 1; d <= x_hi; ++d) v += S.hist[d];  // lines with depth > t
    } else {
      for (int x = 1; x <= x_hi; ++x)
        for (int y = 1; y <= y_hi; ++y) v += S.hist[x * (kMaxD + 1) + y] * seg_count(x, y, t);
    }
    st_dev(&my->cnt[t], v);
  }
  if (t < 3) {
    int v = t == 2 ? 0 : 1;
    for (int q = 0; q < kWaves; ++q) v = max(v, S.smax[q][t]);
    st_dev(&my->mx[t], v);
  }
}

// Levels, segment count, per-task totals of every kind and this chunk's offset
// in each task of its kind, from all chunks' records (written by the previous
// launch); level bases (rows and
// columns) or padded segment offsets (k).  With write_header the workgroup
// also writes the header sizes.
__device__ void layout(const PlanArgs& a, int b, int64_t w, bool write_header, PlanShared& S) {
  const int t = threadIdx.x;
  const PlanLayout& L = a.pl;
  const Entry E = entry_of(a, b);
  const Chunk me = chunk_of(L, w);
  // first record and number of records of a kind (selects, not an indexed
  // array, which would live in scratch memory)
  auto wk0 = [&](int kind) { return kind == 0 ? (int64_t)0 : kind == 1 ? L.wg_a : L.wg_a + L.wg_b; };
  auto wkn = [&](int kind) { return kind == 0 ? L.wg_a : kind == 1 ? L.wg_b : L.wg_k; };
  // records written by the previous launch, read kBatch chunks at a time with
  // all loads in flight (a plain loop would wait for each in turn; the loads
  // are unconditional, at clamped indices, so that none waits behind a branch)
  constexpr int kBatch = 16;
  for (int job = t; job < 3 * kPlanTasks; job += kThreads) {
    const int kind = job / kPlanTasks, task = job % kPlanTasks;
    const int64_t n0 = wk0(kind), nk = wkn(kind);
    long long run = 0;
    for (int64_t r0 = 0; r0 < nk; r0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) v[j] = E.rec[n0 + min64(r0 + j, nk - 1)].cnt[task];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (kind == me.kind && r0 + j == me.rank) S.off[task] = (int)run;
        run += r0 + j < nk ? v[j] : 0;
      }
    }
    S.task_tot[kind][task] = run;
  }
  if (t < 3) {  // lev_a (A rows), lev_b (B columns), emax (k)
    const int kind = t, field = t == 2 ? 2 : 0;
    const int64_t n0 = wk0(kind), nk = wkn(kind);
    int m = t == 2 ? 0 : 1;
    for (int64_t r0 = 0; r0 < nk; r0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) v[j] = E.rec[n0 + min64(r0 + j, nk - 1)].mx[field];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) m = max(m, v[j]);  // a clamped index repeats a record
    }
    if (t < 2) S.lev[t] = min(m, (int)L.levels);
    else S.nseg = min(m, (int)L.segments - 1) + 1;
  }
  __syncthreads();
  if (t < 64) {  // wave 0, lane = task: the prefixes below are wave scans
    const int lane = t;
    const long long m_base = round_up(L.M, L.pad_m), n_base = round_up(L.N, L.pad_n);
    // level bases: base[u] = (padded base) + entries of the levels 1..u-1
    long long base_k[2], end_k[2];
#pragma unroll
    for (int kind = 0; kind < 2; ++kind) {
      const long long v = lane >= 1 && lane < S.lev[kind] ? S.task_tot[kind][lane] : 0;
      const long long incl = wave_incl_scan_i64(v);
      base_k[kind] = (kind == 0 ? m_base : n_base) + incl - v;
      end_k[kind] = (kind == 0 ? m_base : n_base) + __shfl(incl, 63, 64);
    }
    // segment offsets: each segment padded to the K step (lanes from nseg on
    // hold the total, so segoff[nseg] = k_pad)
    const long long seg = lane < S.nseg ? round_up(S.task_tot[2][lane], kKPad) : 0;
    const long long sincl = wave_incl_scan_i64(seg);
    const long long k_pad = __shfl(sincl, 63, 64);
    S.segoff[lane] = sincl - seg;
    if (lane == 0) {
      S.m_base = m_base;
      S.n_base = n_base;
      S.end_rows[0] = end_k[0];
      S.end_rows[1] = end_k[1];
      S.m_alloc = round_up(end_k[0], L.pad_m);
      S.n_alloc = round_up(end_k[1], L.pad_n);
    }
    if (me.kind < 2) S.base[lane] = lane == 0 ? 0 : (me.kind == 0 ? base_k[0] : base_k[1]);
    else S.base[lane] = sincl - seg;
    if (write_header) {
      // the layout fields, into the header and into the host's copy (if any),
      // which also gets the fields of the earlier launches: the host then waits
      // for this launch alone, with no copy queued between it and the unpack
      PlanHeader* hh = a.host_hdr ? reinterpret_cast<PlanHeader*>(a.host_hdr + b * kPlanHeaderStride) : nullptr;
      // put(h, st): every layout field, stored through st (plain stores for the
      // device header, system-scope stores, which write through the caches,
      // for the host copy)
      auto put = [&](PlanHeader* h, auto st) __attribute__((always_inline)) {
        if (lane < S.nseg) {
          st(&h->seg_off[lane], (int64_t)(sincl - seg));
          st(&h->seg_len[lane], (int32_t)S.task_tot[2][lane]);
        }
        if (lane == 0) {
          st(&h->seg_off[S.nseg], (int64_t)k_pad);
          st(&h->n_seg, (int32_t)S.nseg);
          st(&h->k_pad, (int64_t)k_pad);
          st(&h->m_base, (int64_t)m_base);
          st(&h->n_base, (int64_t)n_base);
          st(&h->m_alloc, (int64_t)round_up(end_k[0], L.pad_m));
          st(&h->n_alloc, (int64_t)round_up(end_k[1], L.pad_n));
          st(&h->lev_a, (int32_t)S.lev[0]);
          st(&h->lev_b, (int32_t)S.lev[1]);
          st(&h->emax, (int32_t)(S.nseg - 1));
          st(&h->fmt, (int32_t)a.fmt);
        }
      };
      put(E.ph, [](auto* p, auto v) __attribute__((always_inline)) { *p = v; });
      // B's depth order (device header only: the GEMM reads it): lines deeper
      // than each level and the first B'^T row of each level; the order is a
      // permutation unless every column has the same depth
      if (lane < 32) {
        E.ph->lvcnt_b[lane] = (int32_t)S.task_tot[1][lane];
        E.ph->lvbase_b[lane] = lane == 0 ? 0 : (int64_t)base_k[1];
      }
      {
        const long long exact = lane >= 1 && lane <= S.lev[1] ? S.task_tot[1][lane - 1] - S.task_tot[1][lane] : 0;
        const bool mixed = __ballot(exact > 0 && exact < L.N) != 0;
        if (lane == 0) E.ph->b_perm = mixed ? 1 : 0;
      }
      if (hh) {
        // fields of the earlier launches, all loaded before the first store
        // (a load's wait would also wait for the slow host stores before it)
        const PlanHeader* ph = E.ph;
        int64_t pr[3] = {0, 0, 0}, mu = 0, ku = 0, nu = 0;
        int32_t ca = 0, cb = 0, stt = 0;
        if (lane < kNumPairs) {
          pr[0] = ph->pair[lane][0];
          pr[1] = ph->pair[lane][1];
          pr[2] = ph->pair[lane][2];
        }
        if (lane == 0) {
          ca = ph->choice_a;
          cb = ph->choice_b;
          stt = ph->status;
          mu = ph->m_u;
          ku = ph->k_u;
          nu = ph->n_u;
        }
        auto sys = [](auto* p, auto v) __attribute__((always_inline)) {
          __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        };
        put(hh, sys);
        if (lane < kNumPairs) {
          sys(&hh->pair[lane][0], pr[0]);
          sys(&hh->pair[lane][1], pr[1]);
          sys(&hh->pair[lane][2], pr[2]);
        }
        if (lane == 0) {
          sys(&hh->choice_a, ca);
          sys(&hh->choice_b, cb);
          sys(&hh->status, stt);
          sys(&hh->m_u, mu);
          sys(&hh->k_u, ku);
          sys(&hh->n_u, nu);
        }
        // the tag follows at the end of the workgroup (host_tag_store)
      }
    }
  }
  __syncthreads();
}

// --- (3) positions of a chunk's lines; workgroup 0 also writes the padding --
__device__ void phase_write(const PlanArgs& a, int b, int64_t w, PlanShared& S) {
  const int t = threadIdx.x;
  const PlanLayout& L = a.pl;
  const Entry E = entry_of(a, b);
  const Chunk c = chunk_of(L, w);
  const int ntasks = c.kind == 0 ? S.lev[0] : c.kind == 1 ? S.lev[1] : S.nseg;
  const int64_t i0 = min64(c.first + (int64_t)t * kPer, c.n), i1 = min64(i0 + kPer, c.n);
  int dA[kPer], dB[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t i = min64(i0 + j, c.n - 1);
    if (c.kind == 0) dA[j] = E.da_r[i];
    else if (c.kind == 1) dA[j] = E.db_c[i];
    else {
      dA[j] = E.da_c[i];
      dB[j] = E.db_r[i];
    }
  }
  const int nl = (int)(i1 - i0);
  if (c.kind == 1) {
    // B's columns in depth order: descending depth, then column index.  Task t
    // is the class of depth t + 1; a column of depth d sits at position
    // (columns deeper than d) + (earlier chunks' columns of depth d) + (its rank
    // in this chunk's class), and level u < d of it at B'^T row base[u] + that
    // position (base[0] = 0): the columns deeper than u lead the order.
    for (int tb = 0; tb < ntasks; tb += kTaskBatch) {
      int cnt[kTaskBatch], ex[kTaskBatch];
#pragma unroll
      for (int j = 0; j < kTaskBatch; ++j) {
        int v = 0;
#pragma unroll
        for (int l = 0; l < kPer; ++l)
          if (l < nl) v += dA[l] == tb + j + 1;
        cnt[j] = v;
      }
      block_excl_scan_multi(cnt, ex, S.scan_tot);
#pragma unroll
      for (int j = 0; j < kTaskBatch; ++j) {
        const int d = tb + j + 1;
        if (d > ntasks) continue;
        long long pos = S.task_tot[1][d] + (S.off[d - 1] - S.off[d]) + ex[j];
#pragma unroll
        for (int l = 0; l < kPer; ++l) {
          if (l >= nl || dA[l] != d) continue;
          const int64_t i = i0 + l;
          for (int u = 0; u < ntasks; ++u) {
            const long long row = u == 0 ? pos : S.base[u] + pos;
            E.lvl_b[(int64_t)u * c.n + i] = u < d ? (int32_t)row : -1;
            if (u < d) E.bmap[row] = (int32_t)(i | ((int64_t)u << 24));
          }
          ++pos;
        }
      }
    }
  }
  for (int tb = 0; tb < (c.kind == 1 ? 0 : ntasks); tb += kTaskBatch) {
    int cnt[kTaskBatch], ex[kTaskBatch];
#pragma unroll
    for (int j = 0; j < kTaskBatch; ++j) {
      int v = 0;
#pragma unroll
      for (int l = 0; l < kPer; ++l)
        if (l < nl) v += c.kind < 2 ? (dA[l] > tb + j) : seg_count(dA[l], dB[l], tb + j);
      cnt[j] = v;
    }
    block_excl_scan_multi(cnt, ex, S.scan_tot);
#pragma unroll
    for (int j = 0; j < kTaskBatch; ++j) {
      const int task = tb + j;
      if (task >= ntasks) continue;
      long long pos = ex[j] + S.off[task];  // position inside the task
#pragma unroll
      for (int l = 0; l < kPer; ++l) {
        if (l >= nl) continue;
        const int64_t i = i0 + l;
        if (c.kind < 2) {
          const bool live = dA[l] > task;
          const long long p = S.base[task] + pos;
          (c.kind == 0 ? E.lvl_a : E.lvl_b)[(int64_t)task * c.n + i] = live ? (int32_t)p : -1;
          if (live) (c.kind == 0 ? E.amap : E.bmap)[p] = (int32_t)(i | ((int64_t)task << 24));
          pos += live;
        } else {
          const int cnt_l = seg_count(dA[l], dB[l], task);
          E.kpre[(int64_t)task * (L.K + 1) + i] = (int32_t)pos;
          uint32_t* km = E.kmap + S.base[task] + pos;
          const int lo = max(0, task - (dB[l] - 1));
          for (int v = 0; v < cnt_l; ++v) km[v] = kmap_pack(i, lo + v, task - lo - v, dA[l], dB[l]);
          pos += cnt_l;
        }
      }
    }
  }
  if (w == 0) {
    // rows between M and the padded base and after the last level up to the
    // allocation, zero entries at the end of every segment, and the
    // per-segment totals at kpre[s][K]
    for (int64_t r = L.M + t; r < S.m_base; r += kThreads) E.amap[r] = -1;
    for (int64_t r = S.end_rows[0] + t; r < S.m_alloc; r += kThreads) E.amap[r] = -1;
    for (int64_t r = L.N + t; r < S.n_base; r += kThreads) E.bmap[r] = -1;
    for (int64_t r = S.end_rows[1] + t; r < S.n_alloc; r += kThreads) E.bmap[r] = -1;
    for (int q = 0; q < S.nseg; ++q) {
      const int64_t p0 = S.segoff[q] + S.task_tot[2][q], p1 = S.segoff[q + 1];
      for (int64_t p = p0 + t; p < p1; p += kThreads) E.kmap[p] = kKmapPad;
    }
    if (t < S.nseg) E.kpre[(int64_t)t * (L.K + 1) + L.K] = (int32_t)S.task_tot[2][t];
  }
}

// --- greedy line-at-a-time depths (strategy IMU_GREEDY) ---------------------
// One workgroup per (operand, batch entry).  All depths start at 1, so the
// uncovered codes of each line start as its out-of-range count.  Each step
// raises the line with the most uncovered codes (rows first, then the lowest
// index, on equal counts: the largest key count << 32 | ~line) by one level;
// a row raised to depth d covers exactly its codes with n = d + d_c[k] - 1,
// whose digit counts are recomputed from the operand (the RTN code of x r), so
// only the crossing columns' counts change.  A line stops being chosen once its
// depth reaches its largest digit count, so at most (R + C) * 32 steps run.
constexpr int kGreedyThreads = 1024;
__global__ __launch_bounds__(kGreedyThreads) void greedy_kernel(GreedyArgs g) {
  __shared__ int32_t s_cnt[kGreedyMaxLines];
  __shared__ uint8_t s_dep[kGreedyMaxLines];
  __shared__ unsigned long long s_key[kGreedyThreads / 64];
  __shared__ int32_t s_sum[kGreedyThreads / 64];
  __shared__ unsigned long long s_best;
  const GreedyOp& o = g.op[blockIdx.x];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t R = o.R, C = o.C, NL = R + C;
  const uint8_t* st = o.stats + b * o.stats_stride;
  const float r = reinterpret_cast<const StatsHeader*>(st)->r;
  const int32_t* row_oob = reinterpret_cast<const int32_t*>(st + o.row_oob);
  const int32_t* col_oob = reinterpret_cast<const int32_t*>(st + o.col_oob);
  const uint8_t* xb = static_cast<const uint8_t*>(o.x) + b * o.bstride * (o.dtype == IMU_F32 ? 4 : 2);
  for (int64_t l = tid; l < NL; l += kGreedyThreads) {
    s_dep[l] = 1;
    s_cnt[l] = l < R ? row_oob[l] : col_oob[l - R];
  }
  // digit count of the code of logical element (i, k)
  auto ndig = [&](int64_t i, int64_t k) __attribute__((always_inline)) {
    const int64_t at = o.transposed ? k * o.ld + i : i * o.ld + k;
    const float v = o.dtype == IMU_F32 ? reinterpret_cast<const float*>(xb)[at]
                                       : bf16_to_f32(reinterpret_cast<const uint16_t*>(xb)[at]);
    const float y = __builtin_fabsf(v * r);
    const uint32_t m = g.clip ? (uint32_t)__builtin_rintf(__builtin_fminf(y, (float)g.beta))
                              : (y < 2147483648.0f ? (uint32_t)__builtin_rintf(y) : 0x7FFFFFFFu);
    const int bl = 32 - __clz((int)m);
    return bl == 0 ? 1 : 1 + (bl - 1) / (g.bits - 1);
  };
  __syncthreads();
  const int64_t cap = NL * 32 + 1;
  int64_t step = 0;
  for (;; ++step) {
    unsigned long long key = 0;
    for (int64_t l = tid; l < NL; l += kGreedyThreads)
      key = max(key, (unsigned long long)(uint32_t)s_cnt[l] << 32 | (0xFFFFFFFFu - (uint32_t)l));
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) key = max(key, (unsigned long long)__shfl_xor(key, sh, 64));
    if (lane == 0) s_key[wave] = key;
    __syncthreads();
    if (tid == 0) {
      unsigned long long k2 = 0;
      for (int q = 0; q < kGreedyThreads / 64; ++q) k2 = max(k2, s_key[q]);
      s_best = k2;
      if ((k2 >> 32) != 0 && step < cap) ++s_dep[0xFFFFFFFFu - (uint32_t)k2];
    }
    __syncthreads();
    const unsigned long long best = s_best;
    if ((best >> 32) == 0 || step >= cap) break;
    const int64_t line = 0xFFFFFFFFu - (uint32_t)best;
    const int d = s_dep[line];
    int local = 0;
    if (line < R) {
      for (int64_t k = tid; k < C; k += kGreedyThreads)
        if (ndig(line, k) == d + s_dep[R + k] - 1) {
          --s_cnt[R + k];
          ++local;
        }
    } else {
      const int64_t k = line - R;
      for (int64_t i = tid; i < R; i += kGreedyThreads)
        if (ndig(i, k) == s_dep[i] + d - 1) {
          --s_cnt[i];
          ++local;
        }
    }
    local = wave_sum_i32(local);
    if (lane == 0) s_sum[wave] = local;
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int q = 0; q < kGreedyThreads / 64; ++q) tot += s_sum[q];
      s_cnt[line] -= tot;
    }
    __syncthreads();
  }
  int32_t* gd = reinterpret_cast<int32_t*>(g.plan + g.pl.headers_bytes + b * g.pl.entry_stride + g.pl.gdep);
  for (int64_t l = tid; l < NL; l += kGreedyThreads)
    gd[l < R ? o.rows_off + l : o.cols_off + (l - R)] = s_dep[l];
  if (step >= cap && tid == 0)  // cannot happen for consistent counts; reported by the planner
    atomicOr(reinterpret_cast<unsigned long long*>(
                 &reinterpret_cast<PlanHeader*>(g.plan + b * kPlanHeaderStride)->reserved[2]),
             (unsigned long long)kStatusGreedy);
}

// The three launches.  Records a kernel's own workgroups exchange travel as
// device-scope atomics; records of an earlier launch are read with plain loads.
__global__ __launch_bounds__(kThreads) void plan_sums_kernel(PlanArgs a) {
  __shared__ PlanShared S;
  const int b = blockIdx.y;
  const PlanLayout& L = a.pl;
  const uint32_t G = (uint32_t)(L.wg_a + L.wg_b + L.wg_k);
  phase_sums(a, b, blockIdx.x, S);
  if (!last_to_arrive(arrive_counter(a, b), G, &S.flag)) return;
  choose(a, b, G, true, S);
}
__global__ __launch_bounds__(kThreads) void plan_counts_kernel(PlanArgs a) {
  __shared__ PlanShared S;
  const int b = blockIdx.y;
  const PlanHeader* ph = entry_of(a, b).ph;
  phase_counts(a, b, blockIdx.x, ph->choice_a, ph->choice_b, S);
}
__global__ __launch_bounds__(kThreads) void plan_write_kernel(PlanArgs a) {
  __shared__ PlanShared S;
  const int b = blockIdx.y;
  layout(a, b, blockIdx.x, blockIdx.x == 0, S);
  phase_write(a, b, blockIdx.x, S);
  // Workgroup 0 wrote the host copy of the header (wave 0, during the layout);
  // long after, once those stores have completed, the tag closes the copy: a
  // host that sees the tag sees the whole copy.
  if (blockIdx.x == 0 && a.host_hdr && threadIdx.x < 64) {
    __builtin_amdgcn_s_waitcnt(0);
    if (threadIdx.x == 0)
      __hip_atomic_store(&reinterpret_cast<PlanHeader*>(a.host_hdr + b * kPlanHeaderStride)->reserved[0], a.host_tag,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

}  // namespace

hipError_t launch_greedy(const GreedyArgs& g, int batch, hipStream_t s) {
  if (g.nops < 1 || g.nops > 2 || batch < 1 || batch > 65535) return hipErrorInvalidValue;
  for (int i = 0; i < g.nops; ++i)
    if (g.op[i].R + g.op[i].C > kGreedyMaxLines) return hipErrorInvalidValue;
  hipLaunchKernelGGL(greedy_kernel, dim3((unsigned)g.nops, (unsigned)batch), dim3(kGreedyThreads), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_plan(const PlanArgs& a, hipEvent_t done, hipStream_t s) {
  const PlanLayout& L = a.pl;
  const int64_t G = L.wg_a + L.wg_b + L.wg_k;
  if (G <= 0 || G > 0x7FFFFFFF || L.batch < 1 || L.batch > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)G, (unsigned)L.batch);
  hipLaunchKernelGGL(plan_sums_kernel, grid, dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(plan_counts_kernel, grid, dim3(kThreads), 0, s, a);
  // the event (if any) completes with this launch: no marker of its own in the stream
  if (done) hipExtLaunchKernelGGL(plan_write_kernel, grid, dim3(kThreads), 0, s, nullptr, done, 0, a);
  else hipLaunchKernelGGL(plan_write_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace imu
