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
// kPlanLines, one workgroup per chunk and batch entry:
// (1) plan_sums: the depth of every line under each of the 4 candidates (packed
//     bytes, kept for (2)) and the chunk's share of M'[4], N'[4], K'[4][4]; the
//     last workgroup to finish adds the shares up and picks the pair.
// (2) plan_counts: the chosen depth maps and, per chunk, the entries of every
//     task (each level of A's rows or B's columns: lines deeper than the level;
//     each exponent segment e of K': triples (k, v, v') with v + v' = e); the
//     last workgroup turns them into level bases, padded segment offsets, the
//     header sizes and each chunk's offset in every task.
// (3) plan_write: each chunk scans its lines (a thread owns 4 consecutive
//     lines, one block-wide scan per batch of tasks) and writes the level-major
//     line maps, the per-segment prefixes over k and the K' position table used
//     by the unpack kernels.
// Records pass between the workgroups of one kernel as device-scope atomic
// stores and loads (written through the XCD-local L2); the counter that elects
// the last workgroup is the statistics header's, which is zero between passes.
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
__device__ inline long long ld_dev(const long long* p) {
  return __hip_atomic_load(const_cast<long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int32_t ld_dev(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

__device__ inline long long wave_sum_i64(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    int lo = __shfl_xor((int)(v & 0xFFFFFFFFll), o, 64);
    int hi = __shfl_xor((int)(v >> 32), o, 64);
    v += ((long long)hi << 32) | (unsigned)lo;
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
  return strat == IMU_MIX || (strat == IMU_ROW && c == 0) || (strat == IMU_COL && c == 1);
}

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
  return x;
}

__device__ inline uint32_t* arrive_counter(const PlanArgs& a, int b) {
  return &reinterpret_cast<StatsHeader*>(const_cast<uint8_t*>(a.stats_a) + b * a.stats_stride_a)->arrive;
}

// --- (1) candidate depths and sizes; choice --------------------------------
__global__ __launch_bounds__(kThreads) void plan_sums_kernel(PlanArgs a) {
  __shared__ long long red[kWaves][24];
  __shared__ long long tot[24];
  __shared__ int s_flag;
  const int b = blockIdx.y, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const PlanLayout& L = a.pl;
  const Entry E = entry_of(a, b);
  const Src A = src_of(a.stats_a + b * a.stats_stride_a, a.sla);
  const Src B = src_of(a.stats_b + b * a.stats_stride_b, a.slb);
  const Chunk c = chunk_of(L, blockIdx.x);
  const int gamma = a.gamma;
  long long acc[24];
#pragma unroll
  for (int j = 0; j < 24; ++j) acc[j] = 0;
  uint32_t dx[kPer], dy[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {  // clamped indices: all loads issued before use
    const int64_t i = min64(c.first + t + (int64_t)j * kThreads, c.n - 1);
    if (c.kind == 0) dx[j] = row_depths(A, i, gamma);
    else if (c.kind == 1) dx[j] = col_depths(B, i, gamma);
    else {
      dx[j] = col_depths(A, i, gamma);
      dy[j] = row_depths(B, i, gamma);
    }
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t i = c.first + t + (int64_t)j * kThreads;
    if (i >= c.n) continue;
    if (c.kind == 0) {
      E.cand[i] = dx[j];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += pick(dx[j], q);
    } else if (c.kind == 1) {
      E.cand[L.M + i] = dx[j];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[4 + q] += pick(dx[j], q);
    } else {
      E.cand[L.M + L.N + i] = dx[j];
      E.cand[L.M + L.N + L.K + i] = dy[j];
#pragma unroll
      for (int ca = 0; ca < 4; ++ca)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[8 + ca * 4 + cb] += pick(dx[j], ca) * pick(dy[j], cb);
    }
  }
#pragma unroll
  for (int j = 0; j < 24; ++j) {
    const long long v = wave_sum_i64(acc[j]);
    if (lane == 0) red[wave][j] = v;
  }
  __syncthreads();
  PlanWgRecord* my = E.rec + blockIdx.x;
  if (t < 24) {
    long long v = 0;
    for (int w = 0; w < kWaves; ++w) v += red[w][t];
    st_dev(&my->sum[t], v);
  }
  const uint32_t G = (uint32_t)(L.wg_a + L.wg_b + L.wg_k);
  if (!last_to_arrive(arrive_counter(a, b), G, &s_flag)) return;

  // the last workgroup: totals over all chunks, then the choice
#pragma unroll
  for (int j = 0; j < 24; ++j) acc[j] = 0;
  for (uint32_t w = t; w < G; w += kThreads)
#pragma unroll
    for (int j = 0; j < 24; ++j) acc[j] += ld_dev(&E.rec[w].sum[j]);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 24; ++j) {
    const long long v = wave_sum_i64(acc[j]);
    if (lane == 0) red[wave][j] = v;
  }
  __syncthreads();
  if (t < 24) {
    long long v = 0;
    for (int w = 0; w < kWaves; ++w) v += red[w][t];
    tot[t] = v;
  }
  __syncthreads();
  if (t == 0) {
    PlanHeader* ph = E.ph;
    int best_a = -1, best_b = -1;
    unsigned __int128 best = 0;
    for (int ca = 0; ca < 4; ++ca)
      for (int cb = 0; cb < 4; ++cb) {
        const int slot = ca * 4 + cb;
        if (!allowed(a.strat_a, ca) || !allowed(a.strat_b, cb)) {
          ph->pair[slot][0] = ph->pair[slot][1] = ph->pair[slot][2] = -1;
          continue;
        }
        const long long mu = tot[ca], ku = tot[8 + slot], nu = tot[4 + cb];
        ph->pair[slot][0] = mu;
        ph->pair[slot][1] = ku;
        ph->pair[slot][2] = nu;
        const unsigned __int128 cost =
            (unsigned __int128)(unsigned long long)mu * (unsigned long long)ku * (unsigned long long)nu;
        if (best_a < 0 || cost < best) {
          best = cost;
          best_a = ca;
          best_b = cb;
        }
      }
    ph->choice_a = best_a;
    ph->choice_b = best_b;
    ph->m_u = tot[best_a];
    ph->k_u = tot[8 + best_a * 4 + best_b];
    ph->n_u = tot[4 + best_b];
    ph->status = (int32_t)(reinterpret_cast<const StatsHeader*>(a.stats_a + b * a.stats_stride_a)->status |
                           reinterpret_cast<const StatsHeader*>(a.stats_b + b * a.stats_stride_b)->status);
  }
}

// --- (2) chosen depths, per-chunk task counts; bases, offsets, sizes --------
__global__ __launch_bounds__(kThreads) void plan_counts_kernel(PlanArgs a) {
  __shared__ int hist[(kMaxD + 1) * (kMaxD + 1)];  // depth histogram (rows/cols) or (dA, dB) pairs (k)
  __shared__ int smax[kWaves][4];
  __shared__ int s_flag;
  __shared__ long long gt[2][kPlanTasks];  // lines deeper than u: A rows, B cols
  __shared__ long long seg_len[kPlanTasks];
  __shared__ int lev_s[2], nseg_s;
  const int b = blockIdx.y, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const PlanLayout& L = a.pl;
  const Entry E = entry_of(a, b);
  const Chunk c = chunk_of(L, blockIdx.x);
  const int ca = E.ph->choice_a, cb = E.ph->choice_b;
  for (int i = t; i < (kMaxD + 1) * (kMaxD + 1); i += kThreads) hist[i] = 0;
  __syncthreads();
  uint32_t dx[kPer], dy[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t i = min64(c.first + t + (int64_t)j * kThreads, c.n - 1);
    if (c.kind == 0) dx[j] = E.cand[i];
    else if (c.kind == 1) dx[j] = E.cand[L.M + i];
    else {
      dx[j] = E.cand[L.M + L.N + i];
      dy[j] = E.cand[L.M + L.N + L.K + i];
    }
  }
  int m0 = 1, m1 = 1, m2 = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t i = c.first + t + (int64_t)j * kThreads;
    if (i >= c.n) continue;
    if (c.kind < 2) {
      const int d = pick(dx[j], c.kind == 0 ? ca : cb);
      (c.kind == 0 ? E.da_r : E.db_c)[i] = d;
      m0 = max(m0, d);
      atomicAdd(&hist[d], 1);
    } else {
      const int x = pick(dx[j], ca), y = pick(dy[j], cb);
      E.da_c[i] = x;
      E.db_r[i] = y;
      m0 = max(m0, x);
      m1 = max(m1, y);
      m2 = max(m2, x + y - 2);
      atomicAdd(&hist[x * (kMaxD + 1) + y], 1);
    }
  }
  m0 = wave_max_i32(m0);
  m1 = wave_max_i32(m1);
  m2 = wave_max_i32(m2);
  if (lane == 0) {
    smax[wave][0] = m0;
    smax[wave][1] = m1;
    smax[wave][2] = m2;
  }
  __syncthreads();
  int x_hi = 1, y_hi = 1;
  for (int w = 0; w < kWaves; ++w) {
    x_hi = max(x_hi, smax[w][0]);
    y_hi = max(y_hi, smax[w][1]);
  }
  PlanWgRecord* my = E.rec + blockIdx.x;
  if (t < kPlanTasks) {  // task counts of this chunk
    int v = 0;
    if (c.kind < 2) {
      for (int d = t + 1; d <= x_hi; ++d) v += hist[d];  // lines with depth > t
    } else {
      for (int x = 1; x <= x_hi; ++x)
        for (int y = 1; y <= y_hi; ++y) v += hist[x * (kMaxD + 1) + y] * seg_count(x, y, t);
    }
    st_dev(&my->cnt[t], v);
  }
  if (t < 3) {
    int v = t == 2 ? 0 : 1;
    for (int w = 0; w < kWaves; ++w) v = max(v, smax[w][t]);
    st_dev(&my->mx[t], v);
  }
  const uint32_t G = (uint32_t)(L.wg_a + L.wg_b + L.wg_k);
  if (!last_to_arrive(arrive_counter(a, b), G, &s_flag)) return;

  // the last workgroup: per task, chunk offsets and totals (one thread per
  // task and kind walks that kind's chunks in order)
  const int64_t wk0[3] = {0, L.wg_a, L.wg_a + L.wg_b};
  const int64_t wkn[3] = {L.wg_a, L.wg_b, L.wg_k};
  for (int job = t; job < 3 * kPlanTasks; job += kThreads) {
    const int kind = job / kPlanTasks, task = job % kPlanTasks;
    long long run = 0;
    for (int64_t r = 0; r < wkn[kind]; ++r) {
      PlanWgRecord* rc = E.rec + wk0[kind] + r;
      rc->off[task] = (int32_t)run;  // read by the next kernel
      run += ld_dev(&rc->cnt[task]);
    }
    if (kind < 2) gt[kind][task] = run;
    else seg_len[task] = run;
  }
  if (t < 3) {
    int v = t == 2 ? 0 : 1;
    for (int64_t w = 0; w < (int64_t)G; ++w) {
      const Chunk cw = chunk_of(L, w);
      const int mxv = t == 0 ? ld_dev(&E.rec[w].mx[0]) : ld_dev(&E.rec[w].mx[t == 1 ? 0 : 2]);
      if ((t == 0 && cw.kind == 0) || (t == 1 && cw.kind == 1) || (t == 2 && cw.kind == 2)) v = max(v, mxv);
    }
    if (t < 2) lev_s[t] = min(v, (int)L.levels);
    else nseg_s = min(v, (int)L.segments - 1) + 1;
  }
  __syncthreads();
  if (t == 0) {
    PlanHeader* ph = E.ph;
    const int lev_a = lev_s[0], lev_b = lev_s[1], nseg = nseg_s;
    const int64_t m_base = round_up(L.M, L.pad_m), n_base = round_up(L.N, L.pad_n);
    long long end_a = m_base, end_b = n_base;
    for (int u = 1; u < lev_a; ++u) end_a += gt[0][u];
    for (int u = 1; u < lev_b; ++u) end_b += gt[1][u];
    long long off = 0;
    for (int s = 0; s < nseg; ++s) {
      ph->seg_off[s] = off;
      ph->seg_len[s] = (int32_t)seg_len[s];
      off += round_up(seg_len[s], kKPad);
    }
    ph->seg_off[nseg] = off;
    ph->n_seg = nseg;
    ph->k_pad = off;
    ph->m_base = m_base;
    ph->n_base = n_base;
    ph->m_alloc = round_up(end_a, L.pad_m);
    ph->n_alloc = round_up(end_b, L.pad_n);
    ph->lev_a = lev_a;
    ph->lev_b = lev_b;
    ph->emax = nseg - 1;
  }
}

// --- (3) positions ----------------------------------------------------------
__global__ __launch_bounds__(kThreads) void plan_write_kernel(PlanArgs a) {
  __shared__ int scan_tot[kWaves * kTaskBatch];
  __shared__ long long base_s[kPlanTasks];  // level bases (rows/cols) or segment offsets (k)
  __shared__ int off_s[kPlanTasks];
  const int b = blockIdx.y, t = threadIdx.x;
  const PlanLayout& L = a.pl;
  const Entry E = entry_of(a, b);
  const PlanHeader* ph = E.ph;
  const Chunk c = chunk_of(L, blockIdx.x);
  const int ntasks = c.kind == 0 ? ph->lev_a : c.kind == 1 ? ph->lev_b : ph->n_seg;
  const PlanWgRecord* my = E.rec + blockIdx.x;
  if (t < kPlanTasks) off_s[t] = my->off[t];
  if (t == 0) {
    if (c.kind < 2) {
      // level u > 0 starts after the padded base and the levels 1..u-1, whose
      // sizes are the totals of the previous chunks' last offsets + counts:
      // recomputed here from the records of this kind's last chunk
      const int64_t last = c.kind == 0 ? L.wg_a - 1 : L.wg_a + L.wg_b - 1;
      const PlanWgRecord* lr = E.rec + last;
      long long p = c.kind == 0 ? ph->m_base : ph->n_base;
      base_s[0] = 0;
      for (int u = 1; u < ntasks; ++u) {
        base_s[u] = p;
        p += (long long)lr->off[u] + lr->cnt[u];
      }
    } else {
      for (int s = 0; s < ntasks; ++s) base_s[s] = ph->seg_off[s];
    }
  }
  __syncthreads();
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
  for (int tb = 0; tb < ntasks; tb += kTaskBatch) {
    int cnt[kTaskBatch], ex[kTaskBatch];
#pragma unroll
    for (int j = 0; j < kTaskBatch; ++j) {
      int v = 0;
#pragma unroll
      for (int l = 0; l < kPer; ++l)
        if (l < nl) v += c.kind < 2 ? (dA[l] > tb + j) : seg_count(dA[l], dB[l], tb + j);
      cnt[j] = v;
    }
    block_excl_scan_multi(cnt, ex, scan_tot);
#pragma unroll
    for (int j = 0; j < kTaskBatch; ++j) {
      const int task = tb + j;
      if (task >= ntasks) continue;
      long long pos = ex[j] + off_s[task];  // position inside the task
#pragma unroll
      for (int l = 0; l < kPer; ++l) {
        if (l >= nl) continue;
        const int64_t i = i0 + l;
        if (c.kind < 2) {
          const bool live = dA[l] > task;
          const long long p = base_s[task] + pos;
          (c.kind == 0 ? E.lvl_a : E.lvl_b)[(int64_t)task * c.n + i] = live ? (int32_t)p : -1;
          if (live) (c.kind == 0 ? E.amap : E.bmap)[p] = (int32_t)(i | ((int64_t)task << 24));
          pos += live;
        } else {
          const int cnt_l = seg_count(dA[l], dB[l], task);
          E.kpre[(int64_t)task * (L.K + 1) + i] = (int32_t)pos;
          uint32_t* km = E.kmap + base_s[task] + pos;
          const int lo = max(0, task - (dB[l] - 1));
          for (int v = 0; v < cnt_l; ++v) km[v] = kmap_pack(i, lo + v, task - lo - v, dA[l], dB[l]);
          pos += cnt_l;
        }
      }
    }
  }
  // padding (workgroup 0): rows between M and the padded base, after the last
  // level up to the allocation, zero entries at the end of every segment, and
  // the per-segment totals at kpre[s][K]
  if (blockIdx.x == 0) {
    __shared__ long long end_s[2];
    if (t < 2) {
      const int64_t last = t == 0 ? L.wg_a - 1 : L.wg_a + L.wg_b - 1;
      const PlanWgRecord* lr = E.rec + last;
      const int lev = t == 0 ? ph->lev_a : ph->lev_b;
      long long p = t == 0 ? ph->m_base : ph->n_base;
      for (int u = 1; u < lev; ++u) p += (long long)lr->off[u] + lr->cnt[u];
      end_s[t] = p;
    }
    __syncthreads();
    for (int64_t r = L.M + t; r < ph->m_base; r += kThreads) E.amap[r] = -1;
    for (int64_t r = end_s[0] + t; r < ph->m_alloc; r += kThreads) E.amap[r] = -1;
    for (int64_t r = L.N + t; r < ph->n_base; r += kThreads) E.bmap[r] = -1;
    for (int64_t r = end_s[1] + t; r < ph->n_alloc; r += kThreads) E.bmap[r] = -1;
    const int nseg = ph->n_seg;
    for (int s = 0; s < nseg; ++s) {
      const int64_t p0 = ph->seg_off[s] + ph->seg_len[s], p1 = ph->seg_off[s + 1];
      for (int64_t p = p0 + t; p < p1; p += kThreads) E.kmap[p] = kKmapPad;
    }
    if (t < nseg) E.kpre[(int64_t)t * (L.K + 1) + L.K] = ph->seg_len[t];
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  const PlanLayout& L = a.pl;
  const int64_t G = L.wg_a + L.wg_b + L.wg_k;
  if (G <= 0 || G > 0x7FFFFFFF || L.batch < 1 || L.batch > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)G, (unsigned)L.batch);
  hipLaunchKernelGGL(plan_sums_kernel, grid, dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(plan_counts_kernel, grid, dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(plan_write_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace imu
