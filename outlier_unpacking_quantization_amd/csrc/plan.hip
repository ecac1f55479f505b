// Unpacking planner (gfx950): one 1024-thread workgroup per batch entry.
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
// Phases: (1) the depth of every line under each of the 4 candidates, kept as
// bytes in LDS, and the sums giving M'[4], N'[4] and K'[4][4]; choice of the
// pair; (2) the chosen depth maps (global int32) and their histograms, which
// give every level base and segment size up front; (3) one wave per scan task
// (each level of A's rows, each level of B's columns, each exponent segment of
// K'), each lane scanning a contiguous run, writes final positions: level-major
// line maps, per-segment prefixes over k and the K' position table used by
// the unpack kernels.  Problems whose candidate bytes exceed the LDS budget
// take the same steps reading the statistics from global memory.
#include "common.h"
#include "kernels.h"

namespace imu {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kCandBytes = 112 * 1024;  // LDS budget for candidate depth bytes
constexpr int kMaxD = 32;               // >= max_digits(2) + 1

__device__ inline long long wave_sum_i64(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    int lo = __shfl_xor((int)(v & 0xFFFFFFFFll), o, 64);
    int hi = __shfl_xor((int)(v >> 32), o, 64);
    v += ((long long)hi << 32) | (unsigned)lo;
  }
  return v;
}

constexpr int kTaskBatch = 8;  // scan tasks handled per pass over the line runs

// Block-wide exclusive scans of kTaskBatch counters per thread at once.
// `tot` is LDS scratch of kWaves * kTaskBatch ints.
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

// add 1 to LDS counter `key` for every lane, one atomic per distinct key in the wave
__device__ inline void wave_count(int* counters, int key, bool active) {
  unsigned long long todo = __ballot(active);
  while (todo) {
    const int leader = __ffsll((long long)todo) - 1;
    const int lk = __shfl(key, leader, 64);
    const unsigned long long same = __ballot(active && key == lk) & todo;
    if ((threadIdx.x & 63) == leader) atomicAdd(&counters[lk], __popcll(same));
    todo &= ~same;
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

// Row depths of the 4 candidates (row, col, cr, rc) for row i, packed in bytes.
__device__ inline uint32_t row_depths(const Src& s, int64_t i, int gamma) {
  const int mx = min(max(1, s.row_max[i]), kMaxD);
  const int cr = min(max(1, s.cr_rowdig[i]), kMaxD);
  const int rc = (long long)s.row_oob[i] * s.R > gamma * s.T ? mx : 1;
  return (uint32_t)mx | 1u << 8 | (uint32_t)cr << 16 | (uint32_t)rc << 24;
}
// Column depths of the 4 candidates for column k, packed in bytes.
__device__ inline uint32_t col_depths(const Src& s, int64_t k, int gamma) {
  const int mx = min(max(1, s.col_max[k]), kMaxD);
  const int cr = (long long)s.col_oob[k] * s.C > gamma * s.T ? mx : 1;
  const int rc = min(max(1, s.rc_coldig[k]), kMaxD);
  return 1u | (uint32_t)mx << 8 | (uint32_t)cr << 16 | (uint32_t)rc << 24;
}
__device__ inline int pick(uint32_t packed, int c) { return (packed >> (8 * c)) & 0xFF; }

constexpr int kRound = 4;  // lines per thread whose loads are issued together

// Candidate depths of rows i0 + j*kThreads (j < kRound); all loads first.
__device__ inline void rows_depths_round(const Src& s, int64_t i0, int64_t n, int gamma, uint32_t out[kRound]) {
  int mx[kRound], cr[kRound], ob[kRound];
#pragma unroll
  for (int j = 0; j < kRound; ++j) {  // clamped indices: unconditional loads
    const int64_t i = min64(i0 + (int64_t)j * kThreads, n - 1);
    mx[j] = s.row_max[i];
    cr[j] = s.cr_rowdig[i];
    ob[j] = s.row_oob[i];
  }
#pragma unroll
  for (int j = 0; j < kRound; ++j) {
    const int m = min(max(1, mx[j]), kMaxD);
    const int c = min(max(1, cr[j]), kMaxD);
    const int h = (long long)ob[j] * s.R > gamma * s.T ? m : 1;
    out[j] = (uint32_t)m | 1u << 8 | (uint32_t)c << 16 | (uint32_t)h << 24;
  }
}
// Candidate depths of columns k0 + j*kThreads (j < kRound); all loads first.
__device__ inline void cols_depths_round(const Src& s, int64_t k0, int64_t n, int gamma, uint32_t out[kRound]) {
  int mx[kRound], rc[kRound], ob[kRound];
#pragma unroll
  for (int j = 0; j < kRound; ++j) {  // clamped indices: unconditional loads
    const int64_t k = min64(k0 + (int64_t)j * kThreads, n - 1);
    mx[j] = s.col_max[k];
    rc[j] = s.rc_coldig[k];
    ob[j] = s.col_oob[k];
  }
#pragma unroll
  for (int j = 0; j < kRound; ++j) {
    const int m = min(max(1, mx[j]), kMaxD);
    const int h = (long long)ob[j] * s.C > gamma * s.T ? m : 1;
    const int c = min(max(1, rc[j]), kMaxD);
    out[j] = 1u | (uint32_t)m << 8 | (uint32_t)h << 16 | (uint32_t)c << 24;
  }
}

__device__ inline bool allowed(int strat, int c) {
  return strat == IMU_MIX || (strat == IMU_ROW && c == 0) || (strat == IMU_COL && c == 1);
}

// number of triples (k, v, v') with v + v' = e, v < dA, v' < dB
__device__ inline int seg_count(int dA, int dB, int e) {
  const int lo = max(0, e - (dB - 1)), hi = min(dA - 1, e);
  return max(0, hi - lo + 1);
}

// Chosen depth of one line: from the LDS candidate bytes, or recomputed.
struct DepthView {
  const uint32_t* lds;  // packed candidate bytes, or null
  const int32_t* g;     // global chosen depth map (written in phase 2)
  __device__ int operator()(int64_t i, int c) const { return lds ? pick(lds[i], c) : (int)g[i]; }
};

__global__ __launch_bounds__(kThreads) void plan_kernel(PlanArgs a) {
  __shared__ uint32_t cand[kCandBytes / 4];
  __shared__ long long red[kWaves][24];
  __shared__ long long red_tot[24];
  __shared__ long long gt_a[kMaxD + 1], gt_b[kMaxD + 1];  // lines with depth > u
  __shared__ int smax[kWaves][5];
  __shared__ long long seg_len_s[kMaxSeg];
  __shared__ int choice[2];
  __shared__ int hist_a[kMaxD + 1], hist_b[kMaxD + 1];
  __shared__ int pair_hist[(kMaxD + 1) * (kMaxD + 1)];
  __shared__ long long base_a[kMaxD + 1], base_b[kMaxD + 1];
  __shared__ long long seg_off[kMaxSeg + 1];
  __shared__ int scan_tot[kWaves * kTaskBatch];
  const int b = blockIdx.x;
  const PlanLayout& L = a.pl;
  const Src A = src_of(a.stats_a + b * a.stats_stride_a, a.sla);
  const Src B = src_of(a.stats_b + b * a.stats_stride_b, a.slb);
  const int64_t M = L.M, K = L.K, N = L.N;
  const int gamma = a.gamma;
  PlanHeader* ph = reinterpret_cast<PlanHeader*>(a.plan + b * kPlanHeaderStride);
  uint8_t* e = a.plan + L.headers_bytes + b * L.entry_stride;
  int32_t* da_r = reinterpret_cast<int32_t*>(e + L.da_r);
  int32_t* da_c = reinterpret_cast<int32_t*>(e + L.da_c);
  int32_t* db_r = reinterpret_cast<int32_t*>(e + L.db_r);
  int32_t* db_c = reinterpret_cast<int32_t*>(e + L.db_c);
  int32_t* lvl_a = reinterpret_cast<int32_t*>(e + L.lvl_a);
  int32_t* lvl_b = reinterpret_cast<int32_t*>(e + L.lvl_b);
  int32_t* amap = reinterpret_cast<int32_t*>(e + L.amap);
  int32_t* bmap = reinterpret_cast<int32_t*>(e + L.bmap);
  int32_t* kpre = reinterpret_cast<int32_t*>(e + L.kpre);
  uint32_t* kmap = reinterpret_cast<uint32_t*>(e + L.kmap);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const bool in_lds = 4 * (M + 2 * K + N) <= kCandBytes;
  uint32_t* c_ar = cand;          // [M]  A's rows
  uint32_t* c_ac = cand + M;      // [K]  A's columns
  uint32_t* c_br = c_ac + K;      // [K]  B's rows
  uint32_t* c_bc = c_br + K;      // [N]  B's columns
  if (t == 0) ph->tstamp[0] = wall_clock64();

  // --- 1. candidate depths and the sizes M'[4], N'[4], K'[4][4] ---------------
  // Each round issues the loads of kRound lines per thread before using any.
  long long acc[24];
#pragma unroll
  for (int j = 0; j < 24; ++j) acc[j] = 0;
  for (int64_t i0 = t; i0 < M; i0 += kRound * kThreads) {
    uint32_t d[kRound];
    rows_depths_round(A, i0, M, gamma, d);
#pragma unroll
    for (int j = 0; j < kRound; ++j) {
      const int64_t i = i0 + (int64_t)j * kThreads;
      if (i >= M) continue;
      if (in_lds) c_ar[i] = d[j];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] += pick(d[j], c);
    }
  }
  for (int64_t n0 = t; n0 < N; n0 += kRound * kThreads) {
    uint32_t d[kRound];
    cols_depths_round(B, n0, N, gamma, d);
#pragma unroll
    for (int j = 0; j < kRound; ++j) {
      const int64_t n = n0 + (int64_t)j * kThreads;
      if (n >= N) continue;
      if (in_lds) c_bc[n] = d[j];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[4 + c] += pick(d[j], c);
    }
  }
  for (int64_t k0 = t; k0 < K; k0 += kRound * kThreads) {
    uint32_t x[kRound], y[kRound];
    cols_depths_round(A, k0, K, gamma, x);
    rows_depths_round(B, k0, K, gamma, y);
#pragma unroll
    for (int j = 0; j < kRound; ++j) {
      const int64_t k = k0 + (int64_t)j * kThreads;
      if (k >= K) continue;
      if (in_lds) {
        c_ac[k] = x[j];
        c_br[k] = y[j];
      }
#pragma unroll
      for (int ca = 0; ca < 4; ++ca)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[8 + ca * 4 + cb] += pick(x[j], ca) * pick(y[j], cb);
    }
  }
  if (t == 0) ph->tstamp[5] = wall_clock64();
#pragma unroll
  for (int j = 0; j < 24; ++j) {
    long long v = wave_sum_i64(acc[j]);
    if (lane == 0) red[wave][j] = v;
  }
  if (t == 0) ph->tstamp[6] = wall_clock64();
  for (int i = t; i <= kMaxD; i += kThreads) {
    hist_a[i] = 0;
    hist_b[i] = 0;
  }
  for (int i = t; i < (kMaxD + 1) * (kMaxD + 1); i += kThreads) pair_hist[i] = 0;
  __syncthreads();
  if (t < 24) {
    long long v = 0;
    for (int w = 0; w < kWaves; ++w) v += red[w][t];
    red_tot[t] = v;
  }
  __syncthreads();
  if (t == 0) {
    const long long* tot = red_tot;
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
    choice[0] = best_a;
    choice[1] = best_b;
    ph->choice_a = best_a;
    ph->choice_b = best_b;
    ph->m_u = tot[best_a];
    ph->k_u = tot[8 + best_a * 4 + best_b];
    ph->n_u = tot[4 + best_b];
    ph->status = (int32_t)(reinterpret_cast<const StatsHeader*>(a.stats_a + b * a.stats_stride_a)->status |
                           reinterpret_cast<const StatsHeader*>(a.stats_b + b * a.stats_stride_b)->status);
    ph->tstamp[1] = wall_clock64();
  }
  __syncthreads();
  const int ca = choice[0], cb = choice[1];

  // --- 2. chosen depth maps, their maxima and histograms -----------------------
  int mxa = 1, mxb = 1, mxe = 0, mxx = 1, mxy = 1;
  for (int64_t i0 = 0; i0 < M; i0 += kThreads) {
    const int64_t i = i0 + t;
    const bool ok = i < M;
    const int d = ok ? pick(in_lds ? c_ar[i] : row_depths(A, i, gamma), ca) : 0;
    if (ok) da_r[i] = d;
    mxa = max(mxa, d);
    wave_count(hist_a, d, ok);
  }
  for (int64_t n0 = 0; n0 < N; n0 += kThreads) {
    const int64_t n = n0 + t;
    const bool ok = n < N;
    const int d = ok ? pick(in_lds ? c_bc[n] : col_depths(B, n, gamma), cb) : 0;
    if (ok) db_c[n] = d;
    mxb = max(mxb, d);
    wave_count(hist_b, d, ok);
  }
  for (int64_t k0 = 0; k0 < K; k0 += kThreads) {
    const int64_t k = k0 + t;
    const bool ok = k < K;
    int x = 1, y = 1;
    if (ok) {
      x = pick(in_lds ? c_ac[k] : col_depths(A, k, gamma), ca);
      y = pick(in_lds ? c_br[k] : row_depths(B, k, gamma), cb);
      da_c[k] = x;
      db_r[k] = y;
    }
    mxe = max(mxe, x + y - 2);
    mxx = max(mxx, x);
    mxy = max(mxy, y);
    wave_count(pair_hist, x * (kMaxD + 1) + y, ok);
  }
  mxa = wave_max_i32(mxa);
  mxb = wave_max_i32(mxb);
  mxe = wave_max_i32(mxe);
  mxx = wave_max_i32(mxx);
  mxy = wave_max_i32(mxy);
  if (lane == 0) {
    smax[wave][0] = mxa;
    smax[wave][1] = mxb;
    smax[wave][2] = mxe;
    smax[wave][3] = mxx;
    smax[wave][4] = mxy;
  }
  __syncthreads();  // (workgroup scope) global depth maps visible to the whole workgroup below
  int lev_a = 1, lev_b = 1, emax = 0, xmax = 1, ymax = 1;
  for (int w = 0; w < kWaves; ++w) {
    lev_a = max(lev_a, smax[w][0]);
    lev_b = max(lev_b, smax[w][1]);
    emax = max(emax, smax[w][2]);
    xmax = max(xmax, smax[w][3]);
    ymax = max(ymax, smax[w][4]);
  }
  lev_a = min<int>(lev_a, (int)L.levels);
  lev_b = min<int>(lev_b, (int)L.levels);
  emax = min<int>(emax, (int)L.segments - 1);
  const int nseg = emax + 1;
  const int64_t m_base = round_up(M, L.pad_m), n_base = round_up(N, L.pad_n);
  if (t == 0) ph->tstamp[2] = wall_clock64();

  // segment sizes from the histogram of (A's, B's) inner depth pairs
  if (t < nseg) {
    long long len = 0;
    for (int x = 1; x <= xmax; ++x)
      for (int y = 1; y <= ymax; ++y) len += (long long)pair_hist[x * (kMaxD + 1) + y] * seg_count(x, y, t);
    seg_len_s[t] = len;
  }
  if (t <= kMaxD) {  // lines with depth > t
    long long ga = 0, gb = 0;
    for (int d = t + 1; d <= kMaxD; ++d) {
      ga += hist_a[d];
      gb += hist_b[d];
    }
    gt_a[t] = ga;
    gt_b[t] = gb;
  }
  __syncthreads();
  // level bases and padded segment offsets
  if (t == 0) {
    long long pos = 0;
    for (int u = 0; u < lev_a; ++u) {
      base_a[u] = pos;
      pos = (u == 0) ? m_base : pos + gt_a[u];
    }
    base_a[lev_a] = pos;
    pos = 0;
    for (int u = 0; u < lev_b; ++u) {
      base_b[u] = pos;
      pos = (u == 0) ? n_base : pos + gt_b[u];
    }
    base_b[lev_b] = pos;
    long long off = 0;
    for (int s = 0; s < nseg; ++s) {
      const long long len = seg_len_s[s];
      seg_off[s] = off;
      ph->seg_off[s] = off;
      ph->seg_len[s] = (int32_t)len;
      off += round_up(len, kKPad);
    }
    seg_off[nseg] = off;
    ph->seg_off[nseg] = off;
    ph->n_seg = nseg;
    ph->k_pad = off;
    ph->m_base = m_base;
    ph->n_base = n_base;
    ph->m_alloc = round_up(base_a[lev_a], L.pad_m);
    ph->n_alloc = round_up(base_b[lev_b], L.pad_n);
    ph->lev_a = lev_a;
    ph->lev_b = lev_b;
    ph->emax = emax;
    ph->tstamp[3] = wall_clock64();
  }
  __syncthreads();
  const DepthView VAR{in_lds ? c_ar : nullptr, da_r}, VAC{in_lds ? c_ac : nullptr, da_c};
  const DepthView VBR{in_lds ? c_br : nullptr, db_r}, VBC{in_lds ? c_bc : nullptr, db_c};
  const int64_t m_alloc = round_up(base_a[lev_a], L.pad_m), n_alloc = round_up(base_b[lev_b], L.pad_n);

  // --- 3a. padding entries (disjoint from everything the scans write) ---------
  for (int64_t r = M + t; r < m_base; r += kThreads) amap[r] = -1;
  for (int64_t r = base_a[lev_a] + t; r < m_alloc; r += kThreads) amap[r] = -1;
  for (int64_t r = N + t; r < n_base; r += kThreads) bmap[r] = -1;
  for (int64_t r = base_b[lev_b] + t; r < n_alloc; r += kThreads) bmap[r] = -1;
  for (int s = 0; s < nseg; ++s) {
    const int64_t p0 = seg_off[s] + seg_len_s[s], p1 = seg_off[s + 1];
    for (int64_t p = p0 + t; p < p1; p += kThreads) kmap[p] = kKmapPad;
  }
  if (t == 0) ph->tstamp[7] = wall_clock64();

  // --- 3b. scans: each thread owns a contiguous run of lines; a batch of tasks
  // (levels of A's rows, levels of B's columns, or exponent segments of K') is
  // counted over the run, one block-wide scan gives every run its offsets, and
  // a second pass over the run writes the positions (adjacent threads write
  // adjacent runs, so the stores stay close to coalesced).
  for (int group = 0; group < 3; ++group) {
    const int64_t n = group == 0 ? M : (group == 1 ? N : K);
    const int ntasks = group == 0 ? lev_a : (group == 1 ? lev_b : nseg);
    const int64_t len = ceil_div(n, kThreads);
    const int64_t i0 = min64((int64_t)t * len, n), i1 = min64(i0 + len, n);
    for (int tb = 0; tb < ntasks; tb += kTaskBatch) {
      int cnt[kTaskBatch];
#pragma unroll
      for (int j = 0; j < kTaskBatch; ++j) cnt[j] = 0;
      for (int64_t i = i0; i < i1; ++i) {
        if (group < 2) {
          const int d = group == 0 ? VAR(i, ca) : VBC(i, cb);
#pragma unroll
          for (int j = 0; j < kTaskBatch; ++j) cnt[j] += d > tb + j;
        } else {
          const int dA = VAC(i, ca), dB = VBR(i, cb);
#pragma unroll
          for (int j = 0; j < kTaskBatch; ++j) cnt[j] += seg_count(dA, dB, tb + j);
        }
      }
      int ex[kTaskBatch];
      block_excl_scan_multi(cnt, ex, scan_tot);
      for (int64_t i = i0; i < i1; ++i) {
        if (group < 2) {
          const int d = group == 0 ? VAR(i, ca) : VBC(i, cb);
          int32_t* lvl = group == 0 ? lvl_a : lvl_b;
          int32_t* map = group == 0 ? amap : bmap;
          const long long* base = group == 0 ? base_a : base_b;
#pragma unroll
          for (int j = 0; j < kTaskBatch; ++j) {
            const int u = tb + j;
            if (u < ntasks) {
              const bool live = d > u;
              const long long p = base[u] + ex[j];
              lvl[(int64_t)u * n + i] = live ? (int32_t)p : -1;
              if (live) map[p] = (int32_t)(i | ((int64_t)u << 24));
              ex[j] += live;
            }
          }
        } else {
          const int dA = VAC(i, ca), dB = VBR(i, cb);
#pragma unroll
          for (int j = 0; j < kTaskBatch; ++j) {
            const int s = tb + j;
            if (s < ntasks) {
              const int c = seg_count(dA, dB, s);
              kpre[(int64_t)s * (K + 1) + i] = ex[j];
              uint32_t* km = kmap + seg_off[s] + ex[j];
              const int lo = max(0, s - (dB - 1));
              for (int v = 0; v < c; ++v) km[v] = kmap_pack(i, lo + v, s - lo - v, dA, dB);
              ex[j] += c;
            }
          }
        }
      }
    }
  }
  if (t < nseg) kpre[(int64_t)t * (K + 1) + K] = (int32_t)seg_len_s[t];
  __syncthreads();
  if (t == 0) ph->tstamp[4] = wall_clock64();
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3((unsigned)a.pl.batch), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace imu
