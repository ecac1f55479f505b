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
#include "common.h"
#include "kernels.h"

namespace imu {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ inline long long wave_sum_i64(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    int lo = __shfl_xor((int)(v & 0xFFFFFFFFll), o, 64);
    int hi = __shfl_xor((int)(v >> 32), o, 64);
    v += ((long long)hi << 32) | (unsigned)lo;
  }
  return v;
}

// Block-wide exclusive scan of one int per thread; returns the exclusive
// prefix and writes the block total to *total.  Uses `scratch` (kWaves ints).
__device__ inline int block_excl_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int wbase = 0, tot = 0;
  for (int w = 0; w < kWaves; ++w) {
    int s = scratch[w];
    if (w < wave) wbase += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wbase + incl - v;
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

// Row depth of candidate c (0 row, 1 col, 2 cr, 3 rc) for row i of operand s.
__device__ inline int row_depth(const Src& s, int c, int64_t i, int gamma) {
  switch (c) {
    case 0: return max(1, s.row_max[i]);
    case 1: return 1;
    case 2: return max(1, s.cr_rowdig[i]);
    default: return (long long)s.row_oob[i] * s.R > gamma * s.T ? max(1, s.row_max[i]) : 1;
  }
}
// Column depth of candidate c for column k of operand s.
__device__ inline int col_depth(const Src& s, int c, int64_t k, int gamma) {
  switch (c) {
    case 0: return 1;
    case 1: return max(1, s.col_max[k]);
    case 2: return (long long)s.col_oob[k] * s.C > gamma * s.T ? max(1, s.col_max[k]) : 1;
    default: return max(1, s.rc_coldig[k]);
  }
}

__device__ inline bool allowed(int strat, int c) {
  return strat == IMU_MIX || (strat == IMU_ROW && c == 0) || (strat == IMU_COL && c == 1);
}

// Level-major line positions for one operand side: lvl[u][i] for u < levels.
__device__ void level_maps(const int32_t* d, int64_t n, int levels_used, int64_t base1, int64_t pad,
                           int32_t* lvl, int32_t* map, int64_t* alloc_out, int* scratch) {
  // pass 1: positions
  int64_t base = 0;
  for (int u = 0; u < levels_used; ++u) {
    const int64_t per = ceil_div(n, kThreads);
    const int64_t i0 = min64(threadIdx.x * per, n), i1 = min64(i0 + per, n);
    int cnt = 0;
    for (int64_t i = i0; i < i1; ++i) cnt += d[i] > u;
    int total;
    int ex = block_excl_scan(cnt, scratch, &total);
    int64_t pos = base + ex;
    for (int64_t i = i0; i < i1; ++i) {
      bool live = d[i] > u;
      lvl[(int64_t)u * n + i] = live ? (int32_t)pos : -1;
      pos += live;
    }
    base = (u == 0) ? base1 : base + total;
  }
  const int64_t alloc = round_up(base, pad);
  *alloc_out = alloc;
  __syncthreads();
  for (int64_t r = threadIdx.x; r < alloc; r += kThreads) map[r] = -1;
  __syncthreads();
  for (int u = 0; u < levels_used; ++u)
    for (int64_t i = threadIdx.x; i < n; i += kThreads) {
      int32_t p = lvl[(int64_t)u * n + i];
      if (p >= 0) map[p] = (int32_t)(i | ((int64_t)u << 24));
    }
}

__global__ __launch_bounds__(kThreads) void plan_kernel(PlanArgs a) {
  __shared__ long long red[kWaves][24];
  __shared__ int scratch[kWaves];
  __shared__ int smax[kWaves][3];
  __shared__ int choice[2];
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
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // --- 1. sizes of every candidate: M'[4], N'[4], K'[4][4] --------------------
  long long acc[24];
#pragma unroll
  for (int j = 0; j < 24; ++j) acc[j] = 0;
  for (int64_t i = threadIdx.x; i < M; i += kThreads)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] += row_depth(A, c, i, gamma);
  for (int64_t n = threadIdx.x; n < N; n += kThreads)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[4 + c] += col_depth(B, c, n, gamma);
  for (int64_t k = threadIdx.x; k < K; k += kThreads) {
    int dac[4], dbr[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      dac[c] = col_depth(A, c, k, gamma);
      dbr[c] = row_depth(B, c, k, gamma);
    }
#pragma unroll
    for (int ca = 0; ca < 4; ++ca)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[8 + ca * 4 + cb] += (long long)dac[ca] * dbr[cb];
  }
#pragma unroll
  for (int j = 0; j < 24; ++j) {
    long long v = wave_sum_i64(acc[j]);
    if (lane == 0) red[wave][j] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long tot[24];
    for (int j = 0; j < 24; ++j) {
      tot[j] = 0;
      for (int w = 0; w < kWaves; ++w) tot[j] += red[w][j];
    }
    int best_a = -1, best_b = -1;
    unsigned __int128 best = 0;
    for (int ca = 0; ca < 4; ++ca)
      for (int cb = 0; cb < 4; ++cb) {
        int slot = ca * 4 + cb;
        if (!allowed(a.strat_a, ca) || !allowed(a.strat_b, cb)) {
          ph->pair[slot][0] = ph->pair[slot][1] = ph->pair[slot][2] = -1;
          continue;
        }
        long long mu = tot[ca], ku = tot[8 + slot], nu = tot[4 + cb];
        ph->pair[slot][0] = mu;
        ph->pair[slot][1] = ku;
        ph->pair[slot][2] = nu;
        unsigned __int128 cost = (unsigned __int128)(unsigned long long)mu * (unsigned long long)ku *
                                 (unsigned long long)nu;
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
  }
  __syncthreads();
  const int ca = choice[0], cb = choice[1];

  // --- 2. depth maps of the chosen pair and their maxima ----------------------
  int mxa = 1, mxb = 1, mxe = 0;
  for (int64_t i = threadIdx.x; i < M; i += kThreads) {
    int d = row_depth(A, ca, i, gamma);
    da_r[i] = d;
    mxa = max(mxa, d);
  }
  for (int64_t n = threadIdx.x; n < N; n += kThreads) {
    int d = col_depth(B, cb, n, gamma);
    db_c[n] = d;
    mxb = max(mxb, d);
  }
  for (int64_t k = threadIdx.x; k < K; k += kThreads) {
    int x = col_depth(A, ca, k, gamma), y = row_depth(B, cb, k, gamma);
    da_c[k] = x;
    db_r[k] = y;
    mxe = max(mxe, x + y - 2);
  }
  mxa = wave_max_i32(mxa);
  mxb = wave_max_i32(mxb);
  mxe = wave_max_i32(mxe);
  if (lane == 0) {
    smax[wave][0] = mxa;
    smax[wave][1] = mxb;
    smax[wave][2] = mxe;
  }
  __syncthreads();
  int lev_a = 1, lev_b = 1, emax = 0;
  for (int w = 0; w < kWaves; ++w) {
    lev_a = max(lev_a, smax[w][0]);
    lev_b = max(lev_b, smax[w][1]);
    emax = max(emax, smax[w][2]);
  }
  lev_a = min<int>(lev_a, (int)L.levels);
  lev_b = min<int>(lev_b, (int)L.levels);
  emax = min<int>(emax, (int)L.segments - 1);
  __syncthreads();

  // --- 3. level-major line maps ------------------------------------------------
  int64_t m_alloc, n_alloc;
  const int64_t m_base = round_up(M, L.pad_m), n_base = round_up(N, L.pad_n);
  level_maps(da_r, M, lev_a, m_base, L.pad_m, reinterpret_cast<int32_t*>(e + L.lvl_a),
             reinterpret_cast<int32_t*>(e + L.amap), &m_alloc, scratch);
  __syncthreads();
  level_maps(db_c, N, lev_b, n_base, L.pad_n, reinterpret_cast<int32_t*>(e + L.lvl_b),
             reinterpret_cast<int32_t*>(e + L.bmap), &n_alloc, scratch);
  __syncthreads();

  // --- 4. exponent segments of K': triples (k, v, v') with v + v' = e ---------
  int32_t* kpre = reinterpret_cast<int32_t*>(e + L.kpre);
  int64_t seg_off = 0;
  for (int s = 0; s <= emax; ++s) {
    const int64_t per = ceil_div(K, kThreads);
    const int64_t k0 = min64(threadIdx.x * per, K), k1 = min64(k0 + per, K);
    int cnt = 0;
    for (int64_t k = k0; k < k1; ++k) {
      int lo = max(0, s - (db_r[k] - 1)), hi = min(da_c[k] - 1, s);
      cnt += max(0, hi - lo + 1);
    }
    int total;
    int ex = block_excl_scan(cnt, scratch, &total);
    int pos = ex;
    for (int64_t k = k0; k < k1; ++k) {
      kpre[(int64_t)s * (K + 1) + k] = pos;
      int lo = max(0, s - (db_r[k] - 1)), hi = min(da_c[k] - 1, s);
      pos += max(0, hi - lo + 1);
    }
    if (threadIdx.x == 0) {
      kpre[(int64_t)s * (K + 1) + K] = total;
      ph->seg_off[s] = seg_off;
      ph->seg_len[s] = total;
    }
    seg_off += round_up(total, kKPad);
  }
  if (threadIdx.x == 0) {
    ph->seg_off[emax + 1] = seg_off;
    ph->n_seg = emax + 1;
    ph->k_pad = seg_off;
    ph->m_base = m_base;
    ph->n_base = n_base;
    ph->m_alloc = m_alloc;
    ph->n_alloc = n_alloc;
    ph->lev_a = lev_a;
    ph->lev_b = lev_b;
    ph->emax = emax;
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3((unsigned)a.pl.batch), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace imu
