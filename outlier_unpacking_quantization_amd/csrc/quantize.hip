// Percentile scale, RTN quantization and outlier statistics (gfx950).
//
// Method: the summary page "IM-Unpack: Training and Inference with Arbitrarily
// Low Precision Integers".  The "Measured effects" table quantizes with RTN so
// that the p-percentile magnitude maps to beta (p = 95%); the summary keeps
// heavy hitters as out-of-range integers; "Approach" chooses the unpacking from
// per-line outlier counts.
//
// Every kernel streams the operands once in their stored orientation (16-byte
// loads, 64-lane waves over 512 stored columns, kRowsInFlight rows of loads
// issued before any is used).  One launch serves both operands of a GEMM and
// all batch entries: a small job table gives each (operand, entry) a contiguous
// range of workgroups.
//
// The statistics are formed in the float domain, which gives the same integers
// as rounding every element: with y = fl32(x r) and S = 2^(bits-1) (even),
// rne(y) needs two or more digits iff |y| >= S - 1/2, and the largest digit
// count of a line is the digit count of rne(max |y|) (rne and the digit count
// are monotone in |y|).  Row reductions use wave ballots; column reductions
// stay in registers, then LDS, then one global atomic per column per workgroup.
//
// Percentile: one pass builds an exact 32768-bin histogram of the 15-bit
// magnitude key per workgroup in LDS (128 KB), flushes the non-zero bins with
// global atomics, and the last workgroup to finish an entry selects the k-th
// key from the global histogram (arrival counter; no second launch).  fp32
// refines the low 16 key bits with two more 256-bin passes.
#include "common.h"
#include "kernels.h"

namespace imu {

namespace {

constexpr int kColsPerTile = 512;  // 64 lanes x 8 elements
constexpr int kRowsInFlight = 4;   // row loads issued per wave before use
constexpr int kCountThreads = 512;    // threads of the counting kernel (tiles are 512 columns wide)
constexpr int kResidualThreads = 256; // threads of the residual kernel

// Raw 32-bit patterns (fp32 bits; bf16 widened) of the 8 elements starting at
// column c0 of a stored row, and how many of them lie inside the row.  The
// loads are unconditional (indices clamped into the row) so that a caller can
// issue several rows' loads back to back; elements past the row are garbage
// and must be ignored through the returned count.
template <int DT>
__device__ inline int load8_bits(const typename Elem<DT>::T* row, int64_t c0, int64_t scols, int vec_ok,
                                 uint32_t w[8]) {
  const int n = (int)min64(max64(scols - c0, 0), 8);
  if (vec_ok) {  // scols % 8 == 0: a lane's 8 elements are all inside or all outside
    const int64_t cc = n ? c0 : scols - 8;
    if constexpr (DT == IMU_BF16) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + cc);
      const uint32_t p[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[2 * j] = p[j] << 16;
        w[2 * j + 1] = p[j] & 0xFFFF0000u;
      }
    } else {
      const uint4 a = *reinterpret_cast<const uint4*>(row + cc);
      const uint4 b = *reinterpret_cast<const uint4*>(row + cc + 4);
      w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
      w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    }
    return n;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t c = min64(c0 + j, scols - 1);
    if constexpr (DT == IMU_BF16) w[j] = (uint32_t)row[c] << 16;
    else w[j] = __float_as_uint(row[c]);
  }
  return n;
}

// The same in two halves, so that the loads of the next rows can be in flight
// while the current rows are processed: load_raw issues the loads (same
// clamping as above) into a vector value (bf16: pairs packed low/high as in
// memory), bits8 widens them once they are needed.
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v8u __attribute__((ext_vector_type(8)));
template <int DT>
struct RawOf {
  using V = v8u;
};
template <>
struct RawOf<IMU_BF16> {
  using V = v4u;
};
template <int DT>
__device__ __forceinline__ typename RawOf<DT>::V load_raw(const typename Elem<DT>::T* row, int64_t c0,
                                                          int64_t scols, int vec_ok) {
  typename RawOf<DT>::V u = 0;
  if (vec_ok) {
    const int64_t cc = c0 < scols ? c0 : scols - 8;
    const uint4 a = *reinterpret_cast<const uint4*>(row + cc);
    u.s0 = a.x; u.s1 = a.y; u.s2 = a.z; u.s3 = a.w;
    if constexpr (DT == IMU_F32) {
      const uint4 b = *reinterpret_cast<const uint4*>(row + cc + 4);
      u.s4 = b.x; u.s5 = b.y; u.s6 = b.z; u.s7 = b.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t c = min64(c0 + j, scols - 1);
      if constexpr (DT == IMU_BF16) u[j >> 1] |= (uint32_t)row[c] << (16 * (j & 1));
      else u[j] = __float_as_uint(row[c]);
    }
  }
  return u;
}
template <int DT>
__device__ __forceinline__ void bits8(typename RawOf<DT>::V u, uint32_t (&w)[8]) {
  if constexpr (DT == IMU_BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[2 * j] = u[j] << 16;
      w[2 * j + 1] = u[j] & 0xFFFF0000u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = u[j];
  }
}

// Sum over the wave of a per-lane value in [0, 16), by bit planes of ballots.
__device__ inline int wave_sum_small(int v) {
  int s = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) s += __popcll(__ballot((v >> b) & 1)) << b;
  return s;
}
// Max over the wave of a per-lane value in [0, 32), bit by bit from the top.
__device__ inline int wave_max_small(int v) {
  int m = 0;
#pragma unroll
  for (int bit = 16; bit > 0; bit >>= 1)
    if (__ballot(v >= m + bit)) m += bit;
  return m;
}

// Digit count of rne(a) for a = max |x r| >= 0 (a finite and below 2^31).
template <int BITS>
__device__ inline int digits_of_max(float a) {
  return digit_count<BITS>((uint32_t)__builtin_rintf(a));
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += step) p[i] = v;
}

__global__ void fill_2d_kernel(int32_t* p, int64_t rows, int64_t cols, int64_t ld) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y)
    for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < cols;
         c += (int64_t)gridDim.x * blockDim.x)
      p[r * ld + c] = 0;
}

// Which (operand, batch entry) a workgroup serves, and its index inside that entry.
struct JobPos {
  int op, entry, local, count;
};
__device__ inline JobPos find_job(const QuantJobs& J, int bid) {
  JobPos p{0, 0, 0, 0};
  for (int o = 0; o < J.nops; ++o) {
    const int per = J.op[o].wgs_per_entry;
    const int end = J.op[o].wg_begin + per * J.op[o].batch;
    if (bid < end) {
      const int rel = bid - J.op[o].wg_begin;
      p.op = o;
      p.entry = rel / per;
      p.local = rel % per;
      p.count = per;
      return p;
    }
  }
  return p;  // count 0: not reached for a consistent grid
}

// Select the k-th smallest key of the global histogram (one workgroup of 1024).
// pass 0: 32768 bins (key bits 30..16); pass 1/2: 256 bins (15..8 / 7..0).
// The caller has passed an acquire fence after the arrival counter, so plain
// loads see every other workgroup's flush.  `stage` (>= NB words of LDS) turns
// the coalesced global reads into per-thread runs of consecutive bins.
__device__ void select_from_hist(uint8_t* st, int64_t hist_off, int64_t nelem, int pass, int final_pass,
                                 int beta, int p_num, int p_den, unsigned long long* part,
                                 uint32_t* found, uint32_t* stage) {
  StatsHeader* hd = reinterpret_cast<StatsHeader*>(st);
  uint32_t* gh = reinterpret_cast<uint32_t*>(st + hist_off);
  const int NB = pass == 0 ? kHistBins : 256;
  const int per = (NB + 1023) / 1024;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  unsigned long long k;
  if (pass == 0) {
    // nearest rank: k = ceil(p_num * N / p_den), clamped to [1, N]
    unsigned long long num = (unsigned long long)p_num * (unsigned long long)nelem;
    k = (num + (unsigned long long)p_den - 1) / (unsigned long long)p_den;
    if (k < 1) k = 1;
    if (k > (unsigned long long)nelem) k = nelem;
  } else {
    k = hd->sel_rank;
  }
  __syncthreads();  // every thread is done with its own use of `stage`
  {
    uint32_t tmp[32];  // all loads in flight before the first LDS store
#pragma unroll
    for (int i = 0; i < 32; ++i) tmp[i] = gh[min(t + i * 1024, NB - 1)];
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (t + i * 1024 < NB) stage[t + i * 1024] = tmp[i];
  }
  __syncthreads();
  // this thread's run of `per` consecutive bins
  const int bin0 = t * per, nbin = max(0, min(per, NB - bin0));
  unsigned long long s = 0;
  for (int i = 0; i < nbin; ++i) s += stage[bin0 + i];
  // block-wide inclusive scan of s: within waves, then over wave totals
  unsigned long long incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    unsigned lo = __shfl_up((unsigned)(incl & 0xFFFFFFFFull), o, 64);
    unsigned hi = __shfl_up((unsigned)(incl >> 32), o, 64);
    if (lane >= o) incl += ((unsigned long long)hi << 32) | lo;
  }
  if (lane == 63) part[wave] = incl;
  if (t == 0) found[0] = 0xFFFFFFFFu;
  __syncthreads();
  unsigned long long wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += part[w];
  incl += wbase;
  const unsigned long long excl = incl - s;
  if (excl < k && k <= incl) {
    unsigned long long run = excl;
    for (int i = 0; i < nbin; ++i) {
      const uint32_t c = stage[bin0 + i];
      if (run + c >= k) {
        found[0] = (uint32_t)(bin0 + i);
        part[16] = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  if (t == 0) {
    uint32_t bin = found[0];
    unsigned long long below = part[16];
    if (bin == 0xFFFFFFFFu) {  // cannot happen for a consistent histogram
      hd->status |= kStatusNonfinite;
      bin = 0;
      below = 0;
    }
    const uint32_t rank = (uint32_t)(k - below);
    const uint32_t prefix = pass == 0 ? bin : ((hd->sel_prefix << 8) | bin);
    if (!final_pass) {
      hd->sel_prefix = prefix;
      hd->sel_rank = rank;
    } else {
      const uint32_t key = pass == 0 ? (prefix << 16) : prefix;  // pass 0 is final only for bf16
      const float kth = __uint_as_float(key);
      const float alpha = kth > 0.f ? kth : __uint_as_float(hd->maxkey);
      const int status = hd->status;
      hd->kth = kth;
      hd->alpha = alpha;
      if (alpha > 0.f && !(status & kStatusNonfinite)) {
        // a binary64 quotient rounded once more to binary32 is the correctly
        // rounded binary32 quotient (53 >= 2*24 + 2)
        hd->r = (float)((double)beta / (double)alpha);
        hd->s = (float)((double)alpha / (double)beta);
      } else {
        hd->r = 0.f;
        hd->s = 0.f;
      }
    }
  }
  if (!final_pass) {
    __syncthreads();
    for (int i = t; i < 256; i += blockDim.x) gh[i] = 0;  // the next pass uses 256 bins
  }
}

// --- percentile histogram + fused selection ---------------------------------
template <int DT, int NB, int PASS>
__global__ __launch_bounds__(1024) void hist_kernel(QuantJobs J, int final_pass) {
  using T = typename Elem<DT>::T;
  __shared__ uint32_t h[NB];
  __shared__ uint32_t smax;
  __shared__ int sbad;
  __shared__ uint32_t slast;
  __shared__ unsigned long long part[17];
  __shared__ uint32_t found[1];
  const JobPos jp = find_job(J, blockIdx.x);
  if (jp.count == 0) return;
  const StreamArgs& a = J.op[jp.op].s;
  const T* xb = static_cast<const T*>(a.x) + jp.entry * a.bstride;
  uint8_t* st = a.stats + jp.entry * a.stats_stride;
  StatsHeader* hd = reinterpret_cast<StatsHeader*>(st);
  uint32_t* gh = reinterpret_cast<uint32_t*>(st + a.hist);

  for (int i = threadIdx.x; i < NB; i += blockDim.x) h[i] = 0;
  if (threadIdx.x == 0) {
    smax = 0;
    sbad = 0;
  }
  __syncthreads();

  const uint32_t prefix = PASS == 0 ? 0u : hd->sel_prefix;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  // work units: (stored row, 512-column tile); this workgroup takes a contiguous share
  const uint32_t ctiles = (uint32_t)ceil_div(a.scols, kColsPerTile);
  const int64_t units = a.srows * (int64_t)ctiles;
  const int64_t u0 = units * jp.local / jp.count, u1 = units * (jp.local + 1) / jp.count;
  uint32_t mx = 0;
  int bad = 0;
  auto count = [&](uint32_t bits) {
    const uint32_t k = bits & 0x7FFFFFFFu;
    if constexpr (PASS == 0) {
      mx = max(mx, k);
      bad |= (k >= 0x7F800000u);
      atomicAdd(&h[(k >> 16) & (NB - 1)], 1u);
    } else if constexpr (PASS == 1) {
      if ((k >> 16) == prefix) atomicAdd(&h[(k >> 8) & 0xFFu], 1u);
    } else {
      if ((k >> 8) == prefix) atomicAdd(&h[k & 0xFFu], 1u);
    }
  };
  // two groups of kRowsInFlight units alternate: one group's loads fly while
  // the other is counted
  const int64_t ustep = (int64_t)nwave * kRowsInFlight;
  typename RawOf<DT>::V g0[kRowsInFlight], g1[kRowsInFlight];
#define IMU_ISSUE(g, ub_)                                                                          \
  _Pragma("unroll") for (int rr = 0; rr < kRowsInFlight; ++rr) {                                    \
    const uint32_t u_ = (uint32_t)min64((ub_) + rr, u1 - 1); /* clamped: loads stay unconditional */ \
    const uint32_t sr_ = u_ / ctiles, ct_ = u_ - sr_ * ctiles;                                      \
    g[rr] = load_raw<DT>(xb + (int64_t)sr_ * a.ld, (int64_t)ct_ * kColsPerTile + lane * 8, a.scols, a.vec_ok); \
  }
#define IMU_PROCESS(g, ub_)                                                                        \
  _Pragma("unroll") for (int rr = 0; rr < kRowsInFlight; ++rr) {                                   \
    if ((ub_) + rr < u1) { /* uniform across the wave */                                           \
      const uint32_t u_ = (uint32_t)((ub_) + rr);                                                  \
      const uint32_t sr_ = u_ / ctiles, ct_ = u_ - sr_ * ctiles;                                   \
      const int64_t c0_ = (int64_t)ct_ * kColsPerTile + lane * 8;                                  \
      uint32_t w[8];                                                                               \
      bits8<DT>(g[rr], w);                                                                         \
      if ((int64_t)(ct_ + 1) * kColsPerTile <= a.scols) { /* the whole tile lies inside the row */ \
        _Pragma("unroll") for (int j = 0; j < 8; ++j) count(w[j]);                                 \
      } else {                                                                                     \
        const int n_ = (int)min64(max64(a.scols - c0_, 0), 8);                                     \
        _Pragma("unroll") for (int j = 0; j < 8; ++j) if (j < n_) count(w[j]);                     \
      }                                                                                            \
    }                                                                                              \
  }
  int64_t ub = u0 + (int64_t)wave * kRowsInFlight;
  IMU_ISSUE(g0, ub);
  for (; ub < u1; ub += 2 * ustep) {
    IMU_ISSUE(g1, ub + ustep);
    IMU_PROCESS(g0, ub);
    if (ub + ustep >= u1) break;
    IMU_ISSUE(g0, ub + 2 * ustep);
    IMU_PROCESS(g1, ub + ustep);
  }
#undef IMU_ISSUE
#undef IMU_PROCESS
  if (PASS == 0) {
    mx = wave_max_u32(mx);
    bad = wave_max_i32(bad);
    if (lane == 0) {
      atomicMax(&smax, mx);
      if (bad) atomicOr(&sbad, 1);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < NB; i += blockDim.x) {
    const uint32_t c = h[i];
    if (c) atomicAdd(&gh[i], c);
  }
  if (PASS == 0 && threadIdx.x == 0) {
    atomicMax(&hd->maxkey, smax);
    if (sbad) atomicOr(&hd->status, kStatusNonfinite);
  }
  // The last workgroup of this entry selects.  Every flush above is a
  // device-scope atomic; each thread waits until its own have completed before
  // the arrival counter moves (a device-scope release fence would also write
  // back this XCD's whole L2, which costs tens of us across the grid).  The
  // last workgroup then acquires at device scope, which drops stale cached
  // lines before it reads the histogram.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) slast = atomicAdd(&hd->arrive, 1u) == (uint32_t)(jp.count - 1);
  __syncthreads();
  if (!slast) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (threadIdx.x == 0) hd->arrive = 0;  // ready for the next pass (stream ordered)
  select_from_hist(st, a.hist, a.srows * a.scols, PASS, final_pass, a.beta, a.p_num, a.p_den, part, found, h);
}

// --- fused RTN + outlier statistics -------------------------------------------
// Tile: 512 stored columns x rows_per_wg stored rows.
template <int DT, int BITS, bool QOUT>
__global__ __launch_bounds__(kCountThreads) void round_count_kernel(QuantJobs J, int32_t* q0, int32_t* q1) {
  using T = typename Elem<DT>::T;
  constexpr float kThr = (float)(1 << (BITS - 1)) - 0.5f;  // |y| >= kThr <=> rne(y) out of range
  __shared__ int lcnt[kColsPerTile];
  __shared__ uint32_t lmax[kColsPerTile];  // max |y| as fp32 bits (monotone for y >= 0)
  __shared__ unsigned long long ltot;
  __shared__ int lbad;
  const JobPos jp = find_job(J, blockIdx.x);
  if (jp.count == 0) return;
  const QuantOp& op = J.op[jp.op];
  const StreamArgs& a = op.s;
  const int b = jp.entry;
  const int64_t ctiles = ceil_div(a.scols, kColsPerTile);
  const int64_t ct = jp.local % ctiles, rb = jp.local / ctiles;
  const T* xb = static_cast<const T*>(a.x) + b * a.bstride;
  uint8_t* st = a.stats + b * a.stats_stride;
  StatsHeader* hd = reinterpret_cast<StatsHeader*>(st);
  int32_t* srow_oob = reinterpret_cast<int32_t*>(st + a.srow_oob);
  int32_t* scol_oob = reinterpret_cast<int32_t*>(st + a.scol_oob);
  int32_t* srow_max = reinterpret_cast<int32_t*>(st + a.srow_maxdig);
  int32_t* scol_max = reinterpret_cast<int32_t*>(st + a.scol_maxdig);
  for (int i = threadIdx.x; i < kColsPerTile; i += blockDim.x) {
    lcnt[i] = 0;
    lmax[i] = 0;
  }
  if (threadIdx.x == 0) {
    ltot = 0;
    lbad = 0;
  }
  __syncthreads();
  const float r = hd->r;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int64_t cbase = ct * kColsPerTile;
  const int64_t c0 = cbase + lane * 8;
  const int64_t r0 = rb * op.rows_per_wg;
  const int64_t r1 = min64(r0 + op.rows_per_wg, a.srows);
  int ccnt[8];
  float cmax[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ccnt[j] = 0;
    cmax[j] = -1.f;  // below any |y|; marks "no element seen"
  }
  int tot = 0;
  float amax = 0.f;
  const int64_t R = a.srows, C = a.scols;
  int32_t* qb = nullptr;  // codes of this operand, if they were asked for
  if constexpr (QOUT) {
    int32_t* qo = jp.op == 0 ? q0 : q1;
    if (qo) qb = qo + b * R * C;
  }
  const bool tile_whole = cbase + kColsPerTile <= a.scols;  // no element of this tile is past the row
  const int nin = (int)min64(max64(a.scols - c0, 0), 8);      // this lane's elements inside a row
  // rows of one group: kRowsInFlight consecutive stored rows per wave; two
  // groups alternate so that one group's loads fly while the other is counted
#define IMU_ISSUE(g, sb_)                                                                          \
  _Pragma("unroll") for (int rr = 0; rr < kRowsInFlight; ++rr)                                      \
      g[rr] = load_raw<DT>(xb + min64((sb_) + rr, r1 - 1) * a.ld, c0, a.scols, a.vec_ok);
  // per row: RTN of its elements, out-of-range count and largest digit count;
  // columns keep their counts and maxima in registers
  auto row_stats = [&](const uint32_t (&w)[8], int64_t sr) __attribute__((always_inline)) {
    int lc = 0;
    float lm = 0.f;
    auto elem = [&](int j) {
      const float y = __uint_as_float(w[j]) * r;
      const float ay = __builtin_fabsf(y);
      const int o = ay >= kThr;
      lc += o;
      lm = __builtin_fmaxf(lm, ay);
      ccnt[j] += o;
      cmax[j] = __builtin_fmaxf(cmax[j], ay);
      if (QOUT && qb) {
        const int64_t c = c0 + j;
        const int32_t q = ay < 2147483648.0f ? (int32_t)__builtin_rintf(y) : 0;
        if (!a.transposed) qb[sr * C + c] = q;
        else qb[c * R + sr] = q;
      }
    };
    if (tile_whole) {
#pragma unroll
      for (int j = 0; j < 8; ++j) elem(j);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < nin) elem(j);
    }
    amax = __builtin_fmaxf(amax, lm);
    const int ld = lm < 2147483648.0f ? digits_of_max<BITS>(lm) : 1;
    const int rc = wave_sum_small(lc);
    const int rm = wave_max_small(ld);
    if (lane == 0) {
      if (rc) atomicAdd(&srow_oob[sr], rc);
      atomicMax(&srow_max[sr], rm);
      tot += rc;
    }
  };
#define IMU_PROCESS(g, sb_)                                                                        \
  _Pragma("unroll") for (int rr = 0; rr < kRowsInFlight; ++rr) {                                   \
    if ((sb_) + rr < r1) { /* uniform across the wave */                                           \
      uint32_t w[8];                                                                               \
      bits8<DT>(g[rr], w);                                                               \
      row_stats(w, (sb_) + rr);                                                                    \
    }                                                                                              \
  }
  const int64_t gstep = (int64_t)nwave * kRowsInFlight;
  typename RawOf<DT>::V g0[kRowsInFlight], g1[kRowsInFlight];
  int64_t sb = r0 + (int64_t)wave * kRowsInFlight;
  IMU_ISSUE(g0, sb);
  for (; sb < r1; sb += 2 * gstep) {
    IMU_ISSUE(g1, sb + gstep);
    IMU_PROCESS(g0, sb);
    if (sb + gstep >= r1) break;
    IMU_ISSUE(g0, sb + 2 * gstep);
    IMU_PROCESS(g1, sb + gstep);
  }
#undef IMU_ISSUE
#undef IMU_PROCESS
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (cmax[j] >= 0.f) {
      if (ccnt[j]) atomicAdd(&lcnt[lane * 8 + j], ccnt[j]);
      atomicMax(&lmax[lane * 8 + j], __float_as_uint(cmax[j]) + 1u);  // +1: seen even when |y| = 0
    }
  }
  if (lane == 0 && tot) atomicAdd(&ltot, (unsigned long long)tot);
  if (!(amax < 2147483648.0f)) atomicOr(&lbad, 1);  // also catches NaN
  __syncthreads();
  for (int i = threadIdx.x; i < kColsPerTile; i += blockDim.x) {
    const int64_t c = cbase + i;
    const uint32_t m = lmax[i];
    if (c < a.scols && m) {
      const float cm = __uint_as_float(m - 1u);
      if (lcnt[i]) atomicAdd(&scol_oob[c], lcnt[i]);
      atomicMax(&scol_max[c], cm < 2147483648.0f ? digits_of_max<BITS>(cm) : 1);
    }
  }
  if (threadIdx.x == 0) {
    if (ltot) atomicAdd(&hd->total, ltot);
    if (lbad) atomicOr(&hd->status, kStatusRange);
  }
}

// --- Mix residual: largest digit count of each line outside heavy lines --------
// A stored column is heavy when scol_oob * scols > gamma * T, a stored row when
// srow_oob * srows > gamma * T.  srow_res gets the max over non-heavy columns,
// scol_res the max over non-heavy rows.
template <int DT, int BITS>
__global__ __launch_bounds__(kResidualThreads) void residual_kernel(QuantJobs J) {
  using T = typename Elem<DT>::T;
  __shared__ uint32_t lmax[kColsPerTile];
  const JobPos jp = find_job(J, blockIdx.x);
  if (jp.count == 0) return;
  const QuantOp& op = J.op[jp.op];
  const StreamArgs& a = op.s;
  const int b = jp.entry;
  const int64_t ctiles = ceil_div(a.scols, kColsPerTile);
  const int64_t ct = jp.local % ctiles, rb = jp.local / ctiles;
  const T* xb = static_cast<const T*>(a.x) + b * a.bstride;
  uint8_t* st = a.stats + b * a.stats_stride;
  const StatsHeader* hd = reinterpret_cast<const StatsHeader*>(st);
  const int32_t* srow_oob = reinterpret_cast<const int32_t*>(st + a.srow_oob);
  const int32_t* scol_oob = reinterpret_cast<const int32_t*>(st + a.scol_oob);
  int32_t* srow_res = reinterpret_cast<int32_t*>(st + a.srow_res);
  int32_t* scol_res = reinterpret_cast<int32_t*>(st + a.scol_res);
  for (int i = threadIdx.x; i < kColsPerTile; i += blockDim.x) lmax[i] = 0;
  __syncthreads();
  const float r = hd->r;
  const long long gT = (long long)a.gamma * (long long)hd->total;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int64_t cbase = ct * kColsPerTile;
  const int64_t c0 = cbase + lane * 8;
  const int64_t r0 = rb * op.rows_per_wg;
  const int64_t r1 = min64(r0 + op.rows_per_wg, a.srows);
  bool colheavy[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t c = c0 + j;
    colheavy[j] = c < a.scols && (long long)scol_oob[c] * a.scols > gT;
  }
  float cmax[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) cmax[j] = -1.f;
  const bool tile_whole = cbase + kColsPerTile <= a.scols;
  const int nin = (int)min64(max64(a.scols - c0, 0), 8);  // this lane's elements inside a row
  // two groups of kRowsInFlight rows alternate: one group's loads (elements
  // and row counts) fly while the other is reduced
#define IMU_ISSUE(g, oob, sb_)                                                                     \
  _Pragma("unroll") for (int rr = 0; rr < kRowsInFlight; ++rr) {                                    \
    const int64_t sr_ = min64((sb_) + rr, r1 - 1);                                                  \
    g[rr] = load_raw<DT>(xb + sr_ * a.ld, c0, a.scols, a.vec_ok);                                   \
    oob[rr] = srow_oob[sr_];                                                                        \
  }
  auto row_res = [&](const uint32_t (&w)[8], int64_t sr, bool rowheavy) __attribute__((always_inline)) {
    float lm = -1.f;
    auto elem = [&](int j) {
      const float ay = __builtin_fabsf(__uint_as_float(w[j]) * r);
      if (!colheavy[j]) lm = __builtin_fmaxf(lm, ay);
      if (!rowheavy) cmax[j] = __builtin_fmaxf(cmax[j], ay);
    };
    if (tile_whole) {
#pragma unroll
      for (int j = 0; j < 8; ++j) elem(j);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < nin) elem(j);
    }
    const int ld = lm < 0.f ? 0 : (lm < 2147483648.0f ? digits_of_max<BITS>(lm) : 1);
    const int rm = wave_max_small(ld);
    if (lane == 0 && rm) atomicMax(&srow_res[sr], rm);
  };
#define IMU_PROCESS(g, oob, sb_)                                                                   \
  _Pragma("unroll") for (int rr = 0; rr < kRowsInFlight; ++rr) {                                   \
    if ((sb_) + rr < r1) { /* uniform across the wave */                                           \
      uint32_t w[8];                                                                               \
      bits8<DT>(g[rr], w);                                                                         \
      row_res(w, (sb_) + rr, (long long)oob[rr] * a.srows > gT);                                   \
    }                                                                                              \
  }
  const int64_t gstep = (int64_t)nwave * kRowsInFlight;
  typename RawOf<DT>::V g0[kRowsInFlight], g1[kRowsInFlight];
  int o0[kRowsInFlight], o1[kRowsInFlight];
  int64_t sb = r0 + (int64_t)wave * kRowsInFlight;
  IMU_ISSUE(g0, o0, sb);
  for (; sb < r1; sb += 2 * gstep) {
    IMU_ISSUE(g1, o1, sb + gstep);
    IMU_PROCESS(g0, o0, sb);
    if (sb + gstep >= r1) break;
    IMU_ISSUE(g0, o0, sb + 2 * gstep);
    IMU_PROCESS(g1, o1, sb + gstep);
  }
#undef IMU_ISSUE
#undef IMU_PROCESS
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (cmax[j] >= 0.f) atomicMax(&lmax[lane * 8 + j], __float_as_uint(cmax[j]) + 1u);
  __syncthreads();
  for (int i = threadIdx.x; i < kColsPerTile; i += blockDim.x) {
    const int64_t c = cbase + i;
    const uint32_t m = lmax[i];
    if (c < a.scols && m) {
      const float cm = __uint_as_float(m - 1u);
      atomicMax(&scol_res[c], cm < 2147483648.0f ? digits_of_max<BITS>(cm) : 1);
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_fill_u32(void* p, uint32_t v, int64_t nwords, hipStream_t s) {
  if (nwords <= 0) return hipSuccess;
  const int64_t blocks = min64(ceil_div(nwords, 256), 4096);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint32_t*>(p), v,
                     nwords);
  return hipGetLastError();
}

hipError_t launch_fill_2d(int32_t* p, int64_t rows, int64_t cols, int64_t ld, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  dim3 grid((unsigned)min64(ceil_div(cols, 256), 64), (unsigned)min64(rows, 4096));
  hipLaunchKernelGGL(fill_2d_kernel, grid, dim3(256), 0, s, p, rows, cols, ld);
  return hipGetLastError();
}

// Histogram: about kHistWgs workgroups in total, shared in proportion to size.
static int plan_hist(QuantJobs& J) {
  constexpr int kHistWgs = 256;
  double total = 0;
  for (int o = 0; o < J.nops; ++o) total += (double)J.op[o].s.srows * J.op[o].s.scols * J.op[o].batch;
  int begin = 0;
  for (int o = 0; o < J.nops; ++o) {
    QuantOp& q = J.op[o];
    const double el = (double)q.s.srows * q.s.scols;
    const int64_t units = q.s.srows * ceil_div(q.s.scols, kColsPerTile);
    int64_t per = (int64_t)(kHistWgs * el / total + 0.5);
    per = min64(max64(per, 1), max64(units, 1));
    q.wgs_per_entry = (int)per;
    q.wg_begin = begin;
    begin += (int)per * q.batch;
  }
  return begin;
}

hipError_t launch_hist(int dtype, QuantJobs J, int pass, int final_pass, hipStream_t s) {
  const int grid = plan_hist(J);
  if (dtype == IMU_BF16) {
    hipLaunchKernelGGL((hist_kernel<IMU_BF16, kHistBins, 0>), dim3(grid), dim3(1024), 0, s, J, final_pass);
  } else if (pass == 0) {
    hipLaunchKernelGGL((hist_kernel<IMU_F32, kHistBins, 0>), dim3(grid), dim3(1024), 0, s, J, final_pass);
  } else if (pass == 1) {
    hipLaunchKernelGGL((hist_kernel<IMU_F32, 256, 1>), dim3(grid), dim3(1024), 0, s, J, final_pass);
  } else {
    hipLaunchKernelGGL((hist_kernel<IMU_F32, 256, 2>), dim3(grid), dim3(1024), 0, s, J, final_pass);
  }
  return hipGetLastError();
}

// Count kernels: tiles of 512 columns x rows_per_wg rows, about kCountWgs workgroups
// in total (fewer workgroups: fewer column atomics; more: more loads in flight).
static int plan_tiles(QuantJobs& J, int kCountWgs) {
  double total = 0;
  for (int o = 0; o < J.nops; ++o) total += (double)J.op[o].s.srows * J.op[o].s.scols * J.op[o].batch;
  int begin = 0;
  for (int o = 0; o < J.nops; ++o) {
    QuantOp& q = J.op[o];
    const int64_t ctiles = ceil_div(q.s.scols, kColsPerTile);
    const double el = (double)q.s.srows * q.s.scols * q.batch;
    const int64_t want = max64((int64_t)(kCountWgs * el / total + 0.5), 1);  // workgroups for this operand
    int64_t rblocks = max64(want / (ctiles * q.batch), 1);
    int64_t rpw = ceil_div(q.s.srows, rblocks);
    rpw = max64(rpw, 4);
    rblocks = ceil_div(q.s.srows, rpw);
    q.rows_per_wg = (int)rpw;
    q.wgs_per_entry = (int)(rblocks * ctiles);
    q.wg_begin = begin;
    begin += q.wgs_per_entry * q.batch;
  }
  return begin;
}

template <int DT>
static hipError_t round_count_dt(int bits, const QuantJobs& J, int grid, int32_t* q0, int32_t* q1,
                                 hipStream_t s) {
  switch (bits) {
#define IMU_RC(B)                                                                                  \
  case B:                                                                                          \
    if (q0 || q1)                                                                                  \
      hipLaunchKernelGGL((round_count_kernel<DT, B, true>), dim3(grid), dim3(kCountThreads), 0, s, J, q0, q1); \
    else                                                                                           \
      hipLaunchKernelGGL((round_count_kernel<DT, B, false>), dim3(grid), dim3(kCountThreads), 0, s, J, q0, q1); \
    break;
    IMU_RC(2) IMU_RC(3) IMU_RC(4) IMU_RC(5) IMU_RC(6) IMU_RC(7) IMU_RC(8)
#undef IMU_RC
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_round_count(int dtype, int bits, QuantJobs J, int32_t* q0, int32_t* q1, hipStream_t s) {
  const int grid = plan_tiles(J, 512);
  return dtype == IMU_BF16 ? round_count_dt<IMU_BF16>(bits, J, grid, q0, q1, s)
                           : round_count_dt<IMU_F32>(bits, J, grid, q0, q1, s);
}

template <int DT>
static hipError_t residual_dt(int bits, const QuantJobs& J, int grid, hipStream_t s) {
  switch (bits) {
#define IMU_RS(B)                                                                                  \
  case B:                                                                                          \
    hipLaunchKernelGGL((residual_kernel<DT, B>), dim3(grid), dim3(kResidualThreads), 0, s, J);     \
    break;
    IMU_RS(2) IMU_RS(3) IMU_RS(4) IMU_RS(5) IMU_RS(6) IMU_RS(7) IMU_RS(8)
#undef IMU_RS
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_residual(int dtype, int bits, QuantJobs J, hipStream_t s) {
  const int grid = plan_tiles(J, 1024);  // more, shorter workgroups hide the per-row count loads
  return dtype == IMU_BF16 ? residual_dt<IMU_BF16>(bits, J, grid, s) : residual_dt<IMU_F32>(bits, J, grid, s);
}

}  // namespace imu
