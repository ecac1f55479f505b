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
// The statistics give the same integers as rounding every element: with
// y = fl32(x r) and S = 2^(bits-1) (even), rne(y) needs two or more digits iff
// |y| >= S - 1/2, and the largest digit count of a line is the digit count of
// rne(max |y|) (rne and the digit count are monotone in |y|).  Since
// fl32(|x| r) is itself monotone in |x|, both are decided on integer magnitude
// keys (see "magnitude keys" below) with one product per line.  Row reductions
// use DPP; column reductions stay in registers, then LDS, then one global
// atomic per column per workgroup.
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

// Raw 32-bit patterns of the 8 elements starting at column c0 of a stored row,
// in two halves, so that the loads of the next rows can be in flight while the
// current rows are processed: load_raw issues the loads into a vector value
// (bf16: pairs packed low/high as in memory; fp32: the bits), bits8 widens
// them (bf16 to fp32 bits) once they are needed.  The loads are unconditional
// (indices clamped into the row) so that several rows' loads can be issued
// back to back; elements past the row are garbage for the caller to ignore.
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
// VEC (scols % 8 == 0 and aligned rows): one 16-byte load (two for fp32) per
// lane; otherwise 8 element loads.  A compile-time choice, so that the
// compiler can count the loads in flight exactly (a run-time branch between
// the two makes it wait for all of them before any use).
template <int DT, bool VEC>
__device__ __forceinline__ typename RawOf<DT>::V load_raw(const typename Elem<DT>::T* row, int64_t c0,
                                                          int64_t scols) {
  typename RawOf<DT>::V u = 0;
  if constexpr (VEC) {
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


__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += step) p[i] = v;
}

__global__ void fill_2d_kernel(int32_t* p, int64_t rows, int64_t cols, int64_t ld, int64_t bstride) {
  p += blockIdx.z * bstride;
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

// Inclusive scan of a 64-bit value over the 64 lanes of a wave.
__device__ inline unsigned long long wave_incl_scan_u64(unsigned long long v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned lo = __shfl_up((unsigned)(v & 0xFFFFFFFFull), o, 64);
    const unsigned hi = __shfl_up((unsigned)(v >> 32), o, 64);
    if (lane >= o) v += ((unsigned long long)hi << 32) | lo;
  }
  return v;
}

// Result of a selection pass: the k-th smallest key lies in bin `bin`, with
// `below` keys in lower bins.  Not final: the prefix and the rank left for the
// next pass; final: kth, alpha (the largest |x| when kth is 0), r and s.
__device__ inline void apply_selection(StatsHeader* hd, int pass, int final_pass, uint32_t bin,
                                       unsigned long long below, unsigned long long k, int beta,
                                       uint32_t maxkey, int status) {
  if (bin == 0xFFFFFFFFu) {  // cannot happen for a consistent histogram
    hd->status |= kStatusNonfinite;
    status |= kStatusNonfinite;
    bin = 0;
    below = 0;
  }
  const uint32_t rank = (uint32_t)(k - below);
  const uint32_t prefix = pass == 0 ? bin : ((hd->sel_prefix << 8) | bin);
  if (!final_pass) {
    hd->sel_prefix = prefix;
    hd->sel_rank = rank;
    return;
  }
  const uint32_t key = pass == 0 ? (prefix << 16) : prefix;  // pass 0 is final only for bf16
  const float kth = __uint_as_float(key);
  const float alpha = kth > 0.f ? kth : __uint_as_float(maxkey);
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

// nearest rank: k = ceil(p_num * N / p_den), clamped to [1, N]
__device__ inline unsigned long long nearest_rank(int64_t nelem, int p_num, int p_den) {
  const unsigned long long num = (unsigned long long)p_num * (unsigned long long)nelem;
  unsigned long long k = (num + (unsigned long long)p_den - 1) / (unsigned long long)p_den;
  if (k < 1) k = 1;
  if (k > (unsigned long long)nelem) k = nelem;
  return k;
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
    k = nearest_rank(nelem, p_num, p_den);
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
  if (t == 0) apply_selection(hd, pass, final_pass, found[0], part[16], k, beta, hd->maxkey, hd->status);
  if (!final_pass) {
    __syncthreads();
    for (int i = t; i < 256; i += blockDim.x) gh[i] = 0;  // the next pass uses 256 bins
  }
}

// --- magnitude keys ---------------------------------------------------------
// For r >= 0, fl32(|x| r) is non-decreasing in |x|, and so is the digit count
// of its rounding.  The statistics therefore need no product per element:
// rne(x r) is out of range exactly when |x| is at least the smallest
// magnitude whose product reaches 2^(bits-1) - 1/2, and the largest digit
// count of a line is the digit count of its largest |x| (one product per
// line).  Magnitudes are compared as integer keys, the bit pattern without the
// sign (which orders non-negative floats): bf16 keys have 15 bits and sit two
// to a dword (packed 16-bit arithmetic), fp32 keys have 31.
typedef uint16_t v2u16 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pk_add_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2u16, a) + __builtin_bit_cast(v2u16, b));
}
__device__ inline uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_elementwise_max(__builtin_bit_cast(v2u16, a), __builtin_bit_cast(v2u16, b)));
}

template <int DT>
struct KeyOps {  // fp32: one 31-bit key per dword
  static constexpr int NW = 8;  // dwords of a lane's 8 elements
  static constexpr int NB = 31;
  static constexpr uint32_t kMask = 0x7FFFFFFFu;
  static __device__ float value(uint32_t k) { return __uint_as_float(k); }
};
template <>
struct KeyOps<IMU_BF16> {  // bf16: two 15-bit keys per dword (element 2d low, 2d+1 high)
  static constexpr int NW = 4;
  static constexpr int NB = 15;
  static constexpr uint32_t kMask = 0x7FFF7FFFu;
  static __device__ float value(uint32_t k) { return __uint_as_float(k << 16); }
};

// Key masks of a lane whose first n of 8 elements lie inside the row.
template <int DT>
__device__ inline void key_masks(int n, uint32_t (&km)[KeyOps<DT>::NW]) {
  if constexpr (DT == IMU_BF16) {
#pragma unroll
    for (int d = 0; d < 4; ++d) km[d] = (2 * d < n ? 0x7FFFu : 0u) | (2 * d + 1 < n ? 0x7FFF0000u : 0u);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) km[j] = j < n ? 0x7FFFFFFFu : 0u;
  }
}

// Smallest key k with fl32(value(k) r) >= thr (2^NB if there is none).  The
// keys whose product stays below thr form a prefix of the key order (key 0 is
// one of them: its product is 0), so its last element is found 6 bits at a
// time, the 64 lanes trying the 64 values of the next 6 bits.
template <int DT>
__device__ inline uint32_t key_threshold(float r, float thr) {
  constexpr int NB = KeyOps<DT>::NB;
  const uint64_t lane = threadIdx.x & 63;
  uint32_t p = 0;
#pragma unroll
  for (int s = (NB - 1) / 6 * 6; s >= 0; s -= 6) {
    const uint64_t cand = p + (lane << s);
    const bool under = cand < (1ull << NB) && KeyOps<DT>::value((uint32_t)cand) * r < thr;
    p += (uint32_t)(__popcll(__ballot(under)) - 1) << s;
  }
  return p + 1;
}

struct MaxPk16 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return pk_max_u16(a, b); }
};

// Wave-wide results of the kRowsInFlight = 4 rows of a group, as four
// scalars.  Lane i (< 4) takes row i's value by selects on its lane bits, made
// on values passed by value: selects between loads of one array or struct get
// folded into an access indexed by lane, which the compiler stages in LDS.
static_assert(kRowsInFlight == 4, "row groups of four");
struct Row4 {
  uint32_t v0, v1, v2, v3;
};
__device__ inline uint32_t pick4(uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3, int lane) {
  return (lane & 2) ? ((lane & 1) ? v3 : v2) : ((lane & 1) ? v1 : v0);
}
#define IMU_PICK(r4, lane) pick4((r4).v0, (r4).v1, (r4).v2, (r4).v3, lane)
// sums of per-lane counts below 2^16 / 64 (two rows to a dword)
__device__ inline Row4 wave_sums4(const uint32_t (&c)[4]) {
  const uint32_t a = wave_reduce(c[0] | c[1] << 16, AddU32()), b = wave_reduce(c[2] | c[3] << 16, AddU32());
  return Row4{a & 0xFFFFu, a >> 16, b & 0xFFFFu, b >> 16};
}
template <int DT>
__device__ inline Row4 wave_max_keys4(const uint32_t (&k)[4]) {
  if constexpr (DT == IMU_BF16) {  // 15-bit keys, two rows to a dword
    const uint32_t a = wave_reduce(k[0] | k[1] << 16, MaxPk16()), b = wave_reduce(k[2] | k[3] << 16, MaxPk16());
    return Row4{a & 0xFFFFu, a >> 16, b & 0xFFFFu, b >> 16};
  } else {
    return Row4{wave_reduce(k[0], MaxU32()), wave_reduce(k[1], MaxU32()), wave_reduce(k[2], MaxU32()),
                wave_reduce(k[3], MaxU32())};
  }
}

// --- percentile histogram + fused selection ---------------------------------
// Two-level selection of the first pass: besides the 32768 key bins, every
// workgroup adds its counts per coarse bin of 128 keys to kHistCoarse global
// counters (in the same flush), so the last workgroup reads 256 coarse counts,
// then the 128 bins of the coarse bin holding rank k, instead of all 32768.
static_assert(kHistCoarse * 128 == kHistBins, "two-level histogram");
__device__ __forceinline__ void select_two_level(StatsHeader* hd, const uint32_t* gh, const uint32_t* coarse,
                                                 int64_t nelem, int final_pass, int beta, int p_num, int p_den) {
  const int lane = threadIdx.x & 63;
  const unsigned long long k = nearest_rank(nelem, p_num, p_den);
  uint32_t c4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) c4[j] = coarse[4 * lane + j];
  const unsigned long long csum = (unsigned long long)c4[0] + c4[1] + c4[2] + c4[3];
  const unsigned long long cincl = wave_incl_scan_u64(csum);
  unsigned long long run = cincl - csum;
  const bool chit = run < k && k <= cincl;  // one lane for a consistent histogram
  int j = 0;
  if (chit)
    while (j < 3 && run + c4[j] < k) run += c4[j++];
  const unsigned long long chits = __ballot(chit);
  const int csrc = chits ? __builtin_ctzll(chits) : 0;
  const uint32_t cbin = (uint32_t)__shfl(4 * lane + j, csrc, 64);
  const unsigned long long below = __shfl(run, csrc, 64);
  // the 128 key bins of that coarse bin, two per lane
  const uint32_t f0 = gh[cbin * 128 + 2 * lane], f1 = gh[cbin * 128 + 2 * lane + 1];
  const unsigned long long fsum = (unsigned long long)f0 + f1;
  const unsigned long long fincl = below + wave_incl_scan_u64(fsum), fexcl = fincl - fsum;
  const bool fhit = chits && fexcl < k && k <= fincl;
  const unsigned long long fhits = __ballot(fhit);
  const int fsrc = fhits ? __builtin_ctzll(fhits) : 0;
  const bool lo_half = fexcl + f0 >= k;
  const uint32_t bin = (uint32_t)__shfl(cbin * 128 + 2 * lane + (lo_half ? 0 : 1), fsrc, 64);
  const unsigned long long blw = __shfl(lo_half ? fexcl : fexcl + f0, fsrc, 64);
  if (lane == 0) apply_selection(hd, 0, final_pass, fhits ? bin : 0xFFFFFFFFu, blw, k, beta, hd->maxkey, hd->status);
}

// End of a first pass over 15-bit keys (kHistBins bins in LDS, counted by
// every thread of the workgroup; smax and sbad hold the workgroup's largest
// key and its non-finite flag): the bins and the coarse counts go to the
// entry's global histogram, and the last workgroup of the entry selects the
// percentile key.  Every flush is a device-scope atomic; each thread waits
// until its own have completed before the arrival counter moves (a
// device-scope release fence would also write back this XCD's whole L2,
// which costs tens of us across the grid).  The last workgroup then acquires
// at device scope, which drops stale cached lines before it reads the
// histogram.  Ends with the bins zeroed for a next pass unless final_pass.
__device__ __forceinline__ void finish_first_pass(const uint32_t* h, uint32_t smax, int sbad, uint32_t& slast,
                                                  StatsHeader* hd, uint32_t* gh, int count, int64_t nelem,
                                                  int final_pass, int beta, int p_num, int p_den) {
  constexpr int NB = kHistBins;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // key bins: lane-consecutive bins, so that a wave's atomics fall on two
  // 128-byte lines; 8 LDS reads in flight before their atomics (a loop of
  // read, wait, atomic would pay the LDS latency 32 times).  The workgroup
  // has 1024 threads.
  static_assert(NB % (8 * 1024) == 0, "bins per thread in groups of 8");
#pragma unroll
  for (int j0 = 0; j0 < NB / 1024; j0 += 8) {
    uint32_t c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = h[threadIdx.x + 1024 * (j0 + j)];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c[j]) atomicAdd(&gh[threadIdx.x + 1024 * (j0 + j)], c[j]);
  }
  // coarse counts: thread t sums bins [32t, 32t + 32) (16-byte reads, the
  // chunk order rotated by lane so that 8 lanes read 8 different banks);
  // four threads make one coarse bin, stored after the key bins
  static_assert(NB == 32 * 1024, "one run of 32 bins per thread");
  {
    const int t = threadIdx.x;
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 v = *reinterpret_cast<const uint4*>(&h[32 * t + 4 * ((j + lane) & 7)]);
      c += v.x + v.y + v.z + v.w;
    }
    c += __shfl_xor(c, 1, 64);
    c += __shfl_xor(c, 2, 64);
    if ((t & 3) == 0 && c) atomicAdd(&gh[NB + (t >> 2)], c);
  }
  if (threadIdx.x == 0) {
    atomicMax(&hd->maxkey, smax);
    if (sbad) atomicOr(&hd->status, kStatusNonfinite);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) slast = atomicAdd(&hd->arrive, 1u) == (uint32_t)(count - 1);
  __syncthreads();
  if (!slast) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (threadIdx.x == 0) hd->arrive = 0;  // ready for the next pass (stream ordered)
  if (wave == 0) select_two_level(hd, gh, gh + NB, nelem, final_pass, beta, p_num, p_den);
  if (!final_pass) {  // the next pass uses the first 256 bins
    __syncthreads();
    for (int i = threadIdx.x; i < 256; i += blockDim.x) gh[i] = 0;
  }
}

template <int DT, int NB, int PASS, bool VEC>
__global__ __launch_bounds__(1024) void hist_kernel(QuantJobs J, int final_pass) {
  using T = typename Elem<DT>::T;
  __shared__ __attribute__((aligned(16))) uint32_t h[NB];
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

  const uint32_t prefix = PASS == 0 ? 0u : hd->sel_prefix;
  const int lane = threadIdx.x & 63, nwave = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // unit indices stay scalar
  // work units: (stored row, 512-column tile); this workgroup takes a contiguous share
  const uint32_t ctiles = (uint32_t)ceil_div(a.scols, kColsPerTile);
  const int64_t units = a.srows * (int64_t)ctiles;
  const int64_t u0 = units * jp.local / jp.count, u1 = units * (jp.local + 1) / jp.count;
  uint32_t mx = 0;   // largest key (fp32 bit pattern without sign)
  uint32_t mxp = 0;  // bf16: largest 15-bit keys of the packed path, two halves
  auto count = [&](uint32_t bits) {
    const uint32_t k = bits & 0x7FFFFFFFu;
    if constexpr (PASS == 0) {
      mx = max(mx, k);
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
    g[rr] = load_raw<DT, VEC>(xb + (int64_t)sr_ * a.ld, (int64_t)ct_ * kColsPerTile + lane * 8, a.scols); \
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
        if constexpr (DT == IMU_BF16 && PASS == 0) { /* two 15-bit keys per dword */              \
          _Pragma("unroll") for (int d = 0; d < 4; ++d) {                                          \
            const uint32_t k_ = g[rr][d] & 0x7FFF7FFFu;                                            \
            mxp = pk_max_u16(mxp, k_);                                                             \
            atomicAdd(&h[k_ & 0xFFFFu], 1u);                                                       \
            atomicAdd(&h[k_ >> 16], 1u);                                                           \
          }                                                                                        \
        } else {                                                                                   \
          _Pragma("unroll") for (int j = 0; j < 8; ++j) count(w[j]);                               \
        }                                                                                          \
      } else {                                                                                     \
        const int n_ = (int)min64(max64(a.scols - c0_, 0), 8);                                     \
        _Pragma("unroll") for (int j = 0; j < 8; ++j) if (j < n_) count(w[j]);                     \
      }                                                                                            \
    }                                                                                              \
  }
  int64_t ub = u0 + (int64_t)wave * kRowsInFlight;
  IMU_ISSUE(g0, ub);
  // the LDS histogram is cleared while the first loads fly
  static_assert(NB % 4 == 0, "16-byte clears");
  for (int i = threadIdx.x; i < NB / 4; i += blockDim.x) reinterpret_cast<uint4*>(h)[i] = uint4{0, 0, 0, 0};
  if (threadIdx.x == 0) {
    smax = 0;
    sbad = 0;
  }
  __syncthreads();
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
    mx = max(mx, max(mxp & 0xFFFFu, mxp >> 16) << 16);
    mx = wave_max_u32(mx);
    if (lane == 0) {
      atomicMax(&smax, mx);
      if (mx >= 0x7F800000u) atomicOr(&sbad, 1);  // Inf or NaN
    }
  }
  __syncthreads();
  if constexpr (PASS == 0) {
    finish_first_pass(h, smax, sbad, slast, hd, gh, jp.count, a.srows * a.scols, final_pass, a.beta, a.p_num,
                      a.p_den);
    return;
  }
  for (int i = threadIdx.x; i < NB; i += blockDim.x) {
    const uint32_t c = h[i];
    if (c) atomicAdd(&gh[i], c);
  }
  // The last workgroup of this entry selects (see finish_first_pass).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) slast = atomicAdd(&hd->arrive, 1u) == (uint32_t)(jp.count - 1);
  __syncthreads();
  if (!slast) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (threadIdx.x == 0) hd->arrive = 0;  // ready for the next pass (stream ordered)
  select_from_hist(st, a.hist, a.srows * a.scols, PASS, final_pass, a.beta, a.p_num, a.p_den, part, found, h);
}

// --- row softmax of attention logits + first histogram pass -----------------
// The P operand of the attention-output GEMM P.V ("Key results", third
// bullet) is the row softmax of the logits.  This kernel computes P, stores it
// as bf16 and counts its 15-bit keys in the same pass, so P's percentile
// needs no read of P.  The arithmetic is the binary32 softmax fixed step by
// step (no contraction of a product and a sum into an fma):
//   m = maxNum over the row; t = x - m; y = t * fl(log2 e);
//   e = 0 when y < -100, else 2^n * poly(f), n = rint(y), f = y - n, poly the
//       degree-7 Taylor polynomial of 2^f (coefficients fl((ln 2)^k / k!))
//       by Horner;
//   S = sum of e: lane l adds the row's positions 256 j + 4 l + c in order
//       (j = 0, 1, ..., c = 0..3), then the 64 lane sums are halved pairwise
//       (xor 32, 16, ..., 1);
//   P = bf16 nearest-even of fl(e / S); a NaN becomes 0x7FC0.
// One wave owns a row.  Rows of at most kSmRegChunks * 256 logits are held in
// registers (one read); longer rows are read three times (max, sum, write),
// recomputing the same e.
constexpr int kSmRegChunks = 8;  // 2048 logits per row in registers
constexpr float kSmLog2e = 0x1.715476p+0f;                    // fl(log2 e)
constexpr float kSmC[8] = {0x1p+0f,        0x1.62e430p-1f,  0x1.ebfbe0p-3f,  0x1.c6b08ep-5f,
                           0x1.3b2ab6p-7f, 0x1.5d87fep-10f, 0x1.430912p-13f, 0x1.ffcbfcp-17f};

__device__ inline float sm_exp(float t) {
#pragma clang fp contract(off)
  const float y = t * kSmLog2e;
  if (y != y) return y;
  if (y < -100.0f) return 0.0f;
  const float n = __builtin_rintf(y);  // in [-100, 0]
  const float f = y - n;
  float p = kSmC[7];
#pragma unroll
  for (int k = 6; k >= 0; --k) p = p * f + kSmC[k];
  return p * __int_as_float(((int)n + 127) << 23);  // exact: 2^n and the product are normal
}
__device__ inline uint32_t sm_bf16(float p) {
  const uint32_t u = __float_as_uint(p);
  return p != p ? 0x7FC0u : (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
template <int DT>
__device__ inline void sm_load4(const typename Elem<DT>::T* row, int64_t i, int64_t n, bool vec, float fill,
                                float (&v)[4]) {
  if (vec && i + 3 < n) {
    if constexpr (DT == IMU_F32) {
      const float4 x = *reinterpret_cast<const float4*>(row + i);
      v[0] = x.x, v[1] = x.y, v[2] = x.z, v[3] = x.w;
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(row + i);
      v[0] = __uint_as_float(x.x << 16), v[1] = __uint_as_float(x.x & 0xFFFF0000u);
      v[2] = __uint_as_float(x.y << 16), v[3] = __uint_as_float(x.y & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (DT == IMU_F32) v[c] = i + c < n ? row[i + c] : fill;
      else v[c] = i + c < n ? __uint_as_float((uint32_t)row[i + c] << 16) : fill;
    }
  }
}

template <int DT>
__global__ __launch_bounds__(1024) void softmax_hist_kernel(QuantJobs J, SoftmaxIn in) {
#pragma clang fp contract(off)
  using T = typename Elem<DT>::T;
  __shared__ __attribute__((aligned(16))) uint32_t h[kHistBins];
  __shared__ uint32_t smax;
  __shared__ int sbad;
  __shared__ uint32_t slast;
  const JobPos jp = find_job(J, blockIdx.x);
  if (jp.count == 0) return;
  const StreamArgs& a = J.op[0].s;  // P: bf16, rows x cols, the statistics' operand
  uint16_t* pb = static_cast<uint16_t*>(const_cast<void*>(a.x)) + jp.entry * a.bstride;
  const T* zb = static_cast<const T*>(in.z) + jp.entry * in.bstride;
  uint8_t* st = a.stats + jp.entry * a.stats_stride;
  StatsHeader* hd = reinterpret_cast<StatsHeader*>(st);
  uint32_t* gh = reinterpret_cast<uint32_t*>(st + a.hist);
  const int lane = threadIdx.x & 63, nwave = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t R = a.srows, N = a.scols;
  const int64_t r0 = R * jp.local / jp.count, r1 = R * (jp.local + 1) / jp.count;
  const bool vec = in.vec_ok != 0;
  static_assert(kHistBins % 4 == 0, "16-byte clears");
  for (int i = threadIdx.x; i < kHistBins / 4; i += blockDim.x) reinterpret_cast<uint4*>(h)[i] = uint4{0, 0, 0, 0};
  if (threadIdx.x == 0) smax = 0, sbad = 0;
  __syncthreads();
  uint32_t mx = 0;  // largest key, as a binary32 magnitude pattern
  auto emit = [&](uint16_t* prow, int64_t i, const float (&e)[4], float S) __attribute__((always_inline)) {
    uint32_t b[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      b[c] = sm_bf16(e[c] / S);
      if (i + c < N) {
        atomicAdd(&h[b[c] & 0x7FFFu], 1u);
        mx = max(mx, (b[c] & 0x7FFFu) << 16);
      }
    }
    if (vec && i + 3 < N) {
      *reinterpret_cast<uint2*>(prow + i) = uint2{b[0] | b[1] << 16, b[2] | b[3] << 16};
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (i + c < N) prow[i + c] = (uint16_t)b[c];
    }
  };
  for (int64_t r = r0 + wave; r < r1; r += nwave) {
    const T* zrow = zb + r * in.ld;
    uint16_t* prow = pb + r * a.ld;
    if (N <= 256 * kSmRegChunks) {
      float v[kSmRegChunks][4];
      float m = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < kSmRegChunks; ++j) {
        if (256 * j < N) {
          sm_load4<DT>(zrow, 256 * j + 4 * lane, N, vec, -__builtin_inff(), v[j]);
#pragma unroll
          for (int c = 0; c < 4; ++c) m = fmaxf(m, v[j][c]);
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < kSmRegChunks; ++j) {
        if (256 * j < N) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            v[j][c] = sm_exp(v[j][c] - m);
            if (256 * j + 4 * lane + c < N) acc = acc + v[j][c];
          }
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) acc = acc + __shfl_xor(acc, o, 64);
#pragma unroll
      for (int j = 0; j < kSmRegChunks; ++j)
        if (256 * j < N) emit(prow, 256 * j + 4 * lane, v[j], acc);
    } else {
      float m = -__builtin_inff();
      for (int64_t j0 = 0; j0 < N; j0 += 256) {
        float v[4];
        sm_load4<DT>(zrow, j0 + 4 * lane, N, vec, -__builtin_inff(), v);
#pragma unroll
        for (int c = 0; c < 4; ++c) m = fmaxf(m, v[c]);
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      float acc = 0.0f;
      for (int64_t j0 = 0; j0 < N; j0 += 256) {
        float v[4];
        sm_load4<DT>(zrow, j0 + 4 * lane, N, vec, -__builtin_inff(), v);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (j0 + 4 * lane + c < N) acc = acc + sm_exp(v[c] - m);
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) acc = acc + __shfl_xor(acc, o, 64);
      for (int64_t j0 = 0; j0 < N; j0 += 256) {
        float v[4];
        sm_load4<DT>(zrow, j0 + 4 * lane, N, vec, -__builtin_inff(), v);
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = sm_exp(v[c] - m);
        emit(prow, j0 + 4 * lane, v, acc);
      }
    }
  }
  mx = wave_max_u32(mx);
  if (lane == 0) {
    atomicMax(&smax, mx);
    if (mx >= 0x7F800000u) atomicOr(&sbad, 1);  // a NaN row
  }
  __syncthreads();
  finish_first_pass(h, smax, sbad, slast, hd, gh, jp.count, R * N, 1, a.beta, a.p_num, a.p_den);
}

// --- fused RTN + outlier statistics -------------------------------------------
// Tile: 512 stored columns x rows_per_wg stored rows.  Per row a lane counts
// its out-of-range keys and keeps their largest; the wave reduces a group of
// kRowsInFlight rows at once (DPP) and lanes 0..3 post one row each.  Columns
// keep counts and largest keys in registers (bf16: two columns per dword,
// 16-bit counts, so a workgroup takes at most 65535 rows), then LDS, then one
// global atomic per column per workgroup.  Codes, when asked for, are rounded
// from the elements.
template <int DT, int BITS, bool QOUT, bool VEC>
__global__ __launch_bounds__(kCountThreads) void round_count_kernel(QuantJobs J, int32_t* q0, int32_t* q1) {
  using T = typename Elem<DT>::T;
  using KO = KeyOps<DT>;
  constexpr int NW = KO::NW;
  constexpr float kThr = (float)(1 << (BITS - 1)) - 0.5f;  // |y| >= kThr <=> rne(y) out of range
  __shared__ int lcnt[kColsPerTile];
  __shared__ uint32_t lmax[kColsPerTile];  // largest key + 1 (0: column not seen)
  __shared__ unsigned long long ltot;
  __shared__ uint32_t lamax;
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
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nwave = blockDim.x >> 6;
  const int64_t cbase = ct * kColsPerTile;
  const int64_t c0 = cbase + lane * 8;
  const int64_t r0 = rb * op.rows_per_wg;
  const int64_t r1 = min64(r0 + op.rows_per_wg, a.srows);
  // the first two groups of rows are in flight while the workgroup sets up
#define IMU_ISSUE(g, sb_)                                                                          \
  _Pragma("unroll") for (int rr = 0; rr < kRowsInFlight; ++rr)                                      \
      g[rr] = load_raw<DT, VEC>(xb + min64((sb_) + rr, r1 - 1) * a.ld, c0, a.scols);
  const int64_t gstep = (int64_t)nwave * kRowsInFlight;
  typename RawOf<DT>::V g0[kRowsInFlight], g1[kRowsInFlight];
  int64_t sb = r0 + (int64_t)wave * kRowsInFlight;
  IMU_ISSUE(g0, sb);
  IMU_ISSUE(g1, sb + gstep);
  for (int i = threadIdx.x; i < kColsPerTile; i += blockDim.x) {
    lcnt[i] = 0;
    lmax[i] = 0;
  }
  if (threadIdx.x == 0) {
    ltot = 0;
    lamax = 0;
  }
  __syncthreads();
  const float r = hd->r;
  // clipping at beta < 2^(bits-1) leaves every code in range: no key reaches
  const bool never_oob = a.clip && a.beta < (1 << (BITS - 1));
  const uint32_t kth = never_oob ? (1u << KO::NB) : key_threshold<DT>(r, kThr);
  const uint32_t cadd = (0x8000u - kth) * 0x10001u;  // bf16: a half of k + cadd reaches 0x8000 iff k >= kth
  const int64_t R = a.srows, C = a.scols;
  int32_t* qb = nullptr;  // codes of this operand, if they were asked for
  if constexpr (QOUT) {
    int32_t* qo = jp.op == 0 ? q0 : q1;
    if (qo) qb = qo + b * R * C;
  }
  const bool tile_whole = cbase + kColsPerTile <= a.scols;  // no element of this tile is past the row
  const int nin = (int)min64(max64(a.scols - c0, 0), 8);      // this lane's elements inside a row
  uint32_t km[NW];
  key_masks<DT>(nin, km);
  uint32_t ccnt[NW], cmx[NW];
#pragma unroll
  for (int d = 0; d < NW; ++d) {
    ccnt[d] = 0;
    cmx[d] = 0;
  }
  uint32_t amax = 0;  // largest key of the wave's rows
  uint32_t tot = 0;   // out-of-range codes of the wave's rows
  // one row: the lane's out-of-range count and largest key; column registers
  // returns (count, largest key)
  auto row_keys = [&](const typename RawOf<DT>::V& g, bool whole) __attribute__((always_inline)) {
    uint32_t rc = 0, rm = 0;
#pragma unroll
    for (int d = 0; d < NW; ++d) {
      const uint32_t k = g[d] & (whole ? KO::kMask : km[d]);
      if constexpr (DT == IMU_BF16) {
        const uint32_t m = pk_add_u16(k, cadd) & 0x80008000u;
        rc += __popc(m);
        ccnt[d] += m >> 15;
        rm = pk_max_u16(rm, k);
        cmx[d] = pk_max_u16(cmx[d], k);
      } else {
        const uint32_t o = k >= kth;
        rc += o;
        ccnt[d] += o;
        rm = max(rm, k);
        cmx[d] = max(cmx[d], k);
      }
    }
    if constexpr (DT == IMU_BF16) rm = max(rm & 0xFFFFu, rm >> 16);
    return make_uint2(rc, rm);
  };
  auto row_codes = [&](const typename RawOf<DT>::V& g, int64_t sr) __attribute__((always_inline)) {
    uint32_t w[8];
    bits8<DT>(g, w);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= nin) continue;
      const float y = __uint_as_float(w[j]) * r;
      int32_t q;
      if (a.clip) {  // rne(min(|y|, beta)) = min(rne(|y|), beta); rne is odd-symmetric
        const int32_t m = (int32_t)__builtin_rintf(__builtin_fminf(__builtin_fabsf(y), (float)a.beta));
        q = y < 0.f ? -m : m;
      } else {
        q = __builtin_fabsf(y) < 2147483648.0f ? (int32_t)__builtin_rintf(y) : 0;
      }
      const int64_t c = c0 + j;
      if (!a.transposed) qb[sr * C + c] = q;
      else qb[c * R + sr] = q;
    }
  };
  // a group of rows: lane statistics, then wave totals posted by lanes 0..3
#define IMU_PROCESS(g, sb_)                                                                        \
  {                                                                                                \
    uint32_t rc_[kRowsInFlight], rm_[kRowsInFlight];                                               \
    _Pragma("unroll") for (int rr = 0; rr < kRowsInFlight; ++rr) {                                 \
      if ((sb_) + rr < r1) { /* uniform across the wave */                                         \
        const uint2 v_ = row_keys(g[rr], tile_whole);                                              \
        rc_[rr] = v_.x;                                                                            \
        rm_[rr] = v_.y;                                                                            \
        if (QOUT && qb) row_codes(g[rr], (sb_) + rr);                                              \
      } else {                                                                                     \
        rc_[rr] = 0;                                                                               \
        rm_[rr] = 0;                                                                               \
      }                                                                                            \
    }                                                                                              \
    const Row4 cnt_ = wave_sums4(rc_), key_ = wave_max_keys4<DT>(rm_);                             \
    tot += cnt_.v0 + cnt_.v1 + cnt_.v2 + cnt_.v3;                                                  \
    amax = max(amax, max(max(key_.v0, key_.v1), max(key_.v2, key_.v3)));                           \
    if (lane < kRowsInFlight && (sb_) + lane < r1) {                                               \
      const uint32_t c_ = IMU_PICK(cnt_, lane);                                                         \
      const float f_ = KO::value(IMU_PICK(key_, lane)) * r;                                             \
      if (c_) atomicAdd(&srow_oob[(sb_) + lane], (int)c_);                                         \
      atomicMax(&srow_max[(sb_) + lane], line_digits<BITS>(f_, a.clip, a.beta));       \
    }                                                                                              \
  }
  // two groups alternate: one group's loads fly while the other is reduced
  for (; sb < r1; sb += 2 * gstep) {
    IMU_PROCESS(g0, sb);
    if (sb + gstep >= r1) break;
    IMU_ISSUE(g0, sb + 2 * gstep);  // unconditional (rows clamped), so the loads in flight are known exactly
    IMU_PROCESS(g1, sb + gstep);
    IMU_ISSUE(g1, sb + 3 * gstep);
  }
#undef IMU_ISSUE
#undef IMU_PROCESS
  // columns: registers -> LDS (keys + 1, so that a seen column is non-zero)
#pragma unroll
  for (int d = 0; d < NW; ++d) {
    if constexpr (DT == IMU_BF16) {
      const int c = lane * 8 + 2 * d;
      if (ccnt[d] & 0xFFFFu) atomicAdd(&lcnt[c], (int)(ccnt[d] & 0xFFFFu));
      if (ccnt[d] >> 16) atomicAdd(&lcnt[c + 1], (int)(ccnt[d] >> 16));
      atomicMax(&lmax[c], (cmx[d] & 0xFFFFu) + 1u);
      atomicMax(&lmax[c + 1], (cmx[d] >> 16) + 1u);
    } else {
      const int c = lane * 8 + d;
      if (ccnt[d]) atomicAdd(&lcnt[c], (int)ccnt[d]);
      atomicMax(&lmax[c], cmx[d] + 1u);
    }
  }
  if (lane == 0) {
    if (tot) atomicAdd(&ltot, (unsigned long long)tot);
    atomicMax(&lamax, amax);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kColsPerTile; i += blockDim.x) {
    const int64_t c = cbase + i;
    const uint32_t m = lmax[i];
    if (c < a.scols && m) {
      const float f = KO::value(m - 1u) * r;
      if (lcnt[i]) atomicAdd(&scol_oob[c], lcnt[i]);
      atomicMax(&scol_max[c], line_digits<BITS>(f, a.clip, a.beta));
    }
  }
  if (threadIdx.x == 0) {
    if (ltot) atomicAdd(&hd->total, ltot);
    if (!a.clip && KO::value(lamax) * r >= 2147483648.0f) atomicOr(&hd->status, kStatusRange);
  }
}

// --- Mix residual: largest digit count of each line outside heavy lines --------
// A stored column is heavy when scol_oob * scols > gamma * T, a stored row when
// srow_oob * srows > gamma * T.  srow_res gets the max over non-heavy columns,
// scol_res the max over non-heavy rows; both from largest keys, as above.
template <int DT, int BITS, bool VEC>
__global__ __launch_bounds__(kResidualThreads) void residual_kernel(QuantJobs J) {
  using T = typename Elem<DT>::T;
  using KO = KeyOps<DT>;
  constexpr int NW = KO::NW;
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
  // row counts are read per row with uniform addresses: scalar loads (the
  // counting kernel wrote them before this launch)
  const __attribute__((address_space(4))) int32_t* srow_oob =
      (const __attribute__((address_space(4))) int32_t*)(st + a.srow_oob);
  const int32_t* scol_oob = reinterpret_cast<const int32_t*>(st + a.scol_oob);
  int32_t* srow_res = reinterpret_cast<int32_t*>(st + a.srow_res);
  int32_t* scol_res = reinterpret_cast<int32_t*>(st + a.scol_res);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nwave = blockDim.x >> 6;
  const int64_t cbase = ct * kColsPerTile;
  const int64_t c0 = cbase + lane * 8;
  const int64_t r0 = rb * op.rows_per_wg;
  const int64_t r1 = min64(r0 + op.rows_per_wg, a.srows);
  // the first two groups of rows are in flight while the workgroup sets up;
  // a group's row counts are loaded with its elements, so the loop never
  // waits on a count of its own
#define IMU_ISSUE(g, ro, sb_)                                                                      \
  _Pragma("unroll") for (int rr = 0; rr < kRowsInFlight; ++rr) {                                   \
    g[rr] = load_raw<DT, VEC>(xb + min64((sb_) + rr, r1 - 1) * a.ld, c0, a.scols);                  \
    ro[rr] = srow_oob[min64((sb_) + rr, r1 - 1)];                                                  \
  }
  const int64_t gstep = (int64_t)nwave * kRowsInFlight;
  typename RawOf<DT>::V g0[kRowsInFlight], g1[kRowsInFlight];
  int32_t ro0[kRowsInFlight], ro1[kRowsInFlight];  // row counts of the two groups
  int64_t sb = r0 + (int64_t)wave * kRowsInFlight;
  IMU_ISSUE(g0, ro0, sb);
  IMU_ISSUE(g1, ro1, sb + gstep);
  for (int i = threadIdx.x; i < kColsPerTile; i += blockDim.x) lmax[i] = 0;
  __syncthreads();
  const float r = hd->r;
  const long long gT = (long long)a.gamma * (long long)hd->total;
  const int nin = (int)min64(max64(a.scols - c0, 0), 8);  // this lane's elements inside a row
  uint32_t km[NW], lm[NW];  // key masks: elements inside the row; of those, the non-heavy columns
  key_masks<DT>(nin, km);
  bool light = false;  // the lane has a non-heavy column inside the row
  int coob[8];          // column counts, loaded together (index clamped into the row)
#pragma unroll
  for (int j = 0; j < 8; ++j) coob[j] = scol_oob[min64(c0 + j, a.scols - 1)];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t c = c0 + j;
    const bool heavy = c < a.scols && (long long)coob[j] * a.scols > gT;
    light |= j < nin && !heavy;
    const uint32_t keep = heavy ? 0u : 0xFFFFFFFFu;
    if constexpr (DT == IMU_BF16) {
      if (j & 1) lm[j >> 1] = (lm[j >> 1] & 0xFFFFu) | (km[j >> 1] & keep & 0xFFFF0000u);
      else lm[j >> 1] = km[j >> 1] & keep & 0xFFFFu;
    } else {
      lm[j] = km[j] & keep;
    }
  }
  const bool rows_live = __ballot(light) != 0;  // some row residual is posted
  uint32_t cmx[NW];
#pragma unroll
  for (int d = 0; d < NW; ++d) cmx[d] = 0;
  bool col_seen = false;  // the wave took a non-heavy row
#define IMU_PROCESS(g, ro, sb_)                                                                    \
  {                                                                                                \
    uint32_t rm_[kRowsInFlight];                                                                   \
    _Pragma("unroll") for (int rr = 0; rr < kRowsInFlight; ++rr) {                                 \
      rm_[rr] = 0;                                                                                 \
      if ((sb_) + rr < r1) { /* uniform across the wave */                                         \
        const bool rheavy = (long long)ro[rr] * a.srows > gT;                                      \
        uint32_t m_ = 0;                                                                           \
        _Pragma("unroll") for (int d = 0; d < NW; ++d) {                                           \
          if constexpr (DT == IMU_BF16) m_ = pk_max_u16(m_, g[rr][d] & lm[d]);                     \
          else m_ = max(m_, g[rr][d] & lm[d]);                                                     \
        }                                                                                          \
        if (!rheavy) {                                                                             \
          col_seen = true;                                                                         \
          _Pragma("unroll") for (int d = 0; d < NW; ++d) {                                         \
            if constexpr (DT == IMU_BF16) cmx[d] = pk_max_u16(cmx[d], g[rr][d] & km[d]);           \
            else cmx[d] = max(cmx[d], g[rr][d] & km[d]);                                           \
          }                                                                                        \
        }                                                                                          \
        if constexpr (DT == IMU_BF16) m_ = max(m_ & 0xFFFFu, m_ >> 16);                            \
        rm_[rr] = m_;                                                                              \
      }                                                                                            \
    }                                                                                              \
    if (rows_live) {                                                                               \
      const Row4 key_ = wave_max_keys4<DT>(rm_);                                                   \
      if (lane < kRowsInFlight && (sb_) + lane < r1) {                                             \
        const float f_ = KO::value(IMU_PICK(key_, lane)) * r;                                           \
        atomicMax(&srow_res[(sb_) + lane], line_digits<BITS>(f_, a.clip, a.beta));      \
      }                                                                                            \
    }                                                                                              \
  }
  for (; sb < r1; sb += 2 * gstep) {
    IMU_PROCESS(g0, ro0, sb);
    if (sb + gstep >= r1) break;
    IMU_ISSUE(g0, ro0, sb + 2 * gstep);  // unconditional (rows clamped), so the loads in flight are known exactly
    IMU_PROCESS(g1, ro1, sb + gstep);
    IMU_ISSUE(g1, ro1, sb + 3 * gstep);
  }
#undef IMU_ISSUE
#undef IMU_PROCESS
  if (col_seen) {
#pragma unroll
    for (int d = 0; d < NW; ++d) {
      if constexpr (DT == IMU_BF16) {
        atomicMax(&lmax[lane * 8 + 2 * d], (cmx[d] & 0xFFFFu) + 1u);
        atomicMax(&lmax[lane * 8 + 2 * d + 1], (cmx[d] >> 16) + 1u);
      } else {
        atomicMax(&lmax[lane * 8 + d], cmx[d] + 1u);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kColsPerTile; i += blockDim.x) {
    const int64_t c = cbase + i;
    const uint32_t m = lmax[i];
    if (c < a.scols && m) {
      const float f = KO::value(m - 1u) * r;
      atomicMax(&scol_res[c], line_digits<BITS>(f, a.clip, a.beta));
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

hipError_t launch_fill_2d(int32_t* p, int64_t rows, int64_t cols, int64_t ld, int batch, int64_t bstride,
                          hipStream_t s) {
  if (rows <= 0 || cols <= 0 || batch <= 0) return hipSuccess;
  if (batch > 65535) return hipErrorInvalidValue;
  const int64_t per = max64(1, 4096 / batch);  // row blocks per entry
  dim3 grid((unsigned)min64(ceil_div(cols, 256), 64), (unsigned)min64(rows, per), (unsigned)batch);
  hipLaunchKernelGGL(fill_2d_kernel, grid, dim3(256), 0, s, p, rows, cols, ld, bstride);
  return hipGetLastError();
}

// Histogram: at most about `target` workgroups in total (one per CU: the
// 128 KB histogram allows one), shared in proportion to size and rounded
// down, so that the launch is one round (at least one per batch entry).
static int plan_hist(QuantJobs& J, int target) {
  double total = 0;
  for (int o = 0; o < J.nops; ++o) total += (double)J.op[o].s.srows * J.op[o].s.scols * J.op[o].batch;
  int begin = 0;
  for (int o = 0; o < J.nops; ++o) {
    QuantOp& q = J.op[o];
    const double el = (double)q.s.srows * q.s.scols;
    const int64_t units = q.s.srows * ceil_div(q.s.scols, kColsPerTile);
    int64_t per = (int64_t)(target * el / total);
    per = min64(max64(per, 1), max64(units, 1));
    q.wgs_per_entry = (int)per;
    q.wg_begin = begin;
    begin += (int)per * q.batch;
  }
  return begin;
}

// Whether every operand of a launch takes 16-byte row loads.
static bool all_vec(const QuantJobs& J) {
  bool v = true;
  for (int o = 0; o < J.nops; ++o) v = v && J.op[o].s.vec_ok;
  return v;
}

template <bool VEC>
static hipError_t hist_vec(int dtype, QuantJobs& J, int pass, int final_pass, hipStream_t s) {
  constexpr int kHistWgs = 256;
  const int grid = plan_hist(J, kHistWgs);
  if (dtype == IMU_BF16)
    hipLaunchKernelGGL((hist_kernel<IMU_BF16, kHistBins, 0, VEC>), dim3(grid), dim3(1024), 0, s, J, final_pass);
  else if (pass == 0)
    hipLaunchKernelGGL((hist_kernel<IMU_F32, kHistBins, 0, VEC>), dim3(grid), dim3(1024), 0, s, J, final_pass);
  else if (pass == 1)
    hipLaunchKernelGGL((hist_kernel<IMU_F32, 256, 1, VEC>), dim3(grid), dim3(1024), 0, s, J, final_pass);
  else
    hipLaunchKernelGGL((hist_kernel<IMU_F32, 256, 2, VEC>), dim3(grid), dim3(1024), 0, s, J, final_pass);
  return hipGetLastError();
}

hipError_t launch_hist(int dtype, QuantJobs J, int pass, int final_pass, hipStream_t s) {
  return all_vec(J) ? hist_vec<true>(dtype, J, pass, final_pass, s) : hist_vec<false>(dtype, J, pass, final_pass, s);
}

hipError_t launch_softmax_hist(int zdtype, const SoftmaxIn& in, QuantJobs J, hipStream_t s) {
  // about one 1024-thread workgroup per CU (the 128 KB histogram allows one),
  // split over the batch entries by rows
  QuantOp& q = J.op[0];
  constexpr int kWgs = 256;
  q.wgs_per_entry = (int)min64(max64(ceil_div(kWgs, q.batch), 1), max64(q.s.srows, 1));
  q.wg_begin = 0;
  J.nops = 1;
  const int grid = q.wgs_per_entry * q.batch;
  if (zdtype == IMU_F32) hipLaunchKernelGGL((softmax_hist_kernel<IMU_F32>), dim3(grid), dim3(1024), 0, s, J, in);
  else hipLaunchKernelGGL((softmax_hist_kernel<IMU_BF16>), dim3(grid), dim3(1024), 0, s, J, in);
  return hipGetLastError();
}

// Count kernels: tiles of 512 columns x rows_per_wg rows, about kCountWgs workgroups
// in total (fewer workgroups: fewer column atomics; more: more loads in flight).
// An operand's share is in proportion to the tile lanes it occupies (a row
// narrower than a tile still takes the tile's width), so a narrow operand
// beside a wide one gets short workgroups instead of a few long ones.
static int plan_tiles(QuantJobs& J, int kCountWgs) {
  auto lanes = [](const QuantOp& q) {
    return (double)q.s.srows * (double)(ceil_div(q.s.scols, kColsPerTile) * kColsPerTile) * q.batch;
  };
  double total = 0;
  for (int o = 0; o < J.nops; ++o) total += lanes(J.op[o]);
  int begin = 0;
  for (int o = 0; o < J.nops; ++o) {
    QuantOp& q = J.op[o];
    const int64_t ctiles = ceil_div(q.s.scols, kColsPerTile);
    const int64_t want = max64((int64_t)(kCountWgs * lanes(q) / total + 0.5), 1);  // workgroups for this operand
    int64_t rblocks = max64(ceil_div(want, ctiles * q.batch), 1);
    int64_t rpw = ceil_div(q.s.srows, rblocks);
    rpw = min64(max64(rpw, 4), 32768);  // column counts of the bf16 path are 16-bit
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
    if (q0 || q1) /* codes asked for: element loads for every shape */                           \
      hipLaunchKernelGGL((round_count_kernel<DT, B, true, false>), dim3(grid), dim3(kCountThreads), 0, s, J, q0, q1); \
    else if (all_vec(J))                                                                           \
      hipLaunchKernelGGL((round_count_kernel<DT, B, false, true>), dim3(grid), dim3(kCountThreads), 0, s, J, q0, q1); \
    else                                                                                           \
      hipLaunchKernelGGL((round_count_kernel<DT, B, false, false>), dim3(grid), dim3(kCountThreads), 0, s, J, q0, q1); \
    break;
    IMU_RC(2) IMU_RC(3) IMU_RC(4) IMU_RC(5) IMU_RC(6) IMU_RC(7) IMU_RC(8)
#undef IMU_RC
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_round_count(int dtype, int bits, QuantJobs J, int32_t* q0, int32_t* q1, hipStream_t s) {
  const int grid = plan_tiles(J, 256);  // one workgroup per CU: fewer column flushes
  return dtype == IMU_BF16 ? round_count_dt<IMU_BF16>(bits, J, grid, q0, q1, s)
                           : round_count_dt<IMU_F32>(bits, J, grid, q0, q1, s);
}

template <int DT>
static hipError_t residual_dt(int bits, const QuantJobs& J, int grid, hipStream_t s) {
  switch (bits) {
#define IMU_RS(B)                                                                                  \
  case B:                                                                                          \
    if (all_vec(J))                                                                                \
      hipLaunchKernelGGL((residual_kernel<DT, B, true>), dim3(grid), dim3(kResidualThreads), 0, s, J); \
    else                                                                                           \
      hipLaunchKernelGGL((residual_kernel<DT, B, false>), dim3(grid), dim3(kResidualThreads), 0, s, J); \
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
