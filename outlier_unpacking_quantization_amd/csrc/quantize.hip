// Percentile scale, RTN quantization and outlier statistics (gfx950).
//
// Method: the summary page "IM-Unpack: Training and Inference with Arbitrarily
// Low Precision Integers".  The "Measured effects" table quantizes with RTN so
// that the p-percentile magnitude maps to beta (p = 95%); the summary keeps
// heavy hitters as out-of-range integers; "Approach" chooses the unpacking from
// per-line outlier counts.  Every kernel here streams the operand once from HBM
// in its stored orientation (no transposed copies): 16-byte loads, 64-lane
// waves over 512 stored columns, per-row reductions by cross-lane shuffles and
// per-column reductions in registers, then LDS, then one global atomic per
// column per workgroup.
#include "common.h"
#include "kernels.h"

namespace imu {

namespace {

constexpr int kColsPerTile = 512;  // 64 lanes x 8 elements

template <int DT>
__device__ inline int load8(const typename Elem<DT>::T* row, int64_t c0, int64_t scols, int vec_ok,
                            float v[8]) {
  if (c0 >= scols) return 0;
  if (vec_ok) {
    if constexpr (DT == IMU_BF16) {
      uint4 u = *reinterpret_cast<const uint4*>(row + c0);
      uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(w[j] << 16);
        v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    } else {
      float4 a = *reinterpret_cast<const float4*>(row + c0);
      float4 b = *reinterpret_cast<const float4*>(row + c0 + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    return 8;
  }
  int n = (int)min64(8, scols - c0);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < n) {
      if constexpr (DT == IMU_BF16) v[j] = bf16_to_f32(row[c0 + j]);
      else v[j] = row[c0 + j];
    } else {
      v[j] = 0.f;
    }
  }
  return n;
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

// --- percentile histogram ----------------------------------------------------
// pass 0: 32768 bins on the top 15 bits of the magnitude key (exact for bf16);
// pass 1/2 (fp32 only): 256 bins on key bits [15:8] / [7:0] of the elements
// whose higher bits equal the prefix selected by the previous pass.
template <int DT, int NB>
__global__ __launch_bounds__(1024) void hist_kernel(StreamArgs a, int rows_per_wg, int pass) {
  using T = typename Elem<DT>::T;
  __shared__ uint32_t h[NB];
  __shared__ uint32_t smax;
  __shared__ int sbad;
  const int b = blockIdx.z;
  const T* xb = static_cast<const T*>(a.x) + b * a.bstride;
  uint8_t* st = a.stats + b * a.stats_stride;
  StatsHeader* hd = reinterpret_cast<StatsHeader*>(st);
  uint32_t* gh = reinterpret_cast<uint32_t*>(st + a.hist);

  for (int i = threadIdx.x; i < NB; i += blockDim.x) h[i] = 0;
  if (threadIdx.x == 0) {
    smax = 0;
    sbad = 0;
  }
  __syncthreads();

  const uint32_t prefix = pass == 0 ? 0u : hd->sel_prefix;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int64_t c0 = blockIdx.x * (int64_t)kColsPerTile + lane * 8;
  const int64_t r0 = blockIdx.y * (int64_t)rows_per_wg;
  const int64_t r1 = min64(r0 + rows_per_wg, a.srows);
  uint32_t mx = 0;
  int bad = 0;
  for (int64_t sr = r0 + wave; sr < r1; sr += nwave) {
    float v[8];
    int n = load8<DT>(xb + sr * a.ld, c0, a.scols, a.vec_ok, v);
    for (int j = 0; j < n; ++j) {
      uint32_t k = mag_key(v[j]);
      if (pass == 0) {
        mx = max(mx, k);
        bad |= (k >= 0x7F800000u);
        atomicAdd(&h[(k >> 16) & (NB - 1)], 1u);
      } else if (pass == 1) {
        if ((k >> 16) == prefix) atomicAdd(&h[(k >> 8) & 0xFFu], 1u);
      } else {
        if ((k >> 8) == prefix) atomicAdd(&h[k & 0xFFu], 1u);
      }
    }
  }
  if (pass == 0) {
    mx = wave_max_u32(mx);
    bad = wave_max_i32(bad);
    if (lane == 0) {
      atomicMax(&smax, mx);
      if (bad) atomicOr(&sbad, 1);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < NB; i += blockDim.x) {
    uint32_t c = h[i];
    if (c) atomicAdd(&gh[i], c);
  }
  if (pass == 0 && threadIdx.x == 0) {
    atomicMax(&hd->maxkey, smax);
    if (sbad) atomicOr(&hd->status, kStatusNonfinite);
  }
}

// --- select the k-th smallest magnitude and form r, s -------------------------
__global__ __launch_bounds__(1024) void select_kernel(uint8_t* stats, int64_t stride, int64_t hist_off,
                                                      int64_t nelem, int pass, int final_pass,
                                                      int beta, int p_num, int p_den) {
  __shared__ unsigned long long part[1024];
  __shared__ uint32_t found_bin;
  __shared__ unsigned long long found_below;
  uint8_t* st = stats + blockIdx.x * stride;
  StatsHeader* hd = reinterpret_cast<StatsHeader*>(st);
  uint32_t* gh = reinterpret_cast<uint32_t*>(st + hist_off);
  const int NB = pass == 0 ? kHistBins : 256;
  const int per = (NB + 1023) / 1024;

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
  const int t = threadIdx.x;
  unsigned long long s = 0;
  for (int i = 0; i < per; ++i) {
    int bin = t * per + i;
    if (bin < NB) s += gh[bin];
  }
  part[t] = s;
  if (t == 0) found_bin = 0xFFFFFFFFu;
  __syncthreads();
  // inclusive scan over 1024 partial sums (Hillis-Steele)
  for (int off = 1; off < 1024; off <<= 1) {
    unsigned long long add = t >= off ? part[t - off] : 0ull;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  unsigned long long incl = part[t];
  unsigned long long excl = incl - s;
  if (excl < k && k <= incl) {
    unsigned long long run = excl;
    for (int i = 0; i < per; ++i) {
      int bin = t * per + i;
      if (bin >= NB) break;
      unsigned long long c = gh[bin];
      if (run + c >= k) {
        found_bin = (uint32_t)bin;
        found_below = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  if (t == 0) {
    uint32_t bin = found_bin;
    if (bin == 0xFFFFFFFFu) {  // cannot happen for a consistent histogram
      atomicOr(&hd->status, kStatusNonfinite);
      bin = 0;
    }
    uint32_t rank = (uint32_t)(k - found_below);
    uint32_t prefix = pass == 0 ? bin : ((hd->sel_prefix << 8) | bin);
    if (!final_pass) {
      hd->sel_prefix = prefix;
      hd->sel_rank = rank;
    } else {
      uint32_t key = pass == 0 ? (prefix << 16) : prefix;  // pass 0 final only for bf16
      float kth = __uint_as_float(key);
      float alpha = kth > 0.f ? kth : __uint_as_float(hd->maxkey);
      hd->kth = kth;
      hd->alpha = alpha;
      if (alpha > 0.f && !(hd->status & kStatusNonfinite)) {
        // binary32 quotient; a binary64 quotient rounded once more to binary32
        // is the correctly rounded binary32 quotient (53 >= 2*24 + 2)
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
    for (int i = t; i < 256; i += blockDim.x) gh[i] = 0;  // next pass uses 256 bins
  }
}

// --- fused RTN + outlier statistics -------------------------------------------
template <int DT, int BITS>
__global__ __launch_bounds__(256) void round_count_kernel(StreamArgs a, int rows_per_wg,
                                                          int32_t* q_out) {
  using T = typename Elem<DT>::T;
  __shared__ int lcnt[kColsPerTile];
  __shared__ int lmax[kColsPerTile];
  __shared__ unsigned long long ltot;
  __shared__ int lbad;
  const int b = blockIdx.z;
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
  const int64_t cbase = blockIdx.x * (int64_t)kColsPerTile;
  const int64_t c0 = cbase + lane * 8;
  const int64_t r0 = blockIdx.y * (int64_t)rows_per_wg;
  const int64_t r1 = min64(r0 + rows_per_wg, a.srows);
  int ccnt[8], cmax[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) ccnt[j] = cmax[j] = 0;
  int tot = 0;
  bool bad = false;
  const int64_t R = a.srows, C = a.scols;
  int32_t* qb = q_out ? q_out + b * R * C : nullptr;
  for (int64_t sr = r0 + wave; sr < r1; sr += nwave) {
    float v[8];
    int n = load8<DT>(xb + sr * a.ld, c0, a.scols, a.vec_ok, v);
    int rc = 0, rm = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < n) {
        int32_t q = rtn_code(v[j], r, &bad);
        uint32_t m = q < 0 ? (uint32_t)(-(int64_t)q) : (uint32_t)q;
        int nd = digit_count<BITS>(m);
        int o = nd >= 2;
        rc += o;
        rm = max(rm, nd);
        ccnt[j] += o;
        cmax[j] = max(cmax[j], nd);
        if (qb) {
          int64_t c = c0 + j;
          if (!a.transposed) qb[sr * C + c] = q;
          else qb[c * R + sr] = q;
        }
      }
    }
    rc = wave_sum_i32(rc);
    rm = wave_max_i32(rm);
    if (lane == 0) {
      if (rc) atomicAdd(&srow_oob[sr], rc);
      atomicMax(&srow_max[sr], rm);
      tot += rc;
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (cmax[j]) {
      if (ccnt[j]) atomicAdd(&lcnt[lane * 8 + j], ccnt[j]);
      atomicMax(&lmax[lane * 8 + j], cmax[j]);
    }
  }
  if (lane == 0 && tot) atomicAdd(&ltot, (unsigned long long)tot);
  if (bad) atomicOr(&lbad, 1);
  __syncthreads();
  for (int i = threadIdx.x; i < kColsPerTile; i += blockDim.x) {
    int64_t c = cbase + i;
    if (c < a.scols && lmax[i]) {
      if (lcnt[i]) atomicAdd(&scol_oob[c], lcnt[i]);
      atomicMax(&scol_max[c], lmax[i]);
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
__global__ __launch_bounds__(256) void residual_kernel(StreamArgs a, int rows_per_wg) {
  using T = typename Elem<DT>::T;
  __shared__ int lmax[kColsPerTile];
  const int b = blockIdx.z;
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
  const int64_t cbase = blockIdx.x * (int64_t)kColsPerTile;
  const int64_t c0 = cbase + lane * 8;
  const int64_t r0 = blockIdx.y * (int64_t)rows_per_wg;
  const int64_t r1 = min64(r0 + rows_per_wg, a.srows);
  bool colheavy[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int64_t c = c0 + j;
    colheavy[j] = c < a.scols && (long long)scol_oob[c] * a.scols > gT;
  }
  int cmax[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) cmax[j] = 0;
  bool bad = false;
  for (int64_t sr = r0 + wave; sr < r1; sr += nwave) {
    float v[8];
    int n = load8<DT>(xb + sr * a.ld, c0, a.scols, a.vec_ok, v);
    const bool rowheavy = (long long)srow_oob[sr] * a.srows > gT;
    int rm = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < n) {
        int32_t q = rtn_code(v[j], r, &bad);
        uint32_t m = q < 0 ? (uint32_t)(-(int64_t)q) : (uint32_t)q;
        int nd = digit_count<BITS>(m);
        if (!colheavy[j]) rm = max(rm, nd);
        if (!rowheavy) cmax[j] = max(cmax[j], nd);
      }
    }
    rm = wave_max_i32(rm);
    if (lane == 0 && rm) atomicMax(&srow_res[sr], rm);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (cmax[j]) atomicMax(&lmax[lane * 8 + j], cmax[j]);
  __syncthreads();
  for (int i = threadIdx.x; i < kColsPerTile; i += blockDim.x) {
    int64_t c = cbase + i;
    if (c < a.scols && lmax[i]) atomicMax(&scol_res[c], lmax[i]);
  }
}

int rows_per_wg_for(int64_t srows, int64_t scols, int batch, int target_wgs, int min_rows) {
  int64_t ctiles = ceil_div(scols, kColsPerTile);
  int64_t per = ceil_div(srows * ctiles * batch, target_wgs);
  per = max64(per, min_rows);
  per = min64(per, max64(srows, 1));
  return (int)per;
}

}  // namespace

hipError_t launch_fill_u32(void* p, uint32_t v, int64_t nwords, hipStream_t s) {
  if (nwords <= 0) return hipSuccess;
  int64_t blocks = min64(ceil_div(nwords, 256), 4096);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<uint32_t*>(p), v, nwords);
  return hipGetLastError();
}

hipError_t launch_fill_2d(int32_t* p, int64_t rows, int64_t cols, int64_t ld, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  dim3 grid((unsigned)min64(ceil_div(cols, 256), 64), (unsigned)min64(rows, 4096));
  hipLaunchKernelGGL(fill_2d_kernel, grid, dim3(256), 0, s, p, rows, cols, ld);
  return hipGetLastError();
}

hipError_t launch_hist(int dtype, const StreamArgs& a, int batch, int pass, hipStream_t s) {
  int rpw = rows_per_wg_for(a.srows, a.scols, batch, 512, 16);
  dim3 grid((unsigned)ceil_div(a.scols, kColsPerTile), (unsigned)ceil_div(a.srows, rpw), (unsigned)batch);
  if (dtype == IMU_BF16) {
    hipLaunchKernelGGL((hist_kernel<IMU_BF16, kHistBins>), grid, dim3(1024), 0, s, a, rpw, pass);
  } else if (pass == 0) {
    hipLaunchKernelGGL((hist_kernel<IMU_F32, kHistBins>), grid, dim3(1024), 0, s, a, rpw, pass);
  } else {
    hipLaunchKernelGGL((hist_kernel<IMU_F32, 256>), grid, dim3(1024), 0, s, a, rpw, pass);
  }
  return hipGetLastError();
}

hipError_t launch_select(uint8_t* stats, int64_t stats_stride, int64_t hist_off, int batch,
                         int64_t nelem, int pass, int final_pass, int beta, int p_num, int p_den,
                         hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)batch), dim3(1024), 0, s, stats, stats_stride,
                     hist_off, nelem, pass, final_pass, beta, p_num, p_den);
  return hipGetLastError();
}

template <int DT>
static hipError_t round_count_dt(int bits, const StreamArgs& a, dim3 grid, int rpw, int32_t* q,
                                 hipStream_t s) {
  switch (bits) {
#define IMU_RC(B)                                                                                  \
  case B:                                                                                          \
    hipLaunchKernelGGL((round_count_kernel<DT, B>), grid, dim3(256), 0, s, a, rpw, q);            \
    break;
    IMU_RC(2) IMU_RC(3) IMU_RC(4) IMU_RC(5) IMU_RC(6) IMU_RC(7) IMU_RC(8)
#undef IMU_RC
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_round_count(int dtype, int bits, const StreamArgs& a, int batch, int32_t* q_out,
                              hipStream_t s) {
  int rpw = rows_per_wg_for(a.srows, a.scols, batch, 1024, 8);
  dim3 grid((unsigned)ceil_div(a.scols, kColsPerTile), (unsigned)ceil_div(a.srows, rpw), (unsigned)batch);
  return dtype == IMU_BF16 ? round_count_dt<IMU_BF16>(bits, a, grid, rpw, q_out, s)
                           : round_count_dt<IMU_F32>(bits, a, grid, rpw, q_out, s);
}

template <int DT>
static hipError_t residual_dt(int bits, const StreamArgs& a, dim3 grid, int rpw, hipStream_t s) {
  switch (bits) {
#define IMU_RS(B)                                                                                  \
  case B:                                                                                          \
    hipLaunchKernelGGL((residual_kernel<DT, B>), grid, dim3(256), 0, s, a, rpw);                  \
    break;
    IMU_RS(2) IMU_RS(3) IMU_RS(4) IMU_RS(5) IMU_RS(6) IMU_RS(7) IMU_RS(8)
#undef IMU_RS
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_residual(int dtype, int bits, const StreamArgs& a, int batch, hipStream_t s) {
  int rpw = rows_per_wg_for(a.srows, a.scols, batch, 1024, 8);
  dim3 grid((unsigned)ceil_div(a.scols, kColsPerTile), (unsigned)ceil_div(a.srows, rpw), (unsigned)batch);
  return dtype == IMU_BF16 ? residual_dt<IMU_BF16>(bits, a, grid, rpw, s)
                           : residual_dt<IMU_F32>(bits, a, grid, rpw, s);
}

}  // namespace imu
