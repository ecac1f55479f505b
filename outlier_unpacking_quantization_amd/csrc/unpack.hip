// Digit unpacking of one operand into int8 (gfx950).
//
// Method: summary page "IM-Unpack: Training and Inference with Arbitrarily Low
// Precision Integers": out-of-range integers are decomposed into several
// in-range low bit-width integers placed in extra rows / columns ("Approach"),
// turning each matrix into a larger one (summary paragraph).
//
// Layout written (per batch entry): A' is m_alloc x k_pad, B'^T is n_alloc x
// k_pad, int8, K' contiguous.  Row (line o, level u) sits at lvl[u][o]
// (level-major).  Column j of a row holds the triple kmap[j] = (k, v, v') of the
// exponent segment it lies in (or zero padding).  Digit t of a code whose inner
// line has depth dK goes to inner index min(t, dK-1) and level t - min(t, dK-1),
// so at level 0 every position holds digit (own inner index) and at level u > 0
// only the last inner index dK-1 holds digit dK-1+u.
//
// Two mappings, both writing every byte of every valid row exactly once:
// * inner-contiguous operands (A row-major, B = W^T): each thread owns 16
//   consecutive k, computes their codes once per row and scatters their digit
//   bytes into an LDS copy of each exponent segment (positions from kpre), which
//   the workgroup then streams out with 16-byte stores;
// * outer-contiguous operands (A = X^T, B row-major): lanes walk 64 adjacent
//   lines so every gather is one 128-byte line; bytes are assembled in an LDS
//   tile and written back row by row.
#include "common.h"
#include "kernels.h"

namespace imu {

namespace {

constexpr int kIcWindow = 65536;  // bytes of an unpacked row assembled in LDS at a time
constexpr int kSegReg = 16;       // segment starts of a k-group kept in registers
constexpr int kOcChunk = 256;   // K' positions per tile (outer-contiguous path)
constexpr int kOcStride = kOcChunk / 4 + 1;  // tile row stride in words (bank spread)

template <int DT>
__device__ inline float load_elem(const typename Elem<DT>::T* p) {
  if constexpr (DT == IMU_BF16) return bf16_to_f32(*p);
  else return *p;
}

__device__ inline int64_t entry_offset(const uint8_t* plan, int b, int operand) {
  int64_t off = 0;
  for (int e = 0; e < b; ++e)
    off += unpacked_entry_bytes(reinterpret_cast<const PlanHeader*>(plan + e * kPlanHeaderStride), operand);
  return off;
}

// Byte of unpacked row (line, level u) at the position whose table entry is `ent`.
template <int DT, int BITS>
__device__ inline uint32_t unpack_byte(uint32_t ent, const typename Elem<DT>::T* line, int64_t sk, float r, int u,
                                       bool is_a, const int32_t* own_depth) {
  if (ent == kKmapPad) return 0u;
  const int64_t k = ent & 0x3FFFFFu;
  const int v = (ent >> 22) & 31, vp = (ent >> 27) & 31;
  const int kap = is_a ? v : vp;  // this operand's inner index
  int t = kap;
  if (u > 0) t = (kap == own_depth[k] - 1) ? kap + u : -1;
  if (t < 0) return 0u;
  bool bad = false;
  const int32_t q = rtn_code(load_elem<DT>(line + k * sk), r, &bad);
  return (uint32_t)(uint8_t)(int8_t)digit_of<BITS>(q, t);
}

// Digit bytes of one group of 16 k in exponent segment s of unpacked row level u,
// written into the LDS row window [w0, w1) starting at position `pos`.
template <int BITS>
__device__ inline void emit_group(uint8_t* row_buf, int64_t w0, int64_t w1, int64_t pos, int s, int u, bool is_a,
                                  int nk, const float* xs, const int* dA, const int* dB, float r) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < nk) {
      const int lo = max(0, s - (dB[j] - 1)), hi = min(dA[j] - 1, s);
      if (hi >= lo) {
        const int dK = is_a ? dA[j] : dB[j];
        bool bad = false;
        const int32_t q = rtn_code(xs[j], r, &bad);
        for (int v = lo; v <= hi; ++v, ++pos) {
          if (pos < w0 || pos >= w1) continue;
          const int kap = is_a ? v : s - v;  // this operand's inner index
          const int tt = u == 0 ? kap : (kap == dK - 1 ? kap + u : -1);
          row_buf[pos - w0] = tt < 0 ? (uint8_t)0 : (uint8_t)(int8_t)digit_of<BITS>(q, tt);
        }
      }
    }
  }
}

// Inner-contiguous operands.  Each thread owns groups of 16 consecutive k.  For
// every unpacked row it issues the loads of a group together (16 elements,
// both inner depths, the group's start in each exponent segment), writes the
// group's digit bytes into an LDS copy of the row, and the workgroup streams
// the row out with 16-byte stores.  Rows longer than the LDS buffer are done
// in windows (each window recomputes the bytes that fall into it).
template <int DT, int BITS>
__global__ __launch_bounds__(256) void unpack_ic_kernel(UnpackArgs a, int lines_per_wg) {
  using T = typename Elem<DT>::T;
  __shared__ __attribute__((aligned(16))) uint8_t row_buf[kIcWindow];
  __shared__ int64_t s_off[kMaxSeg + 1];
  __shared__ int32_t s_len[kMaxSeg];
  const int b = blockIdx.y;
  const int64_t o0 = (int64_t)blockIdx.x * lines_per_wg;
  const int64_t o1 = min64(o0 + lines_per_wg, a.n_outer);
  const T* xb = static_cast<const T*>(a.x) + b * a.bstride;
  const float r = reinterpret_cast<const StatsHeader*>(a.stats + b * a.stats_stride)->r;
  const PlanLayout& L = a.pl;
  const uint8_t* pe = a.plan + L.headers_bytes + b * L.entry_stride;
  const PlanHeader* ph = reinterpret_cast<const PlanHeader*>(a.plan + b * kPlanHeaderStride);
  const bool is_a = a.operand == 0;
  const int32_t* da_c = reinterpret_cast<const int32_t*>(pe + L.da_c);
  const int32_t* db_r = reinterpret_cast<const int32_t*>(pe + L.db_r);
  const int32_t* dout = reinterpret_cast<const int32_t*>(pe + (is_a ? L.da_r : L.db_c));
  const int32_t* lvl = reinterpret_cast<const int32_t*>(pe + (is_a ? L.lvl_a : L.lvl_b));
  const int32_t* kpre = reinterpret_cast<const int32_t*>(pe + L.kpre);
  int8_t* out = a.out + entry_offset(a.plan, b, a.operand);
  const int64_t kp = ph->k_pad, K = a.K;
  const int nseg = ph->n_seg;
  const int t = threadIdx.x;
  const int64_t ngroups = ceil_div(K, 16);
  for (int s = t; s <= nseg; s += blockDim.x) {
    s_off[s] = ph->seg_off[s];
    if (s < nseg) s_len[s] = ph->seg_len[s];
  }
  for (int64_t o = o0; o < o1; ++o) {
    const T* line = xb + o * a.so;
    const int d = dout[o];
    for (int u = 0; u < d; ++u) {
      int8_t* row = out + (int64_t)lvl[(int64_t)u * a.n_outer + o] * kp;
      for (int64_t w0 = 0; w0 < kp; w0 += kIcWindow) {
        const int64_t w1 = min64(w0 + kIcWindow, kp);
        __syncthreads();  // the previous window has been copied out (and s_off is staged)
        for (int s = 0; s < nseg; ++s)  // zero padding at the end of each segment
          for (int64_t p = max64(s_off[s] + s_len[s], w0) + t; p < min64(s_off[s + 1], w1); p += blockDim.x)
            row_buf[p - w0] = 0;
        for (int64_t g = t; g < ngroups; g += blockDim.x) {
          const int64_t k0 = g * 16;
          const int nk = (int)min64(16, K - k0);
          // every load of the group first (indices clamped into range)
          float xs[16];
          int dA[16], dB[16], sp[kSegReg];
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int64_t k = min64(k0 + j, K - 1);
            xs[j] = load_elem<DT>(line + k);
            dA[j] = da_c[k];
            dB[j] = db_r[k];
          }
#pragma unroll
          for (int s = 0; s < kSegReg; ++s) sp[s] = kpre[(int64_t)min(s, nseg - 1) * (K + 1) + k0];
#pragma unroll
          for (int sr = 0; sr < kSegReg; ++sr) {  // segments whose start is in registers
            if (sr < nseg)
              emit_group<BITS>(row_buf, w0, w1, s_off[sr] + sp[sr], sr, u, is_a, nk, xs, dA, dB, r);
          }
          for (int s = kSegReg; s < nseg; ++s)
            emit_group<BITS>(row_buf, w0, w1, s_off[s] + kpre[(int64_t)s * (K + 1) + k0], s, u, is_a, nk, xs, dA,
                             dB, r);
        }
        __syncthreads();
        for (int64_t p = w0 + 16 * t; p < w1; p += 16 * blockDim.x)
          *reinterpret_cast<uint4*>(row + p) = *reinterpret_cast<const uint4*>(&row_buf[p - w0]);
      }
    }
  }
}

template <int DT, int BITS>
__global__ __launch_bounds__(256) void unpack_oc_kernel(UnpackArgs a) {
  using T = typename Elem<DT>::T;
  __shared__ uint32_t tab[kOcChunk];
  __shared__ uint32_t tile[64 * kOcStride];
  __shared__ int32_t rowpos[64];
  __shared__ int dmax_s;
  const int b = blockIdx.y;
  const int64_t o0 = (int64_t)blockIdx.x * 64;
  const T* xb = static_cast<const T*>(a.x) + b * a.bstride;
  const float r = reinterpret_cast<const StatsHeader*>(a.stats + b * a.stats_stride)->r;
  const PlanLayout& L = a.pl;
  const uint8_t* pe = a.plan + L.headers_bytes + b * L.entry_stride;
  const PlanHeader* ph = reinterpret_cast<const PlanHeader*>(a.plan + b * kPlanHeaderStride);
  const bool is_a = a.operand == 0;
  const int32_t* own_depth = reinterpret_cast<const int32_t*>(pe + (is_a ? L.da_c : L.db_r));
  const int32_t* dout = reinterpret_cast<const int32_t*>(pe + (is_a ? L.da_r : L.db_c));
  const int32_t* lvl = reinterpret_cast<const int32_t*>(pe + (is_a ? L.lvl_a : L.lvl_b));
  const uint32_t* kmap = reinterpret_cast<const uint32_t*>(pe + L.kmap);
  int8_t* out = a.out + entry_offset(a.plan, b, a.operand);
  const int64_t kp = ph->k_pad;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t o = o0 + lane;
  const bool line_ok = o < a.n_outer;
  const int my_d = line_ok ? dout[o] : 0;
  if (wave == 0) {
    const int m = wave_max_i32(my_d);
    if (lane == 0) dmax_s = m;
  }
  __syncthreads();
  const int dmax = dmax_s;
  const T* line = xb + (line_ok ? o : 0) * a.so;
  for (int64_t j0 = 0; j0 < kp; j0 += kOcChunk) {
    __syncthreads();
    tab[t] = j0 + t < kp ? kmap[j0 + t] : kKmapPad;
    for (int u = 0; u < dmax; ++u) {
      if (t < 64) rowpos[t] = (o0 + t < a.n_outer && dout[o0 + t] > u) ? lvl[(int64_t)u * a.n_outer + o0 + t] : -1;
      __syncthreads();
      if (my_d > u) {
        for (int q = wave; q < kOcChunk / 4; q += 4) {
          uint32_t w = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w |= unpack_byte<DT, BITS>(tab[4 * q + i], line, a.sk, r, u, is_a, own_depth) << (8 * i);
          tile[lane * kOcStride + q] = w;
        }
      }
      __syncthreads();
      for (int item = t; item < 64 * (kOcChunk / 4); item += blockDim.x) {
        const int rr = item / (kOcChunk / 4), wq = item % (kOcChunk / 4);
        const int64_t j = j0 + 4 * wq;
        const int32_t row = rowpos[rr];
        if (row >= 0 && j < kp) *reinterpret_cast<uint32_t*>(out + (int64_t)row * kp + j) = tile[rr * kOcStride + wq];
      }
      __syncthreads();
    }
  }
}

template <int DT>
hipError_t unpack_dt(int bits, const UnpackArgs& a, int batch, hipStream_t s) {
  const bool inner_contiguous = a.sk == 1;
  if (inner_contiguous) {
    const int lines = (int)min64(max64(a.n_outer * batch / 512, 1), 16);
    dim3 grid((unsigned)ceil_div(a.n_outer, lines), (unsigned)batch);
    switch (bits) {
#define IMU_UP(B)                                                                                  \
  case B:                                                                                          \
    hipLaunchKernelGGL((unpack_ic_kernel<DT, B>), grid, dim3(256), 0, s, a, lines);               \
    break;
      IMU_UP(2) IMU_UP(3) IMU_UP(4) IMU_UP(5) IMU_UP(6) IMU_UP(7) IMU_UP(8)
#undef IMU_UP
      default:
        return hipErrorInvalidValue;
    }
  } else {
    dim3 grid((unsigned)ceil_div(a.n_outer, 64), (unsigned)batch);
    switch (bits) {
#define IMU_UP(B)                                                                                  \
  case B:                                                                                          \
    hipLaunchKernelGGL((unpack_oc_kernel<DT, B>), grid, dim3(256), 0, s, a);                       \
    break;
      IMU_UP(2) IMU_UP(3) IMU_UP(4) IMU_UP(5) IMU_UP(6) IMU_UP(7) IMU_UP(8)
#undef IMU_UP
      default:
        return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_unpack(int dtype, int bits, const UnpackArgs& a, int batch, hipStream_t s) {
  return dtype == IMU_BF16 ? unpack_dt<IMU_BF16>(bits, a, batch, s) : unpack_dt<IMU_F32>(bits, a, batch, s);
}

}  // namespace imu
