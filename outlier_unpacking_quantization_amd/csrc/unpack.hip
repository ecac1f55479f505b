// Digit unpacking of one operand into int8 (gfx950).
//
// Method: summary page "IM-Unpack: Training and Inference with Arbitrarily Low
// Precision Integers": out-of-range integers are decomposed into several
// in-range low bit-width integers placed in extra rows / columns ("Approach"),
// turning each matrix into a larger one (summary paragraph).
//
// Layout written (per batch entry): A' is m_alloc x k_pad, B'^T is n_alloc x
// k_pad, int8, K' contiguous.  Row (line o, level u) sits at lvl[u][o]
// (level-major).  Column positions: exponent segment e = v + v' at seg_off[e],
// then k ascending (kpre[e][k]), then A's inner index v ascending.  Digit t of a
// code whose inner line has depth dK goes to inner index min(t, dK-1) and level
// t - min(t, dK-1); A' repeats over B's inner index v', B'^T over A's v.
#include "common.h"
#include "kernels.h"

namespace imu {

namespace {

constexpr int kChunk = 4096;  // K values staged in LDS at a time

template <int DT, int BITS>
__global__ __launch_bounds__(256) void unpack_kernel(UnpackArgs a, int64_t per_xcd) {
  using T = typename Elem<DT>::T;
  __shared__ int32_t qs[kChunk];
  const int b = blockIdx.y;
  // Workgroup ids are dealt round-robin over the 8 XCDs; give each XCD a run of
  // adjacent lines so strided operands share cache lines inside one L2.
  const int64_t bid = blockIdx.x;
  const int64_t o = (bid % 8) * per_xcd + bid / 8;
  if (o >= a.n_outer) return;
  const T* xb = static_cast<const T*>(a.x) + b * a.bstride;
  const float r = reinterpret_cast<const StatsHeader*>(a.stats + b * a.stats_stride)->r;
  const PlanLayout& L = a.pl;
  const uint8_t* pe = a.plan + L.headers_bytes + b * L.entry_stride;
  const PlanHeader* ph = reinterpret_cast<const PlanHeader*>(a.plan + b * kPlanHeaderStride);
  const int32_t* da_c = reinterpret_cast<const int32_t*>(pe + L.da_c);
  const int32_t* db_r = reinterpret_cast<const int32_t*>(pe + L.db_r);
  const int32_t* dout_arr = reinterpret_cast<const int32_t*>(pe + (a.operand == 0 ? L.da_r : L.db_c));
  const int32_t* lvl = reinterpret_cast<const int32_t*>(pe + (a.operand == 0 ? L.lvl_a : L.lvl_b));
  const int32_t* kpre = reinterpret_cast<const int32_t*>(pe + L.kpre);
  int64_t off = 0;
  for (int e = 0; e < b; ++e)
    off += unpacked_entry_bytes(reinterpret_cast<const PlanHeader*>(a.plan + e * kPlanHeaderStride), a.operand);
  int8_t* out = a.out + off;
  const int64_t K = a.K, kp = ph->k_pad, n_outer = a.n_outer;
  const int nseg = ph->n_seg;
  const int dout = dout_arr[o];
  const bool is_a = a.operand == 0;

  for (int64_t kc0 = 0; kc0 < K; kc0 += kChunk) {
    const int64_t kc1 = min64(K, kc0 + kChunk);
    __syncthreads();
    for (int64_t k = kc0 + threadIdx.x; k < kc1; k += blockDim.x) {
      T raw = xb[o * a.so + k * a.sk];
      float v;
      if constexpr (DT == IMU_BF16) v = bf16_to_f32(raw);
      else v = raw;
      bool bad = false;
      qs[k - kc0] = rtn_code(v, r, &bad);
    }
    __syncthreads();
    for (int u = 0; u < dout; ++u) {
      int8_t* row = out + (int64_t)lvl[(int64_t)u * n_outer + o] * kp;
      for (int s = 0; s < nseg; ++s) {
        const int32_t* kps = kpre + (int64_t)s * (K + 1);
        int8_t* seg = row + ph->seg_off[s];
        for (int64_t k = kc0 + threadIdx.x; k < kc1; k += blockDim.x) {
          const int dA = da_c[k], dB = db_r[k];
          const int lo = max(0, s - (dB - 1)), hi = min(dA - 1, s);
          if (hi < lo) continue;
          const int dK = is_a ? dA : dB;
          const int32_t q = qs[k - kc0];
          int8_t* p = seg + kps[k];
          for (int v = lo; v <= hi; ++v) {
            const int kap = is_a ? v : s - v;  // this operand's inner index
            const int t = kap < dK - 1 ? (u == 0 ? kap : -1) : kap + u;
            p[v - lo] = t < 0 ? (int8_t)0 : (int8_t)digit_of<BITS>(q, t);
          }
        }
      }
    }
  }
  // zero bytes that pad each segment to a multiple of kKPad
  for (int u = 0; u < dout; ++u) {
    int8_t* row = out + (int64_t)lvl[(int64_t)u * n_outer + o] * kp;
    for (int s = 0; s < nseg; ++s) {
      const int64_t p0 = ph->seg_off[s] + ph->seg_len[s], p1 = ph->seg_off[s + 1];
      for (int64_t p = p0 + threadIdx.x; p < p1; p += blockDim.x) row[p] = 0;
    }
  }
}

template <int DT>
hipError_t unpack_dt(int bits, const UnpackArgs& a, int batch, hipStream_t s) {
  const int64_t per_xcd = ceil_div(a.n_outer, 8);
  dim3 grid((unsigned)(per_xcd * 8), (unsigned)batch);
  switch (bits) {
#define IMU_UP(B)                                                                                  \
  case B:                                                                                          \
    hipLaunchKernelGGL((unpack_kernel<DT, B>), grid, dim3(256), 0, s, a, per_xcd);                \
    break;
    IMU_UP(2) IMU_UP(3) IMU_UP(4) IMU_UP(5) IMU_UP(6) IMU_UP(7) IMU_UP(8)
#undef IMU_UP
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_unpack(int dtype, int bits, const UnpackArgs& a, int batch, hipStream_t s) {
  return dtype == IMU_BF16 ? unpack_dt<IMU_BF16>(bits, a, batch, s) : unpack_dt<IMU_F32>(bits, a, batch, s);
}

}  // namespace imu
