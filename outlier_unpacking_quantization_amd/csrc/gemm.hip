// Low bit-width GEMM on the unpacked operands with the shift-and-accumulate
// fold and the dequantization epilogue (gfx950, int8 MFMA).
//
// Method: summary page "IM-Unpack: Training and Inference with Arbitrarily Low
// Precision Integers", "Approach": the original integer GEMM is reproduced
// exactly by low bit-width integer GEMMs followed by bit-shift scaling and
// accumulation.  Here every digit is int8 and the products run on
// v_mfma_i32_32x32x32_i8.  K' is split into exponent segments; walking them from
// the highest exponent down, acc = acc * 2^(bits-1) + P_e (Horner), so one set
// of int32 accumulators holds sum_e 2^((bits-1)e) P_e.  The epilogue folds the
// unpacked row (i, u) and column (n, w) into C[i, n] with a further shift of
// (bits-1)(u+w); all int32 arithmetic wraps modulo 2^32.
//
// Operands: A' (m_alloc x k_pad) and B'^T (n_alloc x k_pad), both K-contiguous,
// so both MFMA operands load 16 contiguous bytes per lane.
#include "common.h"
#include "kernels.h"

namespace imu {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 16;  // bytes per staged row (padding spreads LDS banks)

__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) int8_t sA[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) int8_t sB[BN * LDS_STRIDE];
  const PlanHeader* ph = reinterpret_cast<const PlanHeader*>(g.hdr);
  const int tn = blockIdx.x, tm = blockIdx.y;
  const bool base_tile = (int64_t)tm * BM < g.m_base && (int64_t)tn * BN < g.n_base;
  if (g.mode == 2 && base_tile) return;
  const int64_t row0 = (int64_t)tm * BM, col0 = (int64_t)tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nseg = ph->n_seg;
  const int shift = g.bits - 1;

  v16i acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16i{0};

  // global -> LDS: each thread copies 2 x 16 bytes of A and of B per K step
  const int ld_row = tid >> 1, ld_col = (tid & 1) * 32;
  const int8_t* ga = g.a_u + (row0 + ld_row) * g.k_pad + ld_col;
  const int8_t* gb = g.b_u + (col0 + ld_row) * g.k_pad + ld_col;

  for (int s = nseg - 1; s >= 0; --s) {
    if (s < nseg - 1) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = (int)((uint32_t)acc[i][j][r] << shift);
    }
    const int64_t k0 = ph->seg_off[s], k1 = ph->seg_off[s + 1];
    for (int64_t kk = k0; kk < k1; kk += BK) {
      const uint4 a0 = *reinterpret_cast<const uint4*>(ga + kk);
      const uint4 a1 = *reinterpret_cast<const uint4*>(ga + kk + 16);
      const uint4 b0 = *reinterpret_cast<const uint4*>(gb + kk);
      const uint4 b1 = *reinterpret_cast<const uint4*>(gb + kk + 16);
      __syncthreads();
      *reinterpret_cast<uint4*>(&sA[ld_row * LDS_STRIDE + ld_col]) = a0;
      *reinterpret_cast<uint4*>(&sA[ld_row * LDS_STRIDE + ld_col + 16]) = a1;
      *reinterpret_cast<uint4*>(&sB[ld_row * LDS_STRIDE + ld_col]) = b0;
      *reinterpret_cast<uint4*>(&sB[ld_row * LDS_STRIDE + ld_col + 16]) = b1;
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < BK / 32; ++ks) {
        const int koff = ks * 32 + (lane >> 5) * 16;
        v4i af[2], bf[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          af[i] = *reinterpret_cast<const v4i*>(&sA[(wm * 64 + i * 32 + (lane & 31)) * LDS_STRIDE + koff]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bf[j] = *reinterpret_cast<const v4i*>(&sB[(wn * 64 + j * 32 + (lane & 31)) * LDS_STRIDE + koff]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  // epilogue: accumulator register r of lane l holds tile element
  // (8*(r/4) + 4*(l/32) + r%4, l%32) of each 32x32 block
  const float sab = g.sa->s * g.sb->s;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t gr = row0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t gc = col0 + wn * 64 + j * 32 + (lane & 31);
        const int32_t v = acc[i][j][r];
        if (g.mode == 2) {
          const int32_t am = g.amap[gr], bm = g.bmap[gc];
          if (am < 0 || bm < 0) continue;
          const int sh = shift * ((am >> 24) + (bm >> 24));
          if (sh >= 32) continue;
          atomicAdd(&g.c[(int64_t)(am & 0xFFFFFF) * g.ldc + (bm & 0xFFFFFF)], (int)((uint32_t)v << sh));
        } else {
          if (gr >= g.M || gc >= g.N) continue;
          int32_t* cp = &g.c[gr * g.ldc + gc];
          const int32_t cv = g.mode == 1 ? (int32_t)((uint32_t)*cp + (uint32_t)v) : v;
          *cp = cv;
          if (g.out) g.out[gr * g.ldc + gc] = (float)cv * sab;
        }
      }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  const int64_t rows = g.mode == 2 ? g.m_alloc : g.m_base;
  const int64_t cols = g.mode == 2 ? g.n_alloc : g.n_base;
  dim3 grid((unsigned)(cols / BN), (unsigned)(rows / BM));
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace imu
