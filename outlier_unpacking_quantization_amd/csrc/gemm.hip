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
// Operands: A' (m_alloc x k_pad) and B'^T (n_alloc x k_pad), both K-contiguous.
// Workgroup tile 256 x 128, four waves stacked along M, each owning 64 rows x
// 128 columns (2 x 4 blocks of 32 x 32, 128 accumulator registers).  A wave's A
// rows belong to it alone, and A' is stored in MFMA fragment order, so its A
// fragments are contiguous 1 KB loads straight into registers; the B tile (128
// x 128 bytes per K step, read 8 lanes per 128-byte row) is shared by the four
// waves and goes through LDS, double-buffered, rows 144 bytes apart (16-byte
// reads of 8 consecutive rows then touch disjoint banks).  Both operands are
// prefetched two K steps ahead in a register ring (one wave per SIMD, so
// latency is hidden by depth rather than by occupancy).  This keeps LDS
// traffic at about 70% of its read bandwidth when the matrix cores run at peak,
// where staging both operands through LDS would exceed it.  Segments are padded
// to the K step, so a step never straddles two exponents.  Tiles are ordered in
// groups of 8 tile rows and dealt to the 8 XCDs in contiguous runs, so the
// workgroups sharing an XCD's L2 share A and B panels.
#include "common.h"
#include "kernels.h"

namespace imu {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int BSTR = BK + 16;  // LDS bytes per staged B row
constexpr int kGroupM = 8;     // tile rows per ordering group
constexpr int kXcds = 8;
constexpr int kDepth = 2;     // K steps of A and B in flight per thread
static_assert(BK == kKPad, "a K step must not straddle exponent segments");

struct TileCoord {
  int tm, tn;
};

// Workgroup w of a launch over tiles_m x tiles_n tiles -> its tile.  Hardware
// deals workgroups to XCDs round-robin (w % 8); XCD x gets the contiguous run of
// tile ids [start(x), start(x) + count(x)) in grouped order.
__device__ inline TileCoord tile_of(int w, int tiles_m, int tiles_n) {
  const int T = tiles_m * tiles_n;
  const int x = w % kXcds, slot = w / kXcds;
  const int per = T / kXcds, rem = T % kXcds;
  const int id = x * per + min(x, rem) + slot;
  const int group = id / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(kGroupM, tiles_m - first_m);
  const int in = id - group * kGroupM * tiles_n;
  return TileCoord{first_m + in % gm, in / gm};
}

__device__ inline void shift_acc(v16i (&acc)[2][4], int sh) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = sh >= 32 ? 0 : (int)((uint32_t)acc[i][j][r] << sh);
}

__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) int8_t sB[2][BN * BSTR];
  const PlanHeader* ph = reinterpret_cast<const PlanHeader*>(g.hdr);
  const int64_t rows = g.mode == 2 ? g.m_alloc : g.m_base;
  const int64_t cols = g.mode == 2 ? g.n_alloc : g.n_base;
  const int tiles_m = (int)(rows / BM), tiles_n = (int)(cols / BN);
  if ((int)blockIdx.x >= tiles_m * tiles_n) return;
  const TileCoord tc = tile_of(blockIdx.x, tiles_m, tiles_n);
  const bool base_tile = (int64_t)tc.tm * BM < g.m_base && (int64_t)tc.tn * BN < g.n_base;
  if (g.mode == 2 && base_tile) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t kp = g.k_pad;
  const int64_t row0 = (int64_t)tc.tm * BM + wave * 64, col0 = (int64_t)tc.tn * BN;
  const int shift = g.bits - 1;

  // A' is in fragment order: fragment f (rows row0 + 32f ..) of K substep q at
  // step k is the contiguous 1 KB at block (row0/32 + f, k/32 + q); lane l holds
  // bytes [16l, 16l + 16) of it.
  const int8_t* ga = g.a_u + frag_row_offset(row0, kp) + lane * 16;
  const int64_t ga_f1 = (kp >> 5) * 1024;
  // B staging: thread copies rows br + 32j (j < 4), bytes [bc, bc + 16) of the step
  const int br = tid >> 3, bc = (tid & 7) * 16;
  const int8_t* gb = g.b_u + (col0 + br) * kp + bc;
  const int64_t gb_j = 32 * kp;
  const int sb_w = br * BSTR + bc;
  // B fragment j (columns col0 + 32j + lane%32), substep q
  const int sb_r = (lane & 31) * BSTR + 16 * (lane >> 5);

  v16i acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16i{0};

  // Segment cursors (wave-uniform): segments run from the highest exponent
  // down; empty segments are skipped but still count in the shifts.
  const int nseg = ph->n_seg;
  const int64_t* off = ph->seg_off;
  const int64_t steps = kp / BK;
  int ls = nseg - 1;  // load cursor
  while (ls > 0 && off[ls] == off[ls + 1]) --ls;
  int64_t lk = off[ls], lend = off[ls + 1];
  int cs = ls;  // compute cursor
  int64_t ck = lk, cend = lend;
  auto advance = [&](int& s, int64_t& k, int64_t& end) {
    k += BK;
    if (k >= end && s > 0) {
      --s;
      while (s > 0 && off[s] == off[s + 1]) --s;
      k = off[s];
      end = off[s + 1];
    }
  };

  // Register ring over kDepth K steps: slot t holds the A fragments and the B
  // staging registers of the steps j with j % kDepth == t, loaded kDepth steps
  // before their use.  Loads past the last step re-read the last step (they
  // stay unconditional so the ring stays in registers); that data is never used.
  const int64_t k_last = kp - BK;
  v4i ar[kDepth][4][2];
  v4i bs[kDepth][4];
#define IMU_LOAD(t)                                                                          \
  {                                                                                          \
    const int64_t k_ = min64(lk, k_last);                                                    \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                          \
      ar[t][q][0] = *reinterpret_cast<const v4i*>(ga + k_ * 32 + 1024 * q);                  \
      ar[t][q][1] = *reinterpret_cast<const v4i*>(ga + ga_f1 + k_ * 32 + 1024 * q);          \
    }                                                                                        \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) bs[t][j] =                                 \
        *reinterpret_cast<const v4i*>(gb + j * gb_j + k_);                                   \
    advance(ls, lk, lend);                                                                   \
  }
#define IMU_STORE_B(t, buf) \
  _Pragma("unroll") for (int j = 0; j < 4; ++j) *reinterpret_cast<v4i*>(&sB[buf][sb_w + j * 32 * BSTR]) = bs[t][j];
#define IMU_STEP(t)                                                                              \
  if (i0 + t < steps) {                                                                          \
    const int64_t j_ = i0 + t;                                                                   \
    if (cs != prev_s) {                                                                          \
      shift_acc(acc, shift * (prev_s - cs));                                                     \
      prev_s = cs;                                                                               \
    }                                                                                            \
    const int8_t* sbuf = sB[j_ & 1];                                                             \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                              \
      v4i bf[4];                                                                                 \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) bf[j] =                                      \
          *reinterpret_cast<const v4i*>(sbuf + sb_r + j * 32 * BSTR + 32 * q);                   \
      _Pragma("unroll") for (int f = 0; f < 2; ++f)                                              \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                                              \
        acc[f][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ar[t][q][f], bf[j], acc[f][j], 0, 0, 0); \
    }                                                                                            \
    IMU_STORE_B((t + 1) % kDepth, (j_ + 1) & 1);                                                 \
    IMU_LOAD(t);                                                                                 \
    __syncthreads();                                                                             \
    advance(cs, ck, cend);                                                                       \
  }

  static_assert(kDepth == 2, "the ring below is written out for two slots");
  IMU_LOAD(0);
  IMU_LOAD(1);
  IMU_STORE_B(0, 0);
  __syncthreads();
  int prev_s = cs;
  for (int64_t i0 = 0; i0 < steps; i0 += kDepth) {
    IMU_STEP(0);
    IMU_STEP(1);
  }
#undef IMU_LOAD
#undef IMU_STORE_B
#undef IMU_STEP
  if (prev_s > 0) shift_acc(acc, shift * prev_s);  // exponents below the last non-empty segment

  // epilogue: accumulator register r of lane l holds element
  // (8*(r/4) + 4*(l/32) + r%4, l%32) of each 32x32 block
  const float sab = g.sa->s * g.sb->s;
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t gr = row0 + f * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t gc = col0 + j * 32 + (lane & 31);
        const int32_t v = acc[f][j][r];
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
  if (rows % BM || cols % BN) return hipErrorInvalidValue;
  const int64_t tiles = (rows / BM) * (cols / BN);
  if (tiles == 0) return hipSuccess;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace imu
