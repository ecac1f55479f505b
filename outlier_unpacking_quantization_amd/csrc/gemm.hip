// Low bit-width GEMM on the unpacked operands with the shift-and-accumulate
// fold and the dequantization epilogue (gfx950, int8 MFMA); one launch serves
// every batch entry (blockIdx.y).
//
// Method: summary page "IM-Unpack: Training and Inference with Arbitrarily Low
// Precision Integers", "Approach": the original integer GEMM is reproduced
// exactly by low bit-width integer GEMMs followed by bit-shift scaling and
// accumulation.  Here every digit is int8 and the products run on
// v_mfma_i32_32x32x32_i8.  K' is split into exponent segments; walking them from
// the highest exponent down, acc = acc * 2^(bits-1) + P_e (Horner), so one set
// of int32 accumulators holds sum_e 2^((bits-1)e) P_e.  The unpacked row (i, u)
// and column (n, w) fold into C[i, n] with a further shift of (bits-1)(u+w);
// all int32 arithmetic wraps modulo 2^32.  Extra columns (w > 0) of a plan
// without extra rows are folded inside the base tile of their original
// columns: the shift is one more exponent, so the tile walks (level, segment)
// pairs by combined exponent under the same Horner accumulator, with the B'^T
// rows of level w staged into the LDS slots of their own columns.  Extra rows
// fold in a separate pass of extra tiles with atomic adds.
//
// Operands: A' (m_alloc x k_pad) in MFMA fragment order and B'^T (n_alloc x
// k_pad), both K-contiguous.  Workgroup tile 256 x 128, four waves stacked along
// M, each owning 64 rows x 128 columns (2 x 4 blocks of 32 x 32, 128
// accumulator registers).  A wave's A rows belong to it alone, so its A
// fragments are contiguous 1 KB loads straight into registers, refilled one K
// substep at a time one step ahead; the B tile (128 x 128 bytes per K step) is
// shared by the four waves through LDS, double-buffered, rows 144 bytes apart
// (16-byte reads of 8 consecutive rows touch disjoint banks), its global loads
// two steps ahead.  B fragments are double-buffered by substep: the reads of
// substep q+1 are issued before the MFMAs of substep q, and substep 0 of the
// next step is read right after the barrier, under the MFMAs of substep 3.
// Segments are padded to the K step, so a step never straddles two exponents.
// Tiles are dealt to the 8 XCDs (hardware order w % 8) in contiguous runs of a
// grouped order (groups of 4 tile rows), so the workgroups sharing an XCD's L2
// share A and B panels.
#include <hip/hip_ext.h>

#include "common.h"
#include "kernels.h"

namespace imu {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int FR = 2;  // 32-row A fragments per wave
constexpr int BM = 128 * FR, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int BSTR = BK + 16;  // LDS bytes per staged B row
constexpr int kGroupM = 4;     // tile rows per ordering group
constexpr int kXcds = 8;
static_assert(BK == kKPad, "a K step must not straddle exponent segments");

struct TileCoord {
  int tm, tn;
};

// Workgroup w of a launch over tiles_m x tiles_n tiles -> its tile.  XCD
// x = w % 8 gets the contiguous run of ids [start(x), start(x) + count(x)) of the
// order (group of kGroupM tile rows, column, row).
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

// 4 x 4 transpose inside each quad of lanes: on entry lane c of the quad holds
// x[i] = element (i, c), on exit x[i] = element (c, i).  Two exchanges: the
// off-diagonal 2 x 2 blocks with lane c ^ 2, then the off-diagonal elements of
// each 2 x 2 block with lane c ^ 1.
__device__ inline void quad_transpose(int (&x)[4]) {
  const bool hi = (threadIdx.x & 2) != 0, odd = (threadIdx.x & 1) != 0;
  int s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = __builtin_amdgcn_mov_dpp(x[i], 0x4E, 0xF, 0xF, false);  // lane ^ 2
  x[0] = hi ? s[2] : x[0];
  x[1] = hi ? s[3] : x[1];
  x[2] = hi ? x[2] : s[0];
  x[3] = hi ? x[3] : s[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = __builtin_amdgcn_mov_dpp(x[i], 0xB1, 0xF, 0xF, false);  // lane ^ 1
  x[0] = odd ? s[1] : x[0];
  x[1] = odd ? x[1] : s[0];
  x[2] = odd ? s[3] : x[2];
  x[3] = odd ? x[3] : s[2];
}

__device__ inline void shift_acc(v16i (&acc)[FR][4], int sh) {
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = sh >= 32 ? 0 : (int)((uint32_t)acc[i][j][r] << sh);
}

// Position in the walk over K' steps: segment s (walked from the highest
// exponent down, empty segments skipped), K' offset k of the step and the end
// of its segment.  The segment table is read through the constant address
// space: the GEMM never writes it, so the loads are scalar and the cursors stay
// in SGPRs (vector loads here would make the compiler wait for the operand
// prefetches as well).
struct Cursor {
  int s;
  int64_t k, end;
};
typedef __attribute__((address_space(4))) const int64_t* SegTable;
__device__ inline void cursor_advance(Cursor& c, SegTable off) {
  c.k += BK;
  if (c.k >= c.end && c.s > 0) {
    --c.s;
    while (c.s > 0 && off[c.s] == off[c.s + 1]) --c.s;
    c.k = off[c.s];
    c.end = off[c.s + 1];
    // finish the scalar loads here: left pending, they would make the loop
    // wait on lgkmcnt(0) every step, which also drains the LDS reads in flight
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0) only
  }
}
__device__ inline Cursor cursor_top(int nseg, SegTable off) {
  Cursor c;
  c.s = nseg - 1;
  while (c.s > 0 && off[c.s] == off[c.s + 1]) --c.s;
  c.k = off[c.s];
  c.end = off[c.s + 1];
  return c;
}

// The walk of a tile that also folds extra columns (levels w > 0 of its own
// columns): pairs (level w, segment s) in decreasing order of the combined
// exponent w + s, each over its segment's K' steps, so one Horner accumulator
// holds sum 2^((bits-1)(s+w)) P_(w,s).  Empty segments are skipped; once the
// walk is over, k keeps growing (loads clamp it).
struct FoldCursor {
  int s, w, sum;
  int64_t k, end;
};
__device__ inline bool fold_next_pair(FoldCursor& c, int nseg, int nlev, SegTable off) {
  int s = c.s, w = c.w, sum = c.sum;
  for (;;) {
    if (w + 1 <= min(nlev - 1, sum)) {
      ++w;
    } else {
      if (sum == 0) return false;
      --sum;
      w = max(0, sum - (nseg - 1));
    }
    s = sum - w;
    if (off[s] != off[s + 1]) break;
  }
  c.s = s;
  c.w = w;
  c.sum = sum;
  c.k = off[s];
  c.end = off[s + 1];
  return true;
}
__device__ inline void fold_advance(FoldCursor& c, int nseg, int nlev, SegTable off) {
  c.k += BK;
  if (c.k >= c.end && fold_next_pair(c, nseg, nlev, off))
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0) only (see cursor_advance)
}
__device__ inline FoldCursor fold_top(int nseg, int nlev, SegTable off) {
  FoldCursor c;
  c.w = nlev - 1;
  c.sum = (nseg - 1) + (nlev - 1);
  c.s = nseg - 1;
  c.k = off[c.s];
  c.end = off[c.s + 1];
  if (c.k == c.end) fold_next_pair(c, nseg, nlev, off);
  return c;
}

typedef __attribute__((address_space(4))) const PlanHeader* HdrC;
constexpr int kMaxLevels = 32;  // digits of an int32 code in base 2^(bits-1), bits >= 2: at most 31

// FOLD: the base pass also folds the extra columns of entries whose plan has
// extra columns only (their levels w > 0 land on the tile's own columns), so
// those entries need no atomic pass.
template <bool FOLD>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) int8_t sB[2][BN * BSTR];
  __shared__ int32_t s_lvl[kMaxLevels - 1][BN];  // FOLD: B'^T row of (column, level w >= 1), -1 if none
  __shared__ int s_nlev;
  // this workgroup's batch entry: sizes from its plan header (scalar loads)
  const int entry = blockIdx.y;
  const uint8_t* hdr = g.plan + (int64_t)entry * kPlanHeaderStride;
  const HdrC ph = (HdrC)hdr;
  const int64_t m_alloc = ph->m_alloc, n_alloc = ph->n_alloc, m_base = ph->m_base, n_base = ph->n_base;
  const int64_t kp = ph->k_pad;
  const bool rowx = m_alloc > m_base, colx = n_alloc > n_base;
  // the atomic pass serves entries with extra rows (and their extra columns),
  // and entries with extra columns only unless those are folded in the base
  // pass (g.fold_cols)
  const bool atomic_entry = rowx || (colx && !g.fold_cols);
  if (g.mode == 2 && !atomic_entry) return;
  const int mode = g.mode == 2 ? 2 : atomic_entry ? 1 : 0;
  const bool colfold = FOLD && g.mode != 2 && !atomic_entry && colx;
  const int64_t rows = mode == 2 ? m_alloc : m_base;
  const int64_t cols = mode == 2 ? n_alloc : n_base;
  const int tiles_m = (int)(rows / BM), tiles_n = (int)(cols / BN);
  if ((int)blockIdx.x >= tiles_m * tiles_n) return;
  const TileCoord tc = tile_of(blockIdx.x, tiles_m, tiles_n);
  const bool base_tile = (int64_t)tc.tm * BM < m_base && (int64_t)tc.tn * BN < n_base;
  if (mode == 2 && base_tile) return;
  // the entry's operands follow those of the earlier entries
  int64_t a_off = 0, b_off = 0;
  for (int e = 0; e < entry; ++e) {
    const HdrC h = (HdrC)(g.plan + (int64_t)e * kPlanHeaderStride);
    a_off += round_up(h->m_alloc * h->k_pad, 256);
    b_off += round_up(h->n_alloc * h->k_pad, 256);
  }
  const uint8_t* pe = g.plan + g.headers_bytes + entry * g.entry_stride;
  const int32_t* amap = reinterpret_cast<const int32_t*>(pe + g.amap_off);
  const int32_t* bmap = reinterpret_cast<const int32_t*>(pe + g.bmap_off);
  const StatsHeader* sa = reinterpret_cast<const StatsHeader*>(g.stats_a + entry * g.stats_stride_a);
  const StatsHeader* sb = reinterpret_cast<const StatsHeader*>(g.stats_b + entry * g.stats_stride_b);
  int32_t* const c_e = g.c + entry * g.cbs;
  float* const out_e = g.out ? g.out + entry * g.cbs : nullptr;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = (int64_t)tc.tm * BM + wave * (32 * FR), col0 = (int64_t)tc.tn * BN;
  const int shift = g.bits - 1;

  // A' fragment f (rows row0 + 32f ..) of K substep q at step offset k is the
  // contiguous 1 KB at block (row0/32 + f, k/32 + q); lane l holds bytes
  // [16l, 16l + 16) of it.
  const int8_t* ga = g.a_u + a_off + frag_row_offset(row0, kp) + lane * 16;
  const int64_t ga_f = (kp >> 5) * 1024;
  // B staging: thread copies rows br + 32j (j < 4), bytes [bc, bc + 16) of the step
  const int br = tid >> 3, bc = (tid & 7) * 16;
  const int8_t* gb = g.b_u + b_off + (col0 + br) * kp + bc;
  const int64_t gb_j = 32 * kp;
  const int8_t* gbase = g.b_u + b_off + bc;
  const int sb_w = br * BSTR + bc;
  // B fragment j (columns col0 + 32j + lane%32) of substep q
  const int sb_r = (lane & 31) * BSTR + 16 * (lane >> 5);
  const int64_t k_last = kp - BK;  // loads past the walk re-read the last step (never used)

  v16i acc[FR][4];
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16i{0};

  const SegTable off = (SegTable)ph->seg_off;
  const int nseg = ph->n_seg;
  // levels of the tile's columns (1 unless this entry folds extra columns)
  int nlev = 1;
  int64_t gbo[4];    // byte offsets of the B staging rows at lb's level (FOLD)
  uint32_t bvm = 0xF, bvl = 0xF;  // rows present at lb's level / in the last load (FOLD)
  if constexpr (FOLD) {
    if (colfold) {
      const int32_t* dbc = reinterpret_cast<const int32_t*>(pe + g.db_c_off);
      const int32_t* lvlb = reinterpret_cast<const int32_t*>(pe + g.lvl_b_off);
      if (tid == 0) s_nlev = 1;
      __syncthreads();
      if (tid < BN && col0 + tid < g.N) atomicMax(&s_nlev, min(dbc[col0 + tid], kMaxLevels));
      __syncthreads();
      nlev = s_nlev;
      for (int i = tid; i < (nlev - 1) * BN; i += kThreads) {
        const int w = 1 + i / BN;
        const int64_t n = col0 + i % BN;
        s_lvl[w - 1][i % BN] = n < g.N ? lvlb[(int64_t)w * g.N + n] : -1;
      }
      __syncthreads();
    }
  }
  // B staging rows of level w for this thread (FOLD); absent ones re-read the
  // level-0 row and are zeroed when stored
  auto set_level = [&](int w) __attribute__((always_inline)) {
    bvm = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = br + 32 * j;
      int64_t r = col0 + c;
      if (w > 0) {
        const int32_t x = s_lvl[w - 1][c];
        if (x >= 0) r = x;
        bvm |= (uint32_t)(x >= 0) << j;
      } else {
        bvm |= 1u << j;
      }
      gbo[j] = r * kp;
    }
  };
  if constexpr (FOLD) set_level(0);
  const int64_t steps = kp / BK * nlev;
  using Cur = std::conditional_t<FOLD, FoldCursor, Cursor>;
  auto top = [&]() __attribute__((always_inline)) {
    if constexpr (FOLD) return fold_top(nseg, nlev, off);
    else return cursor_top(nseg, off);
  };
  auto adv = [&](Cur& c) __attribute__((always_inline)) {
    if constexpr (FOLD) fold_advance(c, nseg, nlev, off);
    else cursor_advance(c, off);
  };
  auto expo = [](const Cur& c) __attribute__((always_inline)) {
    if constexpr (FOLD) return c.sum;
    else return c.s;
  };
  Cur cc = top();        // compute
  Cur la = cc, lb = cc;  // A loads (one step ahead), B loads (two ahead)
  int lbw = 0;           // level of lb's rows (FOLD)

  v4i ar[4][FR];  // A fragments of the current step, refilled substep by substep
  v4i bs[4];      // B staging registers
  v4i bf[2][4];   // B fragments, double-buffered by substep
#define IMU_LOAD_A(q, k)                                                                       \
  {                                                                                            \
    const int64_t k_ = min64((k), k_last);                                                     \
    _Pragma("unroll") for (int f = 0; f < FR; ++f) ar[q][f] =                                  \
        *reinterpret_cast<const v4i*>(ga + f * ga_f + k_ * 32 + 1024 * (q));                   \
  }
#define IMU_LOAD_B(k)                                                                          \
  {                                                                                            \
    const int64_t k_ = min64((k), k_last);                                                     \
    if constexpr (FOLD) {                                                                      \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) bs[j] = *reinterpret_cast<const v4i*>(gbase + gbo[j] + k_); \
      bvl = bvm;                                                                               \
    } else {                                                                                   \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) bs[j] = *reinterpret_cast<const v4i*>(gb + j * gb_j + k_); \
    }                                                                                          \
  }
#define IMU_STORE_B(buf)                                                                       \
  _Pragma("unroll") for (int j = 0; j < 4; ++j) *reinterpret_cast<v4i*>(&sB[buf][sb_w + j * 32 * BSTR]) = \
      (!FOLD || ((bvl >> j) & 1u)) ? bs[j] : v4i{0, 0, 0, 0};
#define IMU_ADV_B()                                                                            \
  {                                                                                            \
    adv(lb);                                                                                   \
    if constexpr (FOLD) {                                                                      \
      if (lb.w != lbw) {                                                                       \
        lbw = lb.w;                                                                            \
        set_level(lbw);                                                                        \
      }                                                                                        \
    }                                                                                          \
  }
#define IMU_READ_B(d, sbuf, q) \
  _Pragma("unroll") for (int j = 0; j < 4; ++j) bf[d][j] = *reinterpret_cast<const v4i*>((sbuf) + sb_r + j * 32 * BSTR + 32 * (q));
#define IMU_MFMA(d, q)                                                                             \
  _Pragma("unroll") for (int f = 0; f < FR; ++f)                                                   \
  _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                    \
    acc[f][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ar[q][f], bf[d][j], acc[f][j], 0, 0, 0);

#pragma unroll
  for (int q = 0; q < 4; ++q) IMU_LOAD_A(q, la.k);
  adv(la);
  if constexpr (FOLD) set_level(lb.w), lbw = lb.w;
  IMU_LOAD_B(lb.k);
  IMU_ADV_B();
  IMU_STORE_B(0);
  IMU_LOAD_B(lb.k);
  IMU_ADV_B();
  __syncthreads();
  IMU_READ_B(0, sB[0], 0);
  int prev_s = expo(cc);
  for (int64_t i = 0; i < steps; ++i) {
    if (expo(cc) != prev_s) {  // Horner: the exponents between the two steps
      shift_acc(acc, shift * (prev_s - expo(cc)));
      prev_s = expo(cc);
    }
    const int8_t* sbuf = sB[i & 1];
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      IMU_READ_B((q + 1) & 1, sbuf, q + 1);
      __builtin_amdgcn_sched_barrier(0);
      IMU_MFMA(q & 1, q);
      IMU_LOAD_A(q, la.k);
      __builtin_amdgcn_sched_barrier(0);
    }
    IMU_STORE_B((i + 1) & 1);  // B of step i+1 (loaded during step i-1)
    IMU_LOAD_B(lb.k);          // B of step i+2
    IMU_ADV_B();
    __syncthreads();
    IMU_READ_B(0, sB[(i + 1) & 1], 0);
    __builtin_amdgcn_sched_barrier(0);
    IMU_MFMA(1, 3);
    IMU_LOAD_A(3, la.k);
    __builtin_amdgcn_sched_barrier(0);
    adv(la);
    adv(cc);
  }
#undef IMU_LOAD_A
#undef IMU_LOAD_B
#undef IMU_STORE_B
#undef IMU_READ_B
#undef IMU_MFMA
#undef IMU_ADV_B
  if (prev_s > 0) shift_acc(acc, shift * prev_s);  // exponents below the last non-empty segment

  // epilogue: accumulator register r of lane l holds element
  // (8*(r/4) + 4*(l/32) + r%4, l%32) of each 32x32 block.  Rows are visited one
  // at a time (f, r/4, r%4) with the four column blocks j of the row, so only a
  // row's pointers are live.
  const float sab = sa->s * sb->s;
  const int64_t ldc = g.ldc;
  const int64_t r_lane = row0 + 4 * (lane >> 5), c_lane = col0 + (lane & 31);
  if (mode == 2) {  // extra tiles: every element lands on some C[i, n] with its shift
#pragma unroll
    for (int f = 0; f < FR; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t gr = r_lane + f * 32 + 8 * (r >> 2) + (r & 3);
          const int64_t gc = c_lane + j * 32;
          const int32_t am = amap[gr], bm = bmap[gc];
          if (am < 0 || bm < 0) continue;
          const int sh = shift * ((am >> 24) + (bm >> 24));
          if (sh >= 32) continue;
          atomicAdd(&c_e[(int64_t)(am & 0xFFFFFF) * ldc + (bm & 0xFFFFFF)], (int)((uint32_t)acc[f][j][r] << sh));
        }
    return;
  }
  // Base tiles.  A 4 x 4 transpose inside each quad of lanes turns the four
  // rows r4 * 8 + 4 * (l / 32) + 0..3 held at column l % 32 into four
  // consecutive columns of row ... + l % 4, so each lane stores 16 bytes and a
  // store instruction covers eight full 128-byte row segments.  Needs 16-byte
  // aligned rows and the whole tile inside N; otherwise one element per store.
  const bool vec = (ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(c_e) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(out_e) & 15) == 0 && col0 + BN <= g.N;
  if (vec) {
    const int64_t r_v = row0 + 4 * (lane >> 5) + (lane & 3), c_v = col0 + 4 * ((lane & 31) >> 2);
#pragma unroll
    for (int f = 0; f < FR; ++f)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int64_t gr = r_v + f * 32 + 8 * r4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int x[4] = {acc[f][j][4 * r4], acc[f][j][4 * r4 + 1], acc[f][j][4 * r4 + 2], acc[f][j][4 * r4 + 3]};
          quad_transpose(x);
          if (gr < g.M) {
            v4u v = {(uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]};
            v4u* cp = reinterpret_cast<v4u*>(c_e + gr * ldc + c_v + 32 * j);
            if (mode == 1) v += *cp;
            *cp = v;
            if (out_e) {
              const float4 o = {(float)(int32_t)v.x * sab, (float)(int32_t)v.y * sab, (float)(int32_t)v.z * sab,
                                (float)(int32_t)v.w * sab};
              *reinterpret_cast<float4*>(out_e + gr * ldc + c_v + 32 * j) = o;
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    return;
  }
#pragma unroll
  for (int f = 0; f < FR; ++f)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
#pragma unroll
      for (int r3 = 0; r3 < 4; ++r3) {
        const int r = 4 * r4 + r3;
        const int64_t gr = r_lane + f * 32 + 8 * r4 + r3;
        if (gr >= g.M) continue;
        int32_t* crow = c_e + gr * ldc + c_lane;
        float* orow = out_e ? out_e + gr * ldc + c_lane : nullptr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (c_lane + 32 * j >= g.N) continue;
          const int32_t v = acc[f][j][r];
          const int32_t cv = mode == 1 ? (int32_t)((uint32_t)crow[32 * j] + (uint32_t)v) : v;
          crow[32 * j] = cv;
          if (orow) orow[32 * j] = (float)cv * sab;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, int64_t tiles_x, int batch, bool fold, hipStream_t s, hipEvent_t start,
                       hipEvent_t stop) {
  if (tiles_x > 0x7FFFFFFF || batch < 1 || batch > 65535) return hipErrorInvalidValue;
  if (tiles_x <= 0) {  // nothing to launch: the events still get recorded
    if (start) hipEventRecord(start, s);
    if (stop) hipEventRecord(stop, s);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)tiles_x, (unsigned)batch);
  if (fold) {
    if (start || stop) hipExtLaunchKernelGGL(gemm_kernel<true>, grid, dim3(kThreads), 0, s, start, stop, 0, g);
    else hipLaunchKernelGGL(gemm_kernel<true>, grid, dim3(kThreads), 0, s, g);
  } else {
    if (start || stop) hipExtLaunchKernelGGL(gemm_kernel<false>, grid, dim3(kThreads), 0, s, start, stop, 0, g);
    else hipLaunchKernelGGL(gemm_kernel<false>, grid, dim3(kThreads), 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace imu
