// Digit GEMM on the unpacked operands, with the shift-and-accumulate fold and
// the dequantization epilogue (gfx950); one launch serves every batch entry
// (blockIdx.y).
//
// Method: summary page "IM-Unpack: Training and Inference with Arbitrarily Low
// Precision Integers", "Approach".  Each unpacked matrix holds small signed
// digits; a digit of weight 2^((bits-1)t) contributes its product scaled by
// that power, so the scaled sum of the narrow products is the original integer
// product.  The digits are int8 bytes (v_mfma_i32_32x32x32_i8, int32
// accumulators) or, for bits <= 4, e2m3 codes (v_mfma_f32_32x32x64_f8f6f4:
// every product is an integer of magnitude at most 49, and the fp32
// accumulators hold integers, exact while their magnitude stays at most 2^24).
// K' is split into exponent segments; walking them from the highest exponent
// down, acc = acc * 2^(bits-1) + P_e (Horner), so one set of accumulators holds
// sum_e 2^((bits-1)e) P_e.  With fp6 digits each wave keeps an upper bound on
// its |acc| (a K step adds at most 128 (2^(bits-1)-1)^2); when the next step
// or Horner shift could pass 2^24 it takes the true maximum, and if that is
// still too large it adds its exact partial sum, shifted to its exponent, into
// C (int32 arithmetic modulo 2^32) and restarts from zero.  The unpacked row (i, u) and column (n, w) fold
// into C[i, n] with a further shift of (bits-1)(u+w); all int32 arithmetic
// wraps modulo 2^32.  Extra columns (w > 0) of a plan without extra rows are
// folded inside the base tile of their original columns: the shift is one
// more exponent, so the tile walks (level, segment) pairs by combined exponent
// under the same Horner accumulator, with the B'^T rows of level w staged into
// the LDS slots of their own columns.  The plan puts B's columns in depth
// order (descending, then by index), so a tile's 128 columns share their depth
// except at the few tiles where the depth changes, the tile runs only the
// levels its columns have, and level w's rows of the tile are contiguous in
// B'^T; the epilogue stores each column through the order's map.  Extra rows
// fold in a separate pass of extra tiles with atomic adds.
//
// Operands: A' (m_alloc x k_pad) in MFMA fragment order and B'^T (n_alloc x
// k_pad), both K-contiguous.  Workgroup tile 256 x 128, four waves stacked along
// M, each owning 64 rows x 128 columns (2 x 4 blocks of 32 x 32, 128
// accumulator registers).  A K step is 128 positions: 4 substeps of 32 (int8)
// or 2 of 64 (fp6).  A wave's A rows belong to it alone, so its A fragments
// are contiguous loads straight into registers, refilled one K substep at a
// time one step ahead, one load after each MFMA of the substep; the B tile is
// shared by the four waves through LDS, double-buffered (int8 rows 144 bytes
// apart: 16-byte reads of 8 consecutive rows touch disjoint banks; fp6 rows 104
// bytes apart), its global loads two steps ahead.  B fragments are
// double-buffered by substep: the reads of substep q+1 are issued before the
// MFMAs of substep q, and substep 0 of the next step is read right after the
// barrier, under the MFMAs of the last substep.  Segments are padded to the K
// step, so a step never straddles two exponents.  Tiles are dealt to the 8
// XCDs (hardware order w % 8) in contiguous runs of a grouped order (groups of
// G tile rows, G chosen by the host to minimise the L2 fills), so the
// workgroups sharing an XCD's L2 share A and B panels; inside a group the tile
// columns are taken in residue classes mod 8, which spreads the deep (costly)
// columns over all runs.
#include <hip/hip_ext.h>

#include "common.h"
#include "kernels.h"

namespace imu {

namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int BSTR = BK + 16;  // LDS bytes per staged B row
constexpr int BSTR6 = BK / 4 * 3 + 8;  // fp6: 96 bytes of a step plus 8 (row r starts at bank 26 r mod 32)
constexpr uint32_t kF32Exact = 1u << 24;  // integers up to 2^24 in magnitude are exact in binary32
constexpr int kXcds = 8;
static_assert(BK == kKPad, "a K step must not straddle exponent segments");

struct TileCoord {
  int tm, tn;
};

// Tile column at position j of a group's column order: the residue classes
// of the column index mod 8 in turn (0, 8, 16, ..., then 1, 9, ...).  B's
// columns are in depth order, so the deepest (costliest) tile columns come
// first; taking the classes in turn gives every XCD's run a share of each
// depth, and the tiles of a run still share their A and B panels.
__device__ inline int col_interleave(int j, int n) {
  const int q = n >> 3, r = n & 7;  // classes c < r hold q + 1 columns, the others q
  if (j < r * (q + 1)) {
    const int c = j / (q + 1);
    return c + 8 * (j - c * (q + 1));
  }
  const int jj = j - r * (q + 1), c = jj / q;  // q >= 1 here, since j < n
  return r + c + 8 * (jj - c * q);
}

// Workgroup w of a launch over tiles_m x tiles_n tiles -> its tile.  XCD
// x = w % 8 gets the contiguous run of ids [start(x), start(x) + count(x)) of the
// order (group of G tile rows, interleaved column, row).
__device__ inline TileCoord tile_of(int w, int tiles_m, int tiles_n, int G) {
  const int T = tiles_m * tiles_n;
  const int x = w % kXcds, slot = w / kXcds;
  const int per = T / kXcds, rem = T % kXcds;
  const int id = x * per + min(x, rem) + slot;
  const int group = id / (G * tiles_n);
  const int first_m = group * G;
  const int gm = min(G, tiles_m - first_m);
  const int in = id - group * G * tiles_n;
  return TileCoord{first_m + in % gm, col_interleave(in / gm, tiles_n)};
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

template <int FR>
__device__ inline void shift_acc(v16i (&acc)[FR][4], int sh) {
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = sh >= 32 ? 0 : (int)((uint32_t)acc[i][j][r] << sh);
}
// fp6: multiply the accumulators by 2^sh, 0 <= sh <= 24 (exact: a power of
// two, and the products stay finite)
template <int FR>
__device__ inline void shift_acc(v16f (&acc)[FR][4], int sh) {
  const float f = __int_as_float((127 + sh) << 23);
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] *= f;
}
// fp6: largest |acc| of the wave (an integer at most 2^24), wave-uniform
template <int FR>
__device__ inline uint32_t wave_absmax(const v16f (&acc)[FR][4]) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) m = __builtin_fmaxf(m, __builtin_fabsf(acc[i][j][r]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o, 64));
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)m);
}
// an accumulator as the int32 it stands for, times 2^sh, modulo 2^32 (fp6
// accumulators hold integers of magnitude at most 2^24)
__device__ inline int32_t acc_int(int32_t v, int sh) { return sh >= 32 ? 0 : (int32_t)((uint32_t)v << sh); }
__device__ inline int32_t acc_int(float v, int sh) { return sh >= 32 ? 0 : (int32_t)((uint32_t)(int32_t)v << sh); }

// Position in a walk over K' steps.  Without column folding the walk takes
// the segments s from the highest exponent down (empty segments skipped), the
// exponent being e = s.  With it, the walk takes the pairs (level w, segment s)
// in decreasing order of the combined exponent e = w + s, so one Horner
// accumulator holds sum 2^((bits-1)(s+w)) P_(w,s).  k is the K' offset of the
// step; `left` counts the steps up to the end of the segment, so the common
// step is an add and a count, and the segment table (read through the
// constant address space: the GEMM never writes it, so the loads are scalar
// and the cursors stay in SGPRs) is looked at only when a segment ends.  Once
// the walk is over, k keeps growing (loads clamp it) and `left` is too large
// to run out.  K' < 2^31 (K < 2^20 and at most 31 x 31 digit pairs per
// position), so offsets in positions fit 32 bits.
struct Walk {
  int k, left, s, w, e;
};
typedef __attribute__((address_space(4))) const int64_t* SegTable;
constexpr int kWalkOver = 1 << 30;

__device__ inline void walk_enter(Walk& c, SegTable off) {
  c.k = (int)off[c.s];
  c.left = (int)((off[c.s + 1] - off[c.s]) / BK);
}
// Next non-empty segment (pair) after the current one; false when the walk is over.
template <bool FOLD>
__device__ inline bool walk_next(Walk& c, int nseg, int nlev, SegTable off) {
  if constexpr (FOLD) {
    int w = c.w, e = c.e, s;
    for (;;) {
      if (w + 1 <= min(nlev - 1, e)) {
        ++w;
      } else {
        if (e == 0) return false;
        --e;
        w = max(0, e - (nseg - 1));
      }
      s = e - w;
      if (off[s] != off[s + 1]) break;
    }
    c.s = s, c.w = w, c.e = e;
  } else {
    int s = c.s;
    do {
      if (s == 0) return false;
      --s;
    } while (off[s] == off[s + 1]);
    c.s = s, c.e = s;
  }
  walk_enter(c, off);
  return true;
}
template <bool FOLD>
__device__ inline Walk walk_top(int nseg, int nlev, SegTable off) {
  Walk c;
  c.s = nseg - 1;
  c.w = FOLD ? nlev - 1 : 0;
  c.e = c.s + c.w;
  walk_enter(c, off);
  if (c.left == 0 && !walk_next<FOLD>(c, nseg, nlev, off)) c.left = kWalkOver;
  return c;
}
// One step along the walk; true when it entered a new segment.
template <bool FOLD>
__device__ inline bool walk_step(Walk& c, int nseg, int nlev, SegTable off) {
  c.k += BK;
  if (--c.left != 0) return false;
  const bool moved = walk_next<FOLD>(c, nseg, nlev, off);
  if (!moved) c.left = kWalkOver;
  // finish the scalar loads here: left pending, they would make the loop
  // wait on lgkmcnt(0) every step, which also drains the LDS reads in flight
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0) only
  return moved;
}

typedef __attribute__((address_space(4))) const PlanHeader* HdrC;

constexpr int kMaxLevels = 32;

// 64 zero bytes in global memory: a B staging load for a slot that is absent
// at a level (its column has fewer levels) reads here, at the same bytes every
// step, so the staged tile needs no per-step selection.
__device__ __attribute__((aligned(64))) const int8_t kZeroBlock[64] = {};  // digits of an int32 code in base 2^(bits-1), bits >= 2: at most 31

// FOLD: the base pass also folds the extra columns of entries whose plan has
// extra columns only (their levels w > 0 land on the tile's own columns), so
// those entries need no atomic pass.
// F6: fp6 digits (e2m3 codes) on v_mfma_scale_f32_32x32x64_f8f6f4 (unit
// scales): a K step is two substeps of 64 positions; the fp32 accumulators
// run the Horner sum themselves, kept at most 2^24 in magnitude (so exact) by
// the wave's bound and its flushes into C.  With a single set of
// accumulators the kernel fits two workgroups per CU.
// FR: 32-row A fragments per wave, 2 (tile 256 x 128) or, for int8 digits,
// 1 (tile 128 x 128: more, smaller tiles for launches that would leave CUs
// idle, and a third of the registers for more workgroups per CU).
template <bool FOLD, bool F6, int FR>
__global__ __launch_bounds__(kThreads, F6 || FR == 1 ? 2 : 1) void gemm_kernel(GemmArgs g) {
  constexpr int BM = 128 * FR;
  constexpr int SB = F6 ? BSTR6 : BSTR;  // LDS bytes per staged B row
  constexpr int NQ = F6 ? 2 : 4;         // MFMA substeps per K step
  __shared__ __attribute__((aligned(16))) int8_t sB[2][BN * SB];
  // this workgroup's batch entry: sizes from its plan header (scalar loads)
  const int entry = blockIdx.y;
  const uint8_t* hdr = g.plan + (int64_t)entry * kPlanHeaderStride;
  const HdrC ph = (HdrC)hdr;
  const int64_t m_alloc = ph->m_alloc, n_alloc = ph->n_alloc, m_base = ph->m_base, n_base = ph->n_base;
  const int64_t kp = ph->k_pad;
  if (ph->fmt != (F6 ? kDigitsFp6 : kDigitsInt8)) return;  // the host launches the plan's format
  const int64_t rowb = F6 ? kp / 4 * 3 : kp;                // bytes per B'^T row
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
  const TileCoord tc = tile_of(blockIdx.x, tiles_m, tiles_n, g.group_m);
  const bool base_tile = (int64_t)tc.tm * BM < m_base && (int64_t)tc.tn * BN < n_base;
  if (mode == 2 && base_tile) return;
  // the entry's operands follow those of the earlier entries
  int64_t a_off = 0, b_off = 0;
  for (int e = 0; e < entry; ++e) {
    const HdrC h = (HdrC)(g.plan + (int64_t)e * kPlanHeaderStride);
    const int64_t rb = h->fmt == kDigitsFp6 ? h->k_pad / 4 * 3 : h->k_pad;
    a_off += round_up(h->m_alloc * rb, 256);
    b_off += round_up(h->n_alloc * rb, 256);
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
  // contiguous block (row0/32 + f, k/32 + q) of 1 KB (int8: lane l holds bytes
  // [16l, 16l + 16)) or (row0/32 + f, k/64 + q) of 1536 bytes (fp6: lane l
  // holds bytes [24l, 24l + 24)).
  const int8_t* ga = g.a_u + a_off + (F6 ? frag6_row_offset(row0, kp) + lane * 24 : frag_row_offset(row0, kp) + lane * 16);
  const int64_t ga_f = F6 ? (kp >> 6) * 1536 : (kp >> 5) * 1024;
  // B staging.  int8: thread copies rows br + 32j (j < 4), bytes [bc, bc + 16)
  // of the step.  fp6: row br, bytes [bc, bc + 48) of the step's 96.
  constexpr int NB = F6 ? 1 : 4;  // B rows a thread stages
  const int br = F6 ? tid >> 1 : tid >> 3, bc = F6 ? (tid & 1) * 48 : (tid & 7) * 16;
  const int8_t* gb = g.b_u + b_off + (col0 + br) * rowb + bc;
  const int64_t gb_j = 32 * rowb;
  const int8_t* gbase = g.b_u + b_off + bc;
  const int sb_w = br * SB + bc;
  // B fragment j (columns col0 + 32j + lane%32) of substep q
  const int sb_r = (lane & 31) * SB + (F6 ? 24 : 16) * (lane >> 5);
  const int k_last = (int)(kp - BK);  // loads past the walk re-read the last step (never used)

  using Acc = std::conditional_t<F6, v16f, v16i>;
  Acc acc[FR][4];
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = Acc{0};

  const SegTable off = (SegTable)ph->seg_off;
  const int nseg = ph->n_seg;
  // levels of the tile's columns (1 unless this entry folds extra columns)
  int nlev = 1;
  // B staging rows at lb's level (FOLD): source of row j = gbase + gbo[j] +
  // (step byte offset & kmsk[j]); absent rows point at kZeroBlock with mask 0
  int64_t gbo[NB];
  uint32_t kmsk[NB];
  if constexpr (FOLD) {
    // levels present in the tile: B's columns are in depth order, so level w
    // is present iff some slot of the tile lies below lvcnt_b[w]
    if (colfold)
      while (nlev < kMaxLevels && (int64_t)ph->lvcnt_b[nlev] > col0) ++nlev;
  }
  // B staging rows of level w for this thread (FOLD): slot col0 + c of level
  // w > 0 is B'^T row lvbase_b[w] + col0 + c; slots past lvcnt_b[w] are absent
  // (their column has fewer levels) and stage zeros from kZeroBlock
  const int64_t zoff = (int64_t)((intptr_t)kZeroBlock - (intptr_t)gbase);
  auto set_level = [&](int w) __attribute__((always_inline)) {
    const int64_t cnt = w == 0 ? n_alloc : (int64_t)ph->lvcnt_b[w];
    const int64_t base = w == 0 ? 0 : ph->lvbase_b[w];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int c = br + 32 * j;
      const bool live = col0 + c < cnt;
      gbo[j] = live ? (base + col0 + c) * rowb : zoff;
      kmsk[j] = live ? 0xFFFFFFFFu : 0u;
    }
  };
  if constexpr (FOLD) set_level(0);
  const int64_t steps = kp / BK * nlev;

  Walk cc = walk_top<FOLD>(nseg, nlev, off);  // compute
  Walk la = cc, lb = cc;  // A loads (one step ahead), B loads (two ahead)
  int lbw = 0;            // level of lb's rows (FOLD)
  int prev_e = cc.e;   // exponent of the accumulators' contents
  // fp6: upper bound on the wave's |acc| (wave-uniform), what one K step can
  // add to it, and whether the wave has already added a partial sum into C
  uint32_t ub = 0;
  const uint32_t step_add = (uint32_t)(((1 << shift) - 1) * ((1 << shift) - 1) * BK);
  bool flushed = false;

  using Frag = std::conditional_t<F6, v8i, v4i>;  // MFMA operand (fp6: 6 of the 8 dwords)
  Frag ar[NQ][FR];  // A fragments of the current step, refilled substep by substep
  v4i bs[F6 ? 3 : 4];  // B staging registers
  Frag bf[2][4];    // B fragments, double-buffered by substep
#define IMU_LOAD_A(q, k)                                                                       \
  {                                                                                            \
    const int64_t k_ = min((k), k_last);                                                       \
    if constexpr (F6) {                                                                        \
      _Pragma("unroll") for (int f = 0; f < FR; ++f) {                                         \
        const int8_t* pa_ = ga + f * ga_f + k_ * 24 + 1536 * (q);                              \
        const v2i x0 = *reinterpret_cast<const v2i*>(pa_), x1 = *reinterpret_cast<const v2i*>(pa_ + 8), \
                  x2 = *reinterpret_cast<const v2i*>(pa_ + 16);                                \
        ar[q][f] = Frag{x0.x, x0.y, x1.x, x1.y, x2.x, x2.y, 0, 0};                             \
      }                                                                                        \
    } else {                                                                                   \
      _Pragma("unroll") for (int f = 0; f < FR; ++f) ar[q][f] =                                \
          *reinterpret_cast<const Frag*>(ga + f * ga_f + k_ * 32 + 1024 * (q));                \
    }                                                                                          \
  }
#define IMU_LOAD_B(k)                                                                          \
  {                                                                                            \
    const uint32_t kb_ = (uint32_t)(min((k), k_last) / 4) * (F6 ? 3u : 4u);  /* byte offset of the step */ \
    if constexpr (F6) {                                                                        \
      const int8_t* pb_ = FOLD ? gbase + gbo[0] + (kb_ & kmsk[0]) : gb + kb_;                  \
      _Pragma("unroll") for (int j = 0; j < 3; ++j) bs[j] = *reinterpret_cast<const v4i*>(pb_ + 16 * j); \
    } else if constexpr (FOLD) {                                                               \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                                            \
        bs[j] = *reinterpret_cast<const v4i*>(gbase + gbo[j] + (kb_ & kmsk[j]));              \
    } else {                                                                                   \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) bs[j] = *reinterpret_cast<const v4i*>(gb + j * gb_j + kb_); \
    }                                                                                          \
  }
#define IMU_STORE_B(buf)                                                                       \
  if constexpr (F6) {                                                                          \
    _Pragma("unroll") for (int j = 0; j < 3; ++j) {                                            \
      *reinterpret_cast<v2i*>(&sB[buf][sb_w + 16 * j]) = v2i{bs[j].x, bs[j].y};                \
      *reinterpret_cast<v2i*>(&sB[buf][sb_w + 16 * j + 8]) = v2i{bs[j].z, bs[j].w};            \
    }                                                                                          \
  } else {                                                                                     \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) *reinterpret_cast<v4i*>(&sB[buf][sb_w + j * 32 * SB]) = bs[j]; \
  }
#define IMU_ADV_B()                                                                            \
  if (walk_step<FOLD>(lb, nseg, nlev, off)) {                                                  \
    if constexpr (FOLD) {                                                                      \
      if (lb.w != lbw) {                                                                       \
        lbw = lb.w;                                                                            \
        set_level(lbw);                                                                        \
      }                                                                                        \
    }                                                                                          \
  }
#define IMU_READ_B(d, sbuf, q)                                                                 \
  if constexpr (F6) {                                                                          \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                            \
      const int8_t* pr_ = (sbuf) + sb_r + j * 32 * SB + 48 * (q);                              \
      const v2i x0 = *reinterpret_cast<const v2i*>(pr_), x1 = *reinterpret_cast<const v2i*>(pr_ + 8), \
                x2 = *reinterpret_cast<const v2i*>(pr_ + 16);                                  \
      bf[d][j] = Frag{x0.x, x0.y, x1.x, x1.y, x2.x, x2.y, 0, 0};                               \
    }                                                                                          \
  } else {                                                                                     \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) bf[d][j] = *reinterpret_cast<const Frag*>((sbuf) + sb_r + j * 32 * SB + 32 * (q)); \
  }
#define IMU_MFMA(d, q)                                                                             \
  _Pragma("unroll") for (int f = 0; f < FR; ++f)                                                   \
  _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                                  \
    if constexpr (F6)                                                                              \
      acc[f][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ar[q][f], bf[d][j], acc[f][j], 2, 2, 0, 0, 0, 0); \
    else                                                                                           \
      acc[f][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ar[q][f], bf[d][j], acc[f][j], 0, 0, 0);   \
  }

  // C stores of the wave's accumulators, each taken as the integer it holds
  // times 2^esh (modulo 2^32).  add: add to C (entries whose extra rows were
  // folded first, or after an earlier flush of this wave); last: also write the
  // dequantized output.
  auto store_c = [&](int esh, bool add, bool last) __attribute__((always_inline)) {
    // accumulator register r of lane l holds element
    // (8*(r/4) + 4*(l/32) + r%4, l%32) of each 32x32 block.  Rows are visited one
    // at a time (f, r/4, r%4) with the four column blocks j of the row, so only a
    // row's pointers are live.
    const float sab = sa->s * sb->s;
    const int64_t ldc = g.ldc;
    int64_t r_lane = row0 + 4 * (lane >> 5), c_lane = col0 + (lane & 31);
    // a flush sits in the K loop: its addresses are made opaque there, so the
    // compiler cannot hoist (and spill) them ahead of the loop
    if (!last) asm volatile("" : "+v"(r_lane), "+v"(c_lane));
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
            const int sh = esh + shift * ((am >> 24) + (bm >> 24));
            if (sh >= 32) continue;
            atomicAdd(&c_e[(int64_t)(am & 0xFFFFFF) * ldc + (bm & 0xFFFFFF)], acc_int(acc[f][j][r], sh));
          }
      return;
    }
    // Base tiles.  A 4 x 4 transpose inside each quad of lanes turns the four
    // rows r4 * 8 + 4 * (l / 32) + 0..3 held at column l % 32 into four
    // consecutive columns of row ... + l % 4, so each lane stores 16 bytes and a
    // store instruction covers eight full 128-byte row segments.  Needs 16-byte
    // aligned rows and the whole tile inside N; otherwise one element per store.
    // With B's columns in depth order (b_perm) the tile's slots map to scattered
    // columns of C: element stores through the column map.  A flush (not
    // last) also takes element stores, which need fewer registers.
    const bool bperm = ph->b_perm != 0;
    const bool vec = last && !bperm && (ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(c_e) & 15) == 0 &&
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
            int x[4] = {acc_int(acc[f][j][4 * r4], esh), acc_int(acc[f][j][4 * r4 + 1], esh),
                        acc_int(acc[f][j][4 * r4 + 2], esh), acc_int(acc[f][j][4 * r4 + 3], esh)};
            quad_transpose(x);
            if (gr < g.M) {
              v4u v = {(uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]};
              v4u* cp = reinterpret_cast<v4u*>(c_e + gr * ldc + c_v + 32 * j);
              if (add) v += *cp;
              *cp = v;
              if (last && out_e) {
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
    // column of C held by this lane in block j (slot c_lane + 32 j), -1 past N
    int64_t cmapx[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t slot = c_lane + 32 * j;
      cmapx[j] = slot >= g.N ? -1 : bperm ? (int64_t)(bmap[slot] & 0xFFFFFF) : slot;
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
          int32_t* crow = c_e + gr * ldc;
          float* orow = out_e ? out_e + gr * ldc : nullptr;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (cmapx[j] < 0) continue;
            const int32_t v = acc_int(acc[f][j][r], esh);
            const int32_t cv = add ? (int32_t)((uint32_t)crow[cmapx[j]] + (uint32_t)v) : v;
            crow[cmapx[j]] = cv;
            if (last && orow) orow[cmapx[j]] = (float)cv * sab;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  };

  // The prologue issues its loads in the loop's order (the last substep's A
  // fragments after the second B load), so the loads in flight at the loop
  // head are the same on entry and on the back edge: the wait before the B
  // store then covers the B loads only, not the A fragments issued after them.
  // the A loads of a substep go out one after each of its 8 MFMAs
// fp6 (two workgroups per CU): a wave raises its priority while it issues a
// substep's MFMAs, so the two waves of a SIMD take turns at the MFMA pipe
#define IMU_PRIO(p)                                                                            \
  if constexpr (F6) {                                                                          \
    __builtin_amdgcn_s_setprio(p);                                                             \
    __builtin_amdgcn_sched_barrier(0);                                                         \
  }
#define IMU_INTERLEAVE()                                                                       \
  _Pragma("unroll") for (int k_ = 0; k_ < 8; ++k_) {                                          \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); /* one MFMA */                          \
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); /* one vector-memory read */            \
  }
#pragma unroll
  for (int q = 0; q < NQ - 1; ++q) IMU_LOAD_A(q, la.k);
  if constexpr (FOLD) set_level(lb.w), lbw = lb.w;
  IMU_LOAD_B(lb.k);
  IMU_ADV_B();
  IMU_STORE_B(0);
  IMU_LOAD_B(lb.k);
  IMU_ADV_B();
  IMU_LOAD_A(NQ - 1, la.k);
  walk_step<FOLD>(la, nseg, nlev, off);
  __syncthreads();
  IMU_READ_B(0, sB[0], 0);
  const int nsteps = (int)steps;  // kp / BK * nlev < 2^29
  for (int i = 0; i < nsteps; ++i) {
    if constexpr (F6) {
      // Horner shift to this step's exponent, then the step: the accumulators
      // must stay at most 2^24 in magnitude.  If the bound does not allow it,
      // take the true maximum; if that does not allow it either, add the
      // partial sums (at the exponent they hold) into C and restart from zero.
      if (__builtin_expect(cc.e != prev_e || ub > kF32Exact - step_add, 0)) {
        const int sh = shift * (prev_e - cc.e);
        auto fits = [&](uint32_t u) __attribute__((always_inline)) {
          return u == 0 || (sh <= 24 && ((uint64_t)u << sh) + step_add <= kF32Exact);
        };
        if (!fits(ub)) {
          ub = wave_absmax(acc);
          if (!fits(ub)) {
            store_c(shift * prev_e, mode == 1 || flushed, false);
            flushed = true;
#pragma unroll
            for (int f = 0; f < FR; ++f)
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[f][j] = Acc{0};
            ub = 0;
          }
        }
        if (sh != 0) {
          shift_acc(acc, min(sh, 24));  // with sh > 24 the accumulators are zero here
          ub <<= min(sh, 24);
        }
        prev_e = cc.e;
      }
      ub += step_add;
    } else if (cc.e != prev_e) {  // Horner: the exponents between the two steps
      shift_acc(acc, shift * (prev_e - cc.e));
      prev_e = cc.e;
    }
    const int8_t* sbuf = sB[i & 1];
#pragma unroll
    for (int q = 0; q < NQ - 1; ++q) {
      IMU_READ_B((q + 1) & 1, sbuf, q + 1);
      __builtin_amdgcn_sched_barrier(0);
      IMU_PRIO(1);
      IMU_MFMA(q & 1, q);
      IMU_LOAD_A(q, la.k);
      IMU_INTERLEAVE();
      __builtin_amdgcn_sched_barrier(0);
      IMU_PRIO(0);
    }
    IMU_STORE_B((i + 1) & 1);  // B of step i+1 (loaded during step i-1)
    IMU_LOAD_B(lb.k);          // B of step i+2
    IMU_ADV_B();
    __syncthreads();
    IMU_READ_B(0, sB[(i + 1) & 1], 0);
    __builtin_amdgcn_sched_barrier(0);
    IMU_PRIO(1);
    IMU_MFMA(1, NQ - 1);
    IMU_LOAD_A(NQ - 1, la.k);
    IMU_INTERLEAVE();
    __builtin_amdgcn_sched_barrier(0);
    IMU_PRIO(0);
    walk_step<FOLD>(la, nseg, nlev, off);
    walk_step<FOLD>(cc, nseg, nlev, off);
  }
#undef IMU_INTERLEAVE
#undef IMU_PRIO
#undef IMU_LOAD_A
#undef IMU_LOAD_B
#undef IMU_STORE_B
#undef IMU_READ_B
#undef IMU_MFMA
#undef IMU_ADV_B
  // the exponent of the last non-empty segment is the shift still to apply
  store_c(shift * prev_e, mode == 1 || flushed, true);
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
  auto go = [&](auto kernel) {
    if (start || stop) hipExtLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, s, start, stop, 0, g);
    else hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, s, g);
  };
  if (g.fmt == kDigitsFp6 && g.tile_rows == 256) {
    if (fold) go(gemm_kernel<true, true, 2>);
    else go(gemm_kernel<false, true, 2>);
  } else if (g.fmt == kDigitsInt8 && g.tile_rows == 256) {
    if (fold) go(gemm_kernel<true, false, 2>);
    else go(gemm_kernel<false, false, 2>);
  } else if (g.fmt == kDigitsInt8 && g.tile_rows == 128) {
    if (fold) go(gemm_kernel<true, false, 1>);
    else go(gemm_kernel<false, false, 1>);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace imu
