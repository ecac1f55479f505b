// Digit unpacking of one operand into int8 (gfx950).
//
// Method: summary page "IM-Unpack: Training and Inference with Arbitrarily Low
// Precision Integers": out-of-range integers are decomposed into several
// in-range low bit-width integers placed in extra rows / columns ("Approach"),
// turning each matrix into a larger one (summary paragraph).
//
// Layout written (per batch entry): B'^T is n_alloc x k_pad, int8, row-major
// (K' contiguous).  A' (m_alloc x k_pad) is stored in MFMA fragment order: each
// block of 32 rows x 32 bytes of K' is 1 KB, lane l = (row % 32) + 32 * (16-byte
// half) holding 16 consecutive bytes, blocks ordered by row block then K' block
// (frag_row_offset / frag_pos_offset), so the GEMM reads A fragments as
// contiguous 1 KB loads.  Row (line o, level u) sits at lvl[u][o]
// (level-major).  Column j of a row holds the entry kmap[j] = (k, v, v') of the
// exponent segment it lies in (or zero padding).  Digit t of a code whose inner
// line has depth dK goes to inner index min(t, dK-1) and level t - min(t, dK-1),
// so at level 0 every position holds digit (own inner index) and at level u > 0
// only the last inner index dK-1 holds digit dK-1+u.
//
// Work split: a workgroup owns L lines and a run of k windows of W.  Per window
// it stages the lines' codes in LDS as sign-magnitude words (|q| << 1 | sign),
// with one pad word every 32 words, so that lanes reading nearby k hit distinct
// banks, and one zero word per line.  Then, for each level u and exponent
// segment s, it walks the K' positions whose k lies in the window, which are
// the contiguous range [seg_off + kpre[s][kw0], seg_off + kpre[s][kw1]), plus
// the segment's zero padding in the last window.  A thread decodes 4
// consecutive table entries once (LDS slot of k, bit offset of digit t) and
// then, for every line, reads 4 codes, extracts the digits and writes one dword
// (byte stores only where a window boundary cuts the dword), so every byte of
// every valid row is written exactly once.  Inner-contiguous operands (A
// row-major, B = W^T) stage 16 lines x 512 k with 16-byte loads;
// outer-contiguous operands (A = X^T, B row-major) stage 64 lines x 128 k, a
// wave reading 64 adjacent lines of one k.
#include "common.h"
#include "kernels.h"

namespace imu {

namespace {

constexpr int kThreads = 256;
constexpr int kTargetWgs = 2048;  // workgroups aimed for per launch (8 per CU)
constexpr int kInFlight = 4;      // table loads a thread issues before using them
constexpr uint32_t kDrop = 0x80000000u;     // store offset past any buffer: the store is dropped
constexpr int kBufferFlags = 0x00020000;    // buffer descriptor word 3 (raw byte-addressed access)

template <bool OC>
struct Shape {
  static constexpr int L = OC ? 64 : 16;     // lines per workgroup
  static constexpr int W = OC ? 128 : 512;   // k per window
  static constexpr int LS = W + W / 32 + 1;  // LDS words per line (odd)
};

template <int DT>
__device__ inline float load_elem(const typename Elem<DT>::T* p) {
  if constexpr (DT == IMU_BF16) return bf16_to_f32(*p);
  else return *p;
}

// 8 consecutive elements from a 16-byte aligned address.
template <int DT>
__device__ inline void load8_vec(const typename Elem<DT>::T* p, float v[8]) {
  if constexpr (DT == IMU_BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  } else {
    const float4 x0 = *reinterpret_cast<const float4*>(p);
    const float4 x1 = *reinterpret_cast<const float4*>(p + 4);
    v[0] = x0.x, v[1] = x0.y, v[2] = x0.z, v[3] = x0.w;
    v[4] = x1.x, v[5] = x1.y, v[6] = x1.z, v[7] = x1.w;
  }
}

__device__ inline int slot(int kk) { return kk + (kk >> 5); }

// Sign-magnitude word of the RTN code of x (|q| < 2^31, so |q| << 1 fits);
// with clipping the magnitude is min(rne(|x r|), beta).
__device__ inline uint32_t code_word(float x, float r, int clip, int beta) {
  if (clip) {
    const float y = x * r;
    const uint32_t m = (uint32_t)__builtin_rintf(__builtin_fminf(__builtin_fabsf(y), (float)beta));
    return (m << 1) | (uint32_t)(y < 0.f && m != 0);
  }
  bool bad = false;
  const int32_t q = rtn_code(x, r, &bad);
  const uint32_t m = q < 0 ? 0u - (uint32_t)q : (uint32_t)q;
  return (m << 1) | (uint32_t)(q < 0);
}

// The four low digits of the RTN code of x as two's-complement bytes (digit t
// in byte t), for codes with at most four digits (|q| < 2^(4 (BITS-1))).
template <int BITS>
__device__ inline uint32_t digit_word(float x, float r, int clip, int beta) {
  const float y = x * r;  // the RTN product; q = rne(y) (clamped to beta when clipping)
  const float ya = clip ? __builtin_fminf(__builtin_fabsf(y), (float)beta) : __builtin_fabsf(y);
  uint32_t m;             // |q|
  if constexpr (4 * (BITS - 1) <= 22) {
    // |y| < 2^22: adding 1.5 * 2^23 leaves rne(|y|) in the low mantissa bits
    m = __float_as_uint(ya + 12582912.0f) - 0x4B400000u;
  } else {
    m = (uint32_t)__builtin_rintf(ya);
  }
  uint32_t w;
  if constexpr (BITS == 5) {  // nibbles -> bytes
    const uint32_t p = __builtin_amdgcn_perm(m, m, 0x01010000u);  // bytes m0 m0 m1 m1
    w = (p & 0x000F000Fu) | ((p >> 4) & 0x0F000F00u);
  } else {
    constexpr uint32_t kD = BITS - 1, kMask = (1u << kD) - 1u;
    w = (m & kMask) | ((m >> kD) & kMask) << 8 | ((m >> (2 * kD)) & kMask) << 16 | ((m >> (3 * kD)) & kMask) << 24;
  }
  // negative codes: every byte d -> -d (bytes are at most 127, so 0x80 - d
  // never borrows); a zero code has zero bytes either way
  const uint32_t neg = (uint32_t)((int32_t)__float_as_uint(y) >> 31);
  return (w & ~neg) | (((0x80808080u - w) ^ 0x80808080u) & neg);
}

// e2m3 codes of the magnitudes 0..7 held in the bytes of m4 (byte-wise lookup)
__device__ inline uint32_t fp6_mag4(uint32_t m4) { return __builtin_amdgcn_perm(0x1E1C1A18u, 0x14100800u, m4); }

// The fp6 digit format's staging word: the e2m3 codes of the four low digits
// of the RTN code of x (digit t in byte t), for codes with at most four digits.
template <int BITS>
__device__ inline uint32_t digit_word6(float x, float r, int clip, int beta) {
  static_assert(BITS <= 4, "e2m3 holds digits up to 7");
  const float y = x * r;
  const float ya = clip ? __builtin_fminf(__builtin_fabsf(y), (float)beta) : __builtin_fabsf(y);
  const uint32_t m = __float_as_uint(ya + 12582912.0f) - 0x4B400000u;  // rne(|y|), |y| < 2^22
  constexpr uint32_t kD = BITS - 1, kMask = (1u << kD) - 1u;
  const uint32_t mags = (m & kMask) | ((m >> kD) & kMask) << 8 | ((m >> (2 * kD)) & kMask) << 16 |
                        ((m >> (3 * kD)) & kMask) << 24;
  const uint32_t c = fp6_mag4(mags);
  // sign bit 5 on the nonzero codes of a negative x (nonzero codes have bit 3 or 4)
  const uint32_t nz = ((c >> 3) | (c >> 4)) & 0x01010101u;
  const uint32_t neg = (uint32_t)((int32_t)__float_as_uint(y) >> 31);
  return c | ((nz << 5) & neg);
}

// e2m3 code (low byte) of the signed digit whose magnitude starts at bit sh1
// of the sign-magnitude word w; zero digits get code 0.
template <int BITS>
__device__ inline uint32_t fp6_digit(uint32_t w, uint32_t sh1) {
  const uint32_t d = (w >> sh1) & ((1u << (BITS - 1)) - 1u);
  const uint32_t c = fp6_mag4(d) & 0xFFu;
  return c | (c != 0u ? (w & 1u) << 5 : 0u);
}

typedef uint32_t v3u32 __attribute__((ext_vector_type(3)));
// Sixteen codes as four 24-bit runs -> the 12 bytes of the bit stream.
__device__ inline v3u32 pack6x16(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3) {
  return v3u32{p0 | p1 << 24, p1 >> 8 | p2 << 16, p2 >> 16 | p3 << 8};
}

// Two's-complement byte of the signed digit whose magnitude starts at bit sh1
// of the sign-magnitude word w (sh1 = 1 + t (BITS-1) <= 31).
// digit_signed leaves garbage above the low byte (callers that pack bytes with
// v_perm only take the low byte).
template <int BITS>
__device__ inline uint32_t digit_signed(uint32_t w, uint32_t sh1) {
  const uint32_t d = (w >> sh1) & ((1u << (BITS - 1)) - 1u);
  const uint32_t sm = 0u - (w & 1u);
  return (d ^ sm) - sm;
}
template <int BITS>
__device__ inline uint32_t digit_byte(uint32_t w, uint32_t sh1) {
  return digit_signed<BITS>(w, sh1) & 0xFFu;
}

// Buffer-store offset of a row at byte offset ro (-1: absent row).
__device__ inline uint32_t buf_row(int64_t ro) { return ro < 0 ? kDrop : (uint32_t)ro; }

// Output dword of four positions: bytes c8[adr[0..3]] (digit bytes; loaded
// into 16-bit halves, so one shift-or packs them) or the low bytes of the
// digits extracted from sign-magnitude code words.
typedef uint16_t v2u16 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t dword_of_bytes(const uint8_t* c8, const uint32_t (&adr)[4]) {
  const v2u16 even = {c8[adr[0]], c8[adr[2]]}, odd = {c8[adr[1]], c8[adr[3]]};
  return __builtin_bit_cast(uint32_t, even) | __builtin_bit_cast(uint32_t, odd) << 8;
}
template <int BITS>
__device__ inline uint32_t dword_of_digits(const uint32_t* cl, const uint32_t (&adr)[4], const uint32_t (&sh)[4]) {
  const uint32_t b0 = digit_signed<BITS>(cl[adr[0]], sh[0]), b1 = digit_signed<BITS>(cl[adr[1]], sh[1]);
  const uint32_t b2 = digit_signed<BITS>(cl[adr[2]], sh[2]), b3 = digit_signed<BITS>(cl[adr[3]], sh[3]);
  // low bytes of b0..b3 -> bytes 0..3
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u), hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// A 64-bit value that every thread holds alike, as a scalar.
__device__ inline int64_t uniform64(int64_t v) {
  return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)v));
}

// Byte offset of entry b's unpacked operand in the buffer (entries in batch
// order; with after_a, B' entries follow all A' entries).  Returns -1 if any
// entry's plan failed or holds a negative size, so nothing gets placed from
// stale headers.
__device__ inline int64_t entry_offset(const uint8_t* plan, int batch, int b, int operand, bool after_a) {
  int64_t off = 0;
  for (int e = 0; e < batch; ++e) {
    const PlanHeader* h = reinterpret_cast<const PlanHeader*>(plan + e * kPlanHeaderStride);
    const int64_t ba = unpacked_entry_bytes(h, 0), bb = unpacked_entry_bytes(h, 1);
    if (h->status != 0 || ba < 0 || bb < 0) return -1;
    if (after_a) off += ba;
    if (e < b) off += operand == 0 ? ba : bb;
  }
  return off;
}

// The operands of one launch: workgroups [0, wgs[0]) serve op[0], the rest
// op[1]; inside an operand, workgroup w covers line block w % nblk and window
// group w / nblk (wpg windows each).
struct UnpackJobs {
  UnpackArgs op[2];
  int nops;
  int nblk[2], wgs[2], wpg[2];
};

// F6: the fp6 digit format (inner-contiguous shape, bits <= 4): groups of 16
// positions (12 bytes), each written by the window that holds its first
// position; the group that runs past a window's last position (one per
// segment at most) reads the elements of its remaining positions from global
// memory.
// (fp6: three workgroups per CU leave room for the 16-position groups of
// eight lines without spills)
template <int DT, int BITS, bool OC, bool F6>
__global__ __launch_bounds__(kThreads, F6 ? 3 : 4) void unpack_kernel(UnpackJobs J) {
  static_assert(!F6 || (!OC && BITS <= 4), "fp6 digits: inner-contiguous operands, bits <= 4");
  int bid = blockIdx.x, jo = 0;
  if (J.nops > 1 && bid >= J.wgs[0]) {
    bid -= J.wgs[0];
    jo = 1;
  }
  const UnpackArgs& a = J.op[jo];
  const int wins_per_wg = J.wpg[jo];
  const int blk_x = bid % J.nblk[jo], blk_y = bid / J.nblk[jo];
  using T = typename Elem<DT>::T;
  constexpr int L = Shape<OC>::L, W = Shape<OC>::W, LS = Shape<OC>::LS;
  constexpr int D = (31 + BITS - 2) / (BITS - 1);
  constexpr uint32_t kZero = LS - 1;  // zero word of each line
  __shared__ uint32_t codes[L * LS];
  __shared__ int64_t rowoff[L];  // row part of the byte offset of row (line, level u), -1 if absent
  __shared__ int64_t rowoffs[F6 ? D : 1][L];  // F6: the same for every level at once
  __shared__ int s_dout[L];
  __shared__ int32_t s_line[L];  // operand line staged in slot i
  __shared__ int64_t s_off[kMaxSeg + 1];
  __shared__ int64_t s_p0[kMaxSeg + 1], s_p1[kMaxSeg + 1];
  __shared__ int s_ng[kMaxSeg + 1], s_pre[kMaxSeg + 1];

  const int b = blockIdx.z;
  const int64_t o0 = (int64_t)blk_x * L;
  const int64_t K = a.K, nwin = ceil_div(K, W);
  const int64_t w_begin = (int64_t)blk_y * wins_per_wg;
  const int64_t w_end = min64(w_begin + wins_per_wg, nwin);
  if (w_begin >= w_end) return;
  const T* xb = static_cast<const T*>(a.x) + b * a.bstride;
  const StatsHeader* sth = reinterpret_cast<const StatsHeader*>(a.stats + b * a.stats_stride);
  const float r = sth->r;
  // Codes of at most four digits (the largest |x| decides): the staging keeps
  // each element's digits as bytes of one word, and the rows are assembled
  // from byte reads.  Otherwise it keeps sign-magnitude codes and extracts
  // digits per byte.  (Inner-contiguous shape only: the 64-line shape keeps
  // one form, which holds its per-thread table entries in registers.)
  const float fmax = __uint_as_float(sth->maxkey) * r;
  const bool fast = !OC && (a.clip || fmax < 2147483648.0f) && line_digits<BITS>(fmax, a.clip, a.beta) <= 4;
  const PlanLayout& P = a.pl;
  const uint8_t* pe = a.plan + P.headers_bytes + b * P.entry_stride;
  const PlanHeader* ph = reinterpret_cast<const PlanHeader*>(a.plan + b * kPlanHeaderStride);
  const bool is_a = a.operand == 0;
  const int32_t* dout = reinterpret_cast<const int32_t*>(pe + (is_a ? P.da_r : P.db_c));
  const int32_t* lvl = reinterpret_cast<const int32_t*>(pe + (is_a ? P.lvl_a : P.lvl_b));
  const int32_t* kpre = reinterpret_cast<const int32_t*>(pe + P.kpre);
  const uint32_t* kmap = reinterpret_cast<const uint32_t*>(pe + P.kmap);
  // entry placement and guards: nothing is written for an entry whose plan
  // failed or which would not fit in the buffer (the host reports both)
  const int64_t start = entry_offset(a.plan, (int)gridDim.z, b, a.operand, a.after_a != 0);
  if (start < 0 || start + unpacked_entry_bytes(ph, a.operand) > a.cap) return;
  if (ph->fmt != (F6 ? kDigitsFp6 : kDigitsInt8)) return;  // the host launches the plan's format
  int8_t* out = a.out + start;
  // this entry's bytes as a buffer when 32-bit offsets reach all of it
  const int64_t entry_bytes = unpacked_entry_bytes(ph, a.operand);
  const bool use_buf = entry_bytes < (int64_t)kDrop;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(out, (short)0, use_buf ? (int)entry_bytes : 0, kBufferFlags);
  const int64_t kp = ph->k_pad;
  const int nseg = ph->n_seg;
  const int tid = threadIdx.x;
  const int kap_sh = is_a ? 20 : 25, last_sh = is_a ? 30 : 31;
  const int64_t rowb = unpacked_row_bytes(kp, F6 ? kDigitsFp6 : kDigitsInt8);
  // byte offset of unpacked row `row` (the part that does not depend on the position)
  auto row_offset = [&](int64_t row) __attribute__((always_inline)) -> int64_t {
    if (row < 0) return -1;
    if constexpr (F6) return is_a ? frag6_row_offset(row, kp) : row * rowb;
    else return is_a ? frag_row_offset(row, kp) : row * kp;
  };

  for (int s = tid; s <= nseg; s += kThreads) s_off[s] = ph->seg_off[s];
  if (tid < L) {
    // B's lines (columns) in the plan's depth order (inner-contiguous shape):
    // slot o0 + i holds the column at that position, so a workgroup's lines
    // share their depth; otherwise the lines in index order
    int64_t line = min64(o0 + tid, a.n_outer - 1);
    if (!OC && !is_a && ph->b_perm && o0 + tid < a.n_outer)
      line = reinterpret_cast<const int32_t*>(pe + P.bmap)[o0 + tid] & 0xFFFFFF;
    s_line[tid] = (int32_t)line;
    s_dout[tid] = o0 + tid < a.n_outer ? dout[line] : 0;
    codes[tid * LS + kZero] = 0u;
  }
  __syncthreads();
  int umax = 0;
  for (int i = 0; i < L; ++i) umax = max(umax, s_dout[i]);
  if constexpr (F6) {
    // the rows of every level of the workgroup's lines, once (the window
    // loop's first barrier publishes them)
    for (int x = tid; x < umax * L; x += kThreads) {
      const int u = x / L, i = x - u * L;
      const int64_t row = s_dout[i] > u ? (int64_t)lvl[(int64_t)u * a.n_outer + s_line[i]] : (int64_t)-1;
      rowoffs[u][i] = row_offset(row);
    }
  }

  for (int64_t w = w_begin; w < w_end; ++w) {
    const int64_t kw0 = w * W, kw1 = min64(kw0 + W, K);
    const bool last_win = kw1 == K;
    __syncthreads();  // readers of the previous window are done
    // Loads that do not depend on the staged codes are issued first, so one
    // memory round trip covers them and the staging: this window's K' range of
    // every segment, and the level-0 rows of the lines.
    int64_t P0 = 0, P1 = 0;
    if (tid < nseg) {
      const int32_t* kps = kpre + (int64_t)tid * (K + 1);
      P0 = s_off[tid] + kps[kw0];
      P1 = last_win ? s_off[tid + 1] : s_off[tid] + kps[kw1];
    }
    int64_t row_u0 = -1;
    if (tid < L && s_dout[tid] > 0) row_u0 = lvl[s_line[tid]];
    auto stage = [&](auto word) __attribute__((always_inline)) {
      if constexpr (!OC) {
        constexpr int G = W / 8;  // groups of 8 k per line
        constexpr int kIter = L * G / kThreads;
        static_assert(L * G % kThreads == 0, "staging split");
        if (a.vec_ok && kw1 == kw0 + W) {
#pragma unroll
          for (int it = 0; it < kIter; ++it) {
            const int item = tid + it * kThreads;
            const int i = item / G, kk = (item % G) * 8;
            const int64_t o = s_line[i];
            float v[8];
            load8_vec<DT>(xb + o * a.so + kw0 + kk, v);
            uint32_t* dst = &codes[i * LS + slot(kk)];
#pragma unroll
            for (int j = 0; j < 8; ++j) dst[j] = word(v[j]);
          }
        } else {
#pragma unroll
          for (int it = 0; it < kIter; ++it) {
            const int item = tid + it * kThreads;
            const int i = item / G, kk = (item % G) * 8;
            const int64_t o = s_line[i];
            const T* line = xb + o * a.so;
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = load_elem<DT>(line + min64(kw0 + kk + j, K - 1) * a.sk);
            uint32_t* dst = &codes[i * LS + slot(kk)];
#pragma unroll
            for (int j = 0; j < 8; ++j) dst[j] = word(v[j]);
          }
        }
      } else {
        constexpr int kIter = L * W / kThreads;
        static_assert(L * W % kThreads == 0, "staging split");
#pragma unroll 8
        for (int it = 0; it < kIter; ++it) {
          const int item = tid + it * kThreads;
          const int i = item % L, kk = item / L;
          const int64_t o = min64(o0 + i, a.n_outer - 1);
          const int64_t k = min64(kw0 + kk, K - 1);
          codes[i * LS + slot(kk)] = word(load_elem<DT>(xb + o * a.so + k * a.sk));
        }
      }
    };
    const int clip = a.clip, beta = a.beta;
    if constexpr (F6) {
      if (fast) stage([&](float x) { return digit_word6<BITS>(x, r, clip, beta); });
      else stage([&](float x) { return code_word(x, r, clip, beta); });
    } else {
      if (fast) stage([&](float x) { return digit_word<BITS>(x, r, clip, beta); });
      else stage([&](float x) { return code_word(x, r, clip, beta); });
    }
    // this window's K' positions: per segment the range [P0, P1), as groups of
    // 4 positions (16 fully inside the range for F6) flattened over the
    // segments (s_pre: first flat group of each segment), so that all
    // segments' groups are spread over all threads
    if (tid <= nseg) {
      s_p0[tid] = P0;
      s_p1[tid] = P1;
      if constexpr (F6) s_ng[tid] = (int)max64(0, (P1 >> 4) - ((P0 + 15) >> 4));
      else s_ng[tid] = P1 > P0 ? (int)(((P1 + 3) >> 2) - (P0 >> 2)) : 0;
    }
    if (tid < L) rowoff[tid] = row_offset(row_u0);
    __syncthreads();
    if (tid <= nseg) {
      int run = 0;
      for (int q = 0; q < tid; ++q) run += s_ng[q];
      s_pre[tid] = run;
    }
    __syncthreads();
    // F6 walks the levels inside each work item (one pass here)
    for (int u = 0; u < (F6 ? min(umax, 1) : umax); ++u) {
      if (u > 0) {  // rows of the unpacked levels (rare): one more round trip each
        __syncthreads();  // readers of the previous level's rowoff are done
        if (tid < L) {
          const int64_t row = s_dout[tid] > u ? (int64_t)lvl[(int64_t)u * a.n_outer + s_line[tid]] : (int64_t)-1;
          rowoff[tid] = row_offset(row);
        }
        __syncthreads();
      }
      // row offsets as scalars (the same for every thread).  Buffer stores
      // take 32-bit offsets, kDrop for an absent row (kDrop + pos stays past
      // the end): held in SGPRs for 16 lines, re-read from LDS per use for 64.
      // The pointer stores of huge entries re-read the 64-bit offsets.
      constexpr int LR = L <= 16 ? L : 1;
      uint32_t rb_s[LR];
#pragma unroll
      for (int i = 0; i < LR; ++i) rb_s[i] = buf_row(uniform64(rowoff[i]));
#define IMU_RB(i) (L <= 16 ? rb_s[(i) % LR] : buf_row(uniform64(rowoff[i])))
#define IMU_RO(i) uniform64(rowoff[i])
      if constexpr (F6) {
        // work items: (group, part of the lines), NS parts of LP lines each, so
        // that a window's few 16-position groups still spread over all threads
        constexpr int NS = 2, LP = L / NS;
        const int gtot = s_pre[nseg];
        for (int it = tid; it < gtot * NS; it += kThreads) {
          const int gi = it / NS, part = it % NS;
          int lo = 0, hi = nseg - 1;  // segment of flat group gi: last s with s_pre[s] <= gi
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_pre[mid] <= gi) lo = mid;
            else hi = mid - 1;
          }
          const int64_t g = ((s_p0[lo] + 15) >> 4) + (gi - s_pre[lo]);  // group of positions 16g .. 16g + 15
          uint32_t ent[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 e4 = *reinterpret_cast<const uint4*>(kmap + 16 * g + 4 * q);
            ent[4 * q] = e4.x, ent[4 * q + 1] = e4.y, ent[4 * q + 2] = e4.z, ent[4 * q + 3] = e4.w;
          }
          const uint32_t pos = (uint32_t)(is_a ? frag6_pos_offset(16 * g) : 12 * g);
          // per position, once for all levels: LDS word of the element (the
          // zero word for a padding entry or an element outside the window)
          // in bits 0..15, its inner index in bits 16..20 and the last-index
          // flag in bit 21
          uint32_t pi[16];
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const uint32_t e = ent[c];
            const int kk = (int)((int64_t)(e & 0xFFFFFu) - kw0);
            const uint32_t w = e != kKmapPad && kk >= 0 && kk < W ? (uint32_t)slot(kk) : kZero;
            pi[c] = w | ((e >> kap_sh) & 31u) << 16 | ((e >> last_sh) & 1u) << 21;
          }
          const uint32_t* cpart = codes + part * LP * LS;  // the part's first line
          // digit words (FAST) or sign-magnitude code words, one instance each
          auto emit = [&](auto FAST) __attribute__((always_inline)) {
            constexpr bool kFast = decltype(FAST)::value;
            for (int uu = 0; uu < umax; ++uu) {
              // per position: LDS byte of the code of digit t (digit words),
              // or word of the element and shift of digit t (code words)
              uint32_t adr[16], sh[kFast ? 1 : 16];
#pragma unroll
              for (int c = 0; c < 16; ++c) {
                const uint32_t w = pi[c] & 0xFFFFu;
                const int kap = (int)((pi[c] >> 16) & 31u);
                const int t = uu == 0 ? kap : ((pi[c] >> 21) & 1u ? kap + uu : D);
                const bool ok = w != kZero && t < (kFast ? 4 : D);
                if constexpr (kFast) {
                  adr[c] = ok ? 4u * w + (uint32_t)t : 4u * kZero;
                } else {
                  adr[c] = ok ? w : kZero;
                  sh[c] = ok ? (uint32_t)(1 + t * (BITS - 1)) : 1u;
                }
              }
#pragma unroll
              for (int ii = 0; ii < LP; ++ii) {
                const uint32_t* cl = cpart + ii * LS;
                uint32_t cd[16];  // the 16 codes, each below 64
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                  if constexpr (kFast) cd[c] = reinterpret_cast<const uint8_t*>(cl)[adr[c]];
                  else cd[c] = fp6_digit<BITS>(cl[adr[c]], sh[c]);
                }
                // code c at bits [6c, 6c + 6) of the 96-bit group
                const v3u32 v = {cd[0] | cd[1] << 6 | cd[2] << 12 | cd[3] << 18 | cd[4] << 24 | cd[5] << 30,
                                 cd[5] >> 2 | cd[6] << 4 | cd[7] << 10 | cd[8] << 16 | cd[9] << 22 | cd[10] << 28,
                                 cd[10] >> 4 | cd[11] << 2 | cd[12] << 8 | cd[13] << 14 | cd[14] << 20 | cd[15] << 26};
                const int64_t ro = rowoffs[uu][part * LP + ii];
                if (use_buf) {
                  __builtin_amdgcn_raw_buffer_store_b96(v, rs, (int)(buf_row(ro) + pos), 0, 0);
                } else if (ro >= 0) {
                  uint32_t* dst = reinterpret_cast<uint32_t*>(out + ro + pos);
                  dst[0] = v.x, dst[1] = v.y, dst[2] = v.z;
                }
              }
            }
          };
          if (fast) emit(std::true_type{});
          else emit(std::false_type{});
        }
        // Tail groups: per segment, the group holding the range's last
        // position when it runs past the range (and starts inside it).  One
        // thread per (segment, line); positions past the range read their
        // element from global memory.
        for (int item = tid; item < nseg * L; item += kThreads) {
          const int s = item / L, i = item - s * L;
          const int64_t P0 = s_p0[s], P1 = s_p1[s], G = P1 & ~(int64_t)15;
          if ((P1 & 15) == 0 || G < P0 || s_dout[i] == 0) continue;
          const T* xl = xb + (int64_t)s_line[i] * a.so;
          uint32_t ent[16];
#pragma unroll
          for (int c = 0; c < 16; ++c) ent[c] = kmap[G + c];
          float xv[16];
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const bool glob = G + c >= P1 && ent[c] != kKmapPad;
            xv[c] = glob ? load_elem<DT>(xl + (int64_t)(ent[c] & 0xFFFFFu) * a.sk) : 0.f;
          }
          // the code words of the 16 positions (staged or read above), then
          // each level of the line
          uint32_t cw[16];
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const int kk = (int)((int64_t)(ent[c] & 0xFFFFFu) - kw0);  // in [0, W) for staged positions
            cw[c] = G + c < P1 ? codes[i * LS + (kk >= 0 && kk < W ? slot(kk) : (int)kZero)]
                               : code_word(xv[c], r, clip, beta);
          }
          for (int uu = 0; uu < s_dout[i]; ++uu) {
          const int64_t ro = rowoffs[uu][i];
          uint32_t pk[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const uint32_t e = ent[c];
            const int kap = (int)((e >> kap_sh) & 31u);
            const bool last = (e >> last_sh) & 1u;
            const int t = uu == 0 ? kap : (last ? kap + uu : D);
            uint32_t cd = 0;
            if (e != kKmapPad && t < D) {
              const uint32_t sh1 = (uint32_t)(1 + t * (BITS - 1));
              // staged digit words hold the codes of digits 0..3; the others
              // are sign-magnitude code words
              cd = fast && G + c < P1 ? (t < 4 ? (cw[c] >> (8 * t)) & 0xFFu : 0u) : fp6_digit<BITS>(cw[c], sh1);
            }
            pk[c >> 2] |= cd << (6 * (c & 3));
          }
          const v3u32 v = pack6x16(pk[0], pk[1], pk[2], pk[3]);
          if (ro < 0) continue;
          const int64_t at = ro + (is_a ? frag6_pos_offset(G) : G / 16 * 12);
          if (use_buf) {
            __builtin_amdgcn_raw_buffer_store_b96(v, rs, (int)at, 0, 0);
          } else {
            uint32_t* dst = reinterpret_cast<uint32_t*>(out + at);
            dst[0] = v.x, dst[1] = v.y, dst[2] = v.z;
          }
          }
        }
      } else {
        const int gtot = s_pre[nseg];
        for (int gb = 0; gb < gtot; gb += kThreads * kInFlight) {
          // table entries of up to kInFlight groups per thread, loads first
          uint4 e4[kInFlight];
          int64_t gq[kInFlight];
          int sq[kInFlight];
  #pragma unroll
          for (int j = 0; j < kInFlight; ++j) {
            const int gi = min(gb + tid + j * kThreads, gtot - 1);
            int lo = 0, hi = nseg - 1;  // segment of flat group gi: last s with s_pre[s] <= gi
            while (lo < hi) {
              const int mid = (lo + hi + 1) >> 1;
              if (s_pre[mid] <= gi) lo = mid;
              else hi = mid - 1;
            }
            sq[j] = lo;
            gq[j] = (s_p0[lo] >> 2) + (gi - s_pre[lo]);
            e4[j] = *reinterpret_cast<const uint4*>(kmap + 4 * gq[j]);
          }
  #pragma unroll
          for (int j = 0; j < kInFlight; ++j) {
            if (gb + tid + j * kThreads >= gtot) continue;
            const int64_t g = gq[j], P0 = s_p0[sq[j]], P1 = s_p1[sq[j]];
            const uint32_t ent[4] = {e4[j].x, e4[j].y, e4[j].z, e4[j].w};
            // per position: word of the element and shift of digit t (codes),
            // or byte t of the element's word (digit bytes, t < 4)
            uint32_t adr[4], sh[4];
            bool inr[4];
  #pragma unroll
            for (int c = 0; c < 4; ++c) {
              const int64_t p = 4 * g + c;
              inr[c] = p >= P0 && p < P1;
              const uint32_t e = ent[c];
              const int kap = (int)((e >> kap_sh) & 31u);
              const bool last = (e >> last_sh) & 1u;
              const int t = u == 0 ? kap : (last ? kap + u : D);
              const int kk = (int)((int64_t)(e & 0xFFFFFu) - kw0);
              const bool ok = inr[c] && e != kKmapPad && t < (fast ? 4 : D) && kk >= 0 && kk < W;
              adr[c] = fast ? (ok ? 4u * (uint32_t)slot(kk) + (uint32_t)t : 4u * kZero) : (ok ? (uint32_t)slot(kk) : kZero);
              sh[c] = ok ? (uint32_t)(1 + t * (BITS - 1)) : 1u;
            }
            const uint32_t pos = (uint32_t)(is_a ? frag_pos_offset(4 * g) : 4 * g);
            const bool full = inr[0] && inr[3];  // the whole dword lies in the range
            // rows of the group: digit (low byte, two's complement) of position c
            // in line cl from the digit bytes or from the sign-magnitude code
  #define IMU_EMIT_ROWS()                                                                                                           \
            if (use_buf) {                                                                                                          \
              /* Buffer stores at 32-bit offsets into this entry; absent rows and */                                                \
              /* bytes outside the range get an offset past the end, which the */                                                   \
              /* hardware drops, so the lines form one branch-free block in which */                                                \
              /* the LDS reads of later lines overlap the work on earlier ones. */                                                  \
              if (full) {                                                                                                           \
  _Pragma("unroll(L <= 16 ? L : 8)")                                                                                                \
                for (int i = 0; i < L; ++i) {                                                                                       \
                  const uint32_t o = IMU_RB(i) + pos;                                                                               \
                  const uint32_t* cl = codes + i * LS;                                                                              \
                  __builtin_amdgcn_raw_buffer_store_b32(IMU_DWORD(cl), rs, (int)o, 0, 0);                                           \
                }                                                                                                                   \
              } else {                                                                                                              \
  _Pragma("unroll 4")                                                                                                               \
                for (int i = 0; i < L; ++i) {                                                                                       \
                  const uint32_t rb = IMU_RB(i);                                                                                    \
                  const uint32_t* cl = codes + i * LS;                                                                              \
  _Pragma("unroll")                                                                                                                 \
                  for (int c = 0; c < 4; ++c) {                                                                                     \
                    const uint32_t o = inr[c] ? rb + pos + c : kDrop;                                                               \
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)IMU_DIG(cl, c), rs, (int)o, 0, 0);                                \
                  }                                                                                                                 \
                }                                                                                                                   \
              }                                                                                                                     \
            } else if (full) { /* entries of 2 GB and more: pointer stores, one line at a time */                                   \
  _Pragma("unroll")                                                                                                                 \
              for (int i = 0; i < L; ++i) {                                                                                         \
                const int64_t ro = IMU_RO(i);                                                                                       \
                if (ro < 0) continue; /* uniform: row offsets are scalar */                                                         \
                const uint32_t* cl = codes + i * LS;                                                                                \
                uint32_t dw = 0;                                                                                                    \
  _Pragma("unroll")                                                                                                                 \
                for (int c = 0; c < 4; ++c) dw |= (IMU_DIG(cl, c) & 0xFFu) << (8 * c);                                              \
                *reinterpret_cast<uint32_t*>(out + ro + pos) = dw;                                                                  \
              }                                                                                                                     \
            } else {                                                                                                                \
  _Pragma("unroll 4")                                                                                                               \
              for (int i = 0; i < L; ++i) {                                                                                         \
                const int64_t ro = IMU_RO(i);                                                                                       \
                if (ro < 0) continue;                                                                                               \
                const uint32_t* cl = codes + i * LS;                                                                                \
                int8_t* dst = out + ro + pos;                                                                                       \
  _Pragma("unroll")                                                                                                                 \
                for (int c = 0; c < 4; ++c)                                                                                         \
                  if (inr[c]) dst[c] = (int8_t)(uint8_t)(IMU_DIG(cl, c) & 0xFFu);                                                   \
              }                                                                                                                     \
            }
            if (fast) {
  #define IMU_DIG(cl, c) ((uint32_t)reinterpret_cast<const uint8_t*>(cl)[adr[c]])
  #define IMU_DWORD(cl) dword_of_bytes(reinterpret_cast<const uint8_t*>(cl), adr)
              IMU_EMIT_ROWS();
  #undef IMU_DWORD
  #undef IMU_DIG
            } else {
  #define IMU_DIG(cl, c) digit_signed<BITS>((cl)[adr[c]], sh[c])
  #define IMU_DWORD(cl) dword_of_digits<BITS>(cl, adr, sh)
              IMU_EMIT_ROWS();
  #undef IMU_DWORD
  #undef IMU_DIG
            }
  #undef IMU_EMIT_ROWS
          }
        }
      }
#undef IMU_RO
#undef IMU_RB
      __syncthreads();  // before rowoff and the segment ranges are rewritten
    }
  }
}

template <int DT, bool OC>
hipError_t unpack_launch(int bits, bool f6, const UnpackArgs* ops, int nops, int batch, hipStream_t s) {
  constexpr int L = Shape<OC>::L, W = Shape<OC>::W;
  UnpackJobs J{};
  J.nops = nops;
  int64_t total = 0;
  for (int o = 0; o < nops; ++o) {
    const UnpackArgs& a = ops[o];
    J.op[o] = a;
    const int64_t nblk = ceil_div(a.n_outer, L), nwin = ceil_div(a.K, W);
    const int64_t want_y = min64(nwin, max64(1, ceil_div(kTargetWgs, nblk * batch)));
    const int64_t wpg = ceil_div(nwin, want_y);
    const int64_t wgs = nblk * ceil_div(nwin, wpg);
    if (wgs > 0x3FFFFFFF || wpg > 0x7FFFFFFF) return hipErrorInvalidValue;
    J.nblk[o] = (int)nblk;
    J.wpg[o] = (int)wpg;
    J.wgs[o] = (int)wgs;
    total += wgs;
  }
  if (total == 0) return hipSuccess;
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  dim3 grid((unsigned)total, 1, (unsigned)batch);
  if (f6) {
    if constexpr (OC) {
      return hipErrorInvalidValue;
    } else {
      switch (bits) {
#define IMU_UP(B)                                                                                     \
  case B:                                                                                             \
    hipLaunchKernelGGL((unpack_kernel<DT, B, false, true>), grid, dim3(kThreads), 0, s, J);           \
    break;
        IMU_UP(2) IMU_UP(3) IMU_UP(4)
#undef IMU_UP
        default:
          return hipErrorInvalidValue;
      }
    }
    return hipGetLastError();
  }
  switch (bits) {
#define IMU_UP(B)                                                                                     \
  case B:                                                                                             \
    hipLaunchKernelGGL((unpack_kernel<DT, B, OC, false>), grid, dim3(kThreads), 0, s, J);             \
    break;
    IMU_UP(2) IMU_UP(3) IMU_UP(4) IMU_UP(5) IMU_UP(6) IMU_UP(7) IMU_UP(8)
#undef IMU_UP
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT>
hipError_t unpack_dt(int bits, const UnpackArgs* ops, int nops, int batch, hipStream_t s) {
  // operands with the same staging shape share a launch
  if (nops == 2 && (ops[0].sk == 1) != (ops[1].sk == 1)) {
    hipError_t e = unpack_dt<DT>(bits, ops, 1, batch, s);
    return e != hipSuccess ? e : unpack_dt<DT>(bits, ops + 1, 1, batch, s);
  }
  const bool f6 = ops[0].fmt == kDigitsFp6;
  for (int o = 0; o < nops; ++o)
    if (ops[o].fmt != ops[0].fmt || (f6 && (ops[o].sk != 1 || bits > 4))) return hipErrorInvalidValue;
  return ops[0].sk == 1 ? unpack_launch<DT, false>(bits, f6, ops, nops, batch, s)
                        : unpack_launch<DT, true>(bits, f6, ops, nops, batch, s);
}

}  // namespace

hipError_t launch_unpack(int dtype, int bits, const UnpackArgs* ops, int nops, int batch, hipStream_t s) {
  if (nops < 1 || nops > 2) return hipErrorInvalidValue;
  return dtype == IMU_BF16 ? unpack_dt<IMU_BF16>(bits, ops, nops, batch, s)
                           : unpack_dt<IMU_F32>(bits, ops, nops, batch, s);
}

}  // namespace imu
