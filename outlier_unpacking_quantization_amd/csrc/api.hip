// C ABI of the IM-Unpack integer GEMM library: set-up of the per-device
// context, argument validation, buffer carving, kernel launches and the one
// plan-header readback.  Contains no kernels; the device work lives in
// quantize.hip, plan.hip, unpack.hip and gemm.hip.
#include <algorithm>
#include <utility>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "common.h"
#include "kernels.h"

using namespace imu;

namespace {

// Detail of the last error on this thread.  Formatted into a fixed buffer, so
// that no entry point allocates host memory either.
thread_local char g_err[512];
thread_local hipEvent_t g_gemm_ev[2] = {nullptr, nullptr};  // imu_set_gemm_events

__attribute__((format(printf, 2, 3))) imu_status fail(imu_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

#define IMU_HIP(call)                                                                              \
  do {                                                                                             \
    hipError_t e_ = (call);                                                                        \
    if (e_ != hipSuccess) return fail(IMU_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_));        \
  } while (0)

#define IMU_TRY(call)                                                                              \
  do {                                                                                             \
    imu_status s_ = (call);                                                                        \
    if (s_ != IMU_OK) return s_;                                                                   \
  } while (0)

constexpr int64_t kMaxLine = (1ll << 24) - 1;  // line index packed in 24 bits of a map word

struct Operand {
  const imu_matrix* m;
  int64_t R, C;          // logical
  int64_t srows, scols;  // stored
  bool tr;
  int dtype;
  int elem;
};

imu_status check_matrix(const imu_matrix* x, const char* name, Operand* op) {
  if (!x) return fail(IMU_ERR_INVALID_ARG, "%s is NULL", name);
  if (!x->data) return fail(IMU_ERR_INVALID_ARG, "%s.data is NULL", name);
  if (x->dtype != IMU_F32 && x->dtype != IMU_BF16)
    return fail(IMU_ERR_INVALID_ARG, "%s.dtype must be IMU_F32 or IMU_BF16", name);
  if (x->layout != IMU_NORMAL && x->layout != IMU_TRANSPOSED)
    return fail(IMU_ERR_INVALID_ARG, "%s.layout must be IMU_NORMAL or IMU_TRANSPOSED", name);
  if (x->rows < 1 || x->cols < 1)
    return fail(IMU_ERR_INVALID_ARG, "%s must have rows >= 1 and cols >= 1", name);
  if (x->rows > kMaxLine || x->cols > kMaxLine)
    return fail(IMU_ERR_UNSUPPORTED, "%s: rows and cols must be below 2^24", name);
  if ((unsigned long long)x->rows * (unsigned long long)x->cols >= (1ull << 32))
    return fail(IMU_ERR_UNSUPPORTED, "%s: rows*cols must be below 2^32", name);
  if (x->batch < 1 || x->batch > 65535)
    return fail(IMU_ERR_INVALID_ARG, "%s.batch must be in [1, 65535]", name);
  op->m = x;
  op->R = x->rows;
  op->C = x->cols;
  op->tr = x->layout == IMU_TRANSPOSED;
  op->srows = op->tr ? x->cols : x->rows;
  op->scols = op->tr ? x->rows : x->cols;
  op->dtype = x->dtype;
  op->elem = x->dtype == IMU_F32 ? 4 : 2;
  if (x->ld < op->scols) return fail(IMU_ERR_INVALID_ARG, "%s.ld is below the stored row length", name);
  if (x->batch > 1 && x->batch_stride < (op->srows - 1) * x->ld + op->scols)
    return fail(IMU_ERR_INVALID_ARG, "%s.batch_stride overlaps batch entries", name);
  return IMU_OK;
}

imu_status check_params(const imu_params* p) {
  if (!p) return fail(IMU_ERR_INVALID_ARG, "params is NULL");
  if (p->bits < 2 || p->bits > 8) return fail(IMU_ERR_INVALID_ARG, "bits must be in [2, 8]");
  if (p->beta < 1) return fail(IMU_ERR_INVALID_ARG, "beta must be >= 1");
  if (p->p_den < 1 || p->p_den > 1000000) return fail(IMU_ERR_INVALID_ARG, "p_den must be in [1, 1e6]");
  if (p->p_num < 1 || p->p_num > p->p_den) return fail(IMU_ERR_INVALID_ARG, "p = p_num/p_den must be in (0, 1]");
  if (p->gamma < 0 || p->gamma > 1000000) return fail(IMU_ERR_INVALID_ARG, "gamma must be in [0, 1e6]");
  if (p->clip != 0 && p->clip != 1) return fail(IMU_ERR_INVALID_ARG, "clip must be 0 or 1");
  if (p->digits != IMU_DIGITS_AUTO && p->digits != IMU_DIGITS_INT8 && p->digits != IMU_DIGITS_FP6)
    return fail(IMU_ERR_INVALID_ARG, "digits must be IMU_DIGITS_AUTO, IMU_DIGITS_INT8 or IMU_DIGITS_FP6");
  for (int s : {p->strat_a, p->strat_b})
    if (s != IMU_ROW && s != IMU_COL && s != IMU_MIX && s != IMU_GREEDY)
      return fail(IMU_ERR_INVALID_ARG, "strategy must be IMU_ROW, IMU_COL, IMU_MIX or IMU_GREEDY");
  return IMU_OK;
}

// fp6 digits apply when every digit is at most 7 in magnitude (bits <= 4) and
// both operands are K-contiguous, the layout the fp6 unpack is written for.
bool fp6_applies(const Operand& oa, const Operand& ob, const imu_params* p) {
  return p->bits <= 4 && !oa.tr && ob.tr;
}
int digit_fmt(const Operand& oa, const Operand& ob, const imu_params* p) {
  return p->digits != IMU_DIGITS_INT8 && fp6_applies(oa, ob, p) ? kDigitsFp6 : kDigitsInt8;
}

imu_status check_pair(const imu_matrix* a, const imu_matrix* b, const imu_params* p, Operand* oa,
                      Operand* ob) {
  IMU_TRY(check_matrix(a, "a", oa));
  IMU_TRY(check_matrix(b, "b", ob));
  IMU_TRY(check_params(p));
  if (a->cols != b->rows) return fail(IMU_ERR_INVALID_ARG, "a.cols must equal b.rows (K)");
  if (a->cols > kMaxK) return fail(IMU_ERR_UNSUPPORTED, "K must be below 2^20 - 1");
  if (a->batch != b->batch) return fail(IMU_ERR_INVALID_ARG, "a.batch must equal b.batch");
  if ((p->strat_a == IMU_GREEDY && a->rows + a->cols > kGreedyMaxLines) ||
      (p->strat_b == IMU_GREEDY && b->rows + b->cols > kGreedyMaxLines))
    return fail(IMU_ERR_UNSUPPORTED, "the greedy planner holds at most %d rows + columns of an operand",
                kGreedyMaxLines);
  if (p->digits == IMU_DIGITS_FP6 && !fp6_applies(*oa, *ob, p))
    return fail(IMU_ERR_UNSUPPORTED, "fp6 digits need bits <= 4, A IMU_NORMAL and B IMU_TRANSPOSED");
  return IMU_OK;
}

StreamArgs stream_args(const Operand& op, uint8_t* stats, const StatsLayout& L, const imu_params* p) {
  StreamArgs s{};
  const imu_matrix* x = op.m;
  s.x = x->data;
  s.srows = op.srows;
  s.scols = op.scols;
  s.ld = x->ld;
  s.bstride = x->batch_stride;
  const bool aligned = (reinterpret_cast<uintptr_t>(x->data) % 16) == 0;
  s.vec_ok = aligned && op.scols % 8 == 0 && x->ld % 8 == 0 && (x->batch == 1 || x->batch_stride % 8 == 0);
  s.stats = stats;
  s.stats_stride = L.stride;
  s.srow_oob = op.tr ? L.col_oob : L.row_oob;
  s.scol_oob = op.tr ? L.row_oob : L.col_oob;
  s.srow_maxdig = op.tr ? L.col_maxdig : L.row_maxdig;
  s.scol_maxdig = op.tr ? L.row_maxdig : L.col_maxdig;
  s.srow_res = op.tr ? L.rc_coldig : L.cr_rowdig;
  s.scol_res = op.tr ? L.cr_rowdig : L.rc_coldig;
  s.hist = L.hist;
  s.transposed = op.tr ? 1 : 0;
  s.beta = p->beta;
  s.p_num = p->p_num;
  s.p_den = p->p_den;
  s.gamma = p->gamma;
  s.clip = p->clip;
  return s;
}

// Quantize up to two operands; operands of one dtype share every launch.
// `zeroed`: the caller already cleared the statistics buffers.
imu_status quantize_ops(const Operand* const* ops, uint8_t* const* stats, int32_t* const* q, int nops,
                        const imu_params* p, hipStream_t s, bool zeroed) {
  if (!zeroed)
    for (int i = 0; i < nops; ++i)
      IMU_HIP(launch_fill_u32(stats[i], 0u, stats_layout(ops[i]->R, ops[i]->C).stride * ops[i]->m->batch / 4, s));
  for (int dt : {(int)IMU_BF16, (int)IMU_F32}) {
    QuantJobs J{};
    int32_t* qq[2] = {nullptr, nullptr};
    for (int i = 0; i < nops; ++i) {
      if (ops[i]->dtype != dt) continue;
      QuantOp& o = J.op[J.nops];
      o.s = stream_args(*ops[i], stats[i], stats_layout(ops[i]->R, ops[i]->C), p);
      o.batch = (int)ops[i]->m->batch;
      qq[J.nops] = q[i];
      ++J.nops;
    }
    if (!J.nops) continue;
    IMU_HIP(launch_hist(dt, J, 0, dt == IMU_BF16, s));
    if (dt == IMU_F32) {
      IMU_HIP(launch_hist(dt, J, 1, 0, s));
      IMU_HIP(launch_hist(dt, J, 2, 1, s));
    }
    IMU_HIP(launch_round_count(dt, p->bits, J, qq[0], qq[1], s));
  }
  return IMU_OK;
}

// Statistics of one operand as the planner reads them: computed in this call
// (layout of the operand's own shape), or prepared by imu_prepare_operand,
// possibly for the operand's transpose (then the row and column arrays swap
// roles: a row of the operand is a column of the matrix they describe).
struct StatsRef {
  uint8_t* stats;
  StatsLayout L;
  bool prepared;
};

StatsLayout transposed_layout(int64_t R, int64_t C) {
  StatsLayout L = stats_layout(C, R);
  std::swap(L.row_oob, L.col_oob);
  std::swap(L.row_maxdig, L.col_maxdig);
  std::swap(L.cr_rowdig, L.rc_coldig);
  L.R = R;
  L.C = C;
  return L;
}

// Mix residuals of the operands whose statistics were computed in this call,
// then the planner's launches (the plan headers must be zero: see PlanArgs).
imu_status plan_launch(const Operand& oa, const Operand& ob, const imu_params* p, const StatsRef& ra,
                       const StatsRef& rb, uint8_t* plan, uint8_t* host_hdr, int64_t host_tag, hipEvent_t done,
                       hipStream_t s) {
  const int batch = (int)oa.m->batch;
  for (int dt : {(int)IMU_BF16, (int)IMU_F32}) {
    QuantJobs J{};
    if (p->strat_a == IMU_MIX && oa.dtype == dt && !ra.prepared) {
      J.op[J.nops].s = stream_args(oa, ra.stats, ra.L, p);
      J.op[J.nops++].batch = batch;
    }
    if (p->strat_b == IMU_MIX && ob.dtype == dt && !rb.prepared) {
      J.op[J.nops].s = stream_args(ob, rb.stats, rb.L, p);
      J.op[J.nops++].batch = batch;
    }
    if (J.nops) IMU_HIP(launch_residual(dt, p->bits, J, s));
  }
  uint8_t* stats_a = ra.stats;
  uint8_t* stats_b = rb.stats;
  const StatsLayout &la = ra.L, &lb = rb.L;
  const PlanLayout pl = plan_layout(oa.R, oa.C, ob.C, batch, p->bits);
  if (p->strat_a == IMU_GREEDY || p->strat_b == IMU_GREEDY) {
    GreedyArgs g{};
    g.plan = plan;
    g.pl = pl;
    g.bits = p->bits;
    g.clip = p->clip;
    g.beta = p->beta;
    auto add = [&](const Operand& op, const StatsRef& r, int64_t rows_off, int64_t cols_off) {
      GreedyOp& o = g.op[g.nops++];
      o.x = op.m->data;
      o.dtype = op.dtype;
      o.transposed = op.tr ? 1 : 0;
      o.ld = op.m->ld;
      o.bstride = op.m->batch_stride;
      o.R = op.R;
      o.C = op.C;
      o.stats = r.stats;
      o.stats_stride = r.L.stride;
      o.row_oob = r.L.row_oob;
      o.col_oob = r.L.col_oob;
      o.rows_off = rows_off;
      o.cols_off = cols_off;
    };
    // greedy area: A rows [M], A cols [K], B rows [K], B cols [N]
    if (p->strat_a == IMU_GREEDY) add(oa, ra, 0, oa.R);
    if (p->strat_b == IMU_GREEDY) add(ob, rb, oa.R + oa.C, oa.R + 2 * oa.C);
    IMU_HIP(launch_greedy(g, batch, s));
  }
  PlanArgs pa{};
  pa.stats_a = stats_a;
  pa.stats_b = stats_b;
  pa.stats_stride_a = la.stride;
  pa.stats_stride_b = lb.stride;
  pa.sla = la;
  pa.slb = lb;
  pa.plan = plan;
  pa.pl = pl;
  pa.gamma = p->gamma;
  pa.strat_a = p->strat_a;
  pa.strat_b = p->strat_b;
  pa.bits = p->bits;
  pa.fmt = digit_fmt(oa, ob, p);
  pa.host_hdr = host_hdr;
  pa.host_tag = host_tag;
  IMU_HIP(launch_plan(pa, done, s));
  return IMU_OK;
}


// ---------------------------------------------------------------------------
// per-device context (imu_init / imu_release)
// ---------------------------------------------------------------------------
// The planner's last launch writes a copy of the plan headers straight into
// pinned, coherent host memory, each copy closed by a per-call tag, and an
// event completes with that launch (it is attached to the launch, so no marker
// of its own sits between the planner and the unpack; it carries no
// system-scope fence, which would write back the L2 and leave the GPU idle for
// microseconds).  The host waits for the headers alone while later kernels
// keep the GPU busy.  imu_init allocates the buffer and the events once per
// device; imu_release frees them.  Calls on one device from several host
// threads share the buffer and take turns (the mutex) from the planner launch
// to the header read.
constexpr int kMaxDevices = 64;
struct DeviceCtx {
  std::mutex mu;
  bool live = false;
  uint8_t* buf = nullptr;       // host address of the header copies
  uint8_t* dbuf = nullptr;      // the same memory as the device addresses it
  int64_t cap = 0;              // batch entries the buffer holds
  hipEvent_t ev = nullptr;      // completes with the planner's last launch
  hipEvent_t ev_sys = nullptr;  // fallback: an event with the system-scope fence
  int64_t tag = 0;
  int cus = 0;                  // compute units of the device
  uint8_t* scratch = nullptr;   // this device's copy of `scratch` (imu_imunpack_matmul_noalloc)
};
DeviceCtx g_ctx[kMaxDevices];

// Workspace of imu_imunpack_matmul_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never passes its name to a
// kernel (on the host the name is only a stand-in); imu_init looks up each
// device's address with hipGetSymbolAddress and keeps it in the context.
constexpr size_t kNoallocScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];
std::mutex g_init_mu;  // imu_init / imu_release

// The context of the calling thread's current device, or an error when
// imu_init has not set it up (or its buffer is too small for `batch`).
imu_status current_ctx(int64_t batch, DeviceCtx** out) {
  int dev = 0;
  IMU_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(IMU_ERR_UNSUPPORTED, "device %d beyond the library's %d", dev, kMaxDevices);
  DeviceCtx& c = g_ctx[dev];
  if (!c.live) return fail(IMU_ERR_INVALID_ARG, "imu_init was not called for device %d", dev);
  if (batch > c.cap)
    return fail(IMU_ERR_UNSUPPORTED, "batch %lld above the %lld entries imu_init set up on device %d",
                (long long)batch, (long long)c.cap, dev);
  *out = &c;
  return IMU_OK;
}

// Wait until the host copy of every entry's header carries this call's tag:
// the planner's event, then a bounded poll of the tags.  Should they still be
// missing (host memory not coherent with the GPU after all), an event with the
// system-scope fence is recorded and waited for; a tag missing after that is an
// error.
imu_status wait_headers(DeviceCtx& st, int batch, hipStream_t s) {
  auto tagged = [&]() {
    for (int b = 0; b < batch; ++b) {
      const volatile int64_t* t = reinterpret_cast<const volatile int64_t*>(
          st.buf + (size_t)b * kPlanHeaderStride + offsetof(PlanHeader, reserved));
      if (*t != st.tag) return false;
    }
    return true;
  };
  IMU_HIP(hipEventSynchronize(st.ev));
  // The stream is queried every 1024 polls: with calls issued back to back
  // (the previous call's GEMM still queued), a spin without runtime calls was
  // seen to wait out its whole budget, the planner not having run, and then
  // pay the fallback's full-stream wait (7 ms per call instead of 0.66).
  for (int i = 0; i < 100000; ++i) {
    if (tagged()) {
      std::atomic_thread_fence(std::memory_order_acquire);
      return IMU_OK;
    }
    if ((i & 1023) == 1023) (void)hipStreamQuery(s);
  }
  IMU_HIP(hipEventRecord(st.ev_sys, s));  // behind whatever was queued since: still correct
  IMU_HIP(hipEventSynchronize(st.ev_sys));
  if (!tagged()) return fail(IMU_ERR_HIP, "plan headers did not reach the host");
  std::atomic_thread_fence(std::memory_order_acquire);
  return IMU_OK;
}

// Plan launches with the host copy of the headers (the caller holds st.mu);
// returns that copy (valid once wait_headers has returned).
imu_status plan_staged(DeviceCtx& st, const Operand& oa, const Operand& ob, const imu_params* p, const StatsRef& ra,
                       const StatsRef& rb, uint8_t* plan, hipStream_t s, const uint8_t** hdrs) {
  ++st.tag;
  IMU_TRY(plan_launch(oa, ob, p, ra, rb, plan, st.dbuf, st.tag, st.ev, s));
  *hdrs = st.buf;
  return IMU_OK;
}

// Fill info from the staged headers (B' entries follow all A' entries) and
// report a failed plan.  *a_total / *b_total: bytes of all A' / B' entries.
// IMU_LOG=1: one line per batch entry on stderr with the plan a call made
// (candidates chosen, unpacked sizes, exponent segments, layout, digit format).
void log_plan(const Operand& oa, const Operand& ob, const PlanHeader* h, int b) {
  static const char* const kCand[] = {"row", "col", "cr", "rc", "greedy"};
  auto cand = [](int c) { return c >= 0 && c < 5 ? kCand[c] : "?"; };
  char segs[kMaxSeg * 12 + 1];
  int at = 0;
  for (int q = 0; q < h->n_seg && q < kMaxSeg && at < (int)sizeof(segs) - 12; ++q)
    at += std::snprintf(segs + at, sizeof(segs) - at, q ? ",%d" : "%d", h->seg_len[q]);
  segs[at] = 0;
  std::fprintf(stderr,
               "imu plan: entry %d: %lldx%lldx%lld choice %s/%s M'=%lld K'=%lld N'=%lld unpack ratio %.4f; "
               "k_pad %lld, segments [%s]; rows base %lld alloc %lld, columns base %lld alloc %lld; digits %s; "
               "status %d\n",
               b, (long long)oa.R, (long long)oa.C, (long long)ob.C, cand(h->choice_a), cand(h->choice_b),
               (long long)h->m_u, (long long)h->k_u, (long long)h->n_u,
               (double)h->m_u * (double)h->k_u * (double)h->n_u / ((double)oa.R * (double)oa.C * (double)ob.C),
               (long long)h->k_pad, segs, (long long)h->m_base, (long long)h->m_alloc, (long long)h->n_base,
               (long long)h->n_alloc, h->fmt == kDigitsFp6 ? "fp6" : "int8", h->status);
}

imu_status finish_plan(const Operand& oa, const Operand& ob, const uint8_t* hdrs, int batch, imu_plan_info* info,
                       int64_t* a_total, int64_t* b_total) {
  int status = 0;
  int64_t aoff = 0, boff = 0;
  const char* lg = std::getenv("IMU_LOG");
  const bool log = lg && lg[0] == '1';
  for (int b = 0; b < batch; ++b) {
    const PlanHeader* h = reinterpret_cast<const PlanHeader*>(hdrs + (size_t)b * kPlanHeaderStride);
    status |= h->status;
    if (log) log_plan(oa, ob, h, b);
    if (info) {
      imu_plan_info& f = info[b];
      std::memset(&f, 0, sizeof(f));
      f.m = oa.R;
      f.k = oa.C;
      f.n = ob.C;
      f.m_u = h->m_u;
      f.k_u = h->k_u;
      f.n_u = h->n_u;
      f.m_alloc = h->m_alloc;
      f.n_alloc = h->n_alloc;
      f.k_pad = h->k_pad;
      f.m_base = h->m_base;
      f.n_base = h->n_base;
      f.a_offset = aoff;
      f.b_offset = boff;
      f.n_seg = h->n_seg;
      f.choice_a = h->choice_a;
      f.choice_b = h->choice_b;
      f.digits = h->fmt == kDigitsFp6 ? IMU_DIGITS_FP6 : IMU_DIGITS_INT8;
      f.unpack_ratio = (double)h->m_u * (double)h->k_u * (double)h->n_u /
                       ((double)oa.R * (double)oa.C * (double)ob.C);
      std::memcpy(f.pair_sizes, h->pair, sizeof(f.pair_sizes));
    }
    aoff += unpacked_entry_bytes(h, 0);
    boff += unpacked_entry_bytes(h, 1);
  }
  if (a_total) *a_total = aoff;
  if (b_total) *b_total = boff;
  if (status & kStatusNonfinite) return fail(IMU_ERR_NONFINITE, "an input element is NaN or Inf");
  if (status & kStatusRange) return fail(IMU_ERR_RANGE, "|x * r| >= 2^31 for some element");
  if (status & kStatusGreedy) return fail(IMU_ERR_HIP, "the greedy planner did not finish");
  return IMU_OK;
}

imu_status plan_impl(const Operand& oa, const Operand& ob, const imu_params* p, uint8_t* stats_a,
                     uint8_t* stats_b, uint8_t* plan, imu_plan_info* info, hipStream_t s) {
  const int batch = (int)oa.m->batch;
  DeviceCtx* st = nullptr;
  IMU_TRY(current_ctx(batch, &st));
  std::lock_guard<std::mutex> lock(st->mu);
  const uint8_t* hdrs = nullptr;
  const StatsRef ra{stats_a, stats_layout(oa.R, oa.C), false}, rb{stats_b, stats_layout(ob.R, ob.C), false};
  IMU_HIP(launch_fill_u32(plan, 0u, plan_layout(oa.R, oa.C, ob.C, batch, p->bits).headers_bytes / 4, s));
  IMU_TRY(plan_staged(*st, oa, ob, p, ra, rb, plan, s, &hdrs));
  IMU_TRY(wait_headers(*st, batch, s));
  return finish_plan(oa, ob, hdrs, batch, info, nullptr, nullptr);
}

// Unpack one operand; M, K, N give the plan layout.  after_a: B' entries start
// after all A' entries of x_u; cap: bytes available at x_u.
UnpackArgs unpack_args(const Operand& op, int operand, const imu_params* p, const uint8_t* stats,
                       const uint8_t* plan, int64_t M, int64_t K, int64_t N, int8_t* x_u, bool after_a,
                       int64_t cap, int fmt) {
  const StatsLayout L = stats_layout(op.R, op.C);
  const imu_matrix* x = op.m;
  UnpackArgs u{};
  u.x = x->data;
  u.bstride = x->batch_stride;
  // element (outer o, inner k) of the logical operand in memory
  const int64_t ld = x->ld;
  if (operand == 0) {  // A: outer = row i, inner = col k
    u.so = op.tr ? 1 : ld;
    u.sk = op.tr ? ld : 1;
    u.n_outer = op.R;
    u.K = op.C;
  } else {  // B: outer = col n, inner = row k
    u.so = op.tr ? ld : 1;
    u.sk = op.tr ? 1 : ld;
    u.n_outer = op.C;
    u.K = op.R;
  }
  u.operand = operand;
  u.vec_ok = (reinterpret_cast<uintptr_t>(x->data) % 16) == 0 && ld % 8 == 0 &&
             (x->batch == 1 || x->batch_stride % 8 == 0);
  u.stats = stats;
  u.stats_stride = L.stride;
  u.plan = plan;
  u.pl = plan_layout(M, K, N, x->batch, p->bits);
  u.out = x_u;
  u.after_a = after_a ? 1 : 0;
  u.cap = cap;
  u.beta = p->beta;
  u.clip = p->clip;
  u.fmt = fmt;
  return u;
}

imu_status unpack_impl(const Operand& op, int operand, const imu_params* p, const uint8_t* stats,
                       const uint8_t* plan, int64_t M, int64_t K, int64_t N, int8_t* x_u, bool after_a,
                       int64_t cap, int fmt, hipStream_t s) {
  const UnpackArgs u = unpack_args(op, operand, p, stats, plan, M, K, N, x_u, after_a, cap, fmt);
  IMU_HIP(launch_unpack(op.dtype, p->bits, &u, 1, (int)op.m->batch, s));
  return IMU_OK;
}

// Tile-relevant sizes of one batch entry's plan.
struct EntrySizes {
  int64_t m_base, n_base, m_alloc, n_alloc;
  int fmt;
};

// GEMM launches for `batch` entries whose sizes come from get(b) (the staged
// host headers or the caller's info).
template <class Get>
imu_status gemm_impl(const int8_t* a_u, const int8_t* b_u, const imu_params* p, const uint8_t* stats_a,
                     const uint8_t* stats_b, const uint8_t* plan, int64_t M, int64_t K, int64_t N, int64_t batch,
                     Get get, int32_t* c, int64_t ldc, int64_t cbs, float* out, hipStream_t s) {
  const StatsLayout la = stats_layout(M, K), lb = stats_layout(K, N);
  const PlanLayout pl = plan_layout(M, K, N, batch, p->bits);
  if (batch > 65535) return fail(IMU_ERR_INVALID_ARG, "batch above 65535");
  // one launch per pass serves every entry: the grid takes the largest entry
  // Entries with extra rows fold their extra tiles with atomics (C cleared
  // first, then the atomic pass, then the base tiles add).  Entries with extra
  // columns only fold them inside the base pass (each tile also multiplies the
  // levels of its own columns) and store C once, provided the base tiles of
  // the call fill the GPU: with fewer tiles than CUs the folded work would sit
  // on a few CUs, and the atomic pass spreads it over the extra tiles instead.
  int64_t base_tiles = 0, base_total = 0;
  for (int64_t b = 0; b < batch; ++b) {
    const EntrySizes f = get(b);
    if (f.m_base % 256 || f.n_base % 128 || f.m_alloc % 256 || f.n_alloc % 128)
      return fail(IMU_ERR_INVALID_ARG, "plan sizes are not tile multiples");
    if (f.fmt != get(0).fmt || (f.fmt != kDigitsInt8 && f.fmt != kDigitsFp6))
      return fail(IMU_ERR_INVALID_ARG, "the entries' digit formats differ or are unknown");
    base_total += (f.m_base / 256) * (f.n_base / 128);
  }
  int cus = 0;
  {
    DeviceCtx* ctx = nullptr;
    IMU_TRY(current_ctx(0, &ctx));
    cus = ctx->cus;
  }
  // Tile rows: 256, or for int8 digits 128 when the 256-row base tiles would
  // be fewer than the CUs (a launch that would leave CUs idle gets twice the
  // tiles, and its smaller tiles fit more workgroups per CU), or as many as
  // the CUs with some entry folding extra columns (tiles of unequal depth:
  // smaller ones even out the CUs' work).  m_base and m_alloc are multiples
  // of 256, so of either.
  bool folds = false;
  for (int64_t b = 0; b < batch; ++b) {
    const EntrySizes f = get(b);
    folds = folds || (f.n_alloc > f.n_base && f.m_alloc == f.m_base);
  }
  const int64_t tr =
      get(0).fmt == kDigitsInt8 && (base_total < cus || (base_total == cus && folds)) ? 128 : 256;
  base_total = 0;
  for (int64_t b = 0; b < batch; ++b) {
    const EntrySizes f = get(b);
    base_tiles = std::max(base_tiles, (f.m_base / tr) * (f.n_base / 128));
    base_total += (f.m_base / tr) * (f.n_base / 128);
  }
  // IMU_FOLD_COLUMNS=1 / 0 forces the choice (both give the same result)
  const char* fe = std::getenv("IMU_FOLD_COLUMNS");
  const bool fold_cols = fe && fe[0] == '1' ? true : fe && fe[0] == '0' ? false : base_total >= cus;
  int64_t extra_tiles = 0;
  bool any_atomic = false, any_fold = false;
  for (int64_t b = 0; b < batch; ++b) {
    const EntrySizes f = get(b);
    const bool rowx = f.m_alloc > f.m_base, colx = f.n_alloc > f.n_base;
    if (rowx || (colx && !fold_cols)) {
      any_atomic = true;
      extra_tiles = std::max(extra_tiles, (f.m_alloc / tr) * (f.n_alloc / 128));
    } else if (colx) {
      any_fold = true;
    }
  }
  GemmArgs g{};
  g.a_u = a_u;
  g.b_u = b_u;
  g.plan = plan;
  g.headers_bytes = pl.headers_bytes;
  g.entry_stride = pl.entry_stride;
  g.amap_off = pl.amap;
  g.bmap_off = pl.bmap;
  g.stats_a = stats_a;
  g.stats_b = stats_b;
  g.stats_stride_a = la.stride;
  g.stats_stride_b = lb.stride;
  g.c = c;
  g.out = out;
  g.ldc = ldc;
  g.cbs = cbs;
  g.M = M;
  g.N = N;
  g.bits = p->bits;
  g.fold_cols = fold_cols ? 1 : 0;
  g.fmt = get(0).fmt;
  g.tile_rows = (int)tr;
  // Tile order: each XCD takes a run of tiles covering G tile rows; its L2
  // then fills G row panels of A' and about T / (8 G) column panels of B'^T,
  // which is least near G = sqrt(T BN / (8 BM)) (rounded to a power of two).
  {
    int64_t tm = 1, tn = 1;
    for (int64_t b = 0; b < batch; ++b) {
      const EntrySizes f = get(b);
      if ((f.m_base / tr) * (f.n_base / 128) >= tm * tn) {
        tm = f.m_base / tr;
        tn = f.n_base / 128;
      }
    }
    const double ideal = std::sqrt((double)(tm * tn) * 128.0 / (8.0 * (double)tr));
    int gsz = 1;
    while (gsz * 2 <= tm && std::log2(gsz * 2.0) <= std::log2(std::max(ideal, 1.0)) + 0.5) gsz *= 2;
    g.group_m = gsz;
  }
  // Measurement events: attached to the launch when the call makes a single
  // one (no marker of their own in the stream), else recorded around all of
  // the call's launches.
  if (g_gemm_ev[0] && any_atomic) IMU_HIP(hipEventRecord(g_gemm_ev[0], s));
  if (any_atomic) {
    IMU_HIP(launch_fill_2d(c, M, N, ldc, (int)batch, cbs, s));
    g.mode = 2;
    IMU_HIP(launch_gemm(g, extra_tiles, (int)batch, false, s));
    g.mode = 0;
    IMU_HIP(launch_gemm(g, base_tiles, (int)batch, any_fold, s));
    if (g_gemm_ev[1]) IMU_HIP(hipEventRecord(g_gemm_ev[1], s));
  } else {
    g.mode = 0;
    IMU_HIP(launch_gemm(g, base_tiles, (int)batch, any_fold, s, g_gemm_ev[0], g_gemm_ev[1]));
  }
  return IMU_OK;
}

imu_status check_info(const imu_plan_info* info, int64_t batch, int64_t M, int64_t K, int64_t N) {
  if (!info) return fail(IMU_ERR_INVALID_ARG, "info is NULL");
  for (int64_t b = 0; b < batch; ++b)
    if (info[b].m != M || info[b].k != K || info[b].n != N || info[b].k_pad <= 0 ||
        (info[b].digits != IMU_DIGITS_INT8 && info[b].digits != IMU_DIGITS_FP6) || info[b].digits != info[0].digits)
      return fail(IMU_ERR_INVALID_ARG, "info does not describe this problem");
  return IMU_OK;
}

int64_t fixed_bytes(const Operand& oa, const Operand& ob, const imu_params* p) {
  const int64_t batch = oa.m->batch;
  return round_up(stats_layout(oa.R, oa.C).stride * batch, 256) +
         round_up(stats_layout(ob.R, ob.C).stride * batch, 256) +
         round_up(plan_layout(oa.R, oa.C, ob.C, batch, p->bits).total, 256);
}

// The whole path on a caller-provided workspace (see imu_imunpack_matmul).
// pre_a / pre_b: prepared statistics (imu_imunpack_matmul_prepared) or null.
imu_status matmul_impl(const Operand& oa, const Operand& ob, const imu_params* p, int32_t* c, float* out,
                       uint8_t* w, int64_t ws_bytes, size_t* ws_needed, imu_plan_info* info, hipStream_t stream,
                       const imu_prepared* pre_a = nullptr, const imu_prepared* pre_b = nullptr) {
  const int64_t batch = oa.m->batch;
  const int64_t fixed = fixed_bytes(oa, ob, p);
  if (ws_needed) *ws_needed = (size_t)fixed;
  if (!w || ws_bytes < fixed)
    return fail(IMU_ERR_WORKSPACE, "workspace of %lld bytes below the fixed part (statistics and plan) of %lld",
                (long long)ws_bytes, (long long)fixed);
  DeviceCtx* st = nullptr;
  IMU_TRY(current_ctx(batch, &st));
  uint8_t* ws_a = w;
  uint8_t* ws_b = ws_a + round_up(stats_layout(oa.R, oa.C).stride * batch, 256);
  uint8_t* plan = ws_b + round_up(stats_layout(ob.R, ob.C).stride * batch, 256);
  auto ref = [&](const Operand& o, uint8_t* own, const imu_prepared* pre) {
    if (pre && pre->stats)
      return StatsRef{static_cast<uint8_t*>(const_cast<void*>(pre->stats)),
                      pre->transposed ? transposed_layout(o.R, o.C) : stats_layout(o.R, o.C), true};
    return StatsRef{own, stats_layout(o.R, o.C), false};
  };
  const StatsRef ra = ref(oa, ws_a, pre_a), rb = ref(ob, ws_b, pre_b);
  uint8_t* const stats_a = ra.stats;
  uint8_t* const stats_b = rb.stats;
  // the statistics of A and B and the plan headers are adjacent: one clear
  IMU_HIP(launch_fill_u32(ws_a, 0u, (int64_t)(plan - ws_a + plan_layout(oa.R, oa.C, ob.C, batch, p->bits).headers_bytes) / 4,
                          stream));
  {
    const Operand* ops[2];
    uint8_t* stv[2];
    int32_t* q[2] = {nullptr, nullptr};
    int n = 0;
    if (!ra.prepared) ops[n] = &oa, stv[n++] = stats_a;
    if (!rb.prepared) ops[n] = &ob, stv[n++] = stats_b;
    if (n) IMU_TRY(quantize_ops(ops, stv, q, n, p, stream, true));
  }
  // The unpack kernels take their sizes and placement from the plan on the
  // device, so they are queued right behind the plan; the host waits only for
  // the plan headers (staged to pinned memory) while they run, then checks the
  // workspace and sizes the GEMM launch.  If the plan failed or the workspace
  // is too small the unpack kernels write nothing.
  std::lock_guard<std::mutex> lock(st->mu);
  const uint8_t* hdrs = nullptr;
  IMU_TRY(plan_staged(*st, oa, ob, p, ra, rb, plan, stream, &hdrs));
  int8_t* region = reinterpret_cast<int8_t*>(w + fixed);
  const int fmt = digit_fmt(oa, ob, p);  // the format the plan was made for
  const int64_t cap = ws_bytes - fixed;
  if (oa.dtype == ob.dtype) {  // both operands in one launch
    const UnpackArgs u[2] = {unpack_args(oa, 0, p, stats_a, plan, oa.R, oa.C, ob.C, region, false, cap, fmt),
                             unpack_args(ob, 1, p, stats_b, plan, oa.R, oa.C, ob.C, region, true, cap, fmt)};
    IMU_HIP(launch_unpack(oa.dtype, p->bits, u, 2, (int)batch, stream));
  } else {
    IMU_TRY(unpack_impl(oa, 0, p, stats_a, plan, oa.R, oa.C, ob.C, region, false, cap, fmt, stream));
    IMU_TRY(unpack_impl(ob, 1, p, stats_b, plan, oa.R, oa.C, ob.C, region, true, cap, fmt, stream));
  }
  IMU_TRY(wait_headers(*st, (int)batch, stream));
  int64_t a_bytes = 0, b_bytes = 0;
  IMU_TRY(finish_plan(oa, ob, hdrs, (int)batch, info, &a_bytes, &b_bytes));
  const int64_t needed = fixed + a_bytes + b_bytes;
  if (ws_needed) *ws_needed = (size_t)needed;
  if (ws_bytes < needed)
    return fail(IMU_ERR_WORKSPACE, "workspace of %lld bytes below the %lld this plan needs", (long long)ws_bytes,
                (long long)needed);
  int8_t* a_u = region;
  int8_t* b_u = region + a_bytes;
  auto sizes = [hdrs](int64_t b) {
    const PlanHeader* h = reinterpret_cast<const PlanHeader*>(hdrs + (size_t)b * kPlanHeaderStride);
    return EntrySizes{h->m_base, h->n_base, h->m_alloc, h->n_alloc, h->fmt};
  };
  return gemm_impl(a_u, b_u, p, stats_a, stats_b, plan, oa.R, oa.C, ob.C, batch, sizes, c, ob.C, oa.R * ob.C, out,
                   stream);
}

}  // namespace

extern "C" {

imu_status imu_init(int64_t max_batch) {
  if (max_batch < 1 || max_batch > 65535) return fail(IMU_ERR_INVALID_ARG, "max_batch must be in [1, 65535]");
  int dev = 0;
  IMU_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(IMU_ERR_UNSUPPORTED, "device %d beyond the library's %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> g(g_init_mu);
  DeviceCtx& c = g_ctx[dev];
  std::lock_guard<std::mutex> l(c.mu);
  if (!c.live) {
    IMU_HIP(hipEventCreateWithFlags(&c.ev, hipEventDisableTiming | hipEventDisableSystemFence));
    IMU_HIP(hipEventCreateWithFlags(&c.ev_sys, hipEventDisableTiming));
    IMU_HIP(hipDeviceGetAttribute(&c.cus, hipDeviceAttributeMultiprocessorCount, dev));
    void* sp = nullptr;
    IMU_HIP(hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch)));
    c.scratch = static_cast<uint8_t*>(sp);
    c.live = true;
  }
  if (c.cap < max_batch) {
    if (c.buf) {  // no planner launch may still write the old buffer
      IMU_HIP(hipDeviceSynchronize());
      IMU_HIP(hipHostFree(c.buf));
      c.buf = c.dbuf = nullptr;
      c.cap = 0;
    }
    const size_t bytes = (size_t)max_batch * kPlanHeaderStride;
    void* h = nullptr;
    IMU_HIP(hipHostMalloc(&h, bytes, hipHostMallocMapped | hipHostMallocCoherent));
    std::memset(h, 0, bytes);  // no stale tag
    void* d = nullptr;
    IMU_HIP(hipHostGetDevicePointer(&d, h, 0));
    c.buf = static_cast<uint8_t*>(h);
    c.dbuf = static_cast<uint8_t*>(d);
    c.cap = max_batch;
  }
  return IMU_OK;
}

imu_status imu_release(void) {
  int dev = 0;
  IMU_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return IMU_OK;
  std::lock_guard<std::mutex> g(g_init_mu);
  DeviceCtx& c = g_ctx[dev];
  std::lock_guard<std::mutex> l(c.mu);
  if (!c.live) return IMU_OK;
  IMU_HIP(hipDeviceSynchronize());  // nothing may still write the buffer or signal the events
  if (c.buf) IMU_HIP(hipHostFree(c.buf));
  IMU_HIP(hipEventDestroy(c.ev));
  IMU_HIP(hipEventDestroy(c.ev_sys));
  c.buf = c.dbuf = nullptr;
  c.cap = 0;
  c.ev = c.ev_sys = nullptr;
  c.scratch = nullptr;
  c.live = false;
  return IMU_OK;
}

size_t imu_stats_bytes(const imu_matrix* x) {
  Operand op;
  if (check_matrix(x, "x", &op) != IMU_OK) return 0;
  return (size_t)(stats_layout(op.R, op.C).stride * x->batch);
}

imu_status imu_stats_layout(const imu_matrix* x, imu_stats_view* v) {
  Operand op;
  IMU_TRY(check_matrix(x, "x", &op));
  if (!v) return fail(IMU_ERR_INVALID_ARG, "view is NULL");
  const StatsLayout L = stats_layout(op.R, op.C);
  v->stride = L.stride;
  v->row_oob = L.row_oob;
  v->col_oob = L.col_oob;
  v->row_maxdig = L.row_maxdig;
  v->col_maxdig = L.col_maxdig;
  v->cr_rowdig = L.cr_rowdig;
  v->rc_coldig = L.rc_coldig;
  v->hist = L.hist;
  return IMU_OK;
}

size_t imu_plan_bytes(const imu_matrix* a, const imu_matrix* b, const imu_params* p) {
  Operand oa, ob;
  if (check_pair(a, b, p, &oa, &ob) != IMU_OK) return 0;
  return (size_t)plan_layout(oa.R, oa.C, ob.C, a->batch, p->bits).total;
}

imu_status imu_plan_layout(const imu_matrix* a, const imu_matrix* b, const imu_params* p,
                           imu_plan_view* v) {
  Operand oa, ob;
  IMU_TRY(check_pair(a, b, p, &oa, &ob));
  if (!v) return fail(IMU_ERR_INVALID_ARG, "view is NULL");
  const PlanLayout L = plan_layout(oa.R, oa.C, ob.C, a->batch, p->bits);
  v->header_stride = kPlanHeaderStride;
  v->headers_bytes = L.headers_bytes;
  v->entry_stride = L.entry_stride;
  v->da_r = L.da_r;
  v->da_c = L.da_c;
  v->db_r = L.db_r;
  v->db_c = L.db_c;
  v->lvl_a = L.lvl_a;
  v->lvl_b = L.lvl_b;
  v->kpre = L.kpre;
  v->amap = L.amap;
  v->bmap = L.bmap;
  v->levels = L.levels;
  v->segments = L.segments;
  v->m_alloc_max = L.m_alloc_max;
  v->n_alloc_max = L.n_alloc_max;
  return IMU_OK;
}

size_t imu_workspace_fixed_bytes(const imu_matrix* a, const imu_matrix* b, const imu_params* p) {
  Operand oa, ob;
  if (check_pair(a, b, p, &oa, &ob) != IMU_OK) return 0;
  return (size_t)fixed_bytes(oa, ob, p);
}

imu_status imu_quantize_rtn(const imu_matrix* x, const imu_params* p, void* stats, int32_t* q_out,
                            hipStream_t stream) {
  Operand op;
  IMU_TRY(check_matrix(x, "x", &op));
  IMU_TRY(check_params(p));
  if (!stats) return fail(IMU_ERR_INVALID_ARG, "stats is NULL");
  const Operand* ops[1] = {&op};
  uint8_t* st[1] = {static_cast<uint8_t*>(stats)};
  int32_t* q[1] = {q_out};
  return quantize_ops(ops, st, q, 1, p, stream, false);
}

imu_status imu_plan_unpack(const imu_matrix* a, const imu_matrix* b, const imu_params* p, void* stats_a,
                           void* stats_b, void* plan, imu_plan_info* info, hipStream_t stream) {
  Operand oa, ob;
  IMU_TRY(check_pair(a, b, p, &oa, &ob));
  if (!stats_a || !stats_b || !plan) return fail(IMU_ERR_INVALID_ARG, "stats or plan is NULL");
  return plan_impl(oa, ob, p, static_cast<uint8_t*>(stats_a), static_cast<uint8_t*>(stats_b),
                   static_cast<uint8_t*>(plan), info, stream);
}

imu_status imu_unpack(const imu_matrix* x, int32_t operand, const imu_params* p, const void* stats,
                      const void* plan, const imu_plan_info* info, int8_t* x_u, hipStream_t stream) {
  Operand op;
  IMU_TRY(check_matrix(x, "x", &op));
  IMU_TRY(check_params(p));
  if (operand != 0 && operand != 1) return fail(IMU_ERR_INVALID_ARG, "operand must be 0 (A) or 1 (B)");
  if (!stats || !plan || !x_u) return fail(IMU_ERR_INVALID_ARG, "stats, plan or x_u is NULL");
  if (!info) return fail(IMU_ERR_INVALID_ARG, "info is NULL");
  const int64_t M = operand == 0 ? op.R : info[0].m, K = operand == 0 ? op.C : op.R,
                N = operand == 0 ? info[0].n : op.C;
  IMU_TRY(check_info(info, x->batch, M, K, N));
  const int fmt = info[0].digits == IMU_DIGITS_FP6 ? kDigitsFp6 : kDigitsInt8;
  // the fp6 unpack reads K-contiguous operands: A IMU_NORMAL, B IMU_TRANSPOSED
  if (fmt == kDigitsFp6 && (p->bits > 4 || op.tr != (operand == 1)))
    return fail(IMU_ERR_INVALID_ARG, "info holds fp6 digits, which this operand's layout or bits cannot give");
  return unpack_impl(op, operand, p, static_cast<const uint8_t*>(stats), static_cast<const uint8_t*>(plan), M, K,
                     N, x_u, false, INT64_MAX, fmt, stream);
}

imu_status imu_unpacked_gemm(const int8_t* a_u, const int8_t* b_u, const imu_params* p, const void* stats_a,
                             const void* stats_b, const void* plan, const imu_plan_info* info,
                             int64_t batch, int32_t* c, int64_t ldc, int64_t c_batch_stride, float* out,
                             hipStream_t stream) {
  IMU_TRY(check_params(p));
  if (!a_u || !b_u || !stats_a || !stats_b || !plan || !c)
    return fail(IMU_ERR_INVALID_ARG, "a NULL pointer was passed");
  if (!info || batch < 1) return fail(IMU_ERR_INVALID_ARG, "info is NULL or batch < 1");
  IMU_TRY(check_info(info, batch, info[0].m, info[0].k, info[0].n));
  if (ldc < info[0].n) return fail(IMU_ERR_INVALID_ARG, "ldc is below N");
  if (batch > 1 && c_batch_stride < (info[0].m - 1) * ldc + info[0].n)
    return fail(IMU_ERR_INVALID_ARG, "c_batch_stride overlaps batch entries");
  auto sizes = [info](int64_t b) {
    return EntrySizes{info[b].m_base, info[b].n_base, info[b].m_alloc, info[b].n_alloc,
                      info[b].digits == IMU_DIGITS_FP6 ? kDigitsFp6 : kDigitsInt8};
  };
  return gemm_impl(a_u, b_u, p, static_cast<const uint8_t*>(stats_a), static_cast<const uint8_t*>(stats_b),
                   static_cast<const uint8_t*>(plan), info[0].m, info[0].k, info[0].n, batch, sizes, c, ldc,
                   c_batch_stride, out, stream);
}

imu_status imu_imunpack_matmul(const imu_matrix* a, const imu_matrix* b, const imu_params* p, int32_t* c,
                               float* out, void* ws, size_t ws_bytes, size_t* ws_needed,
                               imu_plan_info* info, hipStream_t stream) {
  Operand oa, ob;
  IMU_TRY(check_pair(a, b, p, &oa, &ob));
  if (!c) return fail(IMU_ERR_INVALID_ARG, "c is NULL");
  if (ws_bytes > (size_t)INT64_MAX) return fail(IMU_ERR_INVALID_ARG, "ws_bytes above 2^63");
  return matmul_impl(oa, ob, p, c, out, static_cast<uint8_t*>(ws), (int64_t)ws_bytes, ws_needed, info, stream);
}

imu_status imu_prepare_operand(const imu_matrix* x, const imu_params* p, void* stats, hipStream_t stream) {
  Operand op;
  IMU_TRY(check_matrix(x, "x", &op));
  IMU_TRY(check_params(p));
  if (!stats) return fail(IMU_ERR_INVALID_ARG, "stats is NULL");
  uint8_t* st = static_cast<uint8_t*>(stats);
  const Operand* ops[1] = {&op};
  uint8_t* stv[1] = {st};
  int32_t* q[1] = {nullptr};
  IMU_TRY(quantize_ops(ops, stv, q, 1, p, stream, false));
  QuantJobs J{};
  J.op[0].s = stream_args(op, st, stats_layout(op.R, op.C), p);
  J.op[0].batch = (int)x->batch;
  J.nops = 1;
  IMU_HIP(launch_residual(op.dtype, p->bits, J, stream));
  return IMU_OK;
}

imu_status imu_softmax_prepare(const imu_matrix* logits, const imu_matrix* p_out, const imu_params* p,
                               void* stats, hipStream_t stream) {
  Operand oz, op;
  IMU_TRY(check_matrix(logits, "logits", &oz));
  IMU_TRY(check_matrix(p_out, "p", &op));
  IMU_TRY(check_params(p));
  if (!stats) return fail(IMU_ERR_INVALID_ARG, "stats is NULL");
  if (logits->layout != IMU_NORMAL || p_out->layout != IMU_NORMAL)
    return fail(IMU_ERR_UNSUPPORTED, "the softmax runs along stored rows: logits and p must be IMU_NORMAL");
  if (p_out->dtype != IMU_BF16) return fail(IMU_ERR_INVALID_ARG, "p.dtype must be IMU_BF16");
  if (logits->rows != p_out->rows || logits->cols != p_out->cols || logits->batch != p_out->batch)
    return fail(IMU_ERR_INVALID_ARG, "logits and p must have the same rows, cols and batch");
  // P must not share bytes with the logits (rows longer than 2048 are read again after P is written)
  auto span = [](const imu_matrix* x, int elem) {
    const int64_t n = (x->batch - 1) * (x->batch > 1 ? x->batch_stride : 0) + (x->rows - 1) * x->ld + x->cols;
    const uintptr_t b = reinterpret_cast<uintptr_t>(x->data);
    return std::make_pair(b, b + (uintptr_t)(n * elem));
  };
  const auto zs = span(logits, oz.elem), ps = span(p_out, 2);
  if (zs.first < ps.second && ps.first < zs.second) return fail(IMU_ERR_INVALID_ARG, "p overlaps the logits");
  uint8_t* st = static_cast<uint8_t*>(stats);
  const StatsLayout L = stats_layout(op.R, op.C);
  const int batch = (int)p_out->batch;
  IMU_HIP(launch_fill_u32(st, 0u, L.stride * batch / 4, stream));
  QuantJobs J{};
  J.op[0].s = stream_args(op, st, L, p);
  J.op[0].batch = batch;
  J.nops = 1;
  SoftmaxIn in{};
  in.z = logits->data;
  in.ld = logits->ld;
  in.bstride = batch > 1 ? logits->batch_stride : 0;
  const uintptr_t za = reinterpret_cast<uintptr_t>(logits->data), pa = reinterpret_cast<uintptr_t>(p_out->data);
  const int zal = oz.elem * 4;  // bytes of 4 logits
  in.vec_ok = za % zal == 0 && logits->ld % 4 == 0 && (batch == 1 || logits->batch_stride % 4 == 0) && pa % 8 == 0 &&
              p_out->ld % 4 == 0 && (batch == 1 || p_out->batch_stride % 4 == 0);
  J.op[0].s.bstride = batch > 1 ? p_out->batch_stride : 0;
  IMU_HIP(launch_softmax_hist(oz.dtype, in, J, stream));
  IMU_HIP(launch_round_count(IMU_BF16, p->bits, J, nullptr, nullptr, stream));
  IMU_HIP(launch_residual(IMU_BF16, p->bits, J, stream));
  return IMU_OK;
}

imu_status imu_imunpack_matmul_prepared(const imu_matrix* a, const imu_matrix* b, const imu_params* p,
                                        const imu_prepared* pre_a, const imu_prepared* pre_b, int32_t* c,
                                        float* out, void* ws, size_t ws_bytes, size_t* ws_needed,
                                        imu_plan_info* info, hipStream_t stream) {
  Operand oa, ob;
  IMU_TRY(check_pair(a, b, p, &oa, &ob));
  if (!c) return fail(IMU_ERR_INVALID_ARG, "c is NULL");
  if (ws_bytes > (size_t)INT64_MAX) return fail(IMU_ERR_INVALID_ARG, "ws_bytes above 2^63");
  for (const imu_prepared* pr : {pre_a, pre_b})
    if (pr && pr->transposed != 0 && pr->transposed != 1)
      return fail(IMU_ERR_INVALID_ARG, "imu_prepared.transposed must be 0 or 1");
  return matmul_impl(oa, ob, p, c, out, static_cast<uint8_t*>(ws), (int64_t)ws_bytes, ws_needed, info, stream,
                     pre_a, pre_b);
}

imu_status imu_imunpack_matmul_noalloc(const imu_matrix* a, const imu_matrix* b, const imu_params* p, int32_t* c,
                                       float* out, size_t* ws_needed, imu_plan_info* info, hipStream_t stream) {
  Operand oa, ob;
  IMU_TRY(check_pair(a, b, p, &oa, &ob));
  if (!c) return fail(IMU_ERR_INVALID_ARG, "c is NULL");
  DeviceCtx* st = nullptr;
  IMU_TRY(current_ctx(a->batch, &st));
  const imu_status r = matmul_impl(oa, ob, p, c, out, st->scratch, (int64_t)kNoallocScratchBytes, ws_needed, info,
                                   stream);
  if (r == IMU_ERR_WORKSPACE)
    return fail(IMU_ERR_WORKSPACE, "the problem needs more than the library's fixed %zu-byte scratch (%s)",
                kNoallocScratchBytes, "use imu_imunpack_matmul with a workspace");
  return r;
}

size_t imu_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

const char* imu_status_string(imu_status s) {
  switch (s) {
    case IMU_OK: return "ok";
    case IMU_ERR_INVALID_ARG: return "invalid argument";
    case IMU_ERR_NONFINITE: return "non-finite input";
    case IMU_ERR_RANGE: return "code out of int32 range";
    case IMU_ERR_WORKSPACE: return "workspace too small";
    case IMU_ERR_HIP: return "HIP runtime error";
    case IMU_ERR_UNSUPPORTED: return "unsupported request";
  }
  return "unknown status";
}

const char* imu_last_error(void) { return g_err; }

const char* imu_version(void) { return "imunpack 0.2 (gfx950)"; }

imu_status imu_set_gemm_events(hipEvent_t before, hipEvent_t after) {
  if ((before == nullptr) != (after == nullptr))
    return fail(IMU_ERR_INVALID_ARG, "pass both events or neither");
  g_gemm_ev[0] = before;
  g_gemm_ev[1] = after;
  return IMU_OK;
}

}  // extern "C"
