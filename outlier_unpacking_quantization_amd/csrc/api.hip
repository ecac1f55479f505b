// C ABI of the IM-Unpack integer GEMM library: argument validation, buffer
// carving, kernel launches and the one plan-header readback.  Contains no
// kernels; the device work lives in quantize.hip, plan.hip, unpack.hip and
// gemm.hip.
#include <algorithm>
#include <atomic>
#include <cstddef>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "common.h"
#include "kernels.h"

using namespace imu;

namespace {

thread_local std::string g_err;
thread_local hipEvent_t g_gemm_ev[2] = {nullptr, nullptr};  // imu_set_gemm_events

imu_status fail(imu_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

#define IMU_HIP(call)                                                                              \
  do {                                                                                             \
    hipError_t e_ = (call);                                                                        \
    if (e_ != hipSuccess) return fail(IMU_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
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
  if (!x) return fail(IMU_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!x->data) return fail(IMU_ERR_INVALID_ARG, std::string(name) + ".data is NULL");
  if (x->dtype != IMU_F32 && x->dtype != IMU_BF16)
    return fail(IMU_ERR_INVALID_ARG, std::string(name) + ".dtype must be IMU_F32 or IMU_BF16");
  if (x->layout != IMU_NORMAL && x->layout != IMU_TRANSPOSED)
    return fail(IMU_ERR_INVALID_ARG, std::string(name) + ".layout must be IMU_NORMAL or IMU_TRANSPOSED");
  if (x->rows < 1 || x->cols < 1)
    return fail(IMU_ERR_INVALID_ARG, std::string(name) + " must have rows >= 1 and cols >= 1");
  if (x->rows > kMaxLine || x->cols > kMaxLine)
    return fail(IMU_ERR_UNSUPPORTED, std::string(name) + ": rows and cols must be below 2^24");
  if ((unsigned long long)x->rows * (unsigned long long)x->cols >= (1ull << 32))
    return fail(IMU_ERR_UNSUPPORTED, std::string(name) + ": rows*cols must be below 2^32");
  if (x->batch < 1 || x->batch > 65535)
    return fail(IMU_ERR_INVALID_ARG, std::string(name) + ".batch must be in [1, 65535]");
  op->m = x;
  op->R = x->rows;
  op->C = x->cols;
  op->tr = x->layout == IMU_TRANSPOSED;
  op->srows = op->tr ? x->cols : x->rows;
  op->scols = op->tr ? x->rows : x->cols;
  op->dtype = x->dtype;
  op->elem = x->dtype == IMU_F32 ? 4 : 2;
  if (x->ld < op->scols) return fail(IMU_ERR_INVALID_ARG, std::string(name) + ".ld is below the stored row length");
  if (x->batch > 1 && x->batch_stride < (op->srows - 1) * x->ld + op->scols)
    return fail(IMU_ERR_INVALID_ARG, std::string(name) + ".batch_stride overlaps batch entries");
  return IMU_OK;
}

imu_status check_params(const imu_params* p) {
  if (!p) return fail(IMU_ERR_INVALID_ARG, "params is NULL");
  if (p->bits < 2 || p->bits > 8) return fail(IMU_ERR_INVALID_ARG, "bits must be in [2, 8]");
  if (p->beta < 1) return fail(IMU_ERR_INVALID_ARG, "beta must be >= 1");
  if (p->p_den < 1 || p->p_den > 1000000) return fail(IMU_ERR_INVALID_ARG, "p_den must be in [1, 1e6]");
  if (p->p_num < 1 || p->p_num > p->p_den) return fail(IMU_ERR_INVALID_ARG, "p = p_num/p_den must be in (0, 1]");
  if (p->gamma < 0 || p->gamma > 1000000) return fail(IMU_ERR_INVALID_ARG, "gamma must be in [0, 1e6]");
  for (int s : {p->strat_a, p->strat_b})
    if (s != IMU_ROW && s != IMU_COL && s != IMU_MIX)
      return fail(IMU_ERR_INVALID_ARG, "strategy must be IMU_ROW, IMU_COL or IMU_MIX");
  return IMU_OK;
}

imu_status check_pair(const imu_matrix* a, const imu_matrix* b, const imu_params* p, Operand* oa,
                      Operand* ob) {
  IMU_TRY(check_matrix(a, "a", oa));
  IMU_TRY(check_matrix(b, "b", ob));
  IMU_TRY(check_params(p));
  if (a->cols != b->rows) return fail(IMU_ERR_INVALID_ARG, "a.cols must equal b.rows (K)");
  if (a->cols > kMaxK) return fail(IMU_ERR_UNSUPPORTED, "K must be below 2^20 - 1");
  if (a->batch != b->batch) return fail(IMU_ERR_INVALID_ARG, "a.batch must equal b.batch");
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

imu_status plan_launch(const Operand& oa, const Operand& ob, const imu_params* p, uint8_t* stats_a,
                       uint8_t* stats_b, uint8_t* plan, uint8_t* host_hdr, int64_t host_tag, hipEvent_t done,
                       hipStream_t s) {
  const StatsLayout la = stats_layout(oa.R, oa.C), lb = stats_layout(ob.R, ob.C);
  const int batch = (int)oa.m->batch;
  for (int dt : {(int)IMU_BF16, (int)IMU_F32}) {
    QuantJobs J{};
    if (p->strat_a == IMU_MIX && oa.dtype == dt) {
      J.op[J.nops].s = stream_args(oa, stats_a, la, p);
      J.op[J.nops++].batch = batch;
    }
    if (p->strat_b == IMU_MIX && ob.dtype == dt) {
      J.op[J.nops].s = stream_args(ob, stats_b, lb, p);
      J.op[J.nops++].batch = batch;
    }
    if (J.nops) IMU_HIP(launch_residual(dt, p->bits, J, s));
  }
  PlanArgs pa{};
  pa.stats_a = stats_a;
  pa.stats_b = stats_b;
  pa.stats_stride_a = la.stride;
  pa.stats_stride_b = lb.stride;
  pa.sla = la;
  pa.slb = lb;
  pa.plan = plan;
  pa.pl = plan_layout(oa.R, oa.C, ob.C, batch, p->bits);
  pa.gamma = p->gamma;
  pa.strat_a = p->strat_a;
  pa.strat_b = p->strat_b;
  pa.bits = p->bits;
  pa.host_hdr = host_hdr;
  pa.host_tag = host_tag;
  IMU_HIP(launch_plan(pa, done, s));
  return IMU_OK;
}

// Per-thread pinned, coherent host buffer that the planner's last launch
// writes a copy of the plan headers into, each copy closed by a per-call tag,
// and an event that completes with that launch (it is attached to the launch,
// so no marker of its own sits between the planner and the unpack; it carries
// no system-scope fence, which would write back the L2 and leave the GPU idle
// for microseconds).  The host waits for the headers alone while later kernels
// keep the GPU busy.  Buffer and events live until the process ends.
struct HeaderStage {
  uint8_t* buf = nullptr;       // host address
  uint8_t* dbuf = nullptr;      // the same memory as the device addresses it
  size_t bytes = 0;
  hipEvent_t ev = nullptr;      // completes with the planner's last launch
  hipEvent_t ev_sys = nullptr;  // fallback: an event with the system-scope fence
  int64_t tag = 0;
  int dev = -1;
};
thread_local HeaderStage g_stage;

imu_status header_stage(size_t bytes, uint8_t** out) {
  int dev = 0;
  IMU_HIP(hipGetDevice(&dev));
  HeaderStage& st = g_stage;
  if (st.ev && st.dev != dev) {  // events and mappings belong to a device; the old ones are kept alive
    st.ev = st.ev_sys = nullptr;
    st.bytes = 0;
  }
  if (!st.ev) {
    IMU_HIP(hipEventCreateWithFlags(&st.ev, hipEventDisableTiming | hipEventDisableSystemFence));
    IMU_HIP(hipEventCreateWithFlags(&st.ev_sys, hipEventDisableTiming));
    st.dev = dev;
  }
  if (st.bytes < bytes) {
    void* p = nullptr;
    IMU_HIP(hipHostMalloc(&p, bytes, hipHostMallocMapped | hipHostMallocCoherent));
    std::memset(p, 0, bytes);  // no stale tag
    void* d = nullptr;
    IMU_HIP(hipHostGetDevicePointer(&d, p, 0));
    st.buf = static_cast<uint8_t*>(p);
    st.dbuf = static_cast<uint8_t*>(d);
    st.bytes = bytes;  // the previous buffer is not freed: a launch may still write it
  }
  *out = st.buf;
  return IMU_OK;
}

// Wait until the host copy of every entry's header carries this call's tag:
// the planner's event, then a bounded poll of the tags.  Should they still be
// missing (host memory not coherent with the GPU after all), an event with the
// system-scope fence is recorded and waited for; a tag missing after that is an
// error.
imu_status wait_headers(int batch, hipStream_t s) {
  HeaderStage& st = g_stage;
  auto tagged = [&]() {
    for (int b = 0; b < batch; ++b) {
      const volatile int64_t* t = reinterpret_cast<const volatile int64_t*>(
          st.buf + (size_t)b * kPlanHeaderStride + offsetof(PlanHeader, reserved));
      if (*t != st.tag) return false;
    }
    return true;
  };
  IMU_HIP(hipEventSynchronize(st.ev));
  for (int i = 0; i < 100000; ++i)
    if (tagged()) {
      std::atomic_thread_fence(std::memory_order_acquire);
      return IMU_OK;
    }
  IMU_HIP(hipEventRecord(st.ev_sys, s));  // behind whatever was queued since: still correct
  IMU_HIP(hipEventSynchronize(st.ev_sys));
  if (!tagged()) return fail(IMU_ERR_HIP, "plan headers did not reach the host");
  std::atomic_thread_fence(std::memory_order_acquire);
  return IMU_OK;
}

// Plan launches with the host copy of the headers; returns that copy (valid
// once wait_headers has returned).
imu_status plan_staged(const Operand& oa, const Operand& ob, const imu_params* p, uint8_t* stats_a,
                       uint8_t* stats_b, uint8_t* plan, hipStream_t s, const uint8_t** hdrs) {
  uint8_t* buf = nullptr;
  IMU_TRY(header_stage((size_t)oa.m->batch * kPlanHeaderStride, &buf));
  HeaderStage& st = g_stage;
  ++st.tag;
  IMU_TRY(plan_launch(oa, ob, p, stats_a, stats_b, plan, st.dbuf, st.tag, st.ev, s));
  *hdrs = buf;
  return IMU_OK;
}

// Fill info from the staged headers (B' entries follow all A' entries) and
// report a failed plan.  *a_total / *b_total: bytes of all A' / B' entries.
imu_status finish_plan(const Operand& oa, const Operand& ob, const uint8_t* hdrs, int batch, imu_plan_info* info,
                       int64_t* a_total, int64_t* b_total) {
  int status = 0;
  int64_t aoff = 0, boff = 0;
  for (int b = 0; b < batch; ++b) {
    const PlanHeader* h = reinterpret_cast<const PlanHeader*>(hdrs + (size_t)b * kPlanHeaderStride);
    status |= h->status;
    aoff += unpacked_entry_bytes(h, 0);
  }
  const int64_t a_all = aoff;
  aoff = 0;
  for (int b = 0; b < batch; ++b) {
    const PlanHeader* h = reinterpret_cast<const PlanHeader*>(hdrs + (size_t)b * kPlanHeaderStride);
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
      f.unpack_ratio = (double)h->m_u * (double)h->k_u * (double)h->n_u /
                       ((double)oa.R * (double)oa.C * (double)ob.C);
      std::memcpy(f.pair_sizes, h->pair, sizeof(f.pair_sizes));
    }
    aoff += unpacked_entry_bytes(h, 0);
    boff += unpacked_entry_bytes(h, 1);
  }
  if (a_total) *a_total = a_all;
  if (b_total) *b_total = boff;
  if (status & kStatusNonfinite) return fail(IMU_ERR_NONFINITE, "an input element is NaN or Inf");
  if (status & kStatusRange) return fail(IMU_ERR_RANGE, "|x * r| >= 2^31 for some element");
  return IMU_OK;
}

imu_status plan_impl(const Operand& oa, const Operand& ob, const imu_params* p, uint8_t* stats_a,
                     uint8_t* stats_b, uint8_t* plan, imu_plan_info* info, hipStream_t s) {
  const int batch = (int)oa.m->batch;
  const uint8_t* hdrs = nullptr;
  IMU_TRY(plan_staged(oa, ob, p, stats_a, stats_b, plan, s, &hdrs));
  IMU_TRY(wait_headers(batch, s));
  return finish_plan(oa, ob, hdrs, batch, info, nullptr, nullptr);
}

// Unpack one operand; M, K, N give the plan layout.  after_a: B' entries start
// after all A' entries of x_u; cap: bytes available at x_u.
UnpackArgs unpack_args(const Operand& op, int operand, const imu_params* p, const uint8_t* stats,
                       const uint8_t* plan, int64_t M, int64_t K, int64_t N, int8_t* x_u, bool after_a,
                       int64_t cap) {
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
  return u;
}

imu_status unpack_impl(const Operand& op, int operand, const imu_params* p, const uint8_t* stats,
                       const uint8_t* plan, int64_t M, int64_t K, int64_t N, int8_t* x_u, bool after_a,
                       int64_t cap, hipStream_t s) {
  const UnpackArgs u = unpack_args(op, operand, p, stats, plan, M, K, N, x_u, after_a, cap);
  IMU_HIP(launch_unpack(op.dtype, p->bits, &u, 1, (int)op.m->batch, s));
  return IMU_OK;
}

imu_status gemm_impl(const int8_t* a_u, const int8_t* b_u, const imu_params* p, const uint8_t* stats_a,
                     const uint8_t* stats_b, const uint8_t* plan, const imu_plan_info* info,
                     int64_t batch, int32_t* c, int64_t ldc, int64_t cbs, float* out, hipStream_t s) {
  const int64_t M = info[0].m, K = info[0].k, N = info[0].n;
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
    const imu_plan_info& f = info[b];
    if (f.m_base % 256 || f.n_base % 128 || f.m_alloc % 256 || f.n_alloc % 128)
      return fail(IMU_ERR_INVALID_ARG, "plan sizes are not tile multiples");
    base_tiles = std::max(base_tiles, (f.m_base / 256) * (f.n_base / 128));
    base_total += (f.m_base / 256) * (f.n_base / 128);
  }
  int dev = 0, cus = 0;
  IMU_HIP(hipGetDevice(&dev));
  IMU_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  // IMU_FOLD_COLUMNS=1 / 0 forces the choice (both give the same result)
  const char* fe = std::getenv("IMU_FOLD_COLUMNS");
  const bool fold_cols = fe && fe[0] == '1' ? true : fe && fe[0] == '0' ? false : base_total >= cus;
  int64_t extra_tiles = 0;
  bool any_atomic = false, any_fold = false;
  for (int64_t b = 0; b < batch; ++b) {
    const imu_plan_info& f = info[b];
    const bool rowx = f.m_alloc > f.m_base, colx = f.n_alloc > f.n_base;
    if (rowx || (colx && !fold_cols)) {
      any_atomic = true;
      extra_tiles = std::max(extra_tiles, (f.m_alloc / 256) * (f.n_alloc / 128));
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
  g.db_c_off = pl.db_c;
  g.lvl_b_off = pl.lvl_b;
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
    if (info[b].m != M || info[b].k != K || info[b].n != N || info[b].k_pad <= 0)
      return fail(IMU_ERR_INVALID_ARG, "info does not describe this problem");
  return IMU_OK;
}

int64_t fixed_bytes(const Operand& oa, const Operand& ob, const imu_params* p) {
  const int64_t batch = oa.m->batch;
  return round_up(stats_layout(oa.R, oa.C).stride * batch, 256) +
         round_up(stats_layout(ob.R, ob.C).stride * batch, 256) +
         round_up(plan_layout(oa.R, oa.C, ob.C, batch, p->bits).total, 256);
}

}  // namespace

extern "C" {

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
  return unpack_impl(op, operand, p, static_cast<const uint8_t*>(stats), static_cast<const uint8_t*>(plan), M, K,
                     N, x_u, false, INT64_MAX, stream);
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
  return gemm_impl(a_u, b_u, p, static_cast<const uint8_t*>(stats_a), static_cast<const uint8_t*>(stats_b),
                   static_cast<const uint8_t*>(plan), info, batch, c, ldc, c_batch_stride, out, stream);
}

imu_status imu_imunpack_matmul(const imu_matrix* a, const imu_matrix* b, const imu_params* p, int32_t* c,
                               float* out, void* ws, size_t ws_bytes, size_t* ws_needed,
                               imu_plan_info* info, hipStream_t stream) {
  Operand oa, ob;
  IMU_TRY(check_pair(a, b, p, &oa, &ob));
  if (!c) return fail(IMU_ERR_INVALID_ARG, "c is NULL");
  const int64_t batch = a->batch;
  const int64_t fixed = fixed_bytes(oa, ob, p);
  if (ws_needed) *ws_needed = (size_t)fixed;
  if (!ws || (int64_t)ws_bytes < fixed)
    return fail(IMU_ERR_WORKSPACE, "workspace below the fixed part (statistics and plan)");
  uint8_t* w = static_cast<uint8_t*>(ws);
  uint8_t* stats_a = w;
  uint8_t* stats_b = stats_a + round_up(stats_layout(oa.R, oa.C).stride * batch, 256);
  uint8_t* plan = stats_b + round_up(stats_layout(ob.R, ob.C).stride * batch, 256);
  // statistics of A and B are adjacent: clear both with one launch
  IMU_HIP(launch_fill_u32(stats_a, 0u, (int64_t)(plan - stats_a) / 4, stream));
  const Operand* ops[2] = {&oa, &ob};
  uint8_t* st[2] = {stats_a, stats_b};
  int32_t* q[2] = {nullptr, nullptr};
  IMU_TRY(quantize_ops(ops, st, q, 2, p, stream, true));
  std::vector<imu_plan_info> local;
  if (!info) {
    local.resize((size_t)batch);
    info = local.data();
  }
  // The unpack kernels take their sizes and placement from the plan on the
  // device, so they are queued right behind the plan; the host waits only for
  // the plan headers (staged to pinned memory) while they run, then checks the
  // workspace and sizes the GEMM launch.  If the plan failed or the workspace
  // is too small the unpack kernels write nothing.
  const uint8_t* hdrs = nullptr;
  IMU_TRY(plan_staged(oa, ob, p, stats_a, stats_b, plan, stream, &hdrs));
  int8_t* region = reinterpret_cast<int8_t*>(w + fixed);
  const int64_t cap = (int64_t)ws_bytes - fixed;
  if (oa.dtype == ob.dtype) {  // both operands in one launch
    const UnpackArgs u[2] = {unpack_args(oa, 0, p, stats_a, plan, oa.R, oa.C, ob.C, region, false, cap),
                             unpack_args(ob, 1, p, stats_b, plan, oa.R, oa.C, ob.C, region, true, cap)};
    IMU_HIP(launch_unpack(oa.dtype, p->bits, u, 2, (int)batch, stream));
  } else {
    IMU_TRY(unpack_impl(oa, 0, p, stats_a, plan, oa.R, oa.C, ob.C, region, false, cap, stream));
    IMU_TRY(unpack_impl(ob, 1, p, stats_b, plan, oa.R, oa.C, ob.C, region, true, cap, stream));
  }
  IMU_TRY(wait_headers((int)batch, stream));
  int64_t a_bytes = 0, b_bytes = 0;
  IMU_TRY(finish_plan(oa, ob, hdrs, (int)batch, info, &a_bytes, &b_bytes));
  const int64_t needed = fixed + a_bytes + b_bytes;
  if (ws_needed) *ws_needed = (size_t)needed;
  if ((int64_t)ws_bytes < needed) return fail(IMU_ERR_WORKSPACE, "workspace below the unpacked operands' size");
  int8_t* a_u = region;
  int8_t* b_u = region + a_bytes;
  return gemm_impl(a_u, b_u, p, stats_a, stats_b, plan, info, batch, c, ob.C, oa.R * ob.C, out, stream);
}

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

const char* imu_last_error(void) { return g_err.c_str(); }

const char* imu_version(void) { return "imunpack 0.1 (gfx950)"; }

imu_status imu_set_gemm_events(hipEvent_t before, hipEvent_t after) {
  if ((before == nullptr) != (after == nullptr))
    return fail(IMU_ERR_INVALID_ARG, "pass both events or neither");
  g_gemm_ev[0] = before;
  g_gemm_ev[1] = after;
  return IMU_OK;
}

}  // extern "C"
