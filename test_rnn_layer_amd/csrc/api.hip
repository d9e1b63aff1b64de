// C ABI of the TTT-MLP layer scan: argument checks, workspace planning and
// kernel launches.  The operation and the layouts are specified in
// include/ttt_mlp.h.
#include "../../include/ttt_mlp.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int32_t ok() {
  g_last_error.clear();
  return TTT_OK;
}

// ---------------------------------------------------------------------------
// kernel timing
// ---------------------------------------------------------------------------
struct TimingRecord {
  int kind;
  hipEvent_t start, stop;
};
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<TimingRecord> g_timing_records;
constexpr int kTimingKinds = 5;
double g_timing_ms[kTimingKinds] = {};
int64_t g_timing_n[kTimingKinds] = {};

// Collect the finished records into the per-kind sums (caller holds the lock).
hipError_t drain_timing_locked() {
  hipError_t err = hipSuccess;
  for (auto& r : g_timing_records) {
    hipError_t e = hipEventSynchronize(r.stop);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e == hipSuccess) {
      g_timing_ms[r.kind] += ms;
      g_timing_n[r.kind] += 1;
    } else {
      err = e;
    }
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_timing_records.clear();
  return err;
}

// Set while ttt_mlp_bidir_noalloc enqueues on this thread: its launches record no
// timing events (creating them would be an allocation).
thread_local bool g_untimed = false;

// Launch `fn` on `stream`, bracketed by events when timing is on.
template <class F>
hipError_t timed_launch(int kind, hipStream_t stream, F&& fn) {
  bool on;
  {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    on = g_timing_on && !g_untimed;
  }
  if (!on) return fn();
  TimingRecord r{kind, nullptr, nullptr};
  hipError_t e = hipEventCreate(&r.start);
  if (e != hipSuccess) return e;
  e = hipEventCreate(&r.stop);
  if (e != hipSuccess) {
    (void)hipEventDestroy(r.start);
    return e;
  }
  e = hipEventRecord(r.start, stream);
  if (e == hipSuccess) e = fn();
  if (e == hipSuccess) e = hipEventRecord(r.stop, stream);
  if (e != hipSuccess) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
    return e;
  }
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing_records.push_back(r);
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// configuration checks and workspace plan
// ---------------------------------------------------------------------------
constexpr size_t kAlign = 256;
constexpr size_t kGenericLdsMax = 64 * 1024;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int algo;            // TTT_ALGO_GENERIC, TTT_ALGO_MFMA or TTT_ALGO_COOP
  size_t qkv_off, qkv_bytes;
  size_t wst_off, wst_bytes;  // generic: per-(sequence, head) state; coop: exchange slots + abort flag
  size_t total;
  size_t io_elem;      // bytes per X / Y element
};

int32_t check_config(const ttt_mlp_config* c) {
  if (!c) return fail(TTT_ERR_INVALID_ARG, "cfg is NULL");
  if (c->B < 1) return fail(TTT_ERR_INVALID_ARG, "B must be >= 1 (got %lld)", (long long)c->B);
  if (c->T < 0) return fail(TTT_ERR_INVALID_ARG, "T must be >= 0 (got %lld)", (long long)c->T);
  if (c->H < 1 || c->d < 1 || c->m < 1)
    return fail(TTT_ERR_INVALID_ARG, "H, d, m must be >= 1 (got %d, %d, %d)", c->H, c->d, c->m);
  if (c->b < 1) return fail(TTT_ERR_INVALID_ARG, "mini-batch b must be >= 1 (got %d)", c->b);
  if (!std::isfinite(c->eta) || c->eta < 0.0f)
    return fail(TTT_ERR_INVALID_ARG, "eta must be finite and >= 0 (got %g)", (double)c->eta);
  if (c->loss != TTT_LOSS_MEAN && c->loss != TTT_LOSS_SUM)
    return fail(TTT_ERR_INVALID_ARG, "unknown loss %d", c->loss);
  if (c->gelu != TTT_GELU_ERF && c->gelu != TTT_GELU_TANH)
    return fail(TTT_ERR_INVALID_ARG, "unknown gelu %d", c->gelu);
  if (c->io_dtype != TTT_F32 && c->io_dtype != TTT_BF16)
    return fail(TTT_ERR_INVALID_ARG, "unknown io_dtype %d", c->io_dtype);
  if (c->algo != TTT_ALGO_AUTO && c->algo != TTT_ALGO_GENERIC && c->algo != TTT_ALGO_MFMA &&
      c->algo != TTT_ALGO_COOP)
    return fail(TTT_ERR_INVALID_ARG, "unknown algo %d", c->algo);
  if (c->model != TTT_MODEL_MLP && c->model != TTT_MODEL_LINEAR)
    return fail(TTT_ERR_INVALID_ARG, "unknown model %d", c->model);
  if (c->model == TTT_MODEL_LINEAR && c->m != c->d)
    return fail(TTT_ERR_INVALID_ARG, "the linear model's state is d x d: m must equal d (got d=%d m=%d)", c->d,
                c->m);
  const int64_t D = (int64_t)c->H * c->d;
  if (D > (1 << 20) || c->m > (1 << 16) || c->b > (1 << 16))
    return fail(TTT_ERR_UNSUPPORTED, "D = %lld, m = %d or b = %d too large", (long long)D, c->m, c->b);
  if (c->T > ((int64_t)1 << 40) || c->B > ((int64_t)1 << 20) || c->B * c->H > (1 << 30))
    return fail(TTT_ERR_UNSUPPORTED, "B or T too large");
  return TTT_OK;
}

bool is_linear(const ttt_mlp_config* c) { return c->model == TTT_MODEL_LINEAR; }

// The MFMA scans take bf16 io; the MLP one implements the exact (erf) GELU (the
// tanh form runs on the generic kernel).  They index token rows of one sequence
// with 32-bit integers (T < 2^31).
bool mfma_possible(const ttt_mlp_config* c) {
  const bool shape = is_linear(c) ? ttt::scan_linear_mfma_supported(c->d, c->m, c->b)
                                  : c->gelu == TTT_GELU_ERF && ttt::scan_mfma_supported(c->d, c->m, c->b);
  return c->io_dtype == TTT_BF16 && shape && ((int64_t)c->H * c->d) % 8 == 0 && c->T < ((int64_t)1 << 31);
}

bool coop_possible(const ttt_mlp_config* c) {
  return !is_linear(c) && ttt::scan_coop_supported(c->d, c->m, c->b, c->T);
}

// Whether the cooperative scan's 8 B H workgroups fit co-resident on the current
// device; with no device (planning on a host without a GPU) the plan assumes they do.
bool coop_fits_here(const ttt_mlp_config* c) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n == 0) {
    (void)hipGetLastError();  // a failed query leaves no error behind for the next call
    return true;
  }
  return ttt::scan_coop_fits(c->B, c->H);
}

size_t generic_lds_bytes(const ttt_mlp_config* c) {
  return is_linear(c) ? ttt::scan_linear_generic_lds_bytes(c->d, c->b) : ttt::scan_generic_lds_bytes(c->d, c->m, c->b);
}

// fp32 state elements of one (sequence, head): W1 and W2, or the linear model's W
size_t state_elems(const ttt_mlp_config* c) { return (is_linear(c) ? 1 : 2) * (size_t)c->d * c->m; }

int32_t make_plan(const ttt_mlp_config* c, Plan* p) {
  int32_t st = check_config(c);
  if (st != TTT_OK) return st;
  int algo = c->algo;
  if (algo == TTT_ALGO_AUTO)
    algo = mfma_possible(c)                         ? TTT_ALGO_MFMA
           : coop_possible(c) && coop_fits_here(c) ? TTT_ALGO_COOP
                                                   : TTT_ALGO_GENERIC;
  if (algo == TTT_ALGO_COOP && !coop_possible(c))
    return fail(TTT_ERR_UNSUPPORTED,
                "the cooperative scan needs the MLP model, d=128, m=512, b=1, T < 2^31 (got d=%d m=%d b=%d)", c->d,
                c->m, c->b);
  if (algo == TTT_ALGO_COOP && !coop_fits_here(c))
    return fail(TTT_ERR_UNSUPPORTED, "cooperative scan: %lld workgroups do not fit on this device at once",
                (long long)(c->B * c->H * 8));
  if (algo == TTT_ALGO_MFMA && !mfma_possible(c))
    return fail(TTT_ERR_UNSUPPORTED,
                is_linear(c) ? "the linear MFMA scan needs bf16 io, d=m=64, b=16 (got d=%d m=%d b=%d io=%d)"
                             : "the MFMA scan needs bf16 io, erf GELU, d=64, m=256, b=16 (got d=%d m=%d b=%d io=%d "
                               "gelu=%d)",
                c->d, c->m, c->b, c->io_dtype, c->gelu);
  if (algo == TTT_ALGO_GENERIC && generic_lds_bytes(c) > kGenericLdsMax)
    return fail(TTT_ERR_UNSUPPORTED,
                "generic scan: mini-batch working set of %zu bytes (d=%d m=%d b=%d) exceeds %zu bytes of LDS",
                generic_lds_bytes(c), c->d, c->m, c->b, kGenericLdsMax);
  p->algo = algo;
  p->io_elem = c->io_dtype == TTT_BF16 ? 2 : 4;
  const size_t BHTd = (size_t)c->B * c->H * (size_t)c->T * c->d;
  p->qkv_off = 0;
  if (algo == TTT_ALGO_MFMA) {
    p->qkv_bytes = align_up(ttt::scan_mfma_tile_bytes(c->B, c->T, c->H));
    // the state handed from one chunk of the scan to the next (W1 then W2, or W)
    p->wst_bytes = align_up((size_t)c->B * c->H * state_elems(c) * sizeof(float));
  } else if (algo == TTT_ALGO_COOP) {
    p->qkv_bytes = align_up(3 * BHTd * sizeof(float));
    p->wst_bytes = align_up(ttt::scan_coop_xchg_bytes(c->B, c->H) + sizeof(uint32_t));
  } else {
    p->qkv_bytes = align_up(3 * BHTd * sizeof(float));
    p->wst_bytes = align_up((size_t)c->B * c->H * state_elems(c) * sizeof(float));
  }
  p->wst_off = p->qkv_off + p->qkv_bytes;
  p->total = p->wst_off + p->wst_bytes;
  if (p->total == 0) p->total = kAlign;
  return TTT_OK;
}

hipError_t launch_projection(const ttt::ProjArgs& pa, int mode, hipStream_t s) {
  if (ttt::project_mfma_supported(pa)) return ttt::launch_project_mfma(pa, mode, s);
  return ttt::launch_project_f32out(pa, s);  // mode 0 only: the MFMA scan always has a supported GEMM
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const char* pa = (const char*)a;
  const char* pb = (const char*)b;
  return pa < pb + nb && pb < pa + na;
}

struct Buf {
  const void* p;
  size_t n;
  const char* name;
};

int32_t check_no_overlap(const Buf* outs, int nout, const Buf* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
        return fail(TTT_ERR_INVALID_ARG, "output %s overlaps output %s", outs[i].name, outs[j].name);
    for (int j = 0; j < nin; ++j)
      if (overlaps(outs[i].p, outs[i].n, ins[j].p, ins[j].n))
        return fail(TTT_ERR_INVALID_ARG, "output %s overlaps input %s", outs[i].name, ins[j].name);
  }
  return TTT_OK;
}

ttt::ProjArgs proj_args(const ttt_mlp_config* c, const Plan& pl, const void* xin, const void* theta, int reverse,
                        char* ws) {
  ttt::ProjArgs pa{};
  pa.X = xin;
  pa.theta = theta;
  pa.out = ws + pl.qkv_off;
  pa.B = c->B;
  pa.T = c->T;
  pa.H = c->H;
  pa.d = c->d;
  pa.bf16 = c->io_dtype == TTT_BF16;
  pa.reverse = reverse;
  pa.blk_elems = ttt::scan_mfma_block_elems();
  pa.tt0 = 0;
  pa.tt1 = c->T;
  return pa;
}

ttt::ScanArgs scan_args(const ttt_mlp_config* c, const Plan& pl, const void* xin, const float* W1_0,
                        const float* W2_0, const float* alpha, int reverse, void* y, float* z, float* w1T, float* w2T,
                        char* ws) {
  ttt::ScanArgs sa{};
  sa.qkv = (const float*)(ws + pl.qkv_off);
  sa.qkv_tiles = ws + pl.qkv_off;
  sa.xin = xin;
  sa.y = y;
  sa.z = z;
  sa.alpha = alpha;
  sa.w1_0 = W1_0;
  sa.w2_0 = W2_0;
  sa.w_seq_stride = 0;
  sa.wstate = (float*)(ws + pl.wst_off);
  sa.xchg = (uint64_t*)(ws + pl.wst_off);
  sa.abort_flag = (uint32_t*)(ws + pl.wst_off + ttt::scan_coop_xchg_bytes(c->B, c->H));
  sa.clear_abort = 1;
  sa.w1_T = w1T;
  sa.w2_T = w2T;
  sa.B = c->B;
  sa.T = c->T;
  sa.p0 = 0;
  sa.Tc = c->T;
  sa.H = c->H;
  sa.d = c->d;
  sa.m = c->m;
  sa.b = c->b;
  sa.eta = c->eta;
  sa.gscale = c->loss == TTT_LOSS_MEAN ? 2.0f / (float)c->d : 2.0f;
  sa.gelu_tanh = c->gelu == TTT_GELU_TANH;
  sa.reverse = reverse;
  sa.bf16 = c->io_dtype == TTT_BF16;
  sa.linear = is_linear(c);
  return sa;
}

// One direction on the generic or cooperative path: projection of xin, then
// the scan writing y (and z, W_T).
int32_t run_direction(const ttt_mlp_config* c, const Plan& pl, const void* xin, const void* theta,
                      const float* W1_0, const float* W2_0, const float* alpha, int reverse, void* y,
                      float* z, float* w1T, float* w2T, char* ws, hipStream_t stream, bool first = true) {
  const ttt::ProjArgs pa = proj_args(c, pl, xin, theta, reverse, ws);
  hipError_t e = timed_launch(TTT_KERNEL_PROJECT, stream, [&] { return launch_projection(pa, 0, stream); });
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "projection launch: %s", hipGetErrorString(e));
  ttt::ScanArgs sa = scan_args(c, pl, xin, W1_0, W2_0, alpha, reverse, y, z, w1T, w2T, ws);
  sa.clear_abort = first;
  if (pl.algo == TTT_ALGO_COOP && !ttt::scan_coop_fits(c->B, c->H))
    return fail(TTT_ERR_UNSUPPORTED, "cooperative scan: %lld workgroups do not fit on this device at once",
                (long long)(c->B * c->H * 8));
  e = timed_launch(TTT_KERNEL_SCAN, stream, [&] {
    if (pl.algo == TTT_ALGO_COOP) return ttt::launch_scan_coop(sa, stream);
    return sa.linear ? ttt::launch_scan_linear_generic(sa, stream) : ttt::launch_scan_generic(sa, stream);
  });
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "scan launch: %s", hipGetErrorString(e));
  return TTT_OK;
}

// ---------------------------------------------------------------------------
// MFMA path: chunked scans overlapped with the projections
// ---------------------------------------------------------------------------
// The MFMA scan uses one CU per (sequence, head); the projection GEMM of the
// next chunk of tokens runs on the remaining CUs at the same time.  Each
// direction is cut into chunks of whole 16-token blocks; the projection of
// chunk k runs on a side stream, the scan of chunk k on the caller's stream
// after it, starting from the state the scan of chunk k-1 left in the
// workspace.  In a bidirectional call the projection of a reverse chunk waits
// for the forward scan chunks that wrote its tokens of X' (and read its part of
// the token-block buffer).  Only the first chunk's projection of each
// direction is exposed, so the first chunk is short (512 tokens) and the
// chunks grow by half each time up to about T/12: the projection of chunk k+1
// (on the CUs the scan leaves free, ~0.09 us per token) then still finishes
// within the scan of chunk k (~0.16 us per token).

struct Side {
  hipStream_t stream = nullptr;
  std::vector<hipEvent_t> events;
  int cus = 0;  // compute units of the device
};
std::mutex g_side_mu;  // held while a call enqueues: events are reused between calls
std::map<int, Side> g_side;

hipError_t side_for_device(Side** out, size_t n_events) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  Side& sd = g_side[dev];
  if (!sd.stream) {
    e = hipStreamCreateWithFlags(&sd.stream, hipStreamNonBlocking);  // default priority
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&sd.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
  }
  while (sd.events.size() < n_events) {
    hipEvent_t ev;
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    sd.events.push_back(ev);
  }
  *out = &sd;
  return hipSuccess;
}

// Chunks per direction never exceed 41 for T < 2^31 (512 tokens, growing by half
// up to T/12, then T/12 at a time); ttt_mlp_bidir_noalloc creates the events of
// this many at set-up, so that no later call creates one.
constexpr int kMaxChunks = 48;

struct Chunking {
  std::vector<int64_t> b;  // chunk k covers positions [b[k], b[k+1]); b[0] = 0, b.back() = T
  int64_t count() const { return (int64_t)b.size() - 1; }
  int64_t of(int64_t pos) const {  // chunk holding position pos (0 <= pos < T)
    return (int64_t)(std::upper_bound(b.begin(), b.end(), pos) - b.begin()) - 1;
  }
};

Chunking chunking(int64_t T) {
  constexpr int64_t kFirst = 512, kRows = 256, kParts = 12;  // sizes are multiples of 256 tokens
  const int64_t cap = std::max(kFirst, (T / kParts + kRows - 1) / kRows * kRows);
  Chunking ch;
  ch.b.push_back(0);
  int64_t size = kFirst;
  while (ch.b.back() < T) {
    ch.b.push_back(std::min(T, ch.b.back() + size));
    size = std::min(cap, (size * 3 / 2 + kRows - 1) / kRows * kRows);
  }
  if (T == 0) ch.b.push_back(0);
  return ch;
}

// Projection workgroups beside the scan: at most this many, and no more than the
// CUs the scan leaves free (a workgroup takes a whole CU's LDS, and one that
// waits for a CU would run its share of tiles after the others); no cap when
// fewer than kProjMinWorkgroups are free.  The chip shares one power budget:
// every CU the projection keeps busy lowers the clock the scan runs at, so the
// cap is the fewest workgroups that still keep the projection ahead of the
// scan (bidirectional layer at 307,200 tokens, 48 heads: 96 beats 80 and 112-160;
// re-measured with the faster scan, 88.4 ms per call against 89.9 at 88 and 91.0 at 80).
constexpr int kProjWorkgroupsBesideScan = 96, kProjMinWorkgroups = 64;

int proj_workgroups_beside_scan(int cus, int64_t scan_workgroups) {
  const int64_t free_cus = (int64_t)cus - scan_workgroups;
  const int64_t cap = std::min<int64_t>(kProjWorkgroupsBesideScan, free_cus) / 8 * 8;
  return cap >= kProjMinWorkgroups ? (int)cap : 0;
}

// Overlapping chunk k+1's projection with chunk k's scan pays while the
// projection, squeezed onto the CUs the scan leaves free, keeps pace with the
// scan.  With many (sequence, head) chains there are too few free CUs: each
// direction then projects all its tokens on the whole chip first and scans
// after.  Per token: the projection takes 6 D^2 flops at about 1.1 PFLOP/s on
// the whole chip (cus / free times as long on the free CUs, beside the scan),
// a chain's scan step about 2.3 us per 16 tokens (MLP) or 0.05 us per token
// (linear), measured on MI355X.
bool overlap_pays(const ttt_mlp_config* c, int cus) {
  const int64_t free_cus = (int64_t)cus - c->B * c->H;
  if (free_cus < kProjMinWorkgroups) return false;
  const double D = (double)c->H * c->d;
  const double proj_tok = 6.0 * D * D / 1.1e15;
  const double scan_tok = is_linear(c) ? 0.05e-6 : 2.3e-6 / 16;
  return (double)c->B * proj_tok * ((double)cus / (double)free_cus - 1.0) <= scan_tok;
}

struct Direction {
  const void* xin;
  const float* alpha;
  int reverse;
  void* y;
  float* z;
  float* w1T;
  float* w2T;
};

int32_t run_mfma(const ttt_mlp_config* c, const Plan& pl, const Direction* dirs, int ndir, const void* theta,
                 const float* W1_0, const float* W2_0, char* ws, hipStream_t S) {
  const int64_t T = c->T;
  std::lock_guard<std::mutex> lk(g_side_mu);
  Side* sd = nullptr;
  hipError_t e = side_for_device(&sd, 2);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "side stream: %s", hipGetErrorString(e));
  const bool overlap = overlap_pays(c, sd->cus);
  Chunking ch;
  if (overlap) {
    ch = chunking(T);
  } else {  // one chunk per direction: the projection on the whole chip, then the scan
    ch.b = {0, T};
  }
  const int64_t C = ch.count();
  // events: start, then per direction C projection + C scan events, then end
  e = side_for_device(&sd, 2 + 2 * (size_t)C * ndir);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "side stream: %s", hipGetErrorString(e));
  hipStream_t S2 = sd->stream;
  // the cap pays where the scan is the longer of the two (the MLP); the linear
  // model's scan is a third of its projection, which then takes every free CU
  const int proj_wg = (is_linear(c) || !overlap) ? 0 : proj_workgroups_beside_scan(sd->cus, c->B * c->H);
  hipEvent_t* ev = sd->events.data();
  hipEvent_t ev_start = ev[0], ev_end = ev[1];
  auto ev_proj = [&](int d, int64_t k) { return ev[2 + (2 * d) * C + k]; };
  auto ev_scan = [&](int d, int64_t k) { return ev[2 + (2 * d + 1) * C + k]; };
  float* st1 = (float*)(ws + pl.wst_off);  // chunk-to-chunk state, [B, H, d, m] then [B, H, m, d]
  float* st2 = st1 + (size_t)c->B * c->H * c->d * c->m;
  const int64_t st_stride = (int64_t)c->H * c->d * c->m;

#define TTT_TRY(x, what)                                                              \
  do {                                                                                \
    hipError_t err_ = (x);                                                            \
    if (err_ != hipSuccess) return fail(TTT_ERR_HIP, "%s: %s", what, hipGetErrorString(err_)); \
  } while (0)

  TTT_TRY(hipEventRecord(ev_start, S), "event record");
  TTT_TRY(hipStreamWaitEvent(S2, ev_start, 0), "stream wait");
  for (int d = 0; d < ndir; ++d) {
    const Direction& D = dirs[d];
    // projections of this direction's chunks, on the side stream
    for (int64_t k = 0; k < C; ++k) {
      const int64_t p0 = ch.b[k], p1 = ch.b[k + 1];
      if (d > 0) {
        // X' tokens of this chunk come from forward positions [T-p1, T-p0), and the
        // chunk's token blocks were last read by the forward scan of positions [p0, p1)
        const int64_t need = p1 > p0 ? std::max(ch.of(T - p0 - 1), ch.of(p1 - 1)) : 0;
        TTT_TRY(hipStreamWaitEvent(S2, ev_scan(d - 1, need), 0), "stream wait");
      }
      ttt::ProjArgs pa = proj_args(c, pl, D.xin, theta, D.reverse, ws);
      pa.tt0 = D.reverse ? T - p1 : p0;
      pa.tt1 = D.reverse ? T - p0 : p1;
      // beside the scan, the projection runs on few enough CUs that its power draw
      // does not pull the shared clock down (the first chunk, exposed, takes them all)
      if (k > 0) pa.max_wg = proj_wg;
      TTT_TRY(timed_launch(TTT_KERNEL_PROJECT, S2, [&] { return ttt::launch_project_mfma(pa, 1, S2); }),
              "projection launch");
      if (k == C - 1) TTT_TRY(ttt::launch_zero_block_padding(pa, S2), "padding launch");
      TTT_TRY(hipEventRecord(ev_proj(d, k), S2), "event record");
    }
    // the scan, chunk by chunk on the caller's stream
    for (int64_t k = 0; k < C; ++k) {
      const int64_t p0 = ch.b[k], p1 = ch.b[k + 1];
      TTT_TRY(hipStreamWaitEvent(S, ev_proj(d, k), 0), "stream wait");
      ttt::ScanArgs sa = scan_args(c, pl, D.xin, W1_0, W2_0, D.alpha, D.reverse, D.y, D.z, D.w1T, D.w2T, ws);
      sa.p0 = p0;
      sa.Tc = p1 - p0;
      if (k > 0) {
        sa.w1_0 = st1;
        sa.w2_0 = st2;
        sa.w_seq_stride = st_stride;
      }
      if (k < C - 1) {
        sa.w1_T = st1;
        sa.w2_T = st2;
      }
      TTT_TRY(timed_launch(TTT_KERNEL_SCAN, S,
                           [&] { return sa.linear ? ttt::launch_scan_linear_mfma(sa, S) : ttt::launch_scan_mfma(sa, S); }),
              "scan launch");
      TTT_TRY(hipEventRecord(ev_scan(d, k), S), "event record");
    }
  }
  TTT_TRY(hipEventRecord(ev_end, S2), "event record");
  TTT_TRY(hipStreamWaitEvent(S, ev_end, 0), "stream wait");
#undef TTT_TRY
  return TTT_OK;
}

// ---------------------------------------------------------------------------
// backward (generic fp32 path)
// ---------------------------------------------------------------------------
// The forward pass runs again inside the backward call (projection, then a
// forward scan built from the backward's own steps, which leaves a checkpoint
// of the state every kCkptEvery mini-batches); the backward scan replays one
// segment at a time from its checkpoint.  The checkpoints of a direction take B*H*ceil(T/b/kCkptEvery)
// states, the replayed segment B*H*kCkptEvery states and forward quantities.
constexpr int kCkptEvery = 32;
constexpr size_t kBackwardLdsMax = 160 * 1024;
// With the fp32 matrix-core forward steps (algo AUTO, d = 64, m = 256, b = 16, erf GELU), the
// backward scan's segments are replayed beforehand, kReplayWindow segments of every chain per
// launch on as many workgroups, and the backward scan walks them without replaying.  16: at 48
// chains a replay launch is 768 workgroups, three whole waves of a 256-CU chip (with 4 segments,
// 192 workgroups left 64 CUs idle: 2.00 against 1.96 s per bidir307k backward call).
constexpr int kReplayWindow = 16;

bool bwd_f32mfma(const ttt_mlp_config* c) {
  return c->algo == TTT_ALGO_AUTO && ttt::scan_fwd_f32_supported(c->d, c->m, c->b) && c->gelu != TTT_GELU_TANH;
}

struct BwdPlan {
  Plan fwd;  // the forward pass's Q/K/V and state slices (generic layout)
  // qkv2_off: the reversed pass's Q/K/V (bidirectional), kept beside the forward pass's
  size_t qkv2_off, dqkv_off, dqkv2_off, z_off[2], y_off, xp_off, dxp_off, ckpt_off[2], segst_off, dstate_off,
      scratch_off,
      dwseq_off,
      dal_off, total;
  // the split backward scan: its workgroups per chain (4, 2, or 0: one workgroup per chain), its
  // exchange entries then its abort flag, and with four its second [B, T, 2D] dQ|dK buffer
  int split = 0;
  size_t bxchg_off = 0, dqkvb_off = 0;
  // the replayed segments' second buffer: the next window is replayed into it beside the walk
  size_t segst2_off = 0;
  // the gradient GEMMs' operands: with bf16 io (split3) the exact bf16 split [h | m | l] of a
  // direction's dQ|dK|dV ([B T, 9D]) and theta stacked three times ([9D, D]); with fp32 io none.
  // Then the two rocBLAS workspace slices (caller's stream, side stream).
  bool split3 = false;
  size_t sp_off = 0, th3_off = 0, p3_off = 0, blas_off[2];
};

int32_t make_bwd_plan(const ttt_mlp_config* c, int bidir, BwdPlan* p) {
  int32_t st = check_config(c);
  if (st != TTT_OK) return st;
  if (is_linear(c)) return fail(TTT_ERR_UNSUPPORTED, "the backward covers the MLP model only");
  if (c->algo != TTT_ALGO_AUTO && c->algo != TTT_ALGO_GENERIC)
    return fail(TTT_ERR_UNSUPPORTED, "the backward runs the generic fp32 scans (algo AUTO or GENERIC, got %d)",
                c->algo);
  if (ttt::scan_backward_lds_bytes(c->d, c->m, c->b) > kBackwardLdsMax)
    return fail(TTT_ERR_UNSUPPORTED, "backward: mini-batch working set (d=%d b=%d) exceeds %zu bytes of LDS", c->d,
                c->b, kBackwardLdsMax);
  if (c->d % 4 != 0 || c->m % 4 != 0)
    return fail(TTT_ERR_UNSUPPORTED, "backward: d and m must be multiples of 4 (got d=%d m=%d)", c->d, c->m);
  if (bwd_f32mfma(c) && ttt::scan_replay_f32_slot_elems() != ttt::scan_backward_segment_elems(c->d, c->m, c->b))
    return fail(TTT_ERR_UNSUPPORTED, "backward: the segment replay's slot layout differs from the backward scan's");
  const size_t D = (size_t)c->H * c->d, BTD = (size_t)c->B * c->T * D, BH = (size_t)c->B * c->H;
  const size_t st2 = 2 * (size_t)c->d * c->m * sizeof(float);  // one (W1, W2) state
  const size_t nseg = ((size_t)(c->T + c->b - 1) / c->b + kCkptEvery - 1) / kCkptEvery;
  const size_t io = c->io_dtype == TTT_BF16 ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  Plan& f = p->fwd;
  f.algo = TTT_ALGO_GENERIC;
  f.io_elem = io;
  f.qkv_bytes = align_up(3 * BTD * sizeof(float));
  f.qkv_off = take(3 * BTD * sizeof(float));
  f.wst_bytes = align_up(BH * st2);
  f.wst_off = take(BH * st2);  // the forward scan's state, then the backward's replayed state
  p->qkv2_off = bidir ? take(3 * BTD * sizeof(float)) : 0;
  p->dqkv_off = take(3 * BTD * sizeof(float));
  // the reversed pass's dQ|dK|dV: with fp32 io a buffer of its own, which its deferred dtheta GEMM
  // reads while the forward pass's backward scan writes the other; with bf16 io that GEMM reads
  // their bf16 split, so the two directions share one buffer
  p->dqkv2_off = bidir && c->io_dtype != TTT_BF16 ? take(3 * BTD * sizeof(float)) : p->dqkv_off;
  p->z_off[0] = take(BTD * sizeof(float));
  p->z_off[1] = bidir ? take(BTD * sizeof(float)) : 0;
  p->y_off = take(BTD * io);
  p->xp_off = bidir ? take(BTD * io) : 0;
  p->dxp_off = bidir ? take(BTD * sizeof(float)) : 0;
  p->ckpt_off[0] = take(BH * nseg * st2);
  p->ckpt_off[1] = bidir ? take(BH * nseg * st2) : 0;
  const size_t segst_bytes = BH * (bwd_f32mfma(c) ? kReplayWindow : 1) * kCkptEvery *
                             ttt::scan_backward_segment_elems(c->d, c->m, c->b) * sizeof(float);
  p->segst_off = take(segst_bytes);
  p->segst2_off = bwd_f32mfma(c) ? take(segst_bytes) : 0;
  p->dstate_off = take(BH * st2);
  p->scratch_off = take(BH * ttt::scan_backward_scratch_elems(c->d, c->m, c->b) * sizeof(float));
  p->dwseq_off = take(BH * st2);
  if (bwd_f32mfma(c)) {
    p->split = ttt::scan_backward_split_fits(c->B, c->H, c->d, c->m, c->b, 4)   ? 4
               : ttt::scan_backward_split_fits(c->B, c->H, c->d, c->m, c->b, 2) ? 2
                                                                                 : 0;
    // (the two-part forward pass uses the same entries before the walk)
    if (p->split)
      p->bxchg_off = take(std::max(ttt::scan_backward_split_xchg_elems(c->B, c->H, c->d, c->b, p->split),
                                   ttt::scan_fwd_f32_split_xchg_elems(c->B, c->H)) *
                              sizeof(uint64_t) +
                          256);
    if (p->split == 4) p->dqkvb_off = take(2 * BTD * sizeof(float));
  }
  p->dal_off = take(ttt::dalpha_partial_elems((int)D) * sizeof(float));
  p->split3 = c->io_dtype == TTT_BF16;
  if (p->split3) {
    p->sp_off = take(9 * BTD * sizeof(uint16_t));
    p->th3_off = take(9 * D * D * sizeof(uint16_t));
    p->p3_off = take(9 * D * D * sizeof(float));
  }
  p->blas_off[0] = take(ttt::grad_gemm_workspace_bytes());
  p->blas_off[1] = bidir ? take(ttt::grad_gemm_workspace_bytes()) : 0;
  p->total = off;
  f.total = off;
  return TTT_OK;
}

// Projection of xin into the plan's Q/K/V slice (fp32, [3, B, H, T, d]).
int32_t bwd_project(const ttt_mlp_config* c, const BwdPlan& bp, const void* xin, const void* theta, char* ws,
                    hipStream_t s) {
  const ttt::ProjArgs pa = proj_args(c, bp.fwd, xin, theta, 0, ws);
  hipError_t e = timed_launch(TTT_KERNEL_PROJECT, s, [&] { return launch_projection(pa, 0, s); });
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "projection launch: %s", hipGetErrorString(e));
  return TTT_OK;
}

// The forward pass of one direction, keeping Z and the state checkpoints.
int32_t bwd_forward(const ttt_mlp_config* c, const BwdPlan& bp, const void* xin, const void* theta, const float* W1_0,
                    const float* W2_0, const float* alpha, int reverse, void* y, float* z, float* ckpt, char* ws,
                    hipStream_t s) {
  int32_t st = bwd_project(c, bp, xin, theta, ws, s);
  if (st != TTT_OK) return st;
  ttt::ScanArgs sa = scan_args(c, bp.fwd, xin, W1_0, W2_0, alpha, reverse, y, z, nullptr, nullptr, ws);
  sa.ckpt = ckpt;
  sa.ckpt_every = kCkptEvery;
  sa.scratch = (float*)(ws + bp.scratch_off);
  // AUTO: the fp32 matrix-core forward pass with the state in registers where it applies, on two
  // workgroups per chain where they fit co-resident (exchange entries: the split backward scan's,
  // unused until the walk; the parts' Z: the dQ|dK|dV buffer, likewise)
  const bool f32mfma = bwd_f32mfma(c);
  hipError_t e = hipSuccess;
  const bool split_fwd = f32mfma && bp.split != 0 && c->T > 0 && ttt::scan_fwd_f32_split_fits(c->B, c->H);
  if (split_fwd) {
    const int64_t nx = (int64_t)ttt::scan_fwd_f32_split_xchg_elems(c->B, c->H);
    sa.xchg = (uint64_t*)(ws + bp.bxchg_off);
    sa.abort_flag = (uint32_t*)(sa.xchg + nx);
    sa.zpart = (float*)(ws + bp.dqkv_off);
    e = ttt::launch_zero_u64(sa.xchg, nx + 1, s);
    if (e != hipSuccess) return fail(TTT_ERR_HIP, "clearing launch: %s", hipGetErrorString(e));
  }
  e = timed_launch(TTT_KERNEL_SCAN, s, [&] {
    return f32mfma ? ttt::launch_scan_fwd_f32(sa, s) : ttt::launch_scan_fwd_ckpt(sa, s);
  });
  if (e == hipSuccess && split_fwd) e = ttt::launch_fwd_f32_gate(sa, s);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "scan launch: %s", hipGetErrorString(e));
  return TTT_OK;
}

// The backward of one direction whose forward pass (bwd_forward) left its Q/K/V in
// the workspace: dX = dyin + dQKV theta; dtheta, dW1_0, dW2_0 written or accumulated.
// One direction's backward: the backward scan (dQ|dK|dV into dqkv), dalpha, dX = dY + dqkv theta,
// dtheta (+)= dqkv^T X and the initial state's gradient.  skip_theta leaves this direction's dtheta
// GEMM to the next call; a call with side set runs that deferred GEMM (operands prev_dqkv,
// prev_x; it writes dtheta) on the side stream, released together with this call's backward scan
// (ev_ready) and enqueued after it, so that the scan's workgroups take their CUs first and the
// GEMM fills the rest; this call's own dtheta GEMM then adds to it after ev_done.
// With split3 the deferred GEMM reads the split of the workspace, which the next direction
// overwrites only after it (same stream, or after ev_done); prev_dqkv serves fp32 io.
struct ThetaOverlap {
  bool skip_theta = false;
  hipStream_t side = nullptr;
  hipEvent_t ev_ready = nullptr, ev_done = nullptr;
  const float* prev_dqkv = nullptr;
  const void* prev_x = nullptr;  // the deferred GEMM's X (io dtype)
};

// The replays beside the walk: a second stream and its events (start, replay done and walk done
// per slot buffer), and the device's compute units.
struct ReplayOverlap {
  hipStream_t side = nullptr;
  hipEvent_t start = nullptr, rep[2] = {nullptr, nullptr}, walk[2] = {nullptr, nullptr};
  int cus = 0;
};
// from a device's side stream and its events 2 .. 6 (events 0 and 1 serve ThetaOverlap)
ReplayOverlap replay_overlap(const Side& sd) {
  ReplayOverlap ro;
  ro.side = sd.stream;
  ro.start = sd.events[2];
  ro.rep[0] = sd.events[3];
  ro.rep[1] = sd.events[4];
  ro.walk[0] = sd.events[5];
  ro.walk[1] = sd.events[6];
  ro.cus = sd.cus;
  return ro;
}

// The gradient GEMMs on rocBLAS.  dq: the direction's dQ|dK|dV (fp32 io) or its bf16 split
// (split3); thg: theta (fp32 io) or theta stacked three times (split3); xg: the direction's
// input in the io dtype.
int32_t grad_dx(const BwdPlan& bp, char* ws, int slot, const void* dq, const void* thg, const float* dyin,
                float* dX, int64_t BT, int64_t D, hipStream_t s) {
  const char* err = nullptr;
  hipError_t e = timed_launch(TTT_KERNEL_GRAD_GEMM, s, [&] {
    err = bp.split3 ? ttt::grad_gemm_dx_split(slot, (const uint16_t*)dq, (const uint16_t*)thg, dyin, dX, BT, D,
                                              ws + bp.blas_off[slot], ttt::grad_gemm_workspace_bytes(), s)
                    : ttt::grad_gemm_dx(slot, (const float*)dq, (const float*)thg, dyin, dX, BT, D,
                                        ws + bp.blas_off[slot], ttt::grad_gemm_workspace_bytes(), s);
    return err ? hipErrorUnknown : hipSuccess;
  });
  if (err) return fail(TTT_ERR_HIP, "rocBLAS dX GEMM: %s", err);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "dX GEMM timing: %s", hipGetErrorString(e));
  return TTT_OK;
}

int32_t grad_dtheta(const BwdPlan& bp, char* ws, int slot, const void* dq, const void* xg, float* dtheta,
                    int64_t BT, int64_t D, int accumulate, hipStream_t s) {
  if (BT == 0) {  // no tokens: dtheta is zero, or unchanged
    if (accumulate) return TTT_OK;
    hipError_t e = ttt::launch_gemm_f32(true, false, nullptr, 3 * D, nullptr, D, dtheta, D, nullptr, 3 * D, D, 0, 0, s);
    return e == hipSuccess ? TTT_OK : fail(TTT_ERR_HIP, "dtheta clear: %s", hipGetErrorString(e));
  }
  const char* err = nullptr;
  hipError_t e = timed_launch(TTT_KERNEL_GRAD_GEMM, s, [&] {
    err = bp.split3 ? ttt::grad_gemm_dtheta_split(slot, (const uint16_t*)dq, (const uint16_t*)xg, dtheta,
                                                  (float*)(ws + bp.p3_off), BT, D, accumulate,
                                                  ws + bp.blas_off[slot], ttt::grad_gemm_workspace_bytes(), s)
                    : ttt::grad_gemm_dtheta(slot, (const float*)dq, (const float*)xg, dtheta, BT, D, accumulate,
                                            ws + bp.blas_off[slot], ttt::grad_gemm_workspace_bytes(), s);
    return err ? hipErrorUnknown : hipSuccess;
  });
  if (err) return fail(TTT_ERR_HIP, "rocBLAS dtheta GEMM: %s", err);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "dtheta GEMM timing: %s", hipGetErrorString(e));
  return TTT_OK;
}

// The theta operand of the gradient GEMMs: theta itself (fp32 io) or theta stacked three times
// in the workspace (split3), written on s.
int32_t theta_operand(const BwdPlan& bp, const void* theta, int64_t D, char* ws, hipStream_t s, const void** out) {
  if (!bp.split3) {
    *out = theta;
    return TTT_OK;
  }
  uint16_t* dst = (uint16_t*)(ws + bp.th3_off);
  hipError_t e = ttt::stack3_u16((const uint16_t*)theta, dst, 3 * D * D, s);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "theta stacking launch: %s", hipGetErrorString(e));
  *out = dst;
  return TTT_OK;
}

int32_t bwd_direction(const ttt_mlp_config* c, const BwdPlan& bp, const void* xg, const void* thg,
                      const float* alpha, int reverse, const float* dyin, const float* ckpt, const float* z, float* dX,
                      float* dtheta, float* dW1_0, float* dW2_0, int accumulate, float* dalpha, char* ws,
                      hipStream_t s, float* dqkv, const ThetaOverlap& ov = ThetaOverlap(),
                      const ReplayOverlap& ro = ReplayOverlap()) {
  const int64_t D = (int64_t)c->H * c->d, BT = c->B * c->T;
  float* dw_seq = (float*)(ws + bp.dwseq_off);
  ttt::BwdArgs ba{};
  ba.qkv = (const float*)(ws + bp.fwd.qkv_off);
  ba.dy = dyin;
  ba.alpha = alpha;
  ba.ckpt = ckpt;
  ba.segst = (float*)(ws + bp.segst_off);
  ba.wcur = (float*)(ws + bp.fwd.wst_off);
  ba.dstate = (float*)(ws + bp.dstate_off);
  ba.scratch = (float*)(ws + bp.scratch_off);
  ba.dqkv = dqkv;
  ba.dw_seq = dw_seq;
  ba.B = c->B;
  ba.T = c->T;
  ba.H = c->H;
  ba.d = c->d;
  ba.m = c->m;
  ba.b = c->b;
  ba.ckpt_every = kCkptEvery;
  ba.eta = c->eta;
  ba.gscale = c->loss == TTT_LOSS_MEAN ? 2.0f / (float)c->d : 2.0f;
  ba.gelu_tanh = c->gelu == TTT_GELU_TANH;
  ba.reverse = reverse;
  int32_t st = TTT_OK;
  hipError_t e = hipSuccess;
  const bool replay = bwd_f32mfma(c) && c->T > 0;
  if (replay) {
    // the deferred dtheta GEMM first, on this stream: beside the per-window launches below it
    // would hold the CUs that each relaunch needs
    if (ov.side) {
      st = grad_dtheta(bp, ws, 0, bp.split3 ? (const void*)(ws + bp.sp_off) : ov.prev_dqkv, ov.prev_x, dtheta,
                       BT, D, 0, s);
      if (st != TTT_OK) return st;
    }
    // windows of kReplayWindow segments from the last: replay them (one workgroup per chain and
    // segment), then walk them.  With ro.side, where a chain per CU fits beside the walk's
    // workgroups, window w + 1 is replayed on ro.side during the walk of window w, one segment
    // (B H workgroups) per launch, into the other of two slot buffers.
    const int64_t nseg = ((c->T + c->b - 1) / c->b + kCkptEvery - 1) / kCkptEvery;
    const int64_t nwin = (nseg + kReplayWindow - 1) / kReplayWindow;
    const int64_t BHc = (int64_t)c->B * c->H;
    const bool split = bp.split != 0;
    const bool ovl = ro.side && bp.segst2_off && nwin > 1 && ((split ? bp.split : 1) + 1) * BHc <= ro.cus;
    float* const segbuf[2] = {ba.segst, ovl ? (float*)(ws + bp.segst2_off) : ba.segst};
    const int64_t seg_floats = kCkptEvery * (int64_t)ttt::scan_backward_segment_elems(c->d, c->m, c->b);
    auto window = [&](int64_t w, int64_t* lo, int64_t* hi) {
      *hi = nseg - 1 - w * kReplayWindow;
      *lo = std::max<int64_t>(0, *hi - kReplayWindow + 1);
    };
    ttt::ScanArgs ra = scan_args(c, bp.fwd, nullptr, nullptr, nullptr, nullptr, reverse, nullptr, nullptr, nullptr,
                                 nullptr, ws);
    ra.ckpt = const_cast<float*>(ckpt);
    ra.ckpt_every = kCkptEvery;
    ba.replayed = 1;
    // the split walk (four or two workgroups per chain) where they fit co-resident: dQ and dK
    // are added into dqkv, so it starts from zero, and so do the exchange entries and abort flag
    if (split) {
      const int64_t nx = (int64_t)ttt::scan_backward_split_xchg_elems(c->B, c->H, c->d, c->b, bp.split);
      ba.split = bp.split;
      ba.xchg = (uint64_t*)(ws + bp.bxchg_off);
      ba.abort_flag = (uint32_t*)(ba.xchg + nx);
      ba.dqkv_b = bp.split == 4 ? (float*)(ws + bp.dqkvb_off) : nullptr;
      e = ttt::launch_zero_u64(ba.xchg, nx + 1, s);
      if (e == hipSuccess) e = ttt::launch_zero_u64((uint64_t*)dqkv, 3 * BT * D / 2, s);
      if (e == hipSuccess && ba.dqkv_b) e = ttt::launch_zero_u64((uint64_t*)ba.dqkv_b, BT * D, s);
      if (e != hipSuccess) return fail(TTT_ERR_HIP, "clearing launch: %s", hipGetErrorString(e));
    }
    if (ovl) {  // ro.side starts after this stream's work so far (the forward pass, the clearing)
      e = hipEventRecord(ro.start, s);
      if (e == hipSuccess) e = hipStreamWaitEvent(ro.side, ro.start, 0);
      if (e != hipSuccess) return fail(TTT_ERR_HIP, "side stream: %s", hipGetErrorString(e));
    }
    for (int64_t w = 0; w < nwin; ++w) {
      int64_t lo, hi;
      window(w, &lo, &hi);
      const int buf = ovl ? (int)(w & 1) : 0;
      if (w == 0 || !ovl) {  // the whole window on this stream
        ra.seg_slots = segbuf[buf];
        ra.seg_lo = lo;
        ra.seg_count = (int32_t)(hi - lo + 1);
        ra.seg_stride = 0;
        e = timed_launch(TTT_KERNEL_SCAN, s, [&] { return ttt::launch_scan_replay_f32(ra, s); });
        if (e != hipSuccess) return fail(TTT_ERR_HIP, "segment replay launch: %s", hipGetErrorString(e));
      } else {
        e = hipStreamWaitEvent(s, ro.rep[buf], 0);
        if (e != hipSuccess) return fail(TTT_ERR_HIP, "stream wait: %s", hipGetErrorString(e));
      }
      if (ovl && w + 1 < nwin) {  // the next window, beside this one's walk
        int64_t lo1, hi1;
        window(w + 1, &lo1, &hi1);
        const int b1 = (int)((w + 1) & 1);
        if (w >= 1) e = hipStreamWaitEvent(ro.side, ro.walk[b1], 0);  // window w - 1's walk read it
        for (int64_t sg = lo1; sg <= hi1 && e == hipSuccess; ++sg) {
          ttt::ScanArgs r1 = ra;
          r1.seg_slots = segbuf[b1] + (sg - lo1) * seg_floats;
          r1.seg_lo = sg;
          r1.seg_count = 1;
          r1.seg_stride = (int32_t)(hi1 - lo1 + 1);
          e = timed_launch(TTT_KERNEL_SCAN, ro.side, [&] { return ttt::launch_scan_replay_f32(r1, ro.side); });
        }
        if (e == hipSuccess) e = hipEventRecord(ro.rep[b1], ro.side);
        if (e != hipSuccess) return fail(TTT_ERR_HIP, "segment replay (side stream): %s", hipGetErrorString(e));
      }
      ba.segst = segbuf[buf];
      ba.seg_lo = lo;
      ba.seg_hi = hi;
      ba.seg_count = (int32_t)(hi - lo + 1);
      ba.first = hi == nseg - 1;
      e = timed_launch(TTT_KERNEL_BACKWARD, s, [&] {
        return split ? ttt::launch_scan_backward_split(ba, s) : ttt::launch_scan_backward(ba, s);
      });
      if (e == hipSuccess && ovl) e = hipEventRecord(ro.walk[buf], s);
      if (e != hipSuccess) return fail(TTT_ERR_HIP, "backward scan launch: %s", hipGetErrorString(e));
    }
    if (ba.dqkv_b && !bp.split3) {  // the four-part walk's parts 2 and 3 (else added in the split)
      e = ttt::launch_add_dqk(dqkv, ba.dqkv_b, BT, (int)D, s);
      if (e != hipSuccess) return fail(TTT_ERR_HIP, "dQ|dK sum launch: %s", hipGetErrorString(e));
    }
  } else {
    e = ov.side ? hipEventRecord(ov.ev_ready, s) : hipSuccess;
    if (e != hipSuccess) return fail(TTT_ERR_HIP, "side stream: %s", hipGetErrorString(e));
    e = timed_launch(TTT_KERNEL_BACKWARD, s, [&] { return ttt::launch_scan_backward(ba, s); });
    if (e != hipSuccess) return fail(TTT_ERR_HIP, "backward scan launch: %s", hipGetErrorString(e));
  }
  if (ov.side && !replay) {
    e = hipStreamWaitEvent(ov.side, ov.ev_ready, 0);
    if (e != hipSuccess) return fail(TTT_ERR_HIP, "side stream wait: %s", hipGetErrorString(e));
    st = grad_dtheta(bp, ws, 1, bp.split3 ? (const void*)(ws + bp.sp_off) : ov.prev_dqkv, ov.prev_x, dtheta, BT,
                     D, 0, ov.side);
    if (st != TTT_OK) return st;
    e = hipEventRecord(ov.ev_done, ov.side);
    if (e != hipSuccess) return fail(TTT_ERR_HIP, "side stream event: %s", hipGetErrorString(e));
  }
  e = ttt::launch_dalpha(dyin, z, alpha, (float*)(ws + bp.dal_off), dalpha, BT, (int)D, s);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "dalpha launch: %s", hipGetErrorString(e));
  // the deferred GEMM on the side stream has read the split (or, with fp32 io, adds to dtheta
  // before this direction's GEMM does) once ev_done is reached
  if (ov.side && !replay) {
    e = hipStreamWaitEvent(s, ov.ev_done, 0);
    if (e != hipSuccess) return fail(TTT_ERR_HIP, "stream wait: %s", hipGetErrorString(e));
  }
  const void* dq = dqkv;
  if (bp.split3) {
    uint16_t* sp = (uint16_t*)(ws + bp.sp_off);
    // with the four-part walk, its second dQ|dK buffer is added in first (nothing else reads the
    // fp32 dQ|dK|dV after the walk when the GEMMs take the split)
    const float* dqkv2 = ba.dqkv_b;
    e = timed_launch(TTT_KERNEL_GRAD_GEMM, s,
                     [&] { return ttt::split_bf16x3(dqkv, dqkv2, 2 * D, sp, BT, 3 * D, s); });
    if (e != hipSuccess) return fail(TTT_ERR_HIP, "dQ|dK|dV split launch: %s", hipGetErrorString(e));
    dq = sp;
  }
  st = grad_dx(bp, ws, 0, dq, thg, dyin, dX, BT, D, s);
  if (st != TTT_OK) return st;
  if (!ov.skip_theta) {
    st = grad_dtheta(bp, ws, 0, dq, xg, dtheta, BT, D, accumulate, s);
    if (st != TTT_OK) return st;
  }
  e = ttt::launch_sum_state(dw_seq, dW1_0, dW2_0, c->B, c->H, c->d, c->m, accumulate, s);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "state gradient launch: %s", hipGetErrorString(e));
  return TTT_OK;
}

// ---------------------------------------------------------------------------
// hybrid block: segment-local attention feeding the bidirectional TTT layer
// ---------------------------------------------------------------------------
int32_t check_attention(const ttt_mlp_config* c, int64_t seg_len) {
  int32_t st = check_config(c);
  if (st != TTT_OK) return st;
  if (seg_len < 1) return fail(TTT_ERR_INVALID_ARG, "seg_len must be >= 1 (got %lld)", (long long)seg_len);
  if (c->io_dtype != TTT_BF16 || !ttt::segment_attention_supported(c->d) || ((int64_t)c->H * c->d) % 8 != 0)
    return fail(TTT_ERR_UNSUPPORTED, "segment attention needs bf16 io and head width 64 (got d=%d io=%d)", c->d,
                c->io_dtype);
  return TTT_OK;
}

struct HybridPlan {
  size_t qkv_off, o_off, u_off, ttt_off, ttt_bytes, total;
};

int32_t make_hybrid_plan(const ttt_mlp_config* c, int64_t seg_len, HybridPlan* p) {
  int32_t st = check_attention(c, seg_len);
  if (st != TTT_OK) return st;
  Plan tp;
  st = make_plan(c, &tp);
  if (st != TTT_OK) return st;
  const size_t BTD = (size_t)c->B * c->T * c->H * c->d;
  p->qkv_off = 0;
  p->o_off = p->qkv_off + align_up(3 * BTD * 2);
  p->u_off = p->o_off + align_up(BTD * 2);
  p->ttt_off = p->u_off + align_up(BTD * 2);
  p->ttt_bytes = tp.total;
  p->total = p->ttt_off + align_up(tp.total);
  return TTT_OK;
}

// row-major bf16 GEMM out[B*T, N] = X theta^T (+ resid), theta [N, D]
hipError_t launch_rowmajor_gemm(const ttt_mlp_config* c, const void* X, const void* theta, int N, const void* resid,
                                void* out, hipStream_t s) {
  ttt::ProjArgs pa{};
  pa.X = X;
  pa.theta = theta;
  pa.out = out;
  pa.B = c->B;
  pa.T = c->T;
  pa.H = c->H;
  pa.d = c->d;
  pa.bf16 = 1;
  pa.tt0 = 0;
  pa.tt1 = c->T;
  pa.n_out = N;
  pa.resid = resid;
  return timed_launch(TTT_KERNEL_PROJECT, s, [&] { return ttt::launch_project_mfma(pa, 2, s); });
}

// ---------------------------------------------------------------------------
// the workspace of ttt_mlp_bidir_noalloc: a device array of the library
// ---------------------------------------------------------------------------
// Every GPU the library runs on holds its own copy until the process ends.  It
// is sized for one 3-second segment of the video model at the layer's shape:
// 14,400 tokens, 48 heads of width 64, b = 16 on the MFMA path (the projected
// token blocks, 298.6 MB, and the state handed from one scan launch to the next,
// 6.3 MB).
constexpr size_t kStaticWorkspaceBytes = TTT_STATIC_WORKSPACE_BYTES;

std::mutex g_static_mu;
std::map<int, char*> g_static_ws;  // device -> device address of the array

}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

namespace {

// The array's device address on the current device (looked up once per device,
// with that device current; the host-side name is not a device address), and
// the side stream and events that the MFMA path may need, created here once so
// that no later call creates any.
int32_t static_workspace(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_static_mu);
  auto it = g_static_ws.find(dev);
  if (it != g_static_ws.end()) {
    *out = it->second;
    return TTT_OK;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p)
    return fail(TTT_ERR_HIP, "hipGetSymbolAddress of the static workspace: %s", hipGetErrorString(e));
  {
    std::lock_guard<std::mutex> lk2(g_side_mu);
    Side* sd = nullptr;
    e = side_for_device(&sd, 2 + 2 * (size_t)kMaxChunks * 2);
    if (e != hipSuccess) return fail(TTT_ERR_HIP, "side stream: %s", hipGetErrorString(e));
  }
  g_static_ws[dev] = (char*)p;
  *out = (char*)p;
  return TTT_OK;
}

}  // namespace

extern "C" {

int32_t ttt_mlp_version(void) { return (1 << 16) | 0; }

const char* ttt_mlp_status_string(int32_t status) {
  switch (status) {
    case TTT_OK: return "ok";
    case TTT_ERR_INVALID_ARG: return "invalid argument";
    case TTT_ERR_UNSUPPORTED: return "unsupported configuration";
    case TTT_ERR_WORKSPACE: return "workspace missing or too small";
    case TTT_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* ttt_mlp_last_error(void) { return g_last_error.c_str(); }

int32_t ttt_mlp_workspace_size(const ttt_mlp_config* cfg, int32_t bidir, size_t* bytes) {
  if (!bytes) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  if (bidir != 0 && bidir != 1) return fail(TTT_ERR_INVALID_ARG, "bidir must be 0 or 1");
  Plan pl;
  int32_t st = make_plan(cfg, &pl);
  if (st != TTT_OK) return st;
  *bytes = pl.total;
  return ok();
}

int32_t ttt_mlp_select_algo(const ttt_mlp_config* cfg, int32_t* algo) {
  if (!algo) return fail(TTT_ERR_INVALID_ARG, "algo is NULL");
  Plan pl;
  int32_t st = make_plan(cfg, &pl);
  if (st != TTT_OK) return st;
  *algo = pl.algo;
  return ok();
}

int32_t ttt_mlp_forward(const ttt_mlp_config* cfg, const void* X, const void* theta_qkv,
                        const float* W1_0, const float* W2_0, const float* alpha, int32_t reverse,
                        void* Y, float* Z, float* W1_T, float* W2_T, void* workspace,
                        size_t workspace_bytes, void* stream) {
  Plan pl;
  int32_t st = make_plan(cfg, &pl);
  if (st != TTT_OK) return st;
  const bool no_tokens = cfg->T == 0;  // X and Y may then be NULL
  const bool lin = is_linear(cfg);     // W2_0 and W2_T unused
  if ((!no_tokens && (!X || !Y)) || !theta_qkv || !W1_0 || (!lin && !W2_0) || !alpha)
    return fail(TTT_ERR_INVALID_ARG, "a required pointer (X, theta_qkv, W1_0, W2_0, alpha, Y) is NULL");
  if (lin) W2_T = nullptr;
  if (reverse != 0 && reverse != 1) return fail(TTT_ERR_INVALID_ARG, "reverse must be 0 or 1");
  if (!workspace || workspace_bytes < pl.total)
    return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                pl.total);
  const size_t D = (size_t)cfg->H * cfg->d, BTD = (size_t)cfg->B * cfg->T * D;
  const size_t st_bytes = (size_t)cfg->B * cfg->H * cfg->d * cfg->m * sizeof(float);
  const size_t w0_bytes = (size_t)cfg->H * cfg->d * cfg->m * 4;
  const Buf outs[] = {{Y, BTD * pl.io_elem, "Y"}, {Z, BTD * 4, "Z"}, {W1_T, st_bytes, "W1_T"},
                      {W2_T, st_bytes, "W2_T"}, {workspace, pl.total, "workspace"}};
  const Buf ins[] = {{X, BTD * pl.io_elem, "X"}, {theta_qkv, 3 * D * D * pl.io_elem, "theta_qkv"},
                     {W1_0, w0_bytes, "W1_0"}, {lin ? nullptr : W2_0, w0_bytes, "W2_0"}, {alpha, D * 4, "alpha"}};
  st = check_no_overlap(outs, 5, ins, 5);
  if (st != TTT_OK) return st;
  if (pl.algo == TTT_ALGO_MFMA) {
    const Direction dir{X, alpha, reverse, Y, Z, W1_T, W2_T};
    st = run_mfma(cfg, pl, &dir, 1, theta_qkv, W1_0, W2_0, (char*)workspace, (hipStream_t)stream);
  } else {
    st = run_direction(cfg, pl, X, theta_qkv, W1_0, W2_0, alpha, reverse, Y, Z, W1_T, W2_T, (char*)workspace,
                       (hipStream_t)stream);
  }
  return st == TTT_OK ? ok() : st;
}

int32_t ttt_mlp_bidir(const ttt_mlp_config* cfg, const void* X, const void* theta_qkv,
                      const float* W1_0, const float* W2_0, const float* alpha_f,
                      const float* alpha_b, void* Y, float* Z_f, float* Z_b, float* W1_Tf,
                      float* W2_Tf, float* W1_Tb, float* W2_Tb, void* workspace,
                      size_t workspace_bytes, void* stream) {
  Plan pl;
  int32_t st = make_plan(cfg, &pl);
  if (st != TTT_OK) return st;
  const bool no_tokens = cfg->T == 0;  // X and Y may then be NULL
  const bool lin = is_linear(cfg);     // W2_0 and the W2 outputs unused
  if ((!no_tokens && (!X || !Y)) || !theta_qkv || !W1_0 || (!lin && !W2_0) || !alpha_f || !alpha_b)
    return fail(TTT_ERR_INVALID_ARG,
                "a required pointer (X, theta_qkv, W1_0, W2_0, alpha_f, alpha_b, Y) is NULL");
  if (lin) W2_Tf = W2_Tb = nullptr;
  if (!workspace || workspace_bytes < pl.total)
    return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                pl.total);
  const size_t D = (size_t)cfg->H * cfg->d, BTD = (size_t)cfg->B * cfg->T * D;
  const size_t st_bytes = (size_t)cfg->B * cfg->H * cfg->d * cfg->m * sizeof(float);
  const Buf outs[] = {{Y, BTD * pl.io_elem, "Y"},      {Z_f, BTD * 4, "Z_f"},
                      {Z_b, BTD * 4, "Z_b"},           {W1_Tf, st_bytes, "W1_Tf"},
                      {W2_Tf, st_bytes, "W2_Tf"},      {W1_Tb, st_bytes, "W1_Tb"},
                      {W2_Tb, st_bytes, "W2_Tb"},      {workspace, pl.total, "workspace"}};
  const size_t w0_bytes = (size_t)cfg->H * cfg->d * cfg->m * 4;
  const Buf ins[] = {{X, BTD * pl.io_elem, "X"}, {theta_qkv, 3 * D * D * pl.io_elem, "theta_qkv"},
                     {W1_0, w0_bytes, "W1_0"}, {lin ? nullptr : W2_0, w0_bytes, "W2_0"}, {alpha_f, D * 4, "alpha_f"},
                     {alpha_b, D * 4, "alpha_b"}};
  st = check_no_overlap(outs, 8, ins, 6);
  if (st != TTT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (pl.algo == TTT_ALGO_MFMA) {
    // forward pass into Y, then the reversed pass over X' = Y, written back in place
    const Direction dirs[2] = {{X, alpha_f, 0, Y, Z_f, W1_Tf, W2_Tf}, {Y, alpha_b, 1, Y, Z_b, W1_Tb, W2_Tb}};
    st = run_mfma(cfg, pl, dirs, 2, theta_qkv, W1_0, W2_0, (char*)workspace, s);
    return st == TTT_OK ? ok() : st;
  }
  // forward pass: X' lands in Y
  st = run_direction(cfg, pl, X, theta_qkv, W1_0, W2_0, alpha_f, 0, Y, Z_f, W1_Tf, W2_Tf, (char*)workspace, s);
  if (st != TTT_OK) return st;
  // reversed pass over X' (read from Y, gated output written back in place)
  st = run_direction(cfg, pl, Y, theta_qkv, W1_0, W2_0, alpha_b, 1, Y, Z_b, W1_Tb, W2_Tb, (char*)workspace, s,
                     false);
  return st == TTT_OK ? ok() : st;
}

int32_t ttt_mlp_coop_aborted(const ttt_mlp_config* cfg, int32_t bidir, const void* workspace, size_t workspace_bytes,
                             void* stream, int32_t* aborted) {
  if (!aborted) return fail(TTT_ERR_INVALID_ARG, "aborted is NULL");
  if (bidir != 0 && bidir != 1) return fail(TTT_ERR_INVALID_ARG, "bidir must be 0 or 1");
  Plan pl;
  int32_t st = make_plan(cfg, &pl);
  if (st != TTT_OK) return st;
  if (pl.algo != TTT_ALGO_COOP) {  // only the cooperative scan can stop early
    *aborted = 0;
    return ok();
  }
  if (!workspace || workspace_bytes < pl.total)
    return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                pl.total);
  const char* flag = (const char*)workspace + pl.wst_off + ttt::scan_coop_xchg_bytes(cfg->B, cfg->H);
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, flag, sizeof v, hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "reading the abort flag: %s", hipGetErrorString(e));
  *aborted = v != 0;
  return ok();
}

int32_t ttt_mlp_bidir_noalloc(const ttt_mlp_config* cfg, const void* X, const void* theta_qkv,
                              const float* W1_0, const float* W2_0, const float* alpha_f,
                              const float* alpha_b, void* Y, float* Z_f, float* Z_b, float* W1_Tf,
                              float* W2_Tf, float* W1_Tb, float* W2_Tb, void* stream) {
  Plan pl;
  int32_t st = make_plan(cfg, &pl);
  if (st != TTT_OK) return st;
  if (pl.total > kStaticWorkspaceBytes)
    return fail(TTT_ERR_WORKSPACE,
                "the call needs %zu bytes of workspace; the library's static workspace holds %zu (use "
                "ttt_mlp_bidir with a workspace of its size)",
                pl.total, kStaticWorkspaceBytes);
  char* ws = nullptr;
  st = static_workspace(&ws);
  if (st != TTT_OK) return st;
  g_untimed = true;
  st = ttt_mlp_bidir(cfg, X, theta_qkv, W1_0, W2_0, alpha_f, alpha_b, Y, Z_f, Z_b, W1_Tf, W2_Tf, W1_Tb, W2_Tb, ws,
                     kStaticWorkspaceBytes, stream);
  g_untimed = false;
  return st;
}

int32_t ttt_mlp_backward_workspace_size(const ttt_mlp_config* cfg, int32_t bidir, size_t* bytes) {
  if (!bytes) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  BwdPlan bp;
  int32_t st = make_bwd_plan(cfg, bidir != 0, &bp);
  if (st != TTT_OK) return st;
  *bytes = bp.total;
  return ok();
}

int32_t ttt_mlp_backward(const ttt_mlp_config* cfg, const void* X, const void* theta_qkv, const float* W1_0,
                         const float* W2_0, const float* alpha, int32_t reverse, const float* dY, float* dX,
                         float* dtheta, float* dW1_0, float* dW2_0, float* dalpha, void* workspace,
                         size_t workspace_bytes, void* stream) {
  BwdPlan bp;
  int32_t st = make_bwd_plan(cfg, 0, &bp);
  if (st != TTT_OK) return st;
  const bool no_tokens = cfg->T == 0;
  if ((!no_tokens && (!X || !dY || !dX)) || !theta_qkv || !W1_0 || !W2_0 || !alpha || !dtheta || !dW1_0 ||
      !dW2_0 || !dalpha)
    return fail(TTT_ERR_INVALID_ARG, "a required pointer (X, theta_qkv, W1_0, W2_0, alpha, dY, dX, dtheta, dW1_0, "
                                     "dW2_0, dalpha) is NULL");
  if (!workspace || workspace_bytes < bp.total)
    return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                bp.total);
  const size_t io = bp.fwd.io_elem;
  const size_t D = (size_t)cfg->H * cfg->d, BTD = (size_t)cfg->B * cfg->T * D;
  const size_t w0 = (size_t)cfg->H * cfg->d * cfg->m * 4;
  const Buf outs[] = {{dX, BTD * 4, "dX"},         {dtheta, 3 * D * D * 4, "dtheta"}, {dW1_0, w0, "dW1_0"},
                      {dW2_0, w0, "dW2_0"},        {dalpha, D * 4, "dalpha"},        {workspace, bp.total, "workspace"}};
  const Buf ins[] = {{X, BTD * io, "X"},   {theta_qkv, 3 * D * D * io, "theta_qkv"}, {W1_0, w0, "W1_0"},
                     {W2_0, w0, "W2_0"}, {alpha, D * 4, "alpha"},                 {dY, BTD * 4, "dY"}};
  st = check_no_overlap(outs, 6, ins, 6);
  if (st != TTT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* z = (float*)(ws + bp.z_off[0]);
  float* ck = (float*)(ws + bp.ckpt_off[0]);
  st = bwd_forward(cfg, bp, X, theta_qkv, W1_0, W2_0, alpha, reverse != 0, ws + bp.y_off, z, ck, ws, s);
  if (st != TTT_OK) return st;
  const int64_t D_ = (int64_t)cfg->H * cfg->d;
  const void* thg = nullptr;
  st = theta_operand(bp, theta_qkv, D_, ws, s, &thg);
  if (st != TTT_OK) return st;
  std::lock_guard<std::mutex> lk(g_side_mu);
  Side* sd = nullptr;
  hipError_t e = side_for_device(&sd, 7);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "side stream: %s", hipGetErrorString(e));
  st = bwd_direction(cfg, bp, X, thg, alpha, reverse != 0, dY, ck, z, dX, dtheta, dW1_0, dW2_0, 0, dalpha, ws, s,
                     (float*)(ws + bp.dqkv_off), ThetaOverlap(), replay_overlap(*sd));
  return st == TTT_OK ? ok() : st;
}

int32_t ttt_mlp_bidir_backward(const ttt_mlp_config* cfg, const void* X, const void* theta_qkv, const float* W1_0,
                               const float* W2_0, const float* alpha_f, const float* alpha_b, const float* dY,
                               float* dX, float* dtheta, float* dW1_0, float* dW2_0, float* dalpha_f,
                               float* dalpha_b, void* workspace, size_t workspace_bytes, void* stream) {
  BwdPlan bp;
  int32_t st = make_bwd_plan(cfg, 1, &bp);
  if (st != TTT_OK) return st;
  const bool no_tokens = cfg->T == 0;
  if ((!no_tokens && (!X || !dY || !dX)) || !theta_qkv || !W1_0 || !W2_0 || !alpha_f || !alpha_b || !dtheta ||
      !dW1_0 || !dW2_0 || !dalpha_f || !dalpha_b)
    return fail(TTT_ERR_INVALID_ARG, "a required pointer (X, theta_qkv, W1_0, W2_0, alpha_f, alpha_b, dY, dX, "
                                     "dtheta, dW1_0, dW2_0, dalpha_f, dalpha_b) is NULL");
  if (!workspace || workspace_bytes < bp.total)
    return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                bp.total);
  const size_t io = bp.fwd.io_elem;
  const size_t D = (size_t)cfg->H * cfg->d, BTD = (size_t)cfg->B * cfg->T * D;
  const size_t w0 = (size_t)cfg->H * cfg->d * cfg->m * 4;
  const Buf outs[] = {{dX, BTD * 4, "dX"},           {dtheta, 3 * D * D * 4, "dtheta"}, {dW1_0, w0, "dW1_0"},
                      {dW2_0, w0, "dW2_0"},          {dalpha_f, D * 4, "dalpha_f"},    {dalpha_b, D * 4, "dalpha_b"},
                      {workspace, bp.total, "workspace"}};
  const Buf ins[] = {{X, BTD * io, "X"},         {theta_qkv, 3 * D * D * io, "theta_qkv"}, {W1_0, w0, "W1_0"},
                     {W2_0, w0, "W2_0"},       {alpha_f, D * 4, "alpha_f"},            {alpha_b, D * 4, "alpha_b"},
                     {dY, BTD * 4, "dY"}};
  st = check_no_overlap(outs, 7, ins, 7);
  if (st != TTT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  void* xp = ws + bp.xp_off;  // X', the forward pass's output (io_dtype, as the forward call keeps it)
  float* dxp = (float*)(ws + bp.dxp_off);
  float* zf = (float*)(ws + bp.z_off[0]);
  float* zb = (float*)(ws + bp.z_off[1]);
  float* ckf = (float*)(ws + bp.ckpt_off[0]);
  float* ckb = (float*)(ws + bp.ckpt_off[1]);
  // the two forward passes, keeping X', Z, the checkpoints and both directions' Q/K/V (the
  // reversed pass's in their own buffer: bpb)
  BwdPlan bpb = bp;
  bpb.fwd.qkv_off = bp.qkv2_off;
  st = bwd_forward(cfg, bp, X, theta_qkv, W1_0, W2_0, alpha_f, 0, xp, zf, ckf, ws, s);
  if (st == TTT_OK)
    st = bwd_forward(cfg, bpb, xp, theta_qkv, W1_0, W2_0, alpha_b, 1, ws + bp.y_off, zb, ckb, ws, s);
  // the theta operand of the gradient GEMMs (X and X' serve as they are)
  const int64_t D_ = (int64_t)cfg->H * cfg->d;
  const void* thg = nullptr;
  if (st == TTT_OK) st = theta_operand(bp, theta_qkv, D_, ws, s, &thg);
  // the reversed pass's backward (its Q/K/V, of X', are in the workspace): dX' = dY + ...; its
  // dtheta GEMM is deferred, and the forward pass's dtheta GEMM adds to it afterwards: with the
  // replayed windows it runs on `s` before the forward pass's backward scan, otherwise on the side
  // stream beside that scan (which takes one CU per head)
  std::lock_guard<std::mutex> lk(g_side_mu);
  Side* sd = nullptr;
  hipError_t e = side_for_device(&sd, 7);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "side stream: %s", hipGetErrorString(e));
  const ReplayOverlap ro = replay_overlap(*sd);
  ThetaOverlap ov_b, ov_f;
  ov_b.skip_theta = true;
  ov_f.side = sd->stream;
  ov_f.ev_ready = sd->events[0];
  ov_f.ev_done = sd->events[1];
  ov_f.prev_dqkv = (const float*)(ws + bp.dqkv2_off);
  ov_f.prev_x = xp;
  if (st == TTT_OK)
    st = bwd_direction(cfg, bpb, xp, thg, alpha_b, 1, dY, ckb, zb, dxp, dtheta, dW1_0, dW2_0, 0, dalpha_b, ws, s,
                       (float*)(ws + bp.dqkv2_off), ov_b, ro);
  // the forward pass's backward, with dY = dX'
  if (st == TTT_OK)
    st = bwd_direction(cfg, bp, X, thg, alpha_f, 0, dxp, ckf, zf, dX, dtheta, dW1_0, dW2_0, 1, dalpha_f, ws, s,
                       (float*)(ws + bp.dqkv_off), ov_f, ro);
  return st == TTT_OK ? ok() : st;
}

int32_t ttt_segment_attention(const ttt_mlp_config* cfg, int64_t seg_len, const void* QKV, void* O, void* stream) {
  int32_t st = check_attention(cfg, seg_len);
  if (st != TTT_OK) return st;
  if (cfg->T > 0 && (!QKV || !O)) return fail(TTT_ERR_INVALID_ARG, "QKV and O are required");
  const size_t BTD = (size_t)cfg->B * cfg->T * cfg->H * cfg->d;
  const Buf outs[] = {{O, BTD * 2, "O"}};
  const Buf ins[] = {{QKV, 3 * BTD * 2, "QKV"}};
  st = check_no_overlap(outs, 1, ins, 1);
  if (st != TTT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = timed_launch(TTT_KERNEL_ATTENTION, s, [&] {
    return ttt::launch_segment_attention((const uint16_t*)QKV, (uint16_t*)O, cfg->B, cfg->T, cfg->H, seg_len, s);
  });
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
  return ok();
}

int32_t ttt_hybrid_block_workspace_size(const ttt_mlp_config* cfg, int64_t seg_len, size_t* bytes) {
  if (!bytes) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  HybridPlan hp;
  int32_t st = make_hybrid_plan(cfg, seg_len, &hp);
  if (st != TTT_OK) return st;
  *bytes = hp.total;
  return ok();
}

int32_t ttt_hybrid_block(const ttt_mlp_config* cfg, int64_t seg_len, const void* X, const void* theta_attn,
                         const void* theta_out, const void* theta_qkv, const float* W1_0, const float* W2_0,
                         const float* alpha_f, const float* alpha_b, void* Y, void* workspace, size_t workspace_bytes,
                         void* stream) {
  HybridPlan hp;
  int32_t st = make_hybrid_plan(cfg, seg_len, &hp);
  if (st != TTT_OK) return st;
  const bool lin = is_linear(cfg);
  if ((cfg->T > 0 && (!X || !Y)) || !theta_attn || !theta_out || !theta_qkv || !W1_0 || (!lin && !W2_0) ||
      !alpha_f || !alpha_b)
    return fail(TTT_ERR_INVALID_ARG, "a required pointer (X, theta_attn, theta_out, theta_qkv, W1_0, W2_0, alpha_f, "
                                     "alpha_b, Y) is NULL");
  if (!workspace || workspace_bytes < hp.total)
    return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                hp.total);
  const size_t D = (size_t)cfg->H * cfg->d, BTD = (size_t)cfg->B * cfg->T * D;
  const size_t w0 = (size_t)cfg->H * cfg->d * cfg->m * 4;
  const Buf outs[] = {{Y, BTD * 2, "Y"}, {workspace, hp.total, "workspace"}};
  const Buf ins[] = {{X, BTD * 2, "X"},           {theta_attn, 3 * D * D * 2, "theta_attn"},
                     {theta_out, D * D * 2, "theta_out"}, {theta_qkv, 3 * D * D * 2, "theta_qkv"},
                     {W1_0, w0, "W1_0"},          {lin ? nullptr : W2_0, w0, "W2_0"},
                     {alpha_f, D * 4, "alpha_f"}, {alpha_b, D * 4, "alpha_b"}};
  st = check_no_overlap(outs, 2, ins, 8);
  if (st != TTT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  void* qkv = ws + hp.qkv_off;
  void* o = ws + hp.o_off;
  void* u = ws + hp.u_off;
  if (cfg->T > 0) {
    hipError_t e = launch_rowmajor_gemm(cfg, X, theta_attn, (int)(3 * D), nullptr, qkv, s);  // Q | K | V
    if (e != hipSuccess) return fail(TTT_ERR_HIP, "attention projection launch: %s", hipGetErrorString(e));
    e = timed_launch(TTT_KERNEL_ATTENTION, s, [&] {
      return ttt::launch_segment_attention((const uint16_t*)qkv, (uint16_t*)o, cfg->B, cfg->T, cfg->H, seg_len, s);
    });
    if (e != hipSuccess) return fail(TTT_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
    e = launch_rowmajor_gemm(cfg, o, theta_out, (int)D, X, u, s);  // U = X + O theta_out^T
    if (e != hipSuccess) return fail(TTT_ERR_HIP, "output projection launch: %s", hipGetErrorString(e));
  }
  st = ttt_mlp_bidir(cfg, cfg->T > 0 ? u : nullptr, theta_qkv, W1_0, W2_0, alpha_f, alpha_b, Y, nullptr, nullptr,
                     nullptr, nullptr, nullptr, nullptr, ws + hp.ttt_off, hp.ttt_bytes, stream);
  return st == TTT_OK ? ok() : st;
}

int32_t ttt_mlp_project(const ttt_mlp_config* cfg, const void* X, const void* theta_qkv, float* QKV,
                        void* stream) {
  int32_t st = check_config(cfg);
  if (st != TTT_OK) return st;
  if ((cfg->T > 0 && (!X || !QKV)) || !theta_qkv)
    return fail(TTT_ERR_INVALID_ARG, "X, theta_qkv and QKV are required");
  const size_t esz = cfg->io_dtype == TTT_BF16 ? 2 : 4;
  const size_t D = (size_t)cfg->H * cfg->d, BTD = (size_t)cfg->B * cfg->T * D;
  const Buf outs[] = {{QKV, 3 * BTD * 4, "QKV"}};
  const Buf ins[] = {{X, BTD * esz, "X"}, {theta_qkv, 3 * D * D * esz, "theta_qkv"}};
  st = check_no_overlap(outs, 1, ins, 2);
  if (st != TTT_OK) return st;
  ttt::ProjArgs pa{};
  pa.X = X;
  pa.theta = theta_qkv;
  pa.out = QKV;
  pa.B = cfg->B;
  pa.T = cfg->T;
  pa.H = cfg->H;
  pa.d = cfg->d;
  pa.bf16 = cfg->io_dtype == TTT_BF16;
  pa.reverse = 0;
  pa.tt0 = 0;
  pa.tt1 = cfg->T;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = timed_launch(TTT_KERNEL_PROJECT, s, [&] { return launch_projection(pa, 0, s); });
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "projection launch: %s", hipGetErrorString(e));
  return ok();
}

int32_t ttt_mlp_set_kernel_timing(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing_on = enable != 0;
  return ok();
}

int32_t ttt_mlp_kernel_timing(int32_t kind, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind >= kTimingKinds) return fail(TTT_ERR_INVALID_ARG, "unknown kernel kind %d", kind);
  if (!total_ms || !launches) return fail(TTT_ERR_INVALID_ARG, "total_ms and launches are required");
  std::lock_guard<std::mutex> lk(g_timing_mu);
  hipError_t e = drain_timing_locked();
  *total_ms = g_timing_ms[kind];
  *launches = g_timing_n[kind];
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "timing events: %s", hipGetErrorString(e));
  return ok();
}

int32_t ttt_mlp_reset_kernel_timing(void) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  hipError_t e = drain_timing_locked();
  for (int k = 0; k < kTimingKinds; ++k) {
    g_timing_ms[k] = 0;
    g_timing_n[k] = 0;
  }
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "timing events: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
