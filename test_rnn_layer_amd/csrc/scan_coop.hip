// Per-token scan (b = 1) for inner states too large for one compute unit.
//
// The method is the TTT-MLP layer of "One-Minute Video Generation with
// Test-Time Training" (paper-notes page, key designs, "TTT-MLP layer"): per
// head the hidden state is a two-layer MLP W1 (d x m), W2 (m x d), one
// gradient step per token on l = c/2 ||GELU(k W1) W2 - v||^2 (c = 2/d for the
// mean reading, 2 for the literal sum), read-out z_t = GELU(q_t W1_t) W2_t with
// the state after token t's own step, gate y = x + tanh(alpha) z.  The same
// page's "on-chip tensor parallel" item shards the state of one head over
// several processors and all-reduces between them; this kernel does that on
// gfx950 with workgroups of one cooperative launch.
//
// At d = 128, m = 512 a head's fp32 state is 512 KB, more than one CU's LDS
// and, with working registers, its VGPR file.  The state is split by hidden
// unit over NCU = 8 workgroups (one per CU), 64 units each, held entirely in
// VGPRs; wave w (of 8) owns 8 units of them whole:
//   W1 columns of its units (128 x 8): lane l holds rows 16 (l mod 8) .. +15 of
//     unit 8w + l/8, so the 8 lanes of a unit sum its pre-activation by DPP;
//   W2 rows of its units (8 x 128): lane l holds W2[8w .. 8w+7][l, l+64].
// Per token every workgroup holds the full q, k, v of its head.  a = k W1 and
// aq = q W1 are local to a unit, and so to a wave, so only the contractions over
// hidden units, yhat = GELU(a) W2 and z = GELU(aq) W2, need partial sums: over
// the waves through LDS, then from all NCU workgroups: one exchange per token.
// G2 W2^T of a unit comes out of its wave's own reduction over features, in the
// lanes that own the unit, so G1 and the W1 update stay in registers.
//
// Read-out.  Iteration t runs token t's step with the state W_{t-1}, which is
// also token t-1's post-update state, so token t-1's read-out is computed in
// the same passes: aq_{t-1} = q_{t-1} W1_{t-1} comes out of the previous
// iteration's W1 pass, z_{t-1} = GELU(aq_{t-1}) W2_{t-1} out of this one's
// first W2 pass, and its partials travel with yhat_t's.
//
// Deferred W1 update.  Token t's W1 step W1_t = W1_{t-1} + k_t^T (-eta G1_t) is
// rank one, so a_{t+1} = k_{t+1} W1_t = k_{t+1} W1_{t-1} + (k_{t+1} . k_t)(-eta G1_t),
// and likewise aq_t.  The W1 pass of token t (the update with k_{t-1} and G1_{t-1},
// then the partials of k_{t+1} W1_{t-1}, q_t W1_{t-1} and of the two dot
// products) runs while token t's partials are in flight between the
// workgroups; once G1_t is known only the rank-one correction of each unit's
// pre-activation remains on the token's critical path.
//
// Exchange.  Each value is published as one 64-bit relaxed device-scope
// atomic store (token tag in the high word, fp32 bits in the low word) into a
// slot of the workspace, double-buffered by token parity; readers poll their
// entries with relaxed device-scope atomic loads until the tag matches.  A
// slot is rewritten two tokens later, only after every workgroup of the head
// has consumed it (a workgroup publishes token t+1 only after it has read all
// of token t's partials, which were published after every wave of each
// workgroup had finished with token t-1).  Polls are bounded: a workgroup that
// waits longer than the spin limit raises an abort flag that every poll
// checks; all workgroups then fill the rest of their Y (and Z) slices with NaN
// and exit.  The launch is cooperative, so all workgroups are co-resident.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"
#include "phase_marks.h"

TTT_MARKS_BUFFER(g_marks_scan_coop);

namespace ttt {
namespace {

constexpr int CD = 128;               // head width d
constexpr int CM = 512;               // hidden width m
constexpr int NCU = 8;                // cooperating workgroups per head
constexpr int UNITS = CM / NCU;       // hidden units per workgroup
constexpr int NW = 8;                 // waves per workgroup (two per SIMD)
constexpr int NT = 64 * NW;           // threads per workgroup
constexpr int PW = CD / NW;           // rows of W1 per wave
constexpr int UW = UNITS / NW;        // units of W2 per wave
constexpr int NVAL = 2 * CD;          // exchanged values per workgroup and token: yhat, z partials
constexpr uint32_t SPIN_MAX = 1u << 20;
static_assert(UNITS == 64 && UW == 8 && PW == 16 && CD == 128 && NT == 4 * CD, "lane mapping assumes these sizes");

// Phi(a) = (1 + erf(a / sqrt 2)) / 2, with erf of x = |a| / sqrt 2 >= 0 by Abramowitz
// and Stegun, formula 7.1.26: erf(x) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^(-x^2),
// t = 1 / (1 + p x), |error| <= 1.5e-7 for every x >= 0.  It has no branches (the
// device erff takes two ranges, both of which a wave with mixed arguments runs), and
// its e^(-x^2) = e^(-a^2 / 2) is the factor that GELU'(a) needs as well, returned in *e.
__device__ __forceinline__ float normal_cdf(float a, float* e) {
  const float x = fabsf(a) * 0.7071067811865476f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  float p = 1.061405429f;
  p = fmaf(p, t, -1.453152027f);
  p = fmaf(p, t, 1.421413741f);
  p = fmaf(p, t, -0.284496736f);
  p = fmaf(p, t, 0.254829592f);
  *e = __builtin_amdgcn_exp2f(a * (a * -0.7213475204444817f));  // e^(-a^2/2) = 2^(-a^2 log2(e) / 2)
  const float tail = 0.5f * (p * t) * *e;                         // (1 - erf(x)) / 2 = Phi(-|a|)
  return a >= 0.0f ? 1.0f - tail : tail;
}

__device__ __forceinline__ float gelu_val(float a, bool tanh_form) {
  if (tanh_form) {
    const float u = 0.7978845608028654f * (a + 0.044715f * a * a * a);
    return 0.5f * a * (1.0f + tanhf(u));
  }
  float e;
  return a * normal_cdf(a, &e);
}

__device__ __forceinline__ void gelu_both(float a, bool tanh_form, float* g, float* dg) {
  if (tanh_form) {
    const float a2 = a * a;
    const float u = 0.7978845608028654f * (a + 0.044715f * a2 * a);
    const float th = tanhf(u);
    *g = 0.5f * a * (1.0f + th);
    *dg = 0.5f * (1.0f + th) + 0.5f * a * (1.0f - th * th) * 0.7978845608028654f * (1.0f + 3.0f * 0.044715f * a2);
    return;
  }
  float e;
  const float cdf = normal_cdf(a, &e);
  *g = a * cdf;
  *dg = fmaf(a * 0.3989422804014327f, e, cdf);  // Phi(a) + a phi(a), phi(a) = e^(-a^2/2) / sqrt(2 pi)
}

// Raw bits of an io element; converted where used, so that the load's latency
// is not waited for at the load.
__device__ __forceinline__ uint32_t ld_io_bits(const void* p, int64_t i, bool bf16) {
  if (bf16) return (uint32_t)((const uint16_t*)p)[i];
  return ((const uint32_t*)p)[i];
}

__device__ __forceinline__ float io_bits_to_f32(uint32_t b, bool bf16) { return __uint_as_float(bf16 ? b << 16 : b); }

__device__ __forceinline__ void st_io(void* p, int64_t i, float v, bool bf16) {
  if (bf16)
    ((__bf16*)p)[i] = (__bf16)v;
  else
    ((float*)p)[i] = v;
}

// Exchange transport: relaxed device-scope atomic stores and loads, whose
// coherence between workgroups the memory model guarantees wherever they run.
// Every entry is one 64-bit word (tag and value), so a reader sees either the
// old or the new one whole, and no ordering between entries is needed.  (On
// gfx950 workgroup-scope loads can be served from a stale L1 line even after a
// workgroup-scope invalidate; plain stores with polls that invalidate the L1 at
// device scope before plain loads are correct between workgroups of one XCD and
// faster for a single polling thread, but with every thread of the workgroup
// polling the invalidates cost 14,400 cycles per token against 3,000.  Loads with
// the workgroup-scope bit alone are served from L1 as well, stale also between
// workgroups of one XCD.)
__device__ __forceinline__ void put(uint64_t* e, uint32_t tag, float v) {
  __hip_atomic_store(e, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One round of loads of the n (0..4) entries e_idx[0..n) into e[] (all issued
// before any is looked at, so a round costs one round trip).
__device__ __forceinline__ void poll_issue(const uint64_t* base, int n, const int64_t* e_idx, uint64_t (&e)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    e[i] = __hip_atomic_load(base + e_idx[i < n ? i : 0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Completes a poll of token `tag` whose first round of loads, e[], was issued
// earlier (poll_issue): loads again until all n entries carry the tag, and returns
// their values in out[].  Returns false on abort or time-out.
__device__ bool poll_finish(const uint64_t* base, int n, const int64_t* e_idx, uint32_t tag, uint32_t* abort_flag,
                            uint64_t (&e)[4], float* out) {
  if (n == 0) return true;
  for (uint32_t spin = 0;; ++spin) {
    bool all = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) all = all && (uint32_t)(e[i] >> 32) == tag;
    if (all) break;
    if (spin >= SPIN_MAX) {
      __hip_atomic_store(abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    if ((spin & 15) == 15 && __hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return false;
    if (spin > 0) __builtin_amdgcn_s_sleep(1);
    poll_issue(base, n, e_idx, e);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < n) out[i] = __uint_as_float((uint32_t)e[i]);
  return true;
}

// keep + the value `send` holds in the lane that the DPP control CTRL selects
template <int CTRL>
__device__ __forceinline__ float dpp_add(float keep, float send) {
  return keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), CTRL, 0xf, 0xf, false));
}

// Sum of x over each group of 8 consecutive lanes, in every lane of the group: the
// half-row mirror (lane i with 7 - i) and two quad permutations (lane ^ 2, lane ^ 1).
__device__ __forceinline__ float unit_sum8(float x) {
  x = dpp_add<0x141>(x, x);
  x = dpp_add<0x4e>(x, x);
  return dpp_add<0xb1>(x, x);
}

// Sum of x over the wave's 64 lanes, in every lane: halves of 32 and 16 lanes trade
// with the lane swaps, halves of 8 with a DPP row rotation, then unit_sum8.
__device__ __forceinline__ float wave_sum64(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  x = dpp_add<0x128>(x, x);
  return unit_sum8(x);
}

template <bool TANH>
__global__ __launch_bounds__(NT) void scan_coop_kernel(ScanArgs a) {
  __shared__ float Ypart[NW][4][64];  // per-wave partials of yhat (j = l, l + 64) and z (same)
  __shared__ __attribute__((aligned(16))) float Ks[4][CD];  // k_{t-1} .. k_{t+2} (by token mod 4)
  __shared__ __attribute__((aligned(16))) float Qs[2][CD];  // q_t, q_{t+1} (by token mod 2)
  __shared__ float Xv[NCU][CD];       // gathered yhat partials, by workgroup and feature
  __shared__ float Zv[NCU][16];       // gathered z partials of this workgroup's 16 channels
  __shared__ uint32_t stop_wg;        // set (never cleared) by a thread whose poll failed

  // Workgroup -> (sequence-head bh, slice cu).  The NCU slices of a head get
  // workgroup indices that are equal modulo 8, i.e. the same XCD under the
  // round-robin dispatch of workgroups to XCDs (they then share L2 for the
  // head's q, k, v); indices past B*H are idle.
  const int64_t BH = a.B * a.H;
  const int cu = (int)((blockIdx.x / 8) % NCU);
  const int64_t bh = (int64_t)(blockIdx.x / (8 * NCU)) * 8 + blockIdx.x % 8;
  if (bh >= BH) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t s = bh / a.H;
  const int h = (int)(bh % a.H);
  const int64_t T = a.T;
  const int D = a.H * CD;
  const int u0 = UNITS * cu;
  // this lane's hidden unit (of the wave's UW) and its rows of W1
  const int ul = lane >> 3, r0 = PW * (lane & 7);
  const int unit = u0 + UW * w + ul;
  const bool bf16 = a.bf16;
  const float neta = -a.eta, gs = a.gscale;
  const bool writer = (w == 0) && lane < 16;  // writes channels h*d + 16*cu + lane
  const int ch = h * CD + 16 * cu + (lane & 15);
  auto tok = [&](int64_t t) -> int64_t { return a.reverse ? T - 1 - t : t; };
  auto fill_nan = [&](int64_t t_from) {  // after an abort: the rest of this workgroup's outputs
    if (!writer) return;
    for (int64_t t = t_from; t < T; ++t) {
      const int64_t o = ((int64_t)s * T + tok(t)) * D + ch;
      st_io(a.y, o, __builtin_nanf(""), bf16);
      if (a.z) a.z[o] = __builtin_nanf("");
    }
  };

  bool failed = false;  // this thread saw an abort or a time-out
  const int64_t xslots = bh * 2 * NCU * NVAL;  // first entry of this head's slots

  // ---- state slices
  float W1r[PW];
  float W2r[UW][2];
  {
    const float* w1 = a.w1_0 + (int64_t)h * CD * CM;
    const float* w2 = a.w2_0 + (int64_t)h * CM * CD;
#pragma unroll
    for (int k = 0; k < PW; ++k) W1r[k] = w1[(int64_t)(r0 + k) * CM + unit];
#pragma unroll
    for (int i = 0; i < UW; ++i) {
      W2r[i][0] = w2[(int64_t)(u0 + UW * w + i) * CD + lane];
      W2r[i][1] = w2[(int64_t)(u0 + UW * w + i) * CD + lane + 64];
    }
  }

  const int64_t plane = a.B * a.H * T * CD;
  const float* qb = a.qkv + bh * T * CD;
  const float* kb = qb + plane;
  const float* vb = qb + 2 * plane;
  const float tg = tanhf(a.alpha[ch]);
  // staging: threads 0..127 move k_{t+2}, threads 128..255 q_{t+1} (element tid mod 128)
  // from global memory into their LDS slot, which holds token (t + ahead) mod 4 / mod 2
  const bool stager = tid < 2 * CD;
  const int st_ahead = tid < CD ? 2 : 1, st_mask = tid < CD ? 3 : 1;
  const float* st_src = tid < CD ? kb + tid : qb + (tid & (CD - 1));

  // sum over this lane's 16 rows of x . W1r (x: 16 consecutive floats in LDS)
  auto rows_dot = [&](const float* x) -> float {
    const float4* x4 = (const float4*)x;
    float acc = 0.0f;
#pragma unroll
    for (int k4 = 0; k4 < PW / 4; ++k4) {
      const float4 v = x4[k4];
      acc = fmaf(v.x, W1r[4 * k4], acc);
      acc = fmaf(v.y, W1r[4 * k4 + 1], acc);
      acc = fmaf(v.z, W1r[4 * k4 + 2], acc);
      acc = fmaf(v.w, W1r[4 * k4 + 3], acc);
    }
    return acc;
  };

  if (T > 0) {
    // ---- prologue: the k and q slots zeroed (the deferred update of token -1 and the
    //      pre-activations of the last iteration read slots that hold no token yet), then
    //      k_0, k_1, q_0, and the pre-activation k_0 W1_0 of token 0
    for (int i = tid; i < 4 * CD; i += NT) (&Ks[0][0])[i] = 0.0f;
    for (int i = tid; i < 2 * CD; i += NT) (&Qs[0][0])[i] = 0.0f;
    if (tid == 0) stop_wg = 0u;
    __syncthreads();
    if (tid < CD) {
      Ks[0][tid] = kb[tok(0) * CD + tid];
      Qs[0][tid] = qb[tok(0) * CD + tid];
    } else if (tid < 2 * CD && T > 1) {
      Ks[1][tid - CD] = kb[tok(1) * CD + tid - CD];
    }
    __syncthreads();

    // Carried from one iteration to the next, all in registers: the pre-activations
    // k_{t+1} W1_{t-1} and q_t W1_{t-1} of this lane's unit (every lane of the unit's
    // group of 8 holds them whole), the dot products k_{t+1} . k_t and q_t . k_t
    // (every lane), and -eta G1 of the unit for the previous token, whose W1 update is
    // applied in the next iteration while the exchange is in flight.
    float a_pre = unit_sum8(rows_dot(Ks[0] + r0)), aq_pre = 0.0f;
    float skk = 0.0f, sqk = 0.0f;
    float ng1_prev = 0.0f;
    for (int64_t t = 0; t <= T; ++t) {
      const bool live = t < T;
      TTT_MARK(g_marks_scan_coop, t, 0);
      // operands loaded now and used later in the iteration: v_t, the gate
      // input of token t-1, and (staged into LDS after the first barrier) k_{t+2}, q_{t+1}
      float v0 = 0.0f, v1 = 0.0f, stage = 0.0f;
      uint32_t xo = 0;
      if (live) {
        v0 = vb[tok(t) * CD + lane];
        v1 = vb[tok(t) * CD + lane + 64];
        // one unconditional load per thread (token clamped into range; only
        // valid values are written to LDS)
        const int64_t ts = t + st_ahead < T ? t + st_ahead : T - 1;
        if (stager) stage = st_src[tok(ts) * CD];
      }
      if (writer && t > 0) xo = ld_io_bits(a.xin, ((int64_t)s * T + tok(t - 1)) * D + ch, bf16);
      TTT_MARK(g_marks_scan_coop, t, 1);
      // ---- this lane's unit: a_t = k_t W1_{t-1} = k_t W1_{t-2} + (k_t . k_{t-1}) (-eta G1_{t-1}),
      //      and aq_{t-1} = q_{t-1} W1_{t-1} likewise; their GELU
      float hk = 0.0f, dg = 0.0f, hq = 0.0f;
      {
        const float av = fmaf(skk, ng1_prev, a_pre);
        const float aqv = fmaf(sqk, ng1_prev, aq_pre);
        if (live) gelu_both(av, TANH, &hk, &dg);
        if (t > 0) hq = gelu_val(aqv, TANH);
      }
      // ---- first W2 pass: partial yhat_t and z_{t-1} over this wave's 8 units, whose
      //      activations every lane takes from the first lane of the unit's group
      float hks[UW];
      {
        float y0 = 0.0f, y1 = 0.0f, z0 = 0.0f, z1 = 0.0f;
#pragma unroll
        for (int i = 0; i < UW; ++i) {
          hks[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hk), 8 * i));
          const float hqi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hq), 8 * i));
          y0 = fmaf(hks[i], W2r[i][0], y0);
          y1 = fmaf(hks[i], W2r[i][1], y1);
          z0 = fmaf(hqi, W2r[i][0], z0);
          z1 = fmaf(hqi, W2r[i][1], z1);
        }
        Ypart[w][0][lane] = y0;
        Ypart[w][1][lane] = y1;
        Ypart[w][2][lane] = z0;
        Ypart[w][3][lane] = z1;
      }
      __syncthreads();
      TTT_MARK(g_marks_scan_coop, t, 2);
      // ---- stage k_{t+2}, q_{t+1} (loaded at the top of this iteration); their
      //      slots held k_{t-2}, q_{t-1}, last read in the previous iteration
      if (stager && t + st_ahead < T) {
        float* st_dst = tid < CD ? &Ks[0][tid] : &Qs[0][tid & (CD - 1)];
        st_dst[((t + st_ahead) & st_mask) * CD] = stage;
      }
      // ---- publish this workgroup's partial of value 64 w + lane (waves 0, 1: yhat; 2, 3: z)
      const int64_t slot = xslots + (t & 1) * NCU * NVAL;
      if (w < 4) {
        float p = 0.0f;
#pragma unroll
        for (int q = 0; q < NW; ++q) p += Ypart[q][w][lane];
        put(a.xchg + slot + cu * NVAL + 64 * w + lane, (uint32_t)t, p);
      }
      TTT_MARK(g_marks_scan_coop, t, 3);
      // ---- the gather's entries: thread tid fetches yhat feature tid mod 128 from
      //      workgroups 2 (tid / 128) and 2 (tid / 128) + 1, and (tid < 128) the z
      //      partial of channel tid mod 16 from workgroup tid / 16, all in each round
      //      of loads (one round trip).  The first round goes out in the middle of the
      //      W1 pass below, about when the peers' partials land (measured: 1.44 s per
      //      bigstate307k call, against 1.52 with the first round after the W1 pass,
      //      1.50 after the W1 update, 1.47 after both pre-activations and 1.70 right
      //      after publishing, whose extra rounds of polls lowered the shader clock).
      int64_t e_idx[4] = {0, 0, 0, 0};
      int n_e = 0;
      if (live) {
        for (int i = 0; i < 2; ++i) e_idx[i] = slot + (2 * (tid >> 7) + i) * NVAL + (tid & 127);
        n_e = 2;
      }
      const bool zr = t > 0 && tid < 16 * NCU;
      if (zr) e_idx[n_e++] = slot + (tid >> 4) * NVAL + CD + 16 * cu + (tid & 15);
      uint64_t e_got[4];
      // ---- while the partials travel: token t-1's W1 update of this lane's rows (with
      //      k_{t-1} and its G1), then the pre-activations k_{t+1} W1_{t-1} and
      //      q_t W1_{t-1} of the unit (summed over its 8 lanes) and the dot products
      //      k_{t+1} . k_t and q_t . k_t (summed over the wave; lane l takes features
      //      l and l + 64).  At t = T-1 and T the k and q slots past the end hold stale
      //      values; those results are never used.
      {
        const float4* kp = (const float4*)(Ks[(t + 3) & 3] + r0);  // k_{t-1}
#pragma unroll
        for (int k4 = 0; k4 < PW / 4; ++k4) {
          const float4 pv = kp[k4];
          W1r[4 * k4] = fmaf(ng1_prev, pv.x, W1r[4 * k4]);
          W1r[4 * k4 + 1] = fmaf(ng1_prev, pv.y, W1r[4 * k4 + 1]);
          W1r[4 * k4 + 2] = fmaf(ng1_prev, pv.z, W1r[4 * k4 + 2]);
          W1r[4 * k4 + 3] = fmaf(ng1_prev, pv.w, W1r[4 * k4 + 3]);
        }
        a_pre = unit_sum8(rows_dot(Ks[(t + 1) & 3] + r0));
        __builtin_amdgcn_sched_barrier(0);  // the first round of the gather's loads: here, not moved
        poll_issue(a.xchg, n_e, e_idx, e_got);
        __builtin_amdgcn_sched_barrier(0);
        aq_pre = unit_sum8(rows_dot(Qs[t & 1] + r0));
        const float* kc = Ks[t & 3];
        const float* kn = Ks[(t + 1) & 3];
        const float* qc = Qs[t & 1];
        skk = wave_sum64(fmaf(kn[lane], kc[lane], kn[lane + 64] * kc[lane + 64]));
        sqk = wave_sum64(fmaf(qc[lane], kc[lane], qc[lane + 64] * kc[lane + 64]));
      }
      // ---- the gather completes (the sums follow through LDS in a fixed order)
      {
        float vals[4];
        const bool ok = !failed && poll_finish(a.xchg, n_e, e_idx, (uint32_t)t, a.abort_flag, e_got, vals);
        if (ok && live)
          for (int i = 0; i < 2; ++i) Xv[2 * (tid >> 7) + i][tid & 127] = vals[i];
        if (ok && zr) Zv[tid >> 4][tid & 15] = vals[n_e - 1];
        if (!ok) __hip_atomic_store(&stop_wg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        failed = !ok;
      }
      TTT_MARK(g_marks_scan_coop, t, 4);
      // A failed poll stops the workgroup after this barrier: the stop flag is written
      // only between the first barrier and this one, so every thread reads the same value.
      __syncthreads();
      if (__hip_atomic_load(&stop_wg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) {
        fill_nan(t > 0 ? t - 1 : 0);  // every thread of the workgroup leaves together
        return;
      }
      TTT_MARK(g_marks_scan_coop, t, 5);
      float got[2] = {0.0f, 0.0f};
      if (live) {
#pragma unroll
        for (int q = 0; q < NCU; ++q) {
          got[0] += Xv[q][lane];
          got[1] += Xv[q][lane + 64];
        }
      }
      if (writer && t > 0) {
        float zv = 0.0f;
#pragma unroll
        for (int q = 0; q < NCU; ++q) zv += Zv[q][lane];
        const int64_t o = ((int64_t)s * T + tok(t - 1)) * D + ch;
        st_io(a.y, o, fmaf(tg, zv, io_bits_to_f32(xo, bf16)), bf16);
        if (a.z) a.z[o] = zv;
      }
      if (!live) break;

      // ---- G2 for j = lane, lane + 64; second W2 pass: G2 W2^T partials and the W2 update
      const float g20 = gs * (got[0] - v0), g21 = gs * (got[1] - v1);
      float gp[UW];
#pragma unroll
      for (int i = 0; i < UW; ++i) {
        gp[i] = fmaf(g20, W2r[i][0], g21 * W2r[i][1]);
        const float nh = neta * hks[i];
        W2r[i][0] = fmaf(nh, g20, W2r[i][0]);
        W2r[i][1] = fmaf(nh, g21, W2r[i][1]);
      }
      // ---- sum gp over the 64 lanes (recursive halving, in registers): lane ends
      //      with unit 4 b5 + 2 b4 + b3 = lane / 8 of its wave's 8 (b = bits of the lane
      //      index), the lane's own unit.  Each halving pairs every lane with one lane of
      //      the other half of its group; the lane keeps the units of its half and adds
      //      the partner's partial of them.  Halves of 32 and 16 lanes trade with the lane
      //      swaps (lanes 32..63 of the first operand with lanes 0..31 of the second, and
      //      likewise odd with even rows of 16), halves of 8 through a DPP row rotation;
      //      the 8 lanes that then hold one unit sum it with the half-row mirror and quad
      //      permutations.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(gp[i]), __float_as_uint(gp[4 + i]), false,
                                                         false);
        gp[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(gp[i]), __float_as_uint(gp[2 + i]), false,
                                                         false);
        gp[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      {
        const bool hi = lane & 8;
        gp[0] = dpp_add<0x128>(hi ? gp[1] : gp[0], hi ? gp[0] : gp[1]);  // row_ror:8: lane ^ 8
      }
      TTT_MARK(g_marks_scan_coop, t, 6);
      ng1_prev = neta * unit_sum8(gp[0]) * dg;  // -eta G1_t of this lane's unit: applied to W1 next iteration
      TTT_MARK(g_marks_scan_coop, t, 7);
    }
  }

  // ---- final state
  if (a.w1_T) {
    float* o = a.w1_T + bh * CD * CM;
#pragma unroll
    for (int k = 0; k < PW; ++k) o[(int64_t)(r0 + k) * CM + unit] = W1r[k];
  }
  if (a.w2_T) {
    float* o = a.w2_T + bh * CM * CD;
#pragma unroll
    for (int i = 0; i < UW; ++i) {
      o[(int64_t)(u0 + UW * w + i) * CD + lane] = W2r[i][0];
      o[(int64_t)(u0 + UW * w + i) * CD + lane + 64] = W2r[i][1];
    }
  }
}

// Marks every exchange entry as not yet written (tag 0xffffffff) and, for the first
// launch of a call, clears the abort flag (a bidirectional call's reversed pass keeps
// what its forward pass raised, so the flag reports the whole call).
__global__ void coop_clear_kernel(uint64_t* x, int64_t n, uint32_t* abort_flag, int clear_abort) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = ~(uint64_t)0;
  if (i == 0 && clear_abort) *abort_flag = 0u;
}

int64_t coop_grid(int64_t B, int H) { return 8 * NCU * ((B * H + 7) / 8); }

}  // namespace

bool scan_coop_supported(int d, int m, int b, int64_t T) {
  return d == CD && m == CM && b == 1 && T < ((int64_t)1 << 31);  // token tags stay below 0xffffffff
}

size_t scan_coop_xchg_bytes(int64_t B, int H) { return (size_t)(B * H) * 2 * NCU * NVAL * sizeof(uint64_t); }

bool scan_coop_fits(int64_t B, int H) {
  int dev = 0, cus = 0, coop = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop) return false;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, scan_coop_kernel<false>, NT, 0) != hipSuccess) return false;
  int per_cu_t = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_t, scan_coop_kernel<true>, NT, 0) != hipSuccess) return false;
  const int64_t fit = (int64_t)cus * (per_cu < per_cu_t ? per_cu : per_cu_t);
  return coop_grid(B, H) <= fit;
}

hipError_t launch_scan_coop(const ScanArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)(a.B * a.H) * 2 * NCU * NVAL;
  hipLaunchKernelGGL(coop_clear_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.xchg, n, a.abort_flag,
                     (int)a.clear_abort);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ScanArgs args = a;
  void* kargs[] = {(void*)&args};
  const dim3 grid((unsigned)coop_grid(a.B, a.H)), block(NT);
  if (a.gelu_tanh) return hipLaunchCooperativeKernel((const void*)scan_coop_kernel<true>, grid, block, kargs, 0, s);
  return hipLaunchCooperativeKernel((const void*)scan_coop_kernel<false>, grid, block, kargs, 0, s);
}

}  // namespace ttt

TTT_MARKS_EXPORT(ttt_phase_marks_scan_coop, g_marks_scan_coop);
