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
// VGPRs:
//   W1 slice (128 x 64): lane u of wave w holds W1[32w .. 32w+31][u];
//   W2 slice (64 x 128): lane l of wave w holds W2[16w .. 16w+15][l, l+64].
// Per token every workgroup holds the full q, k, v of its head.  a = k W1 and
// aq = q W1 are local to a unit, so only the contractions over hidden units,
// yhat = GELU(a) W2 and z = GELU(aq) W2, need partial sums from all NCU
// workgroups: one exchange per token.
//
// Read-out.  Iteration t runs token t's step with the state W_{t-1}, which is
// also token t-1's post-update state, so token t-1's read-out is computed in
// the same passes: aq_{t-1} = q_{t-1} W1_{t-1} comes out of the previous
// iteration's W1 pass, z_{t-1} = GELU(aq_{t-1}) W2_{t-1} out of this one's
// first W2 pass, and its partials travel with yhat_t's.
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

namespace ttt {
namespace {

constexpr int CD = 128;               // head width d
constexpr int CM = 512;               // hidden width m
constexpr int NCU = 8;                // cooperating workgroups per head
constexpr int UNITS = CM / NCU;       // hidden units per workgroup
constexpr int NW = 4;                 // waves per workgroup
constexpr int NT = 64 * NW;           // threads per workgroup
constexpr int PW = CD / NW;           // rows of W1 per wave
constexpr int UW = UNITS / NW;        // units of W2 per wave
constexpr int NVAL = 2 * CD;          // exchanged values per workgroup and token: yhat, z partials
constexpr uint32_t SPIN_MAX = 1u << 20;
static_assert(UNITS == 64 && UW == 16 && PW == 32 && CD == 128, "lane mapping assumes these sizes");

__device__ __forceinline__ float gelu_val(float a, bool tanh_form) {
  if (tanh_form) {
    const float u = 0.7978845608028654f * (a + 0.044715f * a * a * a);
    return 0.5f * a * (1.0f + tanhf(u));
  }
  return 0.5f * a * (1.0f + erff(a * 0.7071067811865476f));
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
  const float cdf = 0.5f * (1.0f + erff(a * 0.7071067811865476f));
  *g = a * cdf;
  *dg = cdf + a * 0.3989422804014327f * expf(-0.5f * a * a);
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
// (On gfx950 workgroup-scope loads can be served from a stale L1 line even after
// a workgroup-scope invalidate, and workgroup-scope atomics read L2 correctly but
// are slower per poll.)
__device__ __forceinline__ void put(uint64_t* e, uint32_t tag, float v) {
  __hip_atomic_store(e, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls the n (0..4) entries e_idx[0..n) of token `tag` until all carry the tag
// and returns their values in out[].  A poll issues all its loads before it looks
// at any of them, so it costs one round trip.  Returns false on abort or time-out.
__device__ bool poll(const uint64_t* base, int n, const int64_t* e_idx, uint32_t tag, uint32_t* abort_flag,
                     float* out) {
  if (n == 0) return true;
  uint64_t e[4];
  for (uint32_t spin = 0;; ++spin) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      e[i] = __hip_atomic_load(base + e_idx[i < n ? i : 0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool all = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) all = all && (uint32_t)(e[i] >> 32) == tag;
    if (all) break;
    if (spin >= SPIN_MAX) {
      __hip_atomic_store(abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    if ((spin & 15) == 15 && __hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return false;
    __builtin_amdgcn_s_sleep(1);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < n) out[i] = __uint_as_float((uint32_t)e[i]);
  return true;
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

template <bool TANH>
__global__ __launch_bounds__(NT) void scan_coop_kernel(ScanArgs a) {
  __shared__ float Apart[2][NW][64];  // per-wave partials of a (k W1) and aq (q W1), by unit
  __shared__ float Ypart[NW][4][64];  // per-wave partials of yhat (j = l, l + 64) and z (same)
  __shared__ float GH[UNITS];         // G2 W2^T, by unit
  __shared__ __attribute__((aligned(16))) float Ks[3][CD];  // k_t, k_{t+1}, k_{t+2} (by token mod 3)
  __shared__ __attribute__((aligned(16))) float Qs[2][CD];  // q_t, q_{t+1} (by token mod 2)
  __shared__ float Xv[NCU][CD];       // gathered yhat partials, by workgroup and feature
  __shared__ float Zv[NCU][16];       // gathered z partials of this workgroup's 16 channels

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
    for (int k = 0; k < PW; ++k) W1r[k] = w1[(int64_t)(PW * w + k) * CM + u0 + lane];
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

  if (T > 0) {
    // ---- prologue: k_0, k_1, q_0 into LDS, then the partial a of token 0
    if (tid < CD) {
      Ks[0][tid] = kb[tok(0) * CD + tid];
      Qs[0][tid] = qb[tok(0) * CD + tid];
    } else if (T > 1) {
      Ks[1][tid - CD] = kb[tok(1) * CD + tid - CD];
    }
    __syncthreads();
    {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < PW; ++k) acc = fmaf(Ks[0][PW * w + k], W1r[k], acc);
      Apart[0][w][lane] = acc;
      Apart[1][w][lane] = 0.0f;
    }

    for (int64_t t = 0; t <= T; ++t) {
      const bool live = t < T;
      // operands loaded now and used later in the iteration: v_t, the gate
      // input of token t-1, and (staged into LDS at the end) k_{t+2}, q_{t+1}
      float v0 = 0.0f, v1 = 0.0f, stage = 0.0f;
      uint32_t xo = 0;
      if (live) {
        v0 = vb[tok(t) * CD + lane];
        v1 = vb[tok(t) * CD + lane + 64];
        // one unconditional load per thread (token clamped into range; only
        // valid values are written to LDS): divergent loads into one register
        // would make the second wait for the first
        const int64_t tk = t + 2 < T ? t + 2 : T - 1, tq = t + 1 < T ? t + 1 : T - 1;
        stage = tid < CD ? kb[tok(tk) * CD + tid] : qb[tok(tq) * CD + tid - CD];
      }
      if (writer && t > 0) xo = ld_io_bits(a.xin, ((int64_t)s * T + tok(t - 1)) * D + ch, bf16);

      __syncthreads();  // Apart of this iteration is complete
      // ---- unit u = lane: GELU of a_t and of aq_{t-1}
      float hk = 0.0f, dg = 0.0f, hq = 0.0f;
      {
        float av = 0.0f, aqv = 0.0f;
#pragma unroll
        for (int q = 0; q < NW; ++q) {
          av += Apart[0][q][lane];
          aqv += Apart[1][q][lane];
        }
        if (live) gelu_both(av, TANH, &hk, &dg);
        if (t > 0) hq = gelu_val(aqv, TANH);
      }
      // ---- first W2 pass: partial yhat_t and z_{t-1} over this wave's 16 units
      float hks[UW];
      {
        float y0 = 0.0f, y1 = 0.0f, z0 = 0.0f, z1 = 0.0f;
#pragma unroll
        for (int i = 0; i < UW; ++i) {
          hks[i] = readlane_f(hk, UW * w + i);
          const float hqs = readlane_f(hq, UW * w + i);
          y0 = fmaf(hks[i], W2r[i][0], y0);
          y1 = fmaf(hks[i], W2r[i][1], y1);
          z0 = fmaf(hqs, W2r[i][0], z0);
          z1 = fmaf(hqs, W2r[i][1], z1);
        }
        Ypart[w][0][lane] = y0;
        Ypart[w][1][lane] = y1;
        Ypart[w][2][lane] = z0;
        Ypart[w][3][lane] = z1;
      }
      __syncthreads();
      // ---- stage k_{t+2}, q_{t+1} (loaded at the top of this iteration); their
      //      buffers held k_{t-1}, q_{t-1}, last read in the previous iteration
      if (live) {
        if (tid < CD) {
          if (t + 2 < T) Ks[(t + 2) % 3][tid] = stage;
        } else if (t + 1 < T) {
          Qs[(t + 1) & 1][tid - CD] = stage;
        }
      }
      // ---- publish this workgroup's partial of value 64 w + lane (w < 2: yhat, else z)
      const int64_t slot = xslots + (t & 1) * NCU * NVAL;
      {
        float p = 0.0f;
#pragma unroll
        for (int q = 0; q < NW; ++q) p += Ypart[q][w][lane];
        put(a.xchg + slot + cu * NVAL + 64 * w + lane, (uint32_t)t, p);
      }
      // ---- gather, spread over the workgroup: thread tid fetches yhat feature
      //      tid mod 128 from workgroups 4 (tid / 128) .. +3, and (tid < 128) the z
      //      partial of channel tid mod 16 from workgroup tid / 16; the sums follow
      //      through LDS in a fixed order
      {
        int64_t e_idx[4];
        float vals[4];
        int n = 0;
        if (live) {
          for (int i = 0; i < 4; ++i) e_idx[i] = slot + (4 * (tid >> 7) + i) * NVAL + (tid & 127);
          n = 4;
        }
        bool ok = !failed && poll(a.xchg, n, e_idx, (uint32_t)t, a.abort_flag, vals);
        if (ok && live)
          for (int i = 0; i < 4; ++i) Xv[4 * (tid >> 7) + i][tid & 127] = vals[i];
        if (ok && t > 0 && tid < 16 * NCU) {
          const int64_t ze = slot + (tid >> 4) * NVAL + CD + 16 * cu + (tid & 15);
          float zv;
          ok = poll(a.xchg, 1, &ze, (uint32_t)t, a.abort_flag, &zv);
          if (ok) Zv[tid >> 4][tid & 15] = zv;
        }
        failed = !ok;
      }
      if (__syncthreads_or(failed)) {  // every thread of the workgroup leaves together
        fill_nan(t > 0 ? t - 1 : 0);
        return;
      }
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
      // ---- sum gp over the 64 lanes (recursive halving): lane ends with unit
      //      8 b5 + 4 b4 + 2 b3 + b2 of its wave's 16 (b = bits of the lane index)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool hi = lane & 32;
        const float send = hi ? gp[i] : gp[8 + i], keep = hi ? gp[8 + i] : gp[i];
        gp[i] = keep + __shfl_xor(send, 32);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool hi = lane & 16;
        const float send = hi ? gp[i] : gp[4 + i], keep = hi ? gp[4 + i] : gp[i];
        gp[i] = keep + __shfl_xor(send, 16);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bool hi = lane & 8;
        const float send = hi ? gp[i] : gp[2 + i], keep = hi ? gp[2 + i] : gp[i];
        gp[i] = keep + __shfl_xor(send, 8);
      }
      {
        const bool hi = lane & 4;
        const float send = hi ? gp[0] : gp[1], keep = hi ? gp[1] : gp[0];
        gp[0] = keep + __shfl_xor(send, 4);
      }
      gp[0] += __shfl_xor(gp[0], 2);
      gp[0] += __shfl_xor(gp[0], 1);
      if ((lane & 3) == 0) GH[UW * w + 8 * ((lane >> 5) & 1) + 4 * ((lane >> 4) & 1) + 2 * ((lane >> 3) & 1) +
                             ((lane >> 2) & 1)] = gp[0];
      if (__syncthreads_or(failed)) {  // every thread of the workgroup leaves together
        fill_nan(t > 0 ? t - 1 : 0);
        return;
      }
      // ---- W1 pass: update with k_t and G1 of unit lane, then a_{t+1} = k_{t+1} W1_t, aq_t = q_t W1_t
      {
        // (at t = T-1 the k_{t+1} buffer is stale; that a is never used)
        const float4* kc = (const float4*)(Ks[t % 3] + PW * w);
        const float4* kn = (const float4*)(Ks[(t + 1) % 3] + PW * w);
        const float4* qc = (const float4*)(Qs[t & 1] + PW * w);
        const float ng1 = neta * GH[lane] * dg;
        float an = 0.0f, aq = 0.0f;
#pragma unroll
        for (int k4 = 0; k4 < PW / 4; ++k4) {
          const float4 kv = kc[k4], nv = kn[k4], qv = qc[k4];
          const float kk[4] = {kv.x, kv.y, kv.z, kv.w}, nn[4] = {nv.x, nv.y, nv.z, nv.w},
                      qq[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k = 4 * k4 + e;
            W1r[k] = fmaf(ng1, kk[e], W1r[k]);
            an = fmaf(nn[e], W1r[k], an);
            aq = fmaf(qq[e], W1r[k], aq);
          }
        }
        Apart[0][w][lane] = an;
        Apart[1][w][lane] = aq;
      }
    }
    if (__syncthreads_or(failed)) {
      fill_nan(T - 1);
      return;
    }
  }

  // ---- final state
  if (a.w1_T) {
    float* o = a.w1_T + bh * CD * CM;
#pragma unroll
    for (int k = 0; k < PW; ++k) o[(int64_t)(PW * w + k) * CM + u0 + lane] = W1r[k];
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

// Marks every exchange entry as not yet written (tag 0xffffffff) and clears the abort flag.
__global__ void coop_clear_kernel(uint64_t* x, int64_t n, uint32_t* abort_flag) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = ~(uint64_t)0;
  if (i == 0) *abort_flag = 0u;
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
  hipLaunchKernelGGL(coop_clear_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.xchg, n, a.abort_flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ScanArgs args = a;
  void* kargs[] = {(void*)&args};
  const dim3 grid((unsigned)coop_grid(a.B, a.H)), block(NT);
  if (a.gelu_tanh) return hipLaunchCooperativeKernel((const void*)scan_coop_kernel<true>, grid, block, kargs, 0, s);
  return hipLaunchCooperativeKernel((const void*)scan_coop_kernel<false>, grid, block, kargs, 0, s);
}

}  // namespace ttt
