/*
 * ttt_mlp.h -- C ABI of the MI355X (gfx950) TTT-MLP layer scan.
 *
 * The operation is the TTT-MLP layer of "One-Minute Video Generation with
 * Test-Time Training" (paper-notes page, key designs, "TTT-MLP layer" and
 * "gate + bidirectional"):
 *
 *   per head h (channels [h*d, (h+1)*d) of D = H*d), per token t:
 *     k_t = (X theta_K^T)[t, h],  v_t = (X theta_V^T)[t, h],  q_t = (X theta_Q^T)[t, h]
 *     f(u; W) = GELU(u W1) W2,    W1: d x m,  W2: m x d  (fp32 state, m = 4d in the paper)
 *     loss l(W; x_t) = ||f(k_t; W) - v_t||^2    (TTT_LOSS_SUM, the literal form)
 *                    = (1/d) ||f(k_t; W) - v_t||^2   (TTT_LOSS_MEAN, the default reading)
 *     W_t = W_{t-1} - eta * grad l            (one gradient step per token)
 *     z_t = f(q_t; W_t)                       (read-out with the updated state)
 *     y_t = x_t + tanh(alpha) * z_t           (per-channel gate)
 *   bidirectional: X' = forward pass with alpha_f; Y = reversed pass over X'
 *   with alpha_b; both passes start from the same W_0 and use the same theta.
 *
 * TTT-Linear (model = TTT_MODEL_LINEAR): the same layer with a linear inner
 * model, f(u; W) = u W with W a d x d matrix per head (the linear-state
 * variant of the notes page's ablation table).  Its gradient step is
 * W_t = W_{t-1} - eta * k_t^T c (k_t W_{t-1} - v_t), c = 2/d (mean) or 2 (sum);
 * everything else (projections, read-out, mini-batches, gate, directions) is
 * as above.  W1_0 then holds W_0 [H, d, d] (m must equal d), W1_T the final
 * W [B, H, d, d]; W2_0, W2_T and gelu are not used (W2_0 may be NULL).
 *
 * Mini-batches of b tokens (b = 1 is the per-token rule): every gradient of
 * a mini-batch is taken at the state the mini-batch starts from; token t
 * reads out with that state minus eta times the summed gradients of the
 * tokens s <= t of its mini-batch.  If b does not divide T the last
 * mini-batch is short.  The reversed pass cuts its mini-batches from the
 * start of the reversed sequence (i.e. from token T-1 downwards).
 *
 * Conventions
 *   - Every data pointer is a DEVICE pointer on the current HIP device, and
 *     every buffer belongs to the caller.  The library never allocates or
 *     frees device memory on a compute call; scratch space comes from the
 *     caller's workspace (size from ttt_mlp_workspace_size).
 *   - Dense row-major layouts:
 *       X, Y      [B, T, D]   io_dtype (fp32, or bf16 as raw 16-bit words)
 *       theta_qkv [3, D, D]   io_dtype; theta_Q, theta_K, theta_V, each [out, in]
 *       W1_0      [H, d, m]   fp32, shared by all B sequences
 *       W2_0      [H, m, d]   fp32
 *       alpha     [D]         fp32
 *       Z         [B, T, D]   fp32 pre-gate layer output (optional)
 *       W1_T      [B, H, d, m], W2_T [B, H, m, d]  fp32 final state (optional)
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 *     compute call only enqueues work on it and returns; execution errors
 *     surface at the caller's next synchronisation.  Calls on different
 *     streams with separate workspaces and outputs may run concurrently.
 *   - Errors: argument and shape errors are detected on the host before
 *     anything is enqueued; the call then returns a negative status, writes
 *     no output, and ttt_mlp_last_error() describes the problem.  A failed
 *     kernel launch returns TTT_ERR_HIP.  No C++ exception crosses the ABI.
 *   - Thread safety: all entry points may be called from several threads.
 */
#ifndef TTT_MLP_H
#define TTT_MLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define TTT_OK 0
#define TTT_ERR_INVALID_ARG (-1) /* NULL required pointer, bad size, bad enum, aliasing */
#define TTT_ERR_UNSUPPORTED (-2) /* valid arguments outside what the kernels implement */
#define TTT_ERR_WORKSPACE (-3)   /* workspace NULL or smaller than ttt_mlp_workspace_size */
#define TTT_ERR_HIP (-4)         /* a HIP runtime call or kernel launch failed */

/* io_dtype: element type of X, theta_qkv and Y */
#define TTT_F32 0
#define TTT_BF16 1

/* loss reduction of the inner self-supervised loss */
#define TTT_LOSS_MEAN 0 /* (1/d) ||f(k) - v||^2, gradient scale 2/d */
#define TTT_LOSS_SUM 1  /* ||f(k) - v||^2, gradient scale 2 */

/* inner model */
#define TTT_MODEL_MLP 0    /* f(u; W) = GELU(u W1) W2 */
#define TTT_MODEL_LINEAR 1 /* f(u; W) = u W, W = W1 (d x d) */

/* GELU form of the inner MLP */
#define TTT_GELU_ERF 0  /* a * Phi(a), exact */
#define TTT_GELU_TANH 1 /* 0.5 a (1 + tanh(sqrt(2/pi) (a + 0.044715 a^3))) */

/* scan kernel selection */
#define TTT_ALGO_AUTO 0    /* fastest kernel that supports the shape and dtype (the cooperative
                              scan only where its workgroups fit co-resident on the device) */
#define TTT_ALGO_GENERIC 1 /* fp32 VALU scan, any supported shape */
#define TTT_ALGO_MFMA 2    /* bf16-operand MFMA scan, fp32 state: bf16 io, erf GELU,
                              d = 64, m = 256, b = 16, T < 2^31; for TTT_MODEL_LINEAR
                              d = m = 64, b = 16, bf16 io, T < 2^31 */
#define TTT_ALGO_COOP 3    /* (TTT_MODEL_MLP only) per-token fp32 scan whose state (512 KB per head) is split
                              over 8 cooperating workgroups: d = 128, m = 512, b = 1.
                              Needs B*H*8 co-resident workgroups (cooperative launch);
                              a workgroup that waits for its peers longer than about a
                              second stops, and the outputs it had not written are NaN. */

typedef struct ttt_mlp_config {
  int64_t B;        /* sequences, >= 1 */
  int64_t T;        /* tokens per sequence, >= 0 */
  int32_t H;        /* heads, >= 1 */
  int32_t d;        /* head width, D = H*d */
  int32_t m;        /* hidden width of the inner MLP */
  int32_t b;        /* mini-batch size, >= 1 */
  float eta;        /* inner learning rate, finite, >= 0 */
  int32_t loss;     /* TTT_LOSS_* */
  int32_t gelu;     /* TTT_GELU_* */
  int32_t io_dtype; /* TTT_F32 or TTT_BF16 */
  int32_t algo;     /* TTT_ALGO_* */
  int32_t model;    /* TTT_MODEL_* (0, the MLP, when zero-initialised) */
} ttt_mlp_config;

/* Library version, (major << 16) | minor. */
int32_t ttt_mlp_version(void);

/* Static description of a status code (never NULL). */
const char* ttt_mlp_status_string(int32_t status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* ttt_mlp_last_error(void);

/*
 * Bytes of device workspace a call needs.  bidir = 0 for ttt_mlp_forward,
 * 1 for ttt_mlp_bidir.  Writes *bytes; returns TTT_OK, or an error for an
 * invalid or unsupported configuration (same checks as the compute calls).
 */
int32_t ttt_mlp_workspace_size(const ttt_mlp_config* cfg, int32_t bidir, size_t* bytes);

/*
 * The scan kernel a call with this configuration runs: writes TTT_ALGO_GENERIC,
 * TTT_ALGO_MFMA or TTT_ALGO_COOP to *algo (resolving TTT_ALGO_AUTO), or returns
 * the error the compute calls would return.
 */
int32_t ttt_mlp_select_algo(const ttt_mlp_config* cfg, int32_t* algo);

/*
 * One gated direction of the layer: Y = X + tanh(alpha) * TTT(X).
 *   reverse = 0: tokens t = 0 .. T-1 (causal); 1: t = T-1 .. 0.
 *   X, theta_qkv, W1_0, W2_0, alpha, Y, workspace: required (X and Y may be
 *   NULL when T = 0; the call then only writes the final state, = W_0).
 *   Z, W1_T, W2_T: optional outputs (NULL to skip).
 *   Y must not overlap X, and no output may overlap another buffer.
 */
int32_t ttt_mlp_forward(const ttt_mlp_config* cfg, const void* X, const void* theta_qkv,
                        const float* W1_0, const float* W2_0, const float* alpha, int32_t reverse,
                        void* Y, float* Z, float* W1_T, float* W2_T, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * The bidirectional layer: X' = forward pass (alpha_f) over X, then
 * Y = reversed pass (alpha_b) over X'.  X' is held in Y between the passes
 * (rounded to io_dtype, as a stored activation would be).
 *   Z_f, Z_b: optional pre-gate outputs of the two passes.
 *   W1_Tf/W2_Tf, W1_Tb/W2_Tb: optional final states of the two passes.
 */
int32_t ttt_mlp_bidir(const ttt_mlp_config* cfg, const void* X, const void* theta_qkv,
                      const float* W1_0, const float* W2_0, const float* alpha_f,
                      const float* alpha_b, void* Y, float* Z_f, float* Z_b, float* W1_Tf,
                      float* W2_Tf, float* W1_Tb, float* W2_Tb, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * ttt_mlp_bidir without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The call's scratch space is a device array of the
 * library, TTT_STATIC_WORKSPACE_BYTES (320 MiB) on every GPU the library runs
 * on, held until the process ends; the call allocates nothing and creates no
 * stream or event after its first call on a device (that first call looks up
 * the array's device address and creates the side stream and events).  A
 * configuration whose workspace (ttt_mlp_workspace_size with bidir = 1) exceeds
 * the array returns TTT_ERR_WORKSPACE before anything is enqueued; it holds,
 * for instance, 14,400 tokens at 48 heads of width 64 (b = 16, bf16 io).
 * Kernel timing (ttt_mlp_set_kernel_timing) does not record these calls.
 * Every call on one GPU uses the same array: calls that overlap on one GPU
 * (on different streams, or from several threads) race and give wrong results;
 * serialise them.  No part of the array needs to start at zero, and a call
 * leaves its contents behind.  Arguments, outputs and errors otherwise as for
 * ttt_mlp_bidir.
 */
#define TTT_STATIC_WORKSPACE_BYTES ((size_t)320 << 20)
int32_t ttt_mlp_bidir_noalloc(const ttt_mlp_config* cfg, const void* X, const void* theta_qkv,
                              const float* W1_0, const float* W2_0, const float* alpha_f,
                              const float* alpha_b, void* Y, float* Z_f, float* Z_b, float* W1_Tf,
                              float* W2_Tf, float* W1_Tb, float* W2_Tb, void* stream);

/*
 * Whether the cooperative scan (TTT_ALGO_COOP) of the last ttt_mlp_forward or
 * ttt_mlp_bidir call that used `workspace` stopped early: a workgroup waited for
 * its peers longer than the spin limit, every workgroup of the launch then
 * stopped, and the outputs they had not written yet hold NaN.  The call waits
 * for `stream` (the stream of that call), then writes *aborted = 1 (stopped) or
 * 0.  cfg and bidir are those of that call; for a configuration that runs
 * another scan nothing is read and *aborted = 0.  The flag lives in the
 * workspace, is cleared by the first scan launch of each call and is kept
 * through a bidirectional call's reversed pass, so it covers the whole call
 * until the workspace is used again.
 */
int32_t ttt_mlp_coop_aborted(const ttt_mlp_config* cfg, int32_t bidir, const void* workspace,
                             size_t workspace_bytes, void* stream, int32_t* aborted);

/*
 * The projection step alone (the outer-loop theta_Q/K/V applied to every
 * token), for inspection: QKV [3, B, H, T, d] fp32, QKV[p, s, h, t, :] =
 * (X[s, t, :] theta_p^T)[h*d : (h+1)*d].  Accumulates in fp32.
 */
int32_t ttt_mlp_project(const ttt_mlp_config* cfg, const void* X, const void* theta_qkv,
                        float* QKV, void* stream);

/*
 * Backward of the layer (TTT_MODEL_MLP, d and m multiples of 4; fp32 kernels, algo AUTO or
 * GENERIC).  The outer loop of the notes page's training learns theta, the
 * initial state and the gates through the layer; for the gradient dY of the
 * layer output these calls return the gradients of sum(dY * Y):
 *   dX     [B, T, D] fp32,   dtheta [3, D, D] fp32 ([out, in], as theta_qkv),
 *   dW1_0  [H, d, m] fp32,   dW2_0  [H, m, d] fp32 (summed over the B sequences),
 *   dalpha [D] fp32.
 * dY is [B, T, D] fp32.  Every output is overwritten.  The call runs the
 * forward pass again (projection and scan, keeping a checkpoint of the state
 * every 32 mini-batches in the workspace; with algo AUTO at d = 64, m = 256,
 * b = 16 and the erf GELU that scan runs on the fp32 matrix cores with the
 * state in registers, otherwise, and with algo GENERIC, with the backward's own
 * steps: both fp32, in different summation orders), then the backward scan, which
 * replays one segment of 32 mini-batches at a time from its checkpoint and
 * walks it backwards carrying the gradient of the state (with the fp32 matrix-core
 * steps, windows of 16 segments are replayed beforehand, the next window on the
 * library's second stream of the device beside the walk of this one, ordered
 * by events), then two GEMMs:
 * dX = dY + [dQ dK dV] theta and dtheta = [dQ dK dV]^T X.  With bf16 io (X and
 * theta exact bf16 numbers) the fp32 [dQ dK dV] is split exactly into three bf16
 * parts whose sum it is, and the GEMMs run on the bf16 matrix cores with fp32
 * accumulation (every product exact); with fp32 io they are fp32 GEMMs.
 * Workspace: ttt_mlp_backward_workspace_size (bidir = 0 or 1).
 */
int32_t ttt_mlp_backward_workspace_size(const ttt_mlp_config* cfg, int32_t bidir, size_t* bytes);

/* One gated direction (reverse as for ttt_mlp_forward). */
int32_t ttt_mlp_backward(const ttt_mlp_config* cfg, const void* X, const void* theta_qkv, const float* W1_0,
                         const float* W2_0, const float* alpha, int32_t reverse, const float* dY, float* dX,
                         float* dtheta, float* dW1_0, float* dW2_0, float* dalpha, void* workspace,
                         size_t workspace_bytes, void* stream);

/* The bidirectional layer (as ttt_mlp_bidir: X' is rounded to io_dtype and its
 * rounding is passed through unchanged): dX, dtheta and dW*_0 collect both
 * directions; dalpha_f and dalpha_b are the two gates' gradients.  The reversed
 * pass's dtheta GEMM is deferred: with the fp32 matrix-core forward pass it runs
 * on `stream` before the forward pass's backward scan; otherwise on the library's
 * second stream of the device, beside that scan, ordered by events after this
 * call's earlier work on `stream` and before its later work (its dQ|dK|dV get a
 * buffer of their own in the workspace); calls on one device are serialised
 * while they enqueue. */
int32_t ttt_mlp_bidir_backward(const ttt_mlp_config* cfg, const void* X, const void* theta_qkv, const float* W1_0,
                               const float* W2_0, const float* alpha_f, const float* alpha_b, const float* dY,
                               float* dX, float* dtheta, float* dW1_0, float* dW2_0, float* dalpha_f,
                               float* dalpha_b, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Segment-local attention, the hybrid block's step before the TTT layer (the
 * notes page's framework: self-attention within each 3-second segment, the
 * TTT layer over the whole sequence).  bf16 io, head width d = 64.
 *   QKV [B, T, 3D] bf16: Q | K | V of every token (head h at columns 64 h of
 *   each); O [B, T, D] bf16.  Segments are [s L, (s+1) L) of every sequence,
 *   L = seg_len (the last one shorter); within a segment every query attends
 *   to every key (no causal mask): O = softmax(Q K^T / sqrt(d)) V per head,
 *   fp32 scores, softmax and accumulation.
 */
int32_t ttt_segment_attention(const ttt_mlp_config* cfg, int64_t seg_len, const void* QKV, void* O, void* stream);

/*
 * The hybrid block: U = X + attention(X theta_attn^T) theta_out^T (no biases or
 * norms), then Y = ttt_mlp_bidir over U.  theta_attn [3, D, D] and theta_out
 * [D, D] are bf16, [out, in]; the rest as for ttt_mlp_bidir (bf16 io, d = 64).
 * Workspace: ttt_hybrid_block_workspace_size.
 */
int32_t ttt_hybrid_block_workspace_size(const ttt_mlp_config* cfg, int64_t seg_len, size_t* bytes);
int32_t ttt_hybrid_block(const ttt_mlp_config* cfg, int64_t seg_len, const void* X, const void* theta_attn,
                         const void* theta_out, const void* theta_qkv, const float* W1_0, const float* W2_0,
                         const float* alpha_f, const float* alpha_b, void* Y, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Kernel timing, for measurement.  While enabled, every compute call brackets
 * each kernel launch with HIP events on the stream the kernel runs on.
 * ttt_mlp_kernel_timing waits for the recorded events and returns the summed
 * duration (ms) and launch count of one kernel kind since the last reset.
 *   kind: TTT_KERNEL_PROJECT (the projection GEMM), TTT_KERNEL_SCAN (the scan),
 *   TTT_KERNEL_BACKWARD, TTT_KERNEL_GRAD_GEMM or TTT_KERNEL_ATTENTION (below).
 */
#define TTT_KERNEL_PROJECT 0
#define TTT_KERNEL_SCAN 1
#define TTT_KERNEL_BACKWARD 2  /* the backward scan */
#define TTT_KERNEL_GRAD_GEMM 3 /* the backward's dX and dtheta GEMMs */
#define TTT_KERNEL_ATTENTION 4 /* the segment attention */
int32_t ttt_mlp_set_kernel_timing(int32_t enable);
int32_t ttt_mlp_kernel_timing(int32_t kind, double* total_ms, int64_t* launches);
int32_t ttt_mlp_reset_kernel_timing(void);

#ifdef __cplusplus
}
#endif

#endif /* TTT_MLP_H */
