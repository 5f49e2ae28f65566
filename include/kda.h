/*
 * kda.h - C ABI of libkda, the MI355X (gfx950) KDA decode library.
 *
 * One call advances the Kimi Delta Attention recurrence of every
 * (request, value head) of a decode batch by that request's tokens.  The
 * operation and the tensor contract follow:
 *   - "KdaDecode" (Modular MAX Mojo builtin kernels), Tensor Shapes and
 *     default parameters: packed [1, total_T, ...] token tensors, a slotted
 *     state pool [max_slots, HV, dk, dv] (key-first; the state_layout
 *     parameter also names the value-first transpose, and state_dtype a
 *     non-fp32 pool) mutated in place through state_indices, cu_seqlens
 *     varlen packing, the "original" stable-softplus gate and beta given as
 *     logits;
 *   - "Delta-rule write" (atlas, Kimi-K3 > Kimi Delta Attention), code
 *     excerpt naive_recurrent_kda: per token, decay the state row k by
 *     exp(g[k]), write (beta*k) outer (v - k^T S), read o = q^T S from the
 *     updated state; q and k repeated over G = HV/H value heads; the output
 *     takes v's dtype;
 *   - the same "Delta-rule write" page, modeling_kimi_linear.py excerpt: the
 *     model calls the recurrent kernel with transpose_state_layout=True,
 *     i.e. a value-first state;
 *   - "KDA Block TKG Kernel API Reference" (AWS Neuron NKI): l2_eps = 1e-6,
 *     the query scale folded into the L2-normalised query, and the
 *     lower-bound gate (parameters A_log, dt_bias, lower_bound).
 *
 * Per token t of request b, for value head hv with key head h = hv / G and
 * state S = state_pool[state_indices[b], hv] (S[k][v]; the value-first
 * layout stores its transpose):
 *     qh = scale * q[t,h] / sqrt(sum q[t,h]^2 + l2_eps)
 *     kh =         k[t,h] / sqrt(sum k[t,h]^2 + l2_eps)
 *     x  = raw_gate[t,hv] + dt_bias[hv]                       (per channel)
 *     g  = -exp(a_log[hv]) * softplus(x)           (KDA_GATE_SOFTPLUS)
 *     g  = lower_bound * sigmoid(exp(a_log[hv]) * x)  (KDA_GATE_LOWER_BOUND)
 *     beta = sigmoid(beta_logits[t,hv])
 *     S[k][:] *= exp(g[k]);  u = v[t,hv] - kh^T S;  S += beta * kh u^T
 *     out[t,hv] = qh^T S                         (rounded to nearest-even)
 * and S is written back to the same slot after the request's last token.
 *
 * Memory: every pointer is device memory of the current HIP device, owned
 * by the caller.  The library allocates nothing, keeps no pointer after the
 * call returns and holds no state; it is reentrant.  The work is enqueued on
 * `stream` and the call returns without waiting for it.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t, declared here so that this header needs no HIP include. */
typedef struct ihipStream_t* hipStream_t;

#define KDA_ABI_VERSION 4

/* Status codes.  Zero is success; errors are negative. */
enum kda_status {
  KDA_OK = 0,
  KDA_ERR_NULL = -1,        /* a required pointer (struct or data) is NULL  */
  KDA_ERR_DTYPE = -2,       /* a tensor has a dtype this argument rejects   */
  KDA_ERR_SHAPE = -3,       /* ranks or extents disagree (incl. HV % H)     */
  KDA_ERR_UNSUPPORTED = -4, /* dk or dv outside {16, 32, 64, 128}, data    */
                            /* not 16-byte aligned, or a batch too large   */
                            /* for one launch (T, N or B above 2^31 - 1,   */
                            /* B * HV * max(dv / 32, 1) above 2^26 - 1, or */
                            /* for the convolution B * H above 2^25 - 1)   */
  KDA_ERR_MODE = -5,        /* bad gate mode, lower_bound, l2_eps, scale or */
                            /* state layout                                 */
  KDA_ERR_LAUNCH = -6,      /* the HIP launch itself reported an error      */
  KDA_ERR_PRECONDITION = -7 /* kda_check_host: cu_seqlens / indices invalid */
};

/* Element types of kda_tensor. */
enum kda_dtype {
  KDA_F32 = 0,
  KDA_BF16 = 1,
  KDA_I32 = 2
};

/* Gate activation, "KdaDecode" gate_mode / "KDA Block TKG" lower_bound. */
enum kda_gate_mode {
  KDA_GATE_SOFTPLUS = 0,    /* g = -exp(A_log) * softplus(x)              */
  KDA_GATE_LOWER_BOUND = 1  /* g = lower_bound * sigmoid(exp(A_log) * x)  */
};

/* Layout of one (slot, value head) state tile, "KdaDecode" state_layout. */
enum kda_state_layout {
  KDA_STATE_K_FIRST = 0,    /* [dk][dv]: S[k][v] (the default)             */
  KDA_STATE_V_FIRST = 1     /* [dv][dk]: the transposed layout             */
};

/* Matrix precision of kda_prefill. */
enum kda_matmul {
  KDA_MATMUL_SPLIT_BF16 = 0, /* each fp32 operand as hi + lo bf16, three bf16 */
                             /* products per fp32 product (the default)       */
  KDA_MATMUL_F32 = 1         /* the fp32 matrix instructions                  */
};

/* A dense row-major tensor: `data` points at element [0,...,0]; the extents
 * are shape[0..ndim-1] and the storage is contiguous (no strides). */
typedef struct kda_tensor {
  void* data;
  int32_t dtype;     /* enum kda_dtype */
  int32_t ndim;      /* 1..4           */
  int64_t shape[4];
} kda_tensor;

/* Scalar parameters of a call. */
typedef struct kda_mode {
  int32_t gate_mode;   /* enum kda_gate_mode                                  */
  float lower_bound;   /* lower-bound mode only: finite and <= 0              */
  float l2_eps;        /* >= 0, finite; 0 selects the default 1e-6            */
  float scale;         /* > 0, finite; 0 selects the default dk^-0.5          */
  int32_t state_layout;/* enum kda_state_layout                               */
} kda_mode;

/*
 * kda_decode - advance the decode recurrence; see the operation above.
 *
 * Arguments (B requests, T packed tokens, H key heads, HV value heads,
 * N pool slots, dk = key/query head size, dv = value head size):
 *   out           [1, T, HV, dv]  bf16 or f32, must equal v's dtype.  Written
 *                                 for every token of every request.
 *   q, k          [1, T, H, dk]   bf16 or f32 (same dtype as v).
 *   v             [1, T, HV, dv]  bf16 or f32.
 *   raw_gate      [1, T, HV, dk]  f32, gate pre-activation before dt_bias.
 *   beta_logits   [1, T, HV]      f32.
 *   a_log         [HV]            f32.
 *   dt_bias       [HV, dk]        f32.
 *   cu_seqlens    [B + 1]         i32, device resident.
 *   state_pool    [N, HV, dk, dv] (KDA_STATE_K_FIRST) or [N, HV, dv, dk]
 *                 (KDA_STATE_V_FIRST), f32 or bf16, updated in place.  A
 *                 bf16 pool is widened to fp32 on load, advanced in fp32
 *                 through all of the request's tokens and rounded to
 *                 nearest-even once when written back.
 *   state_indices [B]             i32, device resident.
 *   mode          scalar parameters (see kda_mode).
 *   stream        HIP stream to enqueue on (NULL = the null stream).
 *
 * Preconditions on the device-resident metadata, not checked by this call
 * (checking them would need a device-to-host copy; kda_check_host does it):
 *   cu_seqlens[0] == 0, non-decreasing, cu_seqlens[B] == T; state_indices
 *   pairwise distinct among entries >= 0, and < N.
 * Conventions: state_indices[b] < 0 skips request b: its state is not read
 *   or written and its output rows are set to zero.  A request with no
 *   tokens leaves its state untouched.  The kernel clamps every token range
 *   to [0, T) and treats an index >= N like a negative one, so a violated
 *   precondition never makes it access memory outside the tensors; duplicate
 *   indices, however, race and give undefined state.
 * Errors: every argument check runs before any device work; on a nonzero
 *   return nothing has been enqueued or written.  KDA_ERR_LAUNCH reports a
 *   launch error from the HIP runtime.
 */
int kda_decode(const kda_tensor* out, const kda_tensor* q, const kda_tensor* k,
               const kda_tensor* v, const kda_tensor* raw_gate,
               const kda_tensor* beta_logits, const kda_tensor* a_log,
               const kda_tensor* dt_bias, const kda_tensor* cu_seqlens,
               const kda_tensor* state_pool, const kda_tensor* state_indices,
               const kda_mode* mode, hipStream_t stream);

/*
 * The short causal convolutions in front of the recurrence ("KDA Block TKG
 * Kernel API Reference": parameters conv_w and conv_state, and the
 * Background's short convolutions with SiLU; K = 4 for Kimi K3).  For each
 * stream (q, k, v) and channel c, per token t of a request:
 *     y_t[c] = SiLU(sum_{j<K} w[j][c] * x_{t-K+1+j}[c])
 * where the K-1 inputs before the request's first token come from the
 * stream's window, tap 0 meets the oldest position, and after the request's
 * last token the window holds its last K-1 pre-convolution inputs.  The
 * convolved streams enter the recurrence in fp32, unrounded (the block
 * keeps intermediates on chip, "KDA Block TKG" Background); only the output
 * is rounded to its dtype.  Channels are head-outer (h*dk + d), matching the
 * q/k/v tensors.
 */
typedef struct kda_conv {
  kda_tensor x_q;     /* [1, T, H, dk]  pre-convolution q; bf16 or f32        */
  kda_tensor x_k;     /* [1, T, H, dk]  pre-convolution k; dtype of x_q       */
  kda_tensor x_v;     /* [1, T, HV, dv] pre-convolution v; dtype of x_q       */
  kda_tensor w_q;     /* [K, H*dk]  taps, 2 <= K <= 4; f32 or bf16            */
  kda_tensor w_k;     /* [K, H*dk]  dtype of w_q                              */
  kda_tensor w_v;     /* [K, HV*dv] dtype of w_q                              */
  kda_tensor win_q;   /* [N, K-1, H*dk]  f32 windows, oldest first, IN/OUT    */
  kda_tensor win_k;   /* [N, K-1, H*dk]  slot state_indices[b], like the pool */
  kda_tensor win_v;   /* [N, K-1, HV*dv]                                      */
  kda_tensor q_conv;  /* [1, T, H, dk] OUT: convolved q, f32; may be x_q     */
                      /*   itself when x_q is f32 (convolved in place)        */
  kda_tensor k_conv;  /* [1, T, H, dk] OUT: convolved k, f32; may be x_k      */
} kda_conv;

/*
 * kda_decode_conv - the decode step with the short convolutions in front:
 * convolve q, k and v of every request (windows updated in place) and
 * advance the recurrence on the result, as kda_decode does with
 * q = q_conv, k = k_conv and v = the convolved x_v.  Two kernels are
 * enqueued on `stream`: one convolves q and k per (request, key head,
 * channel); the recurrence kernel convolves v itself, each v channel
 * belonging to exactly one wave.  A skipped request (negative index) gets
 * zero rows in out, q_conv and k_conv and keeps its windows; an empty
 * request changes nothing.  Arguments other than `conv` are those of
 * kda_decode; every check runs before any device work.
 */
int kda_decode_conv(const kda_tensor* out, const kda_conv* conv, const kda_tensor* raw_gate,
                    const kda_tensor* beta_logits, const kda_tensor* a_log,
                    const kda_tensor* dt_bias, const kda_tensor* cu_seqlens,
                    const kda_tensor* state_pool, const kda_tensor* state_indices,
                    const kda_mode* mode, hipStream_t stream);

/*
 * kda_prefill - the same operation and arguments as kda_decode, computed
 * for long requests: each (request, value head) walks its tokens in chunks
 * of 16 on the matrix cores, and the result equals the token-by-token
 * recurrence up to rounding order.  The model runs its whole-sequence step
 * this way (chunk_kda, "Delta-rule write" page, modeling_kimi_linear.py
 * excerpt; the pages leave that kernel's internals open, so only the
 * recurrence's result is fixed).  Per chunk, with Gamma the running sum of
 * the log-decays since the chunk start and S0 the state before it:
 *     U = (I + L)^-1 (V - (kh o exp(Gamma)) S0)         (the corrections)
 *     O = (qh o exp(Gamma)) S0 + R' U
 *     S = diag(exp(Gamma_last)) S0 + Kup^T U
 * where L and R' hold the decayed key-key and query-key products of the
 * chunk scaled by beta (strictly lower and lower triangular), and
 * Kup = beta kh o exp(Gamma_last - Gamma).
 *
 * dk and dv must each be 32, 64 or 128 (else KDA_ERR_UNSUPPORTED).
 * `matmul` is an enum kda_matmul (else KDA_ERR_MODE): the split-bf16 form
 * keeps 16 significant bits per operand; KDA_MATMUL_F32 gives fp32
 * products at about three times the matrix time.  The kernel needs no
 * workspace: each workgroup keeps its state slab in registers and the
 * chunk's operands in LDS.  Preconditions, conventions (skipped and empty
 * requests) and errors are those of kda_decode.
 */
int kda_prefill(const kda_tensor* out, const kda_tensor* q, const kda_tensor* k,
                const kda_tensor* v, const kda_tensor* raw_gate,
                const kda_tensor* beta_logits, const kda_tensor* a_log,
                const kda_tensor* dt_bias, const kda_tensor* cu_seqlens,
                const kda_tensor* state_pool, const kda_tensor* state_indices,
                const kda_mode* mode, int32_t matmul, hipStream_t stream);

/*
 * kda_check_host - validate host copies of the decode metadata.  This is a
 * convention of this library, not an operation of the pages: it checks the
 * preconditions of the "KdaDecode" tensor contract (cu_seqlens varlen
 * packing, state_indices into the slotted pool) that kda_decode cannot check
 * on device-resident data without a device-to-host copy.
 *   cu_seqlens: B + 1 int32 entries; state_indices: B int32 entries.
 * Returns KDA_OK when cu_seqlens[0] == 0, it is non-decreasing and ends at T,
 * and the non-negative indices are distinct and < n_slots; KDA_ERR_NULL for
 * NULL arrays (B > 0), KDA_ERR_SHAPE for B < 0, T < 0 or n_slots < 0, and
 * KDA_ERR_PRECONDITION otherwise.  Pure host code: no HIP call.
 */
int kda_check_host(const int32_t* cu_seqlens, const int32_t* state_indices,
                   int64_t B, int64_t T, int64_t n_slots);

/* Static description of a status code; never NULL.  A convention of this
 * library's error reporting (the pages define no error codes). */
const char* kda_status_string(int status);

/* KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* KDA_H_ */
