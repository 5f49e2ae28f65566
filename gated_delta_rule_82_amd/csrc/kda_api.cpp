// kda_api.cpp - argument checking and the exported C entry points of libkda.
//
// Pure host C++: no HIP call happens here before every check has passed, so
// a bad call returns its error code without touching the device.  The
// tensor contract is the one of the "KdaDecode" page (Tensor Shapes): packed
// [1, total_T, ...] token tensors, [HV] / [HV, dk] gate parameters, int32
// cu_seqlens and state_indices, and a [max_slots, HV, dk, dv] state pool
// (key-first, or its value-first transpose; f32 or bf16).

#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <limits>
#include <vector>

#include "kda.h"
#include "kda_internal.h"

namespace {

bool supported_head_dim(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Rank and non-negative extents; a NULL data pointer only for empty tensors.
int check_tensor(const kda_tensor* t, int ndim) {
  if (t == nullptr) return KDA_ERR_NULL;
  if (t->ndim != ndim) return KDA_ERR_SHAPE;
  bool empty = false;
  for (int i = 0; i < ndim; ++i) {
    if (t->shape[i] < 0) return KDA_ERR_SHAPE;
    empty |= t->shape[i] == 0;
  }
  if (t->data == nullptr && !empty) return KDA_ERR_NULL;
  return KDA_OK;
}

// Whether the product of non-negative factors exceeds `limit` (computed by
// division, so no intermediate product can overflow).
bool product_exceeds(std::initializer_list<int64_t> factors, int64_t limit) {
  for (int64_t f : factors)
    if (f == 0) return false;
  int64_t p = 1;
  for (int64_t f : factors) {
    if (p > limit / f) return true;
    p *= f;
  }
  return false;
}

// One dispatch covers at most this many work-items (a 32-bit count).
constexpr int64_t kMaxWorkItems = std::numeric_limits<uint32_t>::max();

bool aligned(const kda_tensor* t, uintptr_t bytes) {
  return (reinterpret_cast<uintptr_t>(t->data) % bytes) == 0;
}

#define KDA_TRY(expr)              \
  do {                             \
    const int kda_rc_ = (expr);    \
    if (kda_rc_ != KDA_OK) return kda_rc_; \
  } while (0)

}  // namespace

namespace kda {

int launch_prefill(const DecodeArgs& args, int dk, int dv, bool qkv_bf16, bool state_bf16,
                   int state_layout, int matmul, hipStream_t stream) {
  switch (dk) {
    case 32: return launch_prefill_dk<32>(args, dv, qkv_bf16, state_bf16, state_layout, matmul, stream);
    case 64: return launch_prefill_dk<64>(args, dv, qkv_bf16, state_bf16, state_layout, matmul, stream);
    case 128: return launch_prefill_dk<128>(args, dv, qkv_bf16, state_bf16, state_layout, matmul, stream);
    default: return KDA_ERR_UNSUPPORTED;
  }
}

}  // namespace kda

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_DTYPE: return "a tensor has an unsupported or mismatched dtype";
    case KDA_ERR_SHAPE: return "tensor ranks or extents disagree";
    case KDA_ERR_UNSUPPORTED: return "head size not in {16, 32, 64, 128}, misaligned data, or size too large";
    case KDA_ERR_MODE: return "invalid gate mode, lower_bound, l2_eps, scale or state layout";
    case KDA_ERR_LAUNCH: return "the HIP kernel launch failed";
    case KDA_ERR_PRECONDITION: return "cu_seqlens or state_indices violate their preconditions";
    default: return "unknown status";
  }
}

int kda_check_host(const int32_t* cu_seqlens, const int32_t* state_indices, int64_t B,
                   int64_t T, int64_t n_slots) {
  if (B < 0 || T < 0 || n_slots < 0) return KDA_ERR_SHAPE;
  if (cu_seqlens == nullptr) return KDA_ERR_NULL;
  if (B > 0 && state_indices == nullptr) return KDA_ERR_NULL;
  if (cu_seqlens[0] != 0 || cu_seqlens[B] != T) return KDA_ERR_PRECONDITION;
  for (int64_t b = 0; b < B; ++b)
    if (cu_seqlens[b + 1] < cu_seqlens[b]) return KDA_ERR_PRECONDITION;
  std::vector<uint8_t> seen(static_cast<size_t>(n_slots), 0);
  for (int64_t b = 0; b < B; ++b) {
    const int64_t s = state_indices[b];
    if (s < 0) continue;
    if (s >= n_slots || seen[static_cast<size_t>(s)]) return KDA_ERR_PRECONDITION;
    seen[static_cast<size_t>(s)] = 1;
  }
  return KDA_OK;
}

}  // extern "C"

namespace {

// Every check of a decode call; fills `args` and the launch selectors.
// Returns KDA_OK or the first error; touches no device state.
struct Plan {
  kda::DecodeArgs args;
  int dk, dv;
  bool qkv_bf16, state_bf16, empty;
  int layout;
};

int plan_decode(const kda_tensor* out, const kda_tensor* q, const kda_tensor* k,
                const kda_tensor* v, const kda_tensor* raw_gate,
                const kda_tensor* beta_logits, const kda_tensor* a_log,
                const kda_tensor* dt_bias, const kda_tensor* cu_seqlens,
                const kda_tensor* state_pool, const kda_tensor* state_indices,
                const kda_mode* mode, Plan* plan, bool qk_f32 = false) {
  if (mode == nullptr) return KDA_ERR_NULL;
  KDA_TRY(check_tensor(out, 4));
  KDA_TRY(check_tensor(q, 4));
  KDA_TRY(check_tensor(k, 4));
  KDA_TRY(check_tensor(v, 4));
  KDA_TRY(check_tensor(raw_gate, 4));
  KDA_TRY(check_tensor(beta_logits, 3));
  KDA_TRY(check_tensor(a_log, 1));
  KDA_TRY(check_tensor(dt_bias, 2));
  KDA_TRY(check_tensor(cu_seqlens, 1));
  KDA_TRY(check_tensor(state_pool, 4));
  KDA_TRY(check_tensor(state_indices, 1));

  // dtypes: q, k, v share bf16 or f32 (q, k are f32 when qk_f32); out
  // follows v; the rest are fixed
  const int32_t qkv = v->dtype;
  const int32_t qk = qk_f32 ? KDA_F32 : qkv;
  if (qkv != KDA_BF16 && qkv != KDA_F32) return KDA_ERR_DTYPE;
  if (q->dtype != qk || k->dtype != qk || out->dtype != qkv) return KDA_ERR_DTYPE;
  if (raw_gate->dtype != KDA_F32 || beta_logits->dtype != KDA_F32 || a_log->dtype != KDA_F32 ||
      dt_bias->dtype != KDA_F32)
    return KDA_ERR_DTYPE;
  if (state_pool->dtype != KDA_F32 && state_pool->dtype != KDA_BF16) return KDA_ERR_DTYPE;
  if (cu_seqlens->dtype != KDA_I32 || state_indices->dtype != KDA_I32) return KDA_ERR_DTYPE;

  // extents
  const int64_t T = q->shape[1], H = q->shape[2], DK = q->shape[3];
  const int64_t HV = v->shape[2], DV = v->shape[3];
  const int64_t B = state_indices->shape[0];
  const int64_t N = state_pool->shape[0];
  if (q->shape[0] != 1 || k->shape[0] != 1 || v->shape[0] != 1 || out->shape[0] != 1 ||
      raw_gate->shape[0] != 1 || beta_logits->shape[0] != 1)
    return KDA_ERR_SHAPE;
  for (int i = 1; i < 4; ++i)
    if (k->shape[i] != q->shape[i] || out->shape[i] != v->shape[i]) return KDA_ERR_SHAPE;
  if (v->shape[1] != T || raw_gate->shape[1] != T || beta_logits->shape[1] != T)
    return KDA_ERR_SHAPE;
  if (raw_gate->shape[2] != HV || raw_gate->shape[3] != DK) return KDA_ERR_SHAPE;
  if (beta_logits->shape[2] != HV) return KDA_ERR_SHAPE;
  if (a_log->shape[0] != HV || dt_bias->shape[0] != HV || dt_bias->shape[1] != DK)
    return KDA_ERR_SHAPE;
  if (cu_seqlens->shape[0] - 1 != B) return KDA_ERR_SHAPE;
  if (mode->state_layout != KDA_STATE_K_FIRST && mode->state_layout != KDA_STATE_V_FIRST)
    return KDA_ERR_MODE;
  const bool v_first = mode->state_layout == KDA_STATE_V_FIRST;
  if (state_pool->shape[1] != HV || state_pool->shape[2] != (v_first ? DV : DK) ||
      state_pool->shape[3] != (v_first ? DK : DV))
    return KDA_ERR_SHAPE;
  if (H < 1 || HV < 1 || HV % H != 0) return KDA_ERR_SHAPE;

  if (!supported_head_dim(DK) || !supported_head_dim(DV)) return KDA_ERR_UNSUPPORTED;
  // Sizes one launch can take: T, N and B fit the kernels' 32-bit indices,
  // and the grid fits one dispatch, whose extent is a 32-bit count of
  // work-items: 64 per (request, value head, 32-column slab) for the decode
  // and the prefill (the q/k convolution's grid is checked with its other
  // arguments).
  constexpr int64_t kI32 = std::numeric_limits<int32_t>::max();
  const int64_t slabs = DV < 32 ? 1 : DV / 32;
  if (T > kI32 || N > kI32 || B > kI32 || product_exceeds({B, HV, slabs, 64}, kMaxWorkItems))
    return KDA_ERR_UNSUPPORTED;
  // 16-byte alignment: the kernel moves the state with 128-bit accesses and
  // the token rows with 32/64-bit accesses
  const kda_tensor* all[] = {out, q, k, v, raw_gate, beta_logits, a_log, dt_bias,
                             cu_seqlens, state_pool, state_indices};
  for (const kda_tensor* t : all)
    if (!aligned(t, 16)) return KDA_ERR_UNSUPPORTED;

  // scalar parameters
  if (mode->gate_mode != KDA_GATE_SOFTPLUS && mode->gate_mode != KDA_GATE_LOWER_BOUND)
    return KDA_ERR_MODE;
  if (mode->gate_mode == KDA_GATE_LOWER_BOUND &&
      !(std::isfinite(mode->lower_bound) && mode->lower_bound <= 0.0f))
    return KDA_ERR_MODE;
  if (!(std::isfinite(mode->l2_eps) && mode->l2_eps >= 0.0f)) return KDA_ERR_MODE;
  if (!(std::isfinite(mode->scale) && mode->scale >= 0.0f)) return KDA_ERR_MODE;

  plan->empty = B == 0 || T == 0;   // nothing to advance and no output row
  kda::DecodeArgs& args = plan->args;
  args = kda::DecodeArgs{};
  args.out = out->data;
  args.q = q->data;
  args.k = k->data;
  args.v = v->data;
  args.raw_gate = static_cast<const float*>(raw_gate->data);
  args.beta_logits = static_cast<const float*>(beta_logits->data);
  args.a_log = static_cast<const float*>(a_log->data);
  args.dt_bias = static_cast<const float*>(dt_bias->data);
  args.cu_seqlens = static_cast<const int32_t*>(cu_seqlens->data);
  args.state_pool = state_pool->data;
  args.state_indices = static_cast<const int32_t*>(state_indices->data);
  args.B = static_cast<int32_t>(B);
  args.T = static_cast<int32_t>(T);
  args.H = static_cast<int32_t>(H);
  args.HV = static_cast<int32_t>(HV);
  args.G = static_cast<int32_t>(HV / H);
  args.N = static_cast<int32_t>(N);
  args.gate_mode = mode->gate_mode;
  args.lower_bound = mode->gate_mode == KDA_GATE_LOWER_BOUND ? mode->lower_bound : 0.0f;
  args.l2_eps = mode->l2_eps == 0.0f ? 1e-6f : mode->l2_eps;
  args.scale = mode->scale == 0.0f ? 1.0f / std::sqrt(static_cast<float>(DK)) : mode->scale;
  plan->dk = static_cast<int>(DK);
  plan->dv = static_cast<int>(DV);
  plan->qkv_bf16 = qkv == KDA_BF16;
  plan->state_bf16 = state_pool->dtype == KDA_BF16;
  plan->layout = mode->state_layout;
  return KDA_OK;
}


}  // namespace

extern "C" {

int kda_decode(const kda_tensor* out, const kda_tensor* q, const kda_tensor* k,
               const kda_tensor* v, const kda_tensor* raw_gate,
               const kda_tensor* beta_logits, const kda_tensor* a_log,
               const kda_tensor* dt_bias, const kda_tensor* cu_seqlens,
               const kda_tensor* state_pool, const kda_tensor* state_indices,
               const kda_mode* mode, hipStream_t stream) {
  Plan plan;
  KDA_TRY(plan_decode(out, q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens,
                      state_pool, state_indices, mode, &plan));
  if (plan.empty) return KDA_OK;
  return kda::launch_decode(plan.args, plan.dk, plan.dv, plan.qkv_bf16, plan.state_bf16,
                            plan.layout, false, stream);
}

int kda_decode_conv(const kda_tensor* out, const kda_conv* conv, const kda_tensor* raw_gate,
                    const kda_tensor* beta_logits, const kda_tensor* a_log,
                    const kda_tensor* dt_bias, const kda_tensor* cu_seqlens,
                    const kda_tensor* state_pool, const kda_tensor* state_indices,
                    const kda_mode* mode, hipStream_t stream) {
  if (conv == nullptr) return KDA_ERR_NULL;
  // the recurrence sees q = q_conv, k = k_conv and v shaped like x_v
  Plan plan;
  KDA_TRY(plan_decode(out, &conv->q_conv, &conv->k_conv, &conv->x_v, raw_gate, beta_logits,
                      a_log, dt_bias, cu_seqlens, state_pool, state_indices, mode, &plan,
                      /*qk_f32=*/true));
  const kda::DecodeArgs& d = plan.args;
  const int64_t T = d.T, H = conv->q_conv.shape[2], HV = conv->x_v.shape[2];
  const int64_t DK = plan.dk, DV = plan.dv, N = state_pool->shape[0];
  KDA_TRY(check_tensor(&conv->x_q, 4));
  KDA_TRY(check_tensor(&conv->x_k, 4));
  KDA_TRY(check_tensor(&conv->w_q, 2));
  KDA_TRY(check_tensor(&conv->w_k, 2));
  KDA_TRY(check_tensor(&conv->w_v, 2));
  KDA_TRY(check_tensor(&conv->win_q, 3));
  KDA_TRY(check_tensor(&conv->win_k, 3));
  KDA_TRY(check_tensor(&conv->win_v, 3));
  const int32_t act = conv->x_v.dtype;
  if (conv->x_q.dtype != act || conv->x_k.dtype != act) return KDA_ERR_DTYPE;
  const int32_t wdt = conv->w_q.dtype;
  if ((wdt != KDA_F32 && wdt != KDA_BF16) || conv->w_k.dtype != wdt || conv->w_v.dtype != wdt)
    return KDA_ERR_DTYPE;
  if (conv->win_q.dtype != KDA_F32 || conv->win_k.dtype != KDA_F32 || conv->win_v.dtype != KDA_F32)
    return KDA_ERR_DTYPE;
  for (int i = 0; i < 4; ++i)
    if (conv->x_q.shape[i] != conv->q_conv.shape[i] || conv->x_k.shape[i] != conv->q_conv.shape[i])
      return KDA_ERR_SHAPE;
  const int64_t K = conv->w_q.shape[0];
  const int64_t CQ = H * DK, CV = HV * DV;
  if (conv->w_q.shape[1] != CQ || conv->w_k.shape[0] != K || conv->w_k.shape[1] != CQ ||
      conv->w_v.shape[0] != K || conv->w_v.shape[1] != CV)
    return KDA_ERR_SHAPE;
  const kda_tensor* wins[3] = {&conv->win_q, &conv->win_k, &conv->win_v};
  for (int s = 0; s < 3; ++s)
    if (wins[s]->shape[0] != N || wins[s]->shape[1] != K - 1 || wins[s]->shape[2] != (s < 2 ? CQ : CV))
      return KDA_ERR_SHAPE;
  if (K < 2 || K > 4) return KDA_ERR_UNSUPPORTED;
  // the q/k convolution runs 128 work-items per (request, key head)
  if (product_exceeds({static_cast<int64_t>(d.B), H, 128}, kMaxWorkItems)) return KDA_ERR_UNSUPPORTED;
  const kda_tensor* extra[] = {&conv->x_q, &conv->x_k, &conv->w_q, &conv->w_k, &conv->w_v,
                               &conv->win_q, &conv->win_k, &conv->win_v};
  for (const kda_tensor* t : extra)
    if (!aligned(t, 16)) return KDA_ERR_UNSUPPORTED;
  if (plan.empty) return KDA_OK;

  kda::ConvQKArgs c{};
  c.x[0] = conv->x_q.data;
  c.x[1] = conv->x_k.data;
  c.w[0] = conv->w_q.data;
  c.w[1] = conv->w_k.data;
  c.win[0] = static_cast<float*>(conv->win_q.data);
  c.win[1] = static_cast<float*>(conv->win_k.data);
  c.y[0] = conv->q_conv.data;
  c.y[1] = conv->k_conv.data;
  c.cu_seqlens = d.cu_seqlens;
  c.state_indices = d.state_indices;
  c.B = d.B;
  c.T = static_cast<int32_t>(T);
  c.H = static_cast<int32_t>(H);
  c.N = d.N;
  c.conv_k = static_cast<int32_t>(K);
  c.w_bf16 = wdt == KDA_BF16;
  KDA_TRY(kda::launch_conv_qk(c, plan.dk, act == KDA_BF16, stream));

  kda::DecodeArgs args = plan.args;
  args.conv_w_v = conv->w_v.data;
  args.conv_win_v = static_cast<float*>(conv->win_v.data);
  args.conv_k = static_cast<int32_t>(K);
  args.conv_w_bf16 = wdt == KDA_BF16;
  return kda::launch_decode(args, plan.dk, plan.dv, plan.qkv_bf16, plan.state_bf16, plan.layout,
                            true, stream);
}

int kda_prefill(const kda_tensor* out, const kda_tensor* q, const kda_tensor* k,
                const kda_tensor* v, const kda_tensor* raw_gate,
                const kda_tensor* beta_logits, const kda_tensor* a_log,
                const kda_tensor* dt_bias, const kda_tensor* cu_seqlens,
                const kda_tensor* state_pool, const kda_tensor* state_indices,
                const kda_mode* mode, int32_t matmul, hipStream_t stream) {
  Plan plan;
  KDA_TRY(plan_decode(out, q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens,
                      state_pool, state_indices, mode, &plan));
  if (matmul != KDA_MATMUL_SPLIT_BF16 && matmul != KDA_MATMUL_F32) return KDA_ERR_MODE;
  if (plan.dk < 32 || plan.dv < 32) return KDA_ERR_UNSUPPORTED;
  if (plan.empty) return KDA_OK;
  return kda::launch_prefill(plan.args, plan.dk, plan.dv, plan.qkv_bf16, plan.state_bf16,
                             plan.layout, matmul, stream);
}

}  // extern "C"
