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
#include <limits>
#include <vector>

#include "kda.h"
#include "kda_internal.h"

namespace {

bool supported_head_dim(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

int64_t numel(const kda_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

// Rank and non-negative extents; a NULL data pointer only for empty tensors.
int check_tensor(const kda_tensor* t, int ndim) {
  if (t == nullptr) return KDA_ERR_NULL;
  if (t->ndim != ndim) return KDA_ERR_SHAPE;
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] < 0) return KDA_ERR_SHAPE;
  if (t->data == nullptr && numel(t) > 0) return KDA_ERR_NULL;
  return KDA_OK;
}

bool aligned(const kda_tensor* t, uintptr_t bytes) {
  return (reinterpret_cast<uintptr_t>(t->data) % bytes) == 0;
}

#define KDA_TRY(expr)              \
  do {                             \
    const int kda_rc_ = (expr);    \
    if (kda_rc_ != KDA_OK) return kda_rc_; \
  } while (0)

}  // namespace

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

int kda_decode(const kda_tensor* out, const kda_tensor* q, const kda_tensor* k,
               const kda_tensor* v, const kda_tensor* raw_gate,
               const kda_tensor* beta_logits, const kda_tensor* a_log,
               const kda_tensor* dt_bias, const kda_tensor* cu_seqlens,
               const kda_tensor* state_pool, const kda_tensor* state_indices,
               const kda_mode* mode, hipStream_t stream) {
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

  // dtypes: q, k, v share bf16 or f32; out follows v; the rest are fixed
  const int32_t qkv = v->dtype;
  if (qkv != KDA_BF16 && qkv != KDA_F32) return KDA_ERR_DTYPE;
  if (q->dtype != qkv || k->dtype != qkv || out->dtype != qkv) return KDA_ERR_DTYPE;
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
  if (cu_seqlens->shape[0] != B + 1) return KDA_ERR_SHAPE;
  if (mode->state_layout != KDA_STATE_K_FIRST && mode->state_layout != KDA_STATE_V_FIRST)
    return KDA_ERR_MODE;
  const bool v_first = mode->state_layout == KDA_STATE_V_FIRST;
  if (state_pool->shape[1] != HV || state_pool->shape[2] != (v_first ? DV : DK) ||
      state_pool->shape[3] != (v_first ? DK : DV))
    return KDA_ERR_SHAPE;
  if (H < 1 || HV < 1 || HV % H != 0) return KDA_ERR_SHAPE;

  if (!supported_head_dim(DK) || !supported_head_dim(DV)) return KDA_ERR_UNSUPPORTED;
  constexpr int64_t kI32 = std::numeric_limits<int32_t>::max();
  const int64_t slabs = DV < 32 ? 1 : DV / 32;
  if (T > kI32 || N > kI32 || B * HV * slabs > kI32) return KDA_ERR_UNSUPPORTED;
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

  if (B == 0 || T == 0) return KDA_OK;   // nothing to advance and no output row

  kda::DecodeArgs args;
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
  return kda::launch_decode(args, static_cast<int>(DK), static_cast<int>(DV), qkv == KDA_BF16,
                            state_pool->dtype == KDA_BF16, mode->state_layout, stream);
}

}  // extern "C"
