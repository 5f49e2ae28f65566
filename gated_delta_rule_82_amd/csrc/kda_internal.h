// kda_internal.h - what the argument checker hands to the kernel launcher.
#ifndef KDA_INTERNAL_H_
#define KDA_INTERNAL_H_

#include <cstdint>

#include "kda.h"

namespace kda {

// Validated, flattened arguments of one decode call (device pointers).
struct DecodeArgs {
  void* out;                    // [T, HV, dv]   bf16 or f32
  const void* q;                // [T, H, dk]    bf16 or f32
  const void* k;                // [T, H, dk]
  const void* v;                // [T, HV, dv]
  const float* raw_gate;        // [T, HV, dk]
  const float* beta_logits;     // [T, HV]
  const float* a_log;           // [HV]
  const float* dt_bias;         // [HV, dk]
  const int32_t* cu_seqlens;    // [B + 1]
  void* state_pool;             // [N, HV, dk, dv] or [N, HV, dv, dk], f32 or bf16
  const int32_t* state_indices; // [B]
  int32_t B, T, H, HV, G, N;
  int32_t gate_mode;            // enum kda_gate_mode
  float lower_bound, l2_eps, scale;
  // short convolution of the v stream (kda_decode_conv only; v is then the
  // pre-convolution x_v)
  const void* conv_w_v;         // [K, HV*dv] taps
  float* conv_win_v;            // [N, K-1, HV*dv] windows
  int32_t conv_k;               // K, 2..4
  int32_t conv_w_bf16;          // taps stored as bf16
};

// Arguments of the q/k convolution kernel of kda_decode_conv.
struct ConvQKArgs {
  const void* x[2];             // pre-convolution q, k [T, H, dk]
  const void* w[2];             // taps [K, H*dk]
  float* win[2];                // windows [N, K-1, H*dk]
  void* y[2];                   // convolved q, k [T, H, dk]
  const int32_t* cu_seqlens;
  const int32_t* state_indices;
  int32_t B, T, H, N;
  int32_t conv_k;
  int32_t w_bf16;
};

// Enqueue the decode kernel for (dk, dv, q/k/v dtype, state dtype, state
// layout) on `stream`.  Returns KDA_OK, KDA_ERR_UNSUPPORTED (no such
// specialization) or KDA_ERR_LAUNCH.  Defined in kda_decode.hip.
int launch_decode(const DecodeArgs& args, int dk, int dv, bool qkv_bf16, bool state_bf16,
                  int state_layout, bool conv_v, hipStream_t stream);

// Enqueue the chunked prefill kernel (dk, dv in {32, 64, 128}; matmul an
// enum kda_matmul).  Same return codes.  Defined in kda_api.cpp.
int launch_prefill(const DecodeArgs& args, int dk, int dv, bool qkv_bf16, bool state_bf16,
                   int state_layout, int matmul, hipStream_t stream);

// The same for one dk: kda_prefill.hip is compiled once per dk
// (KDA_PREFILL_DK = 32, 64, 128), each object defining its dk's
// specialization, so that the three compile in parallel; launch_prefill
// (kda_api.cpp) picks one.
template <int DK>
int launch_prefill_dk(const DecodeArgs& args, int dv, bool qkv_bf16, bool state_bf16, int state_layout,
                      int matmul, hipStream_t stream);
template <>
int launch_prefill_dk<32>(const DecodeArgs&, int, bool, bool, int, int, hipStream_t);
template <>
int launch_prefill_dk<64>(const DecodeArgs&, int, bool, bool, int, int, hipStream_t);
template <>
int launch_prefill_dk<128>(const DecodeArgs&, int, bool, bool, int, int, hipStream_t);

// Enqueue the q/k convolution kernel.  Same return codes.
int launch_conv_qk(const ConvQKArgs& args, int dk, bool x_bf16, hipStream_t stream);

}  // namespace kda

#endif  // KDA_INTERNAL_H_
