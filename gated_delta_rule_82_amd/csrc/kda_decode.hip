// kda_decode.hip - the KDA decode recurrence for CDNA4 (gfx950).
//
// Operation ("Delta-rule write" page, naive_recurrent_kda code excerpt;
// "KdaDecode" Tensor Shapes and default parameters; "KDA Block TKG"
// l2_eps / scale / lower_bound): per token, decay state row k by
// exp(g[k]), write (beta*k) outer (v - k^T S), and read o = q^T S from the
// updated state.
//
// Work decomposition.  The value columns of a state tile never interact:
// column v of S only meets v[v] and o[v]; every reduction runs over the key
// axis.  So one wavefront owns a 32-value slab of one (request, value head)
// tile for all dk keys and needs no other wave: no cross-wave reduction and
// no workgroup barrier.  A workgroup is that one wave.  How the slab maps to
// lanes depends on the state layout:
//   key-first [dk][dv]  ("K_FIRST", the default): lane (rs, cq) holds keys
//       rs + RS*i and values 4cq..4cq+3; each load instruction of the wave
//       reads RS rows of 128 bytes (32 fp32 values);
//   value-first [dv][dk] (the transposed layout the model asks for): lane
//       (rsub, kc) holds value rows rsub + RPI*i and keys 4kc..4kc+3; each
//       load instruction reads RPI whole rows, one contiguous KiB.
// For dk = dv = 128 a lane carries 64 fp32 state values in VGPRs.
//
// Per token, with alpha = exp(g):
//   a = (kh*alpha)^T S_old,  b = (qh*alpha)^T S_old      (one sweep over S)
//   u = v - a,  o = b + beta*(qh.kh)*u,  S = alpha*S_old + (beta*kh) u^T
// which is the page's decay / write / read sequence with the decay folded
// into the two reduction vectors (exact algebra; only the rounding order
// differs).  The per-channel setup (L2 norms, gate, beta) is computed by the
// wave itself, two channels per lane, and handed to the lanes that need it
// through a small LDS table, double-buffered so one token's table never
// waits for the previous token's readers.  The reductions over lanes use DPP
// and the gfx950 row-swap instructions where the lane pattern allows.
//
// The state makes exactly one trip from HBM and one back per call; tokens
// of the same request keep it in registers (fp32 even for a bf16 pool, which
// is rounded to nearest-even once, on the way out).  Both trips carry the
// nontemporal hint: the tile is touched once per call, and keeping it out of
// L2 / MALL measurably raises the streaming rate.  (The key-first bf16 slab
// is the exception: its rows are half cache lines, which L2 merges.)
//
// Workgroup order is XCD-aware: consecutive workgroup ids land on different
// XCDs, so the id is remapped to give each XCD one contiguous range of
// (tile, slab) pairs and the slabs of a tile meet in one L2.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

// ---------------------------------------------------------------------------
// memory
// ---------------------------------------------------------------------------

// The state is streamed through a raw buffer resource spanning exactly the
// tile: per-row offsets stay in scalar registers (one VGPR offset per lane),
// the hardware range check confines every access to the tile, and the
// cache-policy bit "nt" marks the data as touched once.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr int kCachePolicyNT = 2;
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_resource(void* tile, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(tile, static_cast<short>(0), bytes, kRawBufferWord3);
}

// A lane moves its state in pieces of N consecutive values of one row: N = 4
// fp32 (16 bytes) or N = 4 / 8 bf16 (8 / 16 bytes), widened to fp32 on the
// way in and rounded to nearest-even on the way out.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool SBF16, int N, int POLICY = kCachePolicyNT>
struct StateIO {
  static_assert(N == 4 || (SBF16 && N == 8), "state access width");
  static constexpr int kElem = SBF16 ? 2 : 4;
  __device__ static __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int voff, int soff, float* x) {
    if constexpr (SBF16 && N == 8) {
      const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POLICY);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_to_f32(w[e] & 0xffffu);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    } else if constexpr (SBF16) {
      const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, POLICY);
      x[0] = bf16_to_f32(w.x & 0xffffu);
      x[1] = __uint_as_float(w.x & 0xffff0000u);
      x[2] = bf16_to_f32(w.y & 0xffffu);
      x[3] = __uint_as_float(w.y & 0xffff0000u);
    } else {
      const f32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POLICY);
      x[0] = w.x;
      x[1] = w.y;
      x[2] = w.z;
      x[3] = w.w;
    }
  }
  __device__ static __forceinline__ void store(__amdgpu_buffer_rsrc_t r, int voff, int soff, const float* x) {
    if constexpr (SBF16 && N == 8) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = f32x2_to_bf16x2_rne(x[2 * e], x[2 * e + 1]);
      __builtin_amdgcn_raw_buffer_store_b128(w, r, voff, soff, POLICY);
    } else if constexpr (SBF16) {
      const u32x2 w = {f32x2_to_bf16x2_rne(x[0], x[1]), f32x2_to_bf16x2_rne(x[2], x[3])};
      __builtin_amdgcn_raw_buffer_store_b64(w, r, voff, soff, POLICY);
    } else {
      const f32x4 w = {x[0], x[1], x[2], x[3]};
      __builtin_amdgcn_raw_buffer_store_b128(w, r, voff, soff, POLICY);
    }
  }
};

template <int CPL>
__device__ __forceinline__ void load_f32(const float* p, float (&x)[CPL]) {
  if constexpr (CPL == 2) {
    const float2 w = *reinterpret_cast<const float2*>(p);
    x[0] = w.x;
    x[1] = w.y;
  } else {
    x[0] = p[0];
  }
}

template <bool BF16>
__device__ __forceinline__ float load_scalar(const void* base, int64_t off) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[off]);
  else return static_cast<const float*>(base)[off];
}

template <bool BF16>
__device__ __forceinline__ void store_scalar(void* base, int64_t off, float x) {
  if constexpr (BF16) static_cast<uint16_t*>(base)[off] = static_cast<uint16_t>(f32_to_bf16_rne(x));
  else static_cast<float*>(base)[off] = x;
}

// Two consecutive values at an even element offset.
template <bool BF16>
__device__ __forceinline__ void store_pair(void* base, int64_t off, float x0, float x1) {
  if constexpr (BF16) *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(base) + off) = f32x2_to_bf16x2_rne(x0, x1);
  else *reinterpret_cast<float2*>(static_cast<float*>(base) + off) = make_float2(x0, x1);
}

// ---------------------------------------------------------------------------
// the pieces both layouts share
// ---------------------------------------------------------------------------

// Which tile and slab this workgroup owns, and the request's token range.
struct TileJob {
  int b, hv, h, slab, t0, t1, slot;
};

template <int SLABS>
__device__ __forceinline__ TileJob resolve_job(const DecodeArgs& a) {
  // XCD-aware id -> (tile, slab)
  const uint32_t wg = blockIdx.x;
  const uint32_t nwg = gridDim.x;
  const uint32_t xcd = wg % kXcds;
  const uint32_t per = nwg / kXcds;
  const uint32_t extra = nwg % kXcds;
  const uint32_t logical = xcd * per + (xcd < extra ? xcd : extra) + wg / kXcds;
  TileJob j;
  j.slab = static_cast<int>(logical % SLABS);
  const int tile = static_cast<int>(logical / SLABS);
  j.b = tile / a.HV;
  j.hv = tile - j.b * a.HV;
  j.h = j.hv / a.G;
  int t0 = a.cu_seqlens[j.b];
  int t1 = a.cu_seqlens[j.b + 1];
  t0 = t0 < 0 ? 0 : (t0 > a.T ? a.T : t0);
  t1 = t1 < t0 ? t0 : (t1 > a.T ? a.T : t1);
  j.t0 = t0;
  j.t1 = t1;
  j.slot = a.state_indices[j.b];
  return j;
}

// Skipped request: zero its output rows in this slab, leave every slot alone.
template <int DV, int CW, bool BF16>
__device__ __forceinline__ void zero_rows(const DecodeArgs& a, const TileJob& j, int lane) {
  for (int t = j.t0; t < j.t1; ++t)
    if (lane < CW) store_scalar<BF16>(a.out, (static_cast<int64_t>(t) * a.HV + j.hv) * DV + j.slab * CW + lane, 0.0f);
}

// N (1 or 2) consecutive elements of one row, kept in storage form until
// used, so that a load issued a token ahead is waited for only where its
// value is taken.
template <bool BF16, int N>
struct RawRun {
  static constexpr int W = (BF16 && N == 2) ? 1 : N;
  uint32_t w[W];
  __device__ __forceinline__ void load(const void* base, int64_t off) {
    if constexpr (BF16 && N == 2) {
      w[0] = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + off);
    } else if constexpr (BF16) {
      w[0] = static_cast<const uint16_t*>(base)[off];
    } else if constexpr (N == 2) {
      const u32x2 x = *reinterpret_cast<const u32x2*>(static_cast<const float*>(base) + off);
      w[0] = x[0];
      w[1] = x[1];
    } else {
      w[0] = __float_as_uint(static_cast<const float*>(base)[off]);
    }
  }
  __device__ __forceinline__ void unpack(float (&x)[N]) const {
    if constexpr (BF16 && N == 2) {
      x[0] = bf16_to_f32(w[0] & 0xffffu);
      x[1] = __uint_as_float(w[0] & 0xffff0000u);
    } else if constexpr (BF16) {
      x[0] = bf16_to_f32(w[0]);
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) x[i] = __uint_as_float(w[i]);
    }
  }
};

// One token's inputs for one lane: q, k and the gate pre-activation of its
// CPL setup channels (from channel c0s), the beta logit, and the NVL v
// values at v_ch.  Every lane loads (a lane without channels reads channel
// 0 and drops it), so the loads never sit in a divergent branch.
template <int DK, int DV, bool QKBF16, bool VBF16, int CPL, int NVL>
struct TokenInputs {
  RawRun<QKBF16, CPL> q, k;
  RawRun<false, CPL> x;
  RawRun<VBF16, NVL> v;
  float bl;
  __device__ __forceinline__ void load(const DecodeArgs& a, const TileJob& j, int t, int c0s, int64_t v_ch) {
    const int64_t qk_off = (static_cast<int64_t>(t) * a.H + j.h) * DK + c0s;
    q.load(a.q, qk_off);
    k.load(a.k, qk_off);
    x.load(a.raw_gate, (static_cast<int64_t>(t) * a.HV + j.hv) * DK + c0s);
    v.load(a.v, static_cast<int64_t>(t) * a.HV * DV + v_ch);
    bl = a.beta_logits[static_cast<int64_t>(t) * a.HV + j.hv];
  }
};

// Inputs one token ahead: measured in the same process against loading
// each token's inputs (together) at its start, 1024 requests x 4 tokens x
// 96 heads: bf16 pool value-first 1397 -> 1305 us, key-first 1444 -> 1449
// us; fp32 pool 2270 -> 2285 us (key-first), 2259 -> 2300 us
// (value-first), where the loop is bound by the state's HBM traffic.
template <bool SBF16>
constexpr bool kInputsAhead = SBF16;

struct TokenScalars {
  float beta;   // write strength
  float qk;     // qh . kh, query scale included
  bool fold;    // deferred decay: the pending factors are applied this token
};

// Deferred decay.  The wave keeps its slab as S = D o S^ with D the pending
// decay of each key, so a token's write is one FMA per element,
// S^ += (beta kh / D') u^T, instead of a multiply and an FMA; the reads take
// kh o D' and qh o D'.  D' = D alpha is folded into S^ (and reset to 1) on a
// request's last token and whenever some key's D' would drop below
// kDeferFloor, which keeps every 1 / D' finite.  Measured in the same
// process against the plain update: key-first 64-column bf16 slabs, 96
// heads x 1024 requests x 4 tokens 1323 -> 1279 us; 32-column bf16 slabs,
// 1..8 tokens over 32 heads x 128 requests 77.0 -> 72.7 us; value-first
// bf16, 4 tokens 1353 -> 1323 us, 1..8 tokens 79.9 -> 76.6 us; fp32 pools,
// 1..8 tokens 113.0 -> 110.1 us (key-first) and 109.8 -> 109.2 us
// (value-first), the rest within 0.4%.
constexpr float kDeferFloor = 5.421010862427522e-20f;   // 2^-64

// Per-token setup, CPL channels per lane: L2 norms (wave reductions), gate,
// beta, the deferred decay D' = D alpha (pend holds D across tokens); fills
// red_tab[c] = {kh*D', qh*D'} and upd_tab[c] = {D', beta*kh/D'} for the
// wave's channels, or, on a folding token, {kh, qh} and {D', beta*kh} (the
// kernel then scales its slab's key rows by D').
template <int DK, int CPL, typename In>
__device__ __forceinline__ TokenScalars token_setup(const DecodeArgs& a, const In& in, int c0,
                                                    bool chan_lane, const float (&dtb)[CPL], float amp,
                                                    float2* red_tab, float2* upd_tab,
                                                    float (&pend)[CPL], bool last) {
  float qv[CPL], kv[CPL], xg[CPL];
  in.q.unpack(qv);
  in.k.unpack(kv);
  in.x.unpack(xg);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    qv[c] = chan_lane ? qv[c] : 0.0f;
    kv[c] = chan_lane ? kv[c] : 0.0f;
    xg[c] = chan_lane ? xg[c] : 0.0f;
  }
  TokenScalars s;
  s.beta = sigmoid_f(in.bl);
  float sq = 0.0f, sk = 0.0f, sqk = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    sq = fmaf(qv[c], qv[c], sq);
    sk = fmaf(kv[c], kv[c], sk);
    sqk = fmaf(qv[c], kv[c], sqk);
  }
  sq = wave_sum(sq);
  sk = wave_sum(sk);
  sqk = wave_sum(sqk);
  const float rq = a.scale * rsqrt_f(sq + a.l2_eps);
  const float rk = rsqrt_f(sk + a.l2_eps);
  s.qk = sqk * rq * rk;
  float alpha[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const float x = xg[c] + dtb[c];
    const float g = a.gate_mode == KDA_GATE_SOFTPLUS ? -amp * softplus_f(x)
                                                     : a.lower_bound * sigmoid_f(amp * x);
    alpha[c] = exp_f(g);
  }
  bool small = false;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    alpha[c] *= pend[c];                 // D' = D alpha
    small |= chan_lane && !(alpha[c] >= kDeferFloor);
  }
  s.fold = last || __any(small);
  if (chan_lane) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float kh = kv[c] * rk;
      const float qh = qv[c] * rq;
      // reads take the decay unless it is applied to the slab this token;
      // a deferred write is scaled by 1 / D'
      const float m = s.fold ? 1.0f : alpha[c];
      const float w = s.fold ? 1.0f : __builtin_amdgcn_rcpf(alpha[c]);
      red_tab[c0 + c] = make_float2(kh * m, qh * m);
      upd_tab[c0 + c] = make_float2(alpha[c], s.beta * kh * w);
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) pend[c] = s.fold ? 1.0f : alpha[c];
  return s;
}

template <int N>
constexpr int log2_exact() {
  static_assert(N > 0 && (N & (N - 1)) == 0, "power of two");
  int l = 0;
  while ((1 << l) < N) ++l;
  return l;
}

// ---------------------------------------------------------------------------
// short causal convolution (the step in front of the recurrence)
// ---------------------------------------------------------------------------

constexpr int kMaxConvK = 4;

__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }

__device__ __forceinline__ float load_tap(const void* w, int64_t off, bool bf16) {
  return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(w)[off]) : static_cast<const float*>(w)[off];
}

// One channel's convolution carried through a request's tokens in
// registers: the K-1 previous pre-convolution inputs (oldest first) and the
// K taps (tap 0 meets the oldest position).  Window [N, K-1, C], taps [K, C].
struct ConvChannel {
  float win[kMaxConvK - 1];
  float tap[kMaxConvK];

  __device__ __forceinline__ void load(const void* w, const float* window, int64_t slot, int64_t C,
                                       int64_t ch, int K, bool w_bf16) {
#pragma unroll
    for (int q = 0; q < kMaxConvK; ++q) tap[q] = q < K ? load_tap(w, q * C + ch, w_bf16) : 0.0f;
#pragma unroll
    for (int q = 0; q < kMaxConvK - 1; ++q) win[q] = q < K - 1 ? window[(slot * (K - 1) + q) * C + ch] : 0.0f;
  }

  // Convolve the next input x, roll the window, return SiLU of the sum
  // (fp32, unrounded).  (Register arrays are only indexed by compile-time
  // positions; K selects.)
  __device__ __forceinline__ float step(float x, int K) {
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < kMaxConvK; ++q) {
      const float in = q < K - 1 ? win[q < kMaxConvK - 1 ? q : 0] : x;   // window position q
      if (q < K) acc = fmaf(tap[q], in, acc);
    }
#pragma unroll
    for (int q = 0; q < kMaxConvK - 1; ++q) {
      const float next = q + 1 < kMaxConvK - 1 ? win[q + 1 < kMaxConvK - 1 ? q + 1 : 0] : x;
      win[q] = q < K - 2 ? next : (q == K - 2 ? x : win[q]);
    }
    return silu_f(acc);
  }

  __device__ __forceinline__ void store(float* window, int64_t slot, int64_t C, int64_t ch, int K) const {
#pragma unroll
    for (int q = 0; q < kMaxConvK - 1; ++q)
      if (q < K - 1) window[(slot * (K - 1) + q) * C + ch] = win[q];
  }
};

// The same for N adjacent channels (N = 1 or 2; the first one even), each
// window, tap, input and output row read or written as one N-element
// access: with two channels per lane a wave's access is 512 contiguous
// bytes instead of two 4-byte strided ones.
template <int N>
struct ConvChannels {
  float win[kMaxConvK - 1][N];
  float tap[kMaxConvK][N];

  template <bool BF16>
  static __device__ __forceinline__ void load_run(const void* base, int64_t off, float (&x)[N]) {
    if constexpr (N == 2) {
      if constexpr (BF16) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + off);
        x[0] = bf16_to_f32(w & 0xffffu);
        x[1] = __uint_as_float(w & 0xffff0000u);
      } else {
        const float2 w = *reinterpret_cast<const float2*>(static_cast<const float*>(base) + off);
        x[0] = w.x;
        x[1] = w.y;
      }
    } else {
      x[0] = load_scalar<BF16>(base, off);
    }
  }
  static __device__ __forceinline__ void store_run(float* base, int64_t off, const float (&x)[N]) {
    if constexpr (N == 2) *reinterpret_cast<float2*>(base + off) = make_float2(x[0], x[1]);
    else base[off] = x[0];
  }

  __device__ __forceinline__ void load(const void* w, const float* window, int64_t slot, int64_t C,
                                       int64_t ch, int K, bool w_bf16) {
#pragma unroll
    for (int q = 0; q < kMaxConvK; ++q) {
      if (q < K) {
        if (w_bf16) load_run<true>(w, q * C + ch, tap[q]);
        else load_run<false>(w, q * C + ch, tap[q]);
      } else {
#pragma unroll
        for (int c = 0; c < N; ++c) tap[q][c] = 0.0f;
      }
    }
#pragma unroll
    for (int q = 0; q < kMaxConvK - 1; ++q) {
      if (q < K - 1) {
        load_run<false>(window, (slot * (K - 1) + q) * C + ch, win[q]);
      } else {
#pragma unroll
        for (int c = 0; c < N; ++c) win[q][c] = 0.0f;
      }
    }
  }

  // as ConvChannel::step, per channel
  __device__ __forceinline__ void step(const float (&x)[N], int K, float (&y)[N]) {
#pragma unroll
    for (int c = 0; c < N; ++c) {
      float acc = 0.0f;
#pragma unroll
      for (int q = 0; q < kMaxConvK; ++q) {
        const float in = q < K - 1 ? win[q < kMaxConvK - 1 ? q : 0][c] : x[c];
        if (q < K) acc = fmaf(tap[q][c], in, acc);
      }
#pragma unroll
      for (int q = 0; q < kMaxConvK - 1; ++q) {
        const float next = q + 1 < kMaxConvK - 1 ? win[q + 1 < kMaxConvK - 1 ? q + 1 : 0][c] : x[c];
        win[q][c] = q < K - 2 ? next : (q == K - 2 ? x[c] : win[q][c]);
      }
      y[c] = silu_f(acc);
    }
  }

  __device__ __forceinline__ void store(float* window, int64_t slot, int64_t C, int64_t ch, int K) const {
#pragma unroll
    for (int q = 0; q < kMaxConvK - 1; ++q)
      if (q < K - 1) store_run(window, (slot * (K - 1) + q) * C + ch, win[q]);
  }
};

// q and k of every (request, key head): one workgroup per (request, key
// head, stream), CPL channels per lane, fp32 results.  A lane reads and
// writes only its own channels' windows, so the in-place window update needs
// no ordering.
template <int DK, bool XBF16>
__global__ __launch_bounds__(kWave) void kda_conv_qk(const ConvQKArgs a) {
  constexpr int CPL = DK >= 2 * kWave ? DK / kWave : 1;
  const int lane = threadIdx.x;
  const int s = static_cast<int>(blockIdx.x % 2);
  const int bh = static_cast<int>(blockIdx.x / 2);
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  int t0 = a.cu_seqlens[b];
  int t1 = a.cu_seqlens[b + 1];
  t0 = t0 < 0 ? 0 : (t0 > a.T ? a.T : t0);
  t1 = t1 < t0 ? t0 : (t1 > a.T ? a.T : t1);
  const int slot = a.state_indices[b];
  const int c0 = lane * CPL;
  if (c0 >= DK) return;
  const int64_t C = static_cast<int64_t>(a.H) * DK;
  const int64_t ch = static_cast<int64_t>(h) * DK + c0;
  if (slot < 0 || slot >= a.N) {
    for (int t = t0; t < t1; ++t)
#pragma unroll
      for (int c = 0; c < CPL; ++c) store_scalar<false>(a.y[s], static_cast<int64_t>(t) * C + ch + c, 0.0f);
    return;
  }
  if (t0 == t1) return;
  ConvChannels<CPL> cv;
  cv.load(a.w[s], a.win[s], slot, C, ch, a.conv_k, a.w_bf16 != 0);
  for (int t = t0; t < t1; ++t) {
    const int64_t off = static_cast<int64_t>(t) * C + ch;
    float x[CPL], y[CPL];
    ConvChannels<CPL>::template load_run<XBF16>(a.x[s], off, x);
    cv.step(x, a.conv_k, y);
    ConvChannels<CPL>::store_run(static_cast<float*>(a.y[s]), off, y);
  }
  cv.store(a.win[s], slot, C, ch, a.conv_k);
}

// ---------------------------------------------------------------------------
// transpose-reduce over lane bits
// ---------------------------------------------------------------------------

// Exchange across lane bit BIT (partner lane ^ (1 << BIT)) with the cheapest
// instruction for that bit: a row swap for bits 5 and 4, DPP below.  Lanes
// with the bit clear keep `lo` + the partner's `lo`, the others `hi` + the
// partner's `hi`; with lo == hi it is a plain pairwise sum.
template <int BIT>
__device__ __forceinline__ float xchg_level(bool up, float lo, float hi) {
  if constexpr (BIT == 5) return swap32_add(lo, hi);
  else if constexpr (BIT == 4) return swap16_add(lo, hi);
  else return dpp_level<(1 << BIT)>(up, lo, hi);
}

// HALF-sized transpose levels on lane bits BIT, BIT-1, ...: each level keeps
// half of the values a lane carries and sums it with the partner's copy;
// after LEVELS levels (by default until one value is left) a lane carries
// HALF * 2 / 2^LEVELS values.
template <int HALF, int BIT, int LEVELS = 32>
__device__ __forceinline__ void transpose_levels(float* vals, int lane) {
  const bool up = ((lane >> BIT) & 1) != 0;
#pragma unroll
  for (int m = 0; m < HALF; ++m) vals[m] = xchg_level<BIT>(up, vals[m], vals[m + HALF]);
  if constexpr (HALF > 1 && LEVELS > 1) transpose_levels<HALF / 2, BIT - 1, LEVELS - 1>(vals, lane);
}

// Plain sums over lane bits HI down to LO (none when HI < LO).
template <int HI, int LO>
__device__ __forceinline__ float sum_levels(float x) {
  if constexpr (HI >= LO) {
    x = xchg_level<HI>(false, x, x);
    return sum_levels<HI - 1, LO>(x);
  } else {
    return x;
  }
}

// ---------------------------------------------------------------------------
// key-first layout: state [dk][dv]
// ---------------------------------------------------------------------------

template <int DK, int DV, bool QBF16, bool SBF16, bool CONVV, int CWT = 32>
__global__ __launch_bounds__(kWave) void kda_decode_kfirst(const DecodeArgs a) {
  constexpr int CW = DV < CWT ? DV : CWT;   // value columns of the wave's slab
  constexpr int SLABS = DV / CW;
  // values per lane and key row: 8 bf16 (one 16-byte access) for a bf16
  // pool when dk has a row for each of the 64 / (CW / 8) row groups, else 4
  constexpr int EPL = (SBF16 && DK >= kWave * 8 / CW) ? 8 : 4;
  constexpr int CQ = CW / EPL;            // lanes across the slab's columns
  constexpr int RS = kWave / CQ;          // row groups across the wave
  constexpr int R = DK / RS;              // key rows per lane
  constexpr int NV = 2 * EPL;             // partial sums per lane (a and b)
  constexpr int LOG_CQ = log2_exact<CQ>();
  constexpr int LOG_RS = log2_exact<RS>();
  constexpr int LOG_NV = log2_exact<NV>();
  // With more partial sums than row groups (a 64-column bf16 slab: 16 sums,
  // 8 row groups) the transpose-reduce runs over every row-group bit and
  // leaves NVL fully reduced sums per lane, lane rs holding sums
  // rs * NVL .. rs * NVL + NVL - 1 (a for NVL consecutive columns, or b).
  constexpr int NVL = LOG_NV > LOG_RS ? NV / RS : 1;
  constexpr int CPL = DK >= 2 * kWave ? DK / kWave : 1;   // setup channels per lane
  static_assert(DK % RS == 0 && R >= 1, "tile shape");
  static_assert(NVL == 1 || (NVL == 2 && !CONVV), "two sums per lane only without the v convolution");
  static_assert(CPL * kWave >= DK && CPL <= 2, "setup split");
  // A 32-column bf16 slab row is 64 bytes, half a cache line shared with
  // the next slab's wave: ordinary cached accesses let L2 merge the two
  // halves (measured 341 us against 382 us with the nontemporal hint on the
  // 96-head decode).  Full-line rows (fp32, or 64 bf16 columns) stream best
  // with the hint.
  using IO = StateIO<SBF16, EPL, (SBF16 && CW * 2 < 128) ? 0 : kCachePolicyNT>;

  __shared__ __attribute__((aligned(16))) float2 red_tab[2][DK];
  __shared__ __attribute__((aligned(16))) float2 upd_tab[2][DK];
  __shared__ __attribute__((aligned(16))) float u_tab[CW];

  const int lane = threadIdx.x;
  const int cq = lane % CQ;
  const int rs = lane / CQ;
  const TileJob j = resolve_job<SLABS>(a);
  if (j.slot < 0 || j.slot >= a.N) {
    zero_rows<DV, CW, QBF16>(a, j, lane);
    return;
  }
  if (j.t0 == j.t1) return;

  const int col0 = j.slab * CW + EPL * cq;
  const int c0 = lane * CPL;
  const bool chan_lane = CPL * kWave == DK || c0 < DK;   // every lane when dk >= 64
  float dtb[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) dtb[c] = 0.0f;
  if (chan_lane) load_f32<CPL>(a.dt_bias + static_cast<int64_t>(j.hv) * DK + c0, dtb);
  const float amp = exp_f(a.a_log[j.hv]);

  // state tile: one trip in; lane rows are rs + RS*i
  char* const tile = static_cast<char*>(a.state_pool) +
                     (static_cast<int64_t>(j.slot) * a.HV + j.hv) * (DK * DV * IO::kElem);
  const __amdgpu_buffer_rsrc_t res = tile_resource(tile, DK * DV * IO::kElem);
  const int voff = (rs * DV + col0) * IO::kElem;
  constexpr int kRowStep = RS * DV * IO::kElem;   // bytes between a lane's rows
  float S[R][EPL];
#pragma unroll
  for (int i = 0; i < R; ++i) IO::load(res, voff, i * kRowStep, S[i]);

  // After the reduction lane rs holds values m = m_final .. m_final + NVL - 1
  // (m_final = rs & (NV-1), or rs * NVL): a[col0 + m] when m < EPL, else
  // b[col0 + m - EPL]; row groups rs >= NV carry duplicates.
  const int m_final = NVL == 1 ? (rs & (NV - 1)) : rs * NVL;
  const bool holds_a = m_final < EPL;
  const bool owner = NVL > 1 || rs < NV;
  const int my_col = col0 + (m_final & (EPL - 1));

  // with the convolution in front, the a-lanes convolve their v channel
  const int64_t v_ch = static_cast<int64_t>(j.hv) * DV + my_col;
  ConvChannel cv;
  if constexpr (CONVV)
    if (holds_a) cv.load(a.conv_w_v, a.conv_win_v, j.slot, static_cast<int64_t>(a.HV) * DV, v_ch, a.conv_k, a.conv_w_bf16 != 0);

  // A token's inputs are loaded together (every lane loads v, a column of
  // its own slab), so their latencies overlap; with a bf16 pool, whose
  // token loop is short of memory latency cover, one token ahead (see
  // kInputsAhead).  With the convolution in front, q and k arrive convolved
  // in fp32.
  using In = TokenInputs<DK, DV, QBF16 && !CONVV, QBF16, CPL, NVL>;
  constexpr bool kAhead = kInputsAhead<SBF16>;
  float pend[CPL];   // deferred decay of the lane's setup channels
#pragma unroll
  for (int c = 0; c < CPL; ++c) pend[c] = 1.0f;
  const int c0s = chan_lane ? c0 : 0;
  In nxt;
  if constexpr (kAhead) nxt.load(a, j, j.t0, c0s, v_ch);
  int buf = 0;
  for (int t = j.t0; t < j.t1; ++t, buf ^= 1) {
    In cur;
    if constexpr (kAhead) {
      cur = nxt;
      if (t + 1 < j.t1) nxt.load(a, j, t + 1, c0s, v_ch);   // uniform
    } else {
      cur.load(a, j, t, c0s, v_ch);
    }
    float v_mine[NVL];
    cur.v.unpack(v_mine);
#pragma unroll
    for (int l = 0; l < NVL; ++l) v_mine[l] = holds_a ? v_mine[l] : 0.0f;
    if constexpr (CONVV)
      if (holds_a) v_mine[0] = cv.step(v_mine[0], a.conv_k);
    const TokenScalars ts = token_setup<DK, CPL>(a, cur, c0, chan_lane, dtb, amp, red_tab[buf], upd_tab[buf],
                                                 pend, t + 1 == j.t1);
    __syncthreads();
    if (ts.fold) {   // uniform: apply the pending decay, this token's included
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float f = upd_tab[buf][rs + RS * i].x;
#pragma unroll
        for (int e = 0; e < EPL; ++e) S[i][e] *= f;
      }
    }

    // ---- one sweep: a = (kh*alpha)^T S, b = (qh*alpha)^T S (deferred: against
    // kh*D', qh*D' and S^), partial over rows ----
    float acc[NV];
#pragma unroll
    for (int m = 0; m < NV; ++m) acc[m] = 0.0f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float2 p = red_tab[buf][rs + RS * i];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        acc[e] = fmaf(p.x, S[i][e], acc[e]);
        acc[EPL + e] = fmaf(p.y, S[i][e], acc[EPL + e]);
      }
    }

    // ---- transpose-reduce over the RS row-group lanes (lane bits above LOG_CQ) ----
    float red[NVL];
    if constexpr (NVL == 1) {
      transpose_levels<NV / 2, LOG_CQ + LOG_NV - 1>(acc, lane);
      red[0] = sum_levels<LOG_CQ + LOG_RS - 1, LOG_CQ + LOG_NV>(acc[0]);
    } else {
      transpose_levels<NV / 2, LOG_CQ + LOG_RS - 1, LOG_RS>(acc, lane);
#pragma unroll
      for (int l = 0; l < NVL; ++l) red[l] = acc[l];
    }

    // ---- u = v - a (to every lane of the column group); o = b + beta*(qh.kh)*u ----
    if (holds_a && owner) {
#pragma unroll
      for (int l = 0; l < NVL; ++l) u_tab[EPL * cq + m_final + l] = v_mine[l] - red[l];
    }
    __syncthreads();
    float u[EPL];
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(&u_tab[EPL * cq + e]);
      u[e] = x.x;
      u[e + 1] = x.y;
      u[e + 2] = x.z;
      u[e + 3] = x.w;
    }
    if (!holds_a && owner) {
      const int64_t o_off = (static_cast<int64_t>(t) * a.HV + j.hv) * DV + my_col;
      if constexpr (NVL == 1) {
        store_scalar<QBF16>(a.out, o_off, fmaf(ts.beta * ts.qk, u[m_final & (EPL - 1)], red[0]));
      } else {
        const float o0 = fmaf(ts.beta * ts.qk, u[m_final & (EPL - 1)], red[0]);
        const float o1 = fmaf(ts.beta * ts.qk, u[(m_final & (EPL - 1)) + 1], red[1]);
        store_pair<QBF16>(a.out, o_off, o0, o1);
      }
    }

    // ---- S^ += (beta*kh / D') u^T (the decay is in D' or already applied) ----
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float py = upd_tab[buf][rs + RS * i].y;
#pragma unroll
      for (int e = 0; e < EPL; ++e) S[i][e] = fmaf(py, u[e], S[i][e]);
    }
  }

  // state tile: one trip out, to the same slot
#pragma unroll
  for (int i = 0; i < R; ++i) IO::store(res, voff, i * kRowStep, S[i]);
  if constexpr (CONVV)
    if (holds_a && owner) cv.store(a.conv_win_v, j.slot, static_cast<int64_t>(a.HV) * DV, v_ch, a.conv_k);
}

// ---------------------------------------------------------------------------
// value-first layout: state [dv][dk]
// ---------------------------------------------------------------------------

template <int DK, int DV, bool QBF16, bool SBF16, bool CONVV>
__global__ __launch_bounds__(kWave) void kda_decode_vfirst(const DecodeArgs a) {
  constexpr int CW = DV < 32 ? DV : 32;   // value rows of the wave's slab
  constexpr int SLABS = DV / CW;
  // keys per lane and value row: 8 when the slab has a row for each of the
  // 512 / dk rows one load instruction then covers, else 4.  The 8 keys are
  // two groups of 4: adjacent (one 16-byte access of 8 bf16) for a bf16 pool,
  // dk/2 apart (two 16-byte fp32 accesses, each instruction reading half
  // rows) for an fp32 pool -- which only keeps whole cache lines while a
  // half row is at least 128 bytes, dk >= 64; smaller fp32 rows take 4 keys
  // per lane and each instruction reads whole rows (d = 32 value-first:
  // 724 -> 568 us at the same bytes).
  constexpr int EPL = (kWave * 8 / DK <= CW && (SBF16 || DK >= 64)) ? 8 : 4;
  constexpr int Q = EPL / 4;              // 4-key groups per lane
  constexpr bool ONE_ACCESS = SBF16 && EPL == 8;
  constexpr int KSTEP = ONE_ACCESS ? 8 : 4;       // keys between neighbouring lanes
  constexpr int QSTRIDE = ONE_ACCESS ? 4 : DK / 2;   // keys between a lane's groups
  constexpr int KC = DK / EPL;            // lanes across one row
  constexpr int RPI = kWave / KC;         // rows per load instruction
  constexpr int L = CW / RPI;             // rows per lane
  constexpr int NV = 2 * L;               // partial sums per lane (a and b)
  constexpr int LOG_KC = log2_exact<KC>();
  constexpr int LOG_NV = log2_exact<NV>();
  constexpr int CPL = DK >= 2 * kWave ? DK / kWave : 1;
  static_assert(L >= 1 && LOG_NV <= LOG_KC, "tile shape");
  static_assert(CPL * kWave >= DK && CPL <= 2, "setup split");
  using IO = StateIO<SBF16, ONE_ACCESS ? 8 : 4>;

  __shared__ __attribute__((aligned(16))) float2 red_tab[2][DK];
  __shared__ __attribute__((aligned(16))) float2 upd_tab[2][DK];
  __shared__ __attribute__((aligned(16))) float u_tab[CW];   // [RPI][L]

  const int lane = threadIdx.x;
  const int kc = lane % KC;
  const int rsub = lane / KC;
  const TileJob j = resolve_job<SLABS>(a);
  if (j.slot < 0 || j.slot >= a.N) {
    zero_rows<DV, CW, QBF16>(a, j, lane);
    return;
  }
  if (j.t0 == j.t1) return;

  const int c0 = lane * CPL;
  const bool chan_lane = CPL * kWave == DK || c0 < DK;   // every lane when dk >= 64
  float dtb[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) dtb[c] = 0.0f;
  if (chan_lane) load_f32<CPL>(a.dt_bias + static_cast<int64_t>(j.hv) * DK + c0, dtb);
  const float amp = exp_f(a.a_log[j.hv]);

  // state tile: one trip in; lane rows are row0 + RPI*i, keys key0 + QSTRIDE*q + 0..3
  const int row0 = j.slab * CW + rsub;
  const int key0 = KSTEP * kc;
  char* const tile = static_cast<char*>(a.state_pool) +
                     (static_cast<int64_t>(j.slot) * a.HV + j.hv) * (DK * DV * IO::kElem);
  const __amdgpu_buffer_rsrc_t res = tile_resource(tile, DK * DV * IO::kElem);
  const int voff = (row0 * DK + key0) * IO::kElem;
  constexpr int kRowStep = RPI * DK * IO::kElem;
  constexpr int kGroupStep = QSTRIDE * IO::kElem;
  float S[L][EPL];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    if constexpr (ONE_ACCESS) {
      IO::load(res, voff, i * kRowStep, S[i]);
    } else {
#pragma unroll
      for (int q = 0; q < Q; ++q) IO::load(res, voff + q * kGroupStep, i * kRowStep, &S[i][4 * q]);
    }
  }

  // After the reduction lane kc holds value m (see below): an a-value of
  // row i when m < L, else the b-value of row i = m - L.
  const int m_final = (kc >> (LOG_KC - LOG_NV)) & (NV - 1);
  const bool holds_a = m_final < L;
  const int i_final = m_final & (L - 1);
  const bool owner = (kc & ((1 << (LOG_KC - LOG_NV)) - 1)) == 0;   // not a duplicate
  const int my_row = row0 + RPI * i_final;

  // with the convolution in front, the a-lanes convolve their v channel
  const int64_t v_ch = static_cast<int64_t>(j.hv) * DV + my_row;
  ConvChannel cv;
  if constexpr (CONVV)
    if (holds_a) cv.load(a.conv_w_v, a.conv_win_v, j.slot, static_cast<int64_t>(a.HV) * DV, v_ch, a.conv_k, a.conv_w_bf16 != 0);

  // the token's inputs loaded together, ahead with a bf16 pool (as in the
  // key-first kernel)
  using In = TokenInputs<DK, DV, QBF16 && !CONVV, QBF16, CPL, 1>;
  constexpr bool kAhead = kInputsAhead<SBF16>;
  float pend[CPL];   // deferred decay of the lane's setup channels
#pragma unroll
  for (int c = 0; c < CPL; ++c) pend[c] = 1.0f;
  const int c0s = chan_lane ? c0 : 0;
  In nxt;
  if constexpr (kAhead) nxt.load(a, j, j.t0, c0s, v_ch);
  int buf = 0;
  for (int t = j.t0; t < j.t1; ++t, buf ^= 1) {
    In cur;
    if constexpr (kAhead) {
      cur = nxt;
      if (t + 1 < j.t1) nxt.load(a, j, t + 1, c0s, v_ch);   // uniform
    } else {
      cur.load(a, j, t, c0s, v_ch);
    }
    float vl[1];
    cur.v.unpack(vl);
    float v_mine = holds_a ? vl[0] : 0.0f;
    if constexpr (CONVV)
      if (holds_a) v_mine = cv.step(v_mine, a.conv_k);
    const TokenScalars ts = token_setup<DK, CPL>(a, cur, c0, chan_lane, dtb, amp, red_tab[buf], upd_tab[buf],
                                                 pend, t + 1 == j.t1);
    __syncthreads();
    if (ts.fold) {   // uniform: apply the pending decay (per key), this token's included
      float f[EPL];
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const float4 p01 = *reinterpret_cast<const float4*>(&upd_tab[buf][key0 + QSTRIDE * q]);
        const float4 p23 = *reinterpret_cast<const float4*>(&upd_tab[buf][key0 + QSTRIDE * q + 2]);
        f[4 * q] = p01.x;
        f[4 * q + 1] = p01.z;
        f[4 * q + 2] = p23.x;
        f[4 * q + 3] = p23.z;
      }
#pragma unroll
      for (int i = 0; i < L; ++i)
#pragma unroll
        for (int e = 0; e < EPL; ++e) S[i][e] *= f[e];
    }

    // ---- sweep: per row, a and b partial over this lane's keys ----
    float kq[EPL], qq[EPL];   // kh*alpha, qh*alpha of the lane's keys
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const float4 r01 = *reinterpret_cast<const float4*>(&red_tab[buf][key0 + QSTRIDE * q]);
      const float4 r23 = *reinterpret_cast<const float4*>(&red_tab[buf][key0 + QSTRIDE * q + 2]);
      kq[4 * q] = r01.x;  qq[4 * q] = r01.y;
      kq[4 * q + 1] = r01.z;  qq[4 * q + 1] = r01.w;
      kq[4 * q + 2] = r23.x;  qq[4 * q + 2] = r23.y;
      kq[4 * q + 3] = r23.z;  qq[4 * q + 3] = r23.w;
    }
    float vals[NV];
#pragma unroll
    for (int i = 0; i < L; ++i) {
      float sa = kq[0] * S[i][0], sb = qq[0] * S[i][0];
#pragma unroll
      for (int e = 1; e < EPL; ++e) {
        sa = fmaf(kq[e], S[i][e], sa);
        sb = fmaf(qq[e], S[i][e], sb);
      }
      vals[i] = sa;
      vals[L + i] = sb;
    }

    // ---- transpose-reduce over the KC lanes of a row (lane bits below LOG_KC) ----
    transpose_levels<NV / 2, LOG_KC - 1>(vals, lane);
    const float red = sum_levels<LOG_KC - LOG_NV - 1, 0>(vals[0]);

    // ---- u = v - a (to every lane of the row); o = b + beta*(qh.kh)*u ----
    if (holds_a && owner) u_tab[rsub * L + i_final] = v_mine - red;
    __syncthreads();
    if (!holds_a && owner)
      store_scalar<QBF16>(a.out, (static_cast<int64_t>(t) * a.HV + j.hv) * DV + my_row,
                          fmaf(ts.beta * ts.qk, u_tab[rsub * L + i_final], red));

    // ---- S^ += (beta*kh / D') u^T (the decay is in D' or already applied) ----
    float bk[EPL];   // beta*kh / D' of the lane's keys
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const float4 p01 = *reinterpret_cast<const float4*>(&upd_tab[buf][key0 + QSTRIDE * q]);
      const float4 p23 = *reinterpret_cast<const float4*>(&upd_tab[buf][key0 + QSTRIDE * q + 2]);
      bk[4 * q] = p01.y;
      bk[4 * q + 1] = p01.w;
      bk[4 * q + 2] = p23.y;
      bk[4 * q + 3] = p23.w;
    }
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const float u = u_tab[rsub * L + i];
#pragma unroll
      for (int e = 0; e < EPL; ++e) S[i][e] = fmaf(bk[e], u, S[i][e]);
    }
  }

#pragma unroll
  for (int i = 0; i < L; ++i) {
    if constexpr (ONE_ACCESS) {
      IO::store(res, voff, i * kRowStep, S[i]);
    } else {
#pragma unroll
      for (int q = 0; q < Q; ++q) IO::store(res, voff + q * kGroupStep, i * kRowStep, &S[i][4 * q]);
    }
  }
  if constexpr (CONVV)
    if (holds_a && owner) cv.store(a.conv_win_v, j.slot, static_cast<int64_t>(a.HV) * DV, v_ch, a.conv_k);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

// Occupancy cap for single-token batches on an fp32 pool.  With one token
// per request a wave is almost all state traffic, and at dk = dv = 128 two
// waves per SIMD stream an fp32 pool faster than four (measured on the
// 96-head batch: key-first 545 -> 536 us, value-first 570 -> 549 us; the
// 32-head batch key-first 55.7 -> 52.6 us).  That is about 128 KiB of state
// in flight per CU; at dk = dv = 64 (half the bytes per wave) the same
// amount is four waves per SIMD instead of six (1024 requests x 96 heads:
// key-first 579 -> 566 us, value-first 579 -> 562 us).  Multi-token batches and
// bf16 pools lose with the cap, and so does a value-first batch of fewer
// than kCapMinWaves waves (the 32-head batch, 52.1 -> 54.5 us): those keep
// the full occupancy.  The cap is taken through dynamic LDS that the
// kernel never touches: capped_lds(N) bytes per one-wave workgroup let N
// workgroups fill a CU's 160 KiB.
constexpr int64_t kCapMinWaves = 16384;   // four rounds at four waves per SIMD
constexpr size_t kCuLds = 163840;

constexpr size_t capped_lds(int workgroups_per_cu) {   // a little over 160 KiB / (N + 1)
  return kCuLds * 10 / (10 * workgroups_per_cu + 8) / 64 * 64;
}
static_assert(capped_lds(8) == 18560, "two waves per SIMD");

template <int DK, int DV>
constexpr size_t static_lds() {   // the kernels' tables: red_tab, upd_tab, u_tab
  return 2 * 2 * DK * sizeof(float2) + (DV < 32 ? DV : 32) * sizeof(float);
}

template <int DK, int DV, bool QBF16, bool SBF16, int LAYOUT, bool CONVV, int CWT = 32>
hipError_t launch_one(const DecodeArgs& args, hipStream_t stream) {
  constexpr int CW = DV < CWT ? DV : CWT;
  const int64_t nwg = static_cast<int64_t>(args.B) * args.HV * (DV / CW);
  void* kargs[] = {const_cast<DecodeArgs*>(&args)};
  const void* fn = LAYOUT == KDA_STATE_K_FIRST
                       ? reinterpret_cast<const void*>(&kda_decode_kfirst<DK, DV, QBF16, SBF16, CONVV, CWT>)
                       : reinterpret_cast<const void*>(&kda_decode_vfirst<DK, DV, QBF16, SBF16, CONVV>);
  // workgroups per CU that hold about 128 KiB of state: 8 at d = 128, 16 at 64
  constexpr int kCapWgs = 32768 / (DK * CW);
  static_assert(SBF16 || static_lds<DK, DV>() < capped_lds(kCapWgs), "cap above the tables");
  const bool cap = DK >= 64 && DV >= 64 && !SBF16 && args.T <= args.B &&
                   (LAYOUT == KDA_STATE_K_FIRST || nwg >= kCapMinWaves);
  // Multi-token batches at dk = dv = 64 on an fp32 pool keep six waves per
  // SIMD, where the kernel's 72 registers would allow seven (1024 requests x
  // 4 tokens x 96 heads: 632 us at seven, 611 us at six).
  constexpr int kMultiWgs = 24;
  const bool cap_multi = DK == 64 && DV == 64 && !SBF16 && args.T > args.B;
  static_assert(static_lds<DK, DV>() < capped_lds(kMultiWgs), "cap above the tables");
  const size_t dyn_lds = cap ? capped_lds(kCapWgs) - static_lds<DK, DV>()
                             : cap_multi ? capped_lds(kMultiWgs) - static_lds<DK, DV>() : 0;
  return hipLaunchKernel(fn, dim3(static_cast<uint32_t>(nwg)), dim3(kWave), kargs, dyn_lds, stream);
}

using LaunchFn = hipError_t (*)(const DecodeArgs&, hipStream_t);

// Key-first kernel on a bf16 pool: 64-column slabs make every slab row a
// whole 128-byte line (32 bf16 columns are half a line, split between two
// waves), at two waves per (request, head) tile and twice the registers per
// lane (about 185: two waves per SIMD).  They win on large batches (96
// heads x 256 requests, one token: 339 -> 280 us; 96 heads x 1024
// requests: 2 tokens 1365 -> 1123 us, 4 tokens 1449 -> 1311 us; 96 heads x
// 512 requests x 8 tokens 1110 -> 1017 us; 1..8 tokens over 96 heads x 128
// requests 224 -> 199 us) and lose where fewer, heavier waves leave the
// chip short of work: 32 heads x 64 requests, one token, +4%; 1..8 tokens
// over 32 heads x 128 requests (16384 32-column slabs) +3.7%.  So they are
// taken from kCapMinWaves 32-column slabs for one-token batches and from
// twice that for longer ones (96 heads x 64 requests x 4 tokens, 24576
// slabs, gains 3% with them and keeps 32 columns).
template <int DK, int DV, bool QBF16>
hipError_t launch_kfirst_bf16(const DecodeArgs& args, hipStream_t stream) {
  if constexpr (DV >= 64) {
    const int64_t waves = static_cast<int64_t>(args.B) * args.HV * (DV / 32);
    if (waves >= (args.T <= args.B ? kCapMinWaves : 2 * kCapMinWaves))
      return launch_one<DK, DV, QBF16, true, KDA_STATE_K_FIRST, false, 64>(args, stream);
  }
  return launch_one<DK, DV, QBF16, true, KDA_STATE_K_FIRST, false, 32>(args, stream);
}

template <int DK, int DV, bool QBF16, bool SBF16>
LaunchFn pick_layout(int layout, bool conv_v) {
  if (layout == KDA_STATE_V_FIRST)
    return conv_v ? &launch_one<DK, DV, QBF16, SBF16, KDA_STATE_V_FIRST, true>
                  : &launch_one<DK, DV, QBF16, SBF16, KDA_STATE_V_FIRST, false>;
  if (conv_v) return &launch_one<DK, DV, QBF16, SBF16, KDA_STATE_K_FIRST, true>;
  if constexpr (SBF16) return &launch_kfirst_bf16<DK, DV, QBF16>;
  return &launch_one<DK, DV, QBF16, SBF16, KDA_STATE_K_FIRST, false>;
}

template <int DK, int DV>
LaunchFn pick(bool qbf16, bool sbf16, int layout, bool conv_v) {
  if (qbf16) return sbf16 ? pick_layout<DK, DV, true, true>(layout, conv_v)
                          : pick_layout<DK, DV, true, false>(layout, conv_v);
  return sbf16 ? pick_layout<DK, DV, false, true>(layout, conv_v)
               : pick_layout<DK, DV, false, false>(layout, conv_v);
}

template <int DK>
LaunchFn pick_dv(int dv, bool qbf16, bool sbf16, int layout, bool conv_v) {
  switch (dv) {
    case 16: return pick<DK, 16>(qbf16, sbf16, layout, conv_v);
    case 32: return pick<DK, 32>(qbf16, sbf16, layout, conv_v);
    case 64: return pick<DK, 64>(qbf16, sbf16, layout, conv_v);
    case 128: return pick<DK, 128>(qbf16, sbf16, layout, conv_v);
    default: return nullptr;
  }
}

template <int DK, bool XBF16>
hipError_t launch_conv(const ConvQKArgs& args, hipStream_t stream) {
  const int64_t nwg = static_cast<int64_t>(args.B) * args.H * 2;
  void* kargs[] = {const_cast<ConvQKArgs*>(&args)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&kda_conv_qk<DK, XBF16>),
                         dim3(static_cast<uint32_t>(nwg)), dim3(kWave), kargs, 0, stream);
}

}  // namespace

int launch_decode(const DecodeArgs& args, int dk, int dv, bool qkv_bf16, bool state_bf16,
                  int state_layout, bool conv_v, hipStream_t stream) {
  LaunchFn fn = nullptr;
  switch (dk) {
    case 16: fn = pick_dv<16>(dv, qkv_bf16, state_bf16, state_layout, conv_v); break;
    case 32: fn = pick_dv<32>(dv, qkv_bf16, state_bf16, state_layout, conv_v); break;
    case 64: fn = pick_dv<64>(dv, qkv_bf16, state_bf16, state_layout, conv_v); break;
    case 128: fn = pick_dv<128>(dv, qkv_bf16, state_bf16, state_layout, conv_v); break;
    default: break;
  }
  if (fn == nullptr) return KDA_ERR_UNSUPPORTED;
  return fn(args, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

int launch_conv_qk(const ConvQKArgs& args, int dk, bool x_bf16, hipStream_t stream) {
  hipError_t (*fn)(const ConvQKArgs&, hipStream_t) = nullptr;
  switch (dk) {
    case 16: fn = x_bf16 ? &launch_conv<16, true> : &launch_conv<16, false>; break;
    case 32: fn = x_bf16 ? &launch_conv<32, true> : &launch_conv<32, false>; break;
    case 64: fn = x_bf16 ? &launch_conv<64, true> : &launch_conv<64, false>; break;
    case 128: fn = x_bf16 ? &launch_conv<128, true> : &launch_conv<128, false>; break;
    default: break;
  }
  if (fn == nullptr) return KDA_ERR_UNSUPPORTED;
  return fn(args, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace kda
