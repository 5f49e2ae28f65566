// kda_decode.hip - the KDA decode recurrence for CDNA4 (gfx950).
//
// Operation ("Delta-rule write" page, naive_recurrent_kda code excerpt;
// "KdaDecode" Tensor Shapes; "KDA Block TKG" l2_eps / scale / lower_bound):
// per token, decay the key-first state row k by exp(g[k]), write
// (beta*k) outer (v - k^T S), and read o = q^T S from the updated state.
//
// Work decomposition.  The columns of a state tile never interact: column c
// of S only meets v[c] and o[c]; every reduction runs over the key axis.  So
// one wavefront owns a 32-column slab (all dk rows) of one (request, value
// head) tile and needs no other wave: no cross-wave reduction and no
// workgroup barrier.  A workgroup is that one wave.  Lane (rs, cq) of the
// wave holds rows rs + RS*i (i < R) and columns 4cq..4cq+3 of the slab as R
// float4 registers, so each load instruction of the wave reads RS whole
// 128-byte row segments; for dk = dv = 128 that is 16 x 128-bit loads per
// lane and 64 VGPRs of state.
//
// Per token, with alpha = exp(g):
//   a = (kh*alpha)^T S_old,  b = (qh*alpha)^T S_old      (one sweep over S)
//   u = v - a,  o = b + beta*(qh.kh)*u,  S = alpha*S_old + (beta*kh) u^T
// which is the page's decay / write / read sequence with the decay folded
// into the two reduction vectors (exact algebra; only the rounding order
// differs).  The per-channel setup (L2 norms, gate, beta) is computed by the
// wave itself, two channels per lane, and handed to the row owners through
// a small LDS table, double-buffered so one token's table never waits for
// the previous token's readers.  The reductions over the row-group lanes
// use DPP and the gfx950 row-swap instructions, not LDS round trips.  The state makes exactly one trip from HBM and one back
// per call; tokens of the same request keep it in registers.  Those two
// trips carry the nontemporal hint: the tile is touched once per call, and
// keeping it out of L2 / MALL measurably raises the streaming rate.
//
// Workgroup order is XCD-aware: consecutive workgroup ids land on different
// XCDs, so the id is remapped to give each XCD one contiguous range of
// (tile, slab) pairs and the slabs of a tile meet in one L2.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kWave = 64;
constexpr int kXcds = 8;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// The state is streamed: each tile is read once and written once per call,
// so its accesses carry the nontemporal hint (cache policy bit "nt") and go
// through a buffer resource spanning exactly the tile.  The resource keeps
// the per-row offsets in scalar registers (one VGPR offset per lane) and the
// hardware range check confines every access to the tile.
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kCachePolicyNT = 2;
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_resource(float* tile, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(tile, static_cast<short>(0), bytes, kRawBufferWord3);
}

__device__ __forceinline__ float4 load_state(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const f32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCachePolicyNT);
  return make_float4(x.x, x.y, x.z, x.w);
}

__device__ __forceinline__ void store_state(__amdgpu_buffer_rsrc_t r, int voff, int soff, float4 v) {
  const f32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(x, r, voff, soff, kCachePolicyNT);
}

// Transcendentals use the hardware exp2 / log2 / rcp / rsqrt instructions
// (about 1 ulp each).  ln(1 + y) keeps full relative accuracy for small y
// through the correction of Goldberg, "What every computer scientist should
// know about floating-point arithmetic" (1991), Theorem 4:
// ln(1 + y) = y * ln(w) / (w - 1) with w = fl(1 + y), and = y when w == 1.
__device__ __forceinline__ float exp_f(float x) { return __expf(x); }

__device__ __forceinline__ float log1p_f(float y) {
  const float w = 1.0f + y;
  return w == 1.0f ? y : __logf(w) * (y / (w - 1.0f));
}

__device__ __forceinline__ float softplus_f(float x) {
  return fmaxf(x, 0.0f) + log1p_f(exp_f(-fabsf(x)));
}

__device__ __forceinline__ float sigmoid_f(float x) {
  return __builtin_amdgcn_rcpf(1.0f + exp_f(-x));
}

__device__ __forceinline__ float rsqrt_f(float x) { return __builtin_amdgcn_rsqf(x); }

// Cross-lane moves.  DPP reads a neighbour lane inside a 16-lane row;
// v_permlane16_swap / v_permlane32_swap (gfx950) exchange whole rows.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppSwapPairs = 0xB1;    // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppSwapHalves = 0x4E;   // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowRor4 = 0x124;     // lane (i + 4) mod 16 of the row
constexpr int kDppRowRor8 = 0x128;     // lane (i + 8) mod 16 = lane ^ 8

// Both return keep + the partner's value, where lanes in the lower half of
// each pair of rows keep `lo` and the upper half keep `hi`:
//   swap16: rows 16 lanes apart (lane ^ 16); swap32: lane ^ 32.
__device__ __forceinline__ float swap16_add(float lo, float hi) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ float swap32_add(float lo, float hi) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kDppSwapPairs>(x);
  x += dpp<kDppSwapHalves>(x);
  x += dpp<kDppRowRor4>(x);
  x += dpp<kDppRowRor8>(x);
  x = swap16_add(x, x);
  return swap32_add(x, x);
}

// Channels [c0, c0 + CPL) of one token row of q / k (bf16 or f32).
template <bool BF16, int CPL>
__device__ __forceinline__ void load_qk(const void* base, int64_t off, float (&x)[CPL]) {
  if constexpr (BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + off;
    if constexpr (CPL == 2) {
      uint32_t w = *reinterpret_cast<const uint32_t*>(p);
      x[0] = bf16_to_f32(w & 0xffffu);
      x[1] = __uint_as_float(w & 0xffff0000u);
    } else {
      x[0] = bf16_to_f32(p[0]);
    }
  } else {
    const float* p = static_cast<const float*>(base) + off;
    if constexpr (CPL == 2) {
      float2 w = *reinterpret_cast<const float2*>(p);
      x[0] = w.x;
      x[1] = w.y;
    } else {
      x[0] = p[0];
    }
  }
}

template <int CPL>
__device__ __forceinline__ void load_f32(const float* p, float (&x)[CPL]) {
  if constexpr (CPL == 2) {
    float2 w = *reinterpret_cast<const float2*>(p);
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
  if constexpr (BF16) static_cast<uint16_t*>(base)[off] = f32_to_bf16_rne(x);
  else static_cast<float*>(base)[off] = x;
}

template <int DK, int DV, bool BF16, int GATE>
__global__ __launch_bounds__(kWave) void kda_decode_kernel(const DecodeArgs a) {
  constexpr int CW = DV < 32 ? DV : 32;   // columns of the wave's slab
  constexpr int SLABS = DV / CW;
  constexpr int CQ = CW / 4;              // float4 column groups per slab
  constexpr int RS = kWave / CQ;          // row groups across the wave
  constexpr int R = DK / RS;              // rows per lane
  constexpr int CPL = DK >= 2 * kWave ? DK / kWave : 1;   // setup channels per lane
  static_assert(DK % RS == 0 && R >= 1, "tile shape");
  static_assert(CPL * kWave >= DK && CPL <= 2, "setup split");

  // per-channel setup tables {kh*alpha, qh*alpha} and {alpha, beta*kh},
  // double-buffered by token parity, and the slab's u vector
  __shared__ __attribute__((aligned(16))) float2 red_tab[2][DK];
  __shared__ __attribute__((aligned(16))) float2 upd_tab[2][DK];
  __shared__ __attribute__((aligned(16))) float u_tab[CW];

  const int lane = threadIdx.x;
  const int cq = lane % CQ;
  const int rs = lane / CQ;

  // XCD-aware id -> (tile, slab)
  const uint32_t wg = blockIdx.x;
  const uint32_t nwg = gridDim.x;
  const uint32_t xcd = wg % kXcds;
  const uint32_t per = nwg / kXcds;
  const uint32_t extra = nwg % kXcds;
  const uint32_t logical = xcd * per + (xcd < extra ? xcd : extra) + wg / kXcds;
  const int slab = static_cast<int>(logical % SLABS);
  const int tile = static_cast<int>(logical / SLABS);
  const int b = tile / a.HV;
  const int hv = tile - b * a.HV;
  const int h = hv / a.G;

  int t0 = a.cu_seqlens[b];
  int t1 = a.cu_seqlens[b + 1];
  t0 = t0 < 0 ? 0 : (t0 > a.T ? a.T : t0);
  t1 = t1 < t0 ? t0 : (t1 > a.T ? a.T : t1);
  const int slot = a.state_indices[b];
  const int col0 = slab * CW + 4 * cq;

  if (slot < 0 || slot >= a.N) {
    // skipped request: zero its output rows, leave every slot alone
    for (int t = t0; t < t1; ++t)
      if (lane < CW) store_scalar<BF16>(a.out, (static_cast<int64_t>(t) * a.HV + hv) * DV + slab * CW + lane, 0.0f);
    return;
  }
  if (t0 == t1) return;

  // token-invariant per-head parameters
  const int c0 = lane * CPL;
  const bool chan_lane = c0 < DK;
  float dtb[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) dtb[j] = 0.0f;
  if (chan_lane) load_f32<CPL>(a.dt_bias + static_cast<int64_t>(hv) * DK + c0, dtb);
  const float amp = exp_f(a.a_log[hv]);

  // state tile: one trip in
  float* const S_ptr = a.state_pool + (static_cast<int64_t>(slot) * a.HV + hv) * (DK * DV);
  const __amdgpu_buffer_rsrc_t S_res = tile_resource(S_ptr, DK * DV * 4);
  const int S_voff = (rs * DV + col0) * 4;
  constexpr int kRowStep = RS * DV * 4;   // bytes between a lane's rows
  float4 S[R];
#pragma unroll
  for (int i = 0; i < R; ++i) S[i] = load_state(S_res, S_voff, i * kRowStep);

  const bool holds_a = (rs & 4) == 0;          // after the reduction, see below
  const int my_col = col0 + (rs & 3);

  int buf = 0;
  for (int t = t0; t < t1; ++t, buf ^= 1) {
    // ---- per-token setup: L2 norms, gate, beta (two channels per lane) ----
    float qv[CPL], kv[CPL], xg[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) qv[j] = kv[j] = xg[j] = 0.0f;
    const int64_t qk_off = (static_cast<int64_t>(t) * a.H + h) * DK + c0;
    const int64_t g_off = (static_cast<int64_t>(t) * a.HV + hv) * DK + c0;
    if (chan_lane) {
      load_qk<BF16, CPL>(a.q, qk_off, qv);
      load_qk<BF16, CPL>(a.k, qk_off, kv);
      load_f32<CPL>(a.raw_gate + g_off, xg);
    }
    const float beta = sigmoid_f(a.beta_logits[static_cast<int64_t>(t) * a.HV + hv]);
    const float v_mine = holds_a ? load_scalar<BF16>(a.v, (static_cast<int64_t>(t) * a.HV + hv) * DV + my_col) : 0.0f;

    float sq = 0.0f, sk = 0.0f, sqk = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      sq = fmaf(qv[j], qv[j], sq);
      sk = fmaf(kv[j], kv[j], sk);
      sqk = fmaf(qv[j], kv[j], sqk);
    }
    sq = wave_sum(sq);
    sk = wave_sum(sk);
    sqk = wave_sum(sqk);
    const float rq = a.scale * rsqrt_f(sq + a.l2_eps);
    const float rk = rsqrt_f(sk + a.l2_eps);
    const float qk = sqk * rq * rk;             // qh . kh (scale included)

    if (chan_lane) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const float x = xg[j] + dtb[j];
        float g;
        if constexpr (GATE == KDA_GATE_SOFTPLUS) g = -amp * softplus_f(x);
        else g = a.lower_bound * sigmoid_f(amp * x);
        const float alpha = exp_f(g);
        const float kh = kv[j] * rk;
        const float qh = qv[j] * rq;
        red_tab[buf][c0 + j] = make_float2(kh * alpha, qh * alpha);
        upd_tab[buf][c0 + j] = make_float2(alpha, beta * kh);
      }
    }
    __syncthreads();

    // ---- one sweep: a = (kh*alpha)^T S, b = (qh*alpha)^T S, partial over rows ----
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float2 p = red_tab[buf][rs + RS * i];
      acc[0] = fmaf(p.x, S[i].x, acc[0]);
      acc[1] = fmaf(p.x, S[i].y, acc[1]);
      acc[2] = fmaf(p.x, S[i].z, acc[2]);
      acc[3] = fmaf(p.x, S[i].w, acc[3]);
      acc[4] = fmaf(p.y, S[i].x, acc[4]);
      acc[5] = fmaf(p.y, S[i].y, acc[5]);
      acc[6] = fmaf(p.y, S[i].z, acc[6]);
      acc[7] = fmaf(p.y, S[i].w, acc[7]);
    }

    // ---- transpose-reduce over the RS row-group lanes ----
    // Lanes of a column group sit CQ apart.  Each butterfly level halves the
    // values a lane carries, so after three levels lane rs holds value
    // rs & 7: a[col0 + (rs&3)] when rs&4 == 0, else b[col0 + (rs&3)].
    float red;
    if constexpr (CQ == 8) {
      // row-group bits are lane bits 5, 4, 3: two row swaps and one DPP move
      float v4[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) v4[m] = swap32_add(acc[m], acc[m + 4]);
      float v2[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) v2[m] = swap16_add(v4[m], v4[m + 2]);
      const bool up = (rs & 1) != 0;
      red = (up ? v2[1] : v2[0]) + dpp<kDppRowRor8>(up ? v2[0] : v2[1]);
    } else {
      float v4[4];
      {
        const bool up = (rs & 4) != 0;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float send = up ? acc[m] : acc[m + 4];
          const float keep = up ? acc[m + 4] : acc[m];
          v4[m] = keep + __shfl_xor(send, 4 * CQ, kWave);
        }
      }
      float v2[2];
      {
        const bool up = (rs & 2) != 0;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const float send = up ? v4[m] : v4[m + 2];
          const float keep = up ? v4[m + 2] : v4[m];
          v2[m] = keep + __shfl_xor(send, 2 * CQ, kWave);
        }
      }
      const bool up = (rs & 1) != 0;
      red = (up ? v2[1] : v2[0]) + __shfl_xor(up ? v2[0] : v2[1], CQ, kWave);
#pragma unroll
      for (int m = 8 * CQ; m < kWave; m <<= 1) red += __shfl_xor(red, m, kWave);
    }

    // ---- u = v - a (to every lane of the column group); o = b + beta*(qh.kh)*u ----
    if (holds_a && rs < 4) u_tab[4 * cq + rs] = v_mine - red;
    __syncthreads();
    const float4 u4 = *reinterpret_cast<const float4*>(&u_tab[4 * cq]);
    if (!holds_a && rs < 8) {
      const float uj = (rs & 2) ? ((rs & 1) ? u4.w : u4.z) : ((rs & 1) ? u4.y : u4.x);
      store_scalar<BF16>(a.out, (static_cast<int64_t>(t) * a.HV + hv) * DV + my_col,
                         fmaf(beta * qk, uj, red));
    }
    const float u[4] = {u4.x, u4.y, u4.z, u4.w};

    // ---- S = alpha*S + (beta*kh) u^T ----
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float2 p = upd_tab[buf][rs + RS * i];
      S[i].x = fmaf(p.y, u[0], p.x * S[i].x);
      S[i].y = fmaf(p.y, u[1], p.x * S[i].y);
      S[i].z = fmaf(p.y, u[2], p.x * S[i].z);
      S[i].w = fmaf(p.y, u[3], p.x * S[i].w);
    }
  }

  // state tile: one trip out, to the same slot
#pragma unroll
  for (int i = 0; i < R; ++i) store_state(S_res, S_voff, i * kRowStep, S[i]);
}

template <int DK, int DV, bool BF16, int GATE>
hipError_t launch_one(const DecodeArgs& args, hipStream_t stream) {
  constexpr int CW = DV < 32 ? DV : 32;
  const int64_t nwg = static_cast<int64_t>(args.B) * args.HV * (DV / CW);
  void* kargs[] = {const_cast<DecodeArgs*>(&args)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&kda_decode_kernel<DK, DV, BF16, GATE>),
                         dim3(static_cast<uint32_t>(nwg)), dim3(kWave), kargs, 0, stream);
}

using LaunchFn = hipError_t (*)(const DecodeArgs&, hipStream_t);

template <int DK, int DV>
constexpr LaunchFn pick(bool bf16, int gate) {
  return bf16 ? (gate == KDA_GATE_SOFTPLUS ? &launch_one<DK, DV, true, KDA_GATE_SOFTPLUS>
                                           : &launch_one<DK, DV, true, KDA_GATE_LOWER_BOUND>)
              : (gate == KDA_GATE_SOFTPLUS ? &launch_one<DK, DV, false, KDA_GATE_SOFTPLUS>
                                           : &launch_one<DK, DV, false, KDA_GATE_LOWER_BOUND>);
}

template <int DK>
LaunchFn pick_dv(int dv, bool bf16, int gate) {
  switch (dv) {
    case 16: return pick<DK, 16>(bf16, gate);
    case 32: return pick<DK, 32>(bf16, gate);
    case 64: return pick<DK, 64>(bf16, gate);
    case 128: return pick<DK, 128>(bf16, gate);
    default: return nullptr;
  }
}

}  // namespace

int launch_decode(const DecodeArgs& args, int dk, int dv, bool bf16, int gate_mode,
                  hipStream_t stream) {
  LaunchFn fn = nullptr;
  switch (dk) {
    case 16: fn = pick_dv<16>(dv, bf16, gate_mode); break;
    case 32: fn = pick_dv<32>(dv, bf16, gate_mode); break;
    case 64: fn = pick_dv<64>(dv, bf16, gate_mode); break;
    case 128: fn = pick_dv<128>(dv, bf16, gate_mode); break;
    default: break;
  }
  if (fn == nullptr) return KDA_ERR_UNSUPPORTED;
  return fn(args, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace kda
