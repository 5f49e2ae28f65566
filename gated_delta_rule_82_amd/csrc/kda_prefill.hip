// kda_prefill.hip - the KDA recurrence over whole requests (prefill), chunk
// by chunk on the CDNA4 matrix cores (gfx950).
//
// Operation: the same per-token recurrence as kda_decode ("Delta-rule
// write" page, naive_recurrent_kda code excerpt; "KdaDecode" tensor
// contract; "KDA Block TKG" l2_eps / scale / lower_bound).  The model runs
// this step as chunk_kda for a whole sequence ("Delta-rule write" page,
// modeling_kimi_linear.py excerpt); the pages do not pin that kernel's
// internals, so what is fixed is the token-by-token result.
//
// Chunk form.  Take C = 16 tokens at a time.  With Gamma_t[d] the running
// sum of the log-decays g since the chunk start (inclusive of token t),
// S0 the state before the chunk and kh, qh the normalised keys and scaled
// queries:
//   X  = V - Kt S0            Kt[t]  = kh_t * exp(Gamma_t)
//   Y  = Qt S0                Qt[t]  = qh_t * exp(Gamma_t)
//   (I + L) U = X             L[t,s] = beta_s P[t,s]          (s < t)
//   O  = Y + R' U             R'[t,s] = beta_s R[t,s]         (s <= t)
//   S  = diag(exp(Gamma_last)) S0 + Kup^T U,
//                             Kup[s] = beta_s kh_s exp(Gamma_last - Gamma_s)
//   P[t,s] = sum_d kh_t[d] kh_s[d] exp(Gamma_t[d] - Gamma_s[d]), R the same
//   with qh_t.  U holds the per-token corrections v_t - kh_t^T(decayed S);
// unrolling the recurrence over the chunk gives exactly these equations, so
// the result differs from the token loop only in rounding order.  The L2
// norms are per-token scale factors, so every product above runs on the raw
// q, k and the norms are applied to its rows or columns afterwards:
//   X = V - diag(rk) (Kt_raw S0),  O = diag(rq) (Qt_raw S0 + R_raw U'),
//   S = diag(exp(Gamma_last)) S0 + Kup_raw^T U',  U' = diag(beta rk) U,
//   L = diag(rk) P_raw diag(rk beta).
// A ragged last chunk is padded with tokens whose v, beta and g are zero (q
// and k repeat the last real token's row): with beta = 0 a padding token
// writes nothing to the state, and as L and R are lower triangular no real
// token's row reads one, so they change nothing.
//
// P_raw and R_raw are sums over the key channels, so each wave adds up the
// part of its own channels.  For a channel set whose decay span
// max(-Gamma_last[d]) is at most kSafeSpan, that part is one matrix product
// of Kp = k exp(Gamma - c) and Ks = k exp(c - Gamma) with c = Gamma_last / 2:
// every factor then lies within exp(+-kSafeSpan / 2) = exp(+-60): finite for
// any |k| below 1e12, and the bf16 remainder of the smallest factor is a
// normal number for any |k| above 1e-9.  A wider span (a strong softplus gate) splits the
// chunk's lower triangle hierarchically into blocks that each factor with
// every exponent bounded (see wide_level): two to five products instead of
// one, for any decay span.
//
// Work decomposition.  A workgroup owns one (request, value head) tile and
// walks the request's chunks in order; wave w owns value columns
// [32w, 32w + 32), and its state slab S[:, 32w:32w+32] stays in the wave's
// MFMA accumulators for the whole request.  An accumulator tile holds rows
// 4*(lane/16) + i (i = 0..3) of column lane % 16; an A (B) operand holds,
// per lane, row (column) lane % 16 and a set of reduction indices chosen by
// lane / 16.  The reduction order inside a product is free, so each product
// is oriented to take its operands where they already are:
//   * acc(M) is the B operand of M and the A operand of M^T.  X = Kt_raw S
//     and Y^T = S^T Qt_raw^T both read the state straight from its
//     accumulators; U = T X reads X, O^T = Y^T + U'^T R_raw^T and the state
//     update Kup_raw^T U' read U'.  O comes out transposed, so each lane
//     stores four consecutive values of one output row.
//   * The per-chunk elementwise work runs in the operand layout itself: lane
//     (token lane % 16, quarter lane / 16) handles 8 consecutive channels of
//     its token.  P and R partials are then one product of registers (A and
//     B from the same lanes), the decay prefix over tokens is a DPP scan
//     within each 16-lane row, and V enters X through a product with an
//     identity B operand instead of a gather.
// Per chunk: every wave builds its channels' operands and partials and
// publishes them in LDS (Kt, Qt, Kup^T, exp(Gamma_last), norms, P and R
// partials); after one workgroup barrier each wave assembles L, solves
// T = (I + L)^-1 itself (forward substitution over the rows, each final row
// broadcast along the 16-lane rows by DPP) and runs X, Y^T, U, O^T and the
// state update on its slab; a second barrier frees the tables for the next
// chunk.  The next chunk's inputs are loaded into
// registers while the current one is processed, and the barriers fence LDS
// only, so those loads stay in flight.  The state makes one trip from HBM
// and one back per request.
//
// Matrix precision.  KDA_MATMUL_F32 uses the fp32 matrix instruction
// (v_mfma_f32_16x16x4_f32): fp32 products, fp32 sums.  KDA_MATMUL_SPLIT_BF16
// writes each fp32 operand as hi + lo, both bf16 (round to nearest even).
// A K = 32 product sums hi*hi + hi*lo + lo*hi on the bf16 matrix
// instruction (16x16x32): each operand keeps 16 significant bits and the
// dropped lo*lo term is below 2^-16 of the product, at a third of the fp32
// instruction's cost per product.  A K = 16 product packs hi and lo along
// K and takes two instructions, lo*lo included (see mma).  (This is the
// classic split-precision product, e.g. Henry, Tang and Heinecke,
// "Leveraging the bfloat16 artificial intelligence datatype for
// higher-precision computations", ARITH 2019.)

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kChunk = 16;          // tokens per chunk: one MFMA M / K tile
// Value columns per products wave: 32 (two MFMA N tiles), one workgroup per
// 128-column tile; or 16 (one tile), two workgroups per tile, each with half
// the columns and the whole elementwise stage (for batches of few tiles).
constexpr int kSlabCols = 32;
constexpr int kNarrowSlabCols = 16;
constexpr int kGroupChannels = 32;  // key channels per elementwise channel group
constexpr float kSafeSpan = 120.0f; // largest decay span of the one-product P, R
// The table factors exp(Gamma_t) and exp(Gamma_last - Gamma_t) use
// differences of prefix sums; in fp32 they carry an error near
// ulp(|Gamma|), harmless while a chunk's decay span stays within kExactSpan
// (in log2 units; ulp(512) = 2^-14 gives factor errors of order 1e-5).  A
// wider span, or a non-finite one, splits each token's log2-decay g into an
// integer, whose prefix sums are exact in fp32, and a remainder in (-1, 0],
// whose prefix sums stay within 16 (ulp 2^-20); g is first raised to
// -kGateFloor (exp2 of it is already 0 in fp32), which keeps an infinite
// decay finite and the integer sums below 2^24.
constexpr float kExactSpan = 512.0f;
constexpr float kGateStep = 1.0f;
constexpr float kGateFloor = 1048576.0f;   // 2^20
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kPT = kChunk + 4;     // pitch of the 16-column LDS tables

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Barrier for LDS traffic only: outstanding global loads (the next chunk's
// inputs) and stores (outputs) are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders this wave's own LDS writes before its later LDS reads of other
// lanes' data (the hardware keeps a wave's LDS operations in order; this
// keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
}

// ---------------------------------------------------------------------------
// operand fragments and the two matrix precisions
// ---------------------------------------------------------------------------

// N fp32 operand values of one lane: the reduction indices (lane / 16, j)
// of a 16x16xK product, K = 4N (N = 8: K = 32; N = 4: K = 16).
template <int PREC, int N>
struct Frag;

template <int N>
struct Frag<KDA_MATMUL_F32, N> {
  float v[N];
};

template <int N>
struct Frag<KDA_MATMUL_SPLIT_BF16, N> {
  typedef __bf16 vec __attribute__((ext_vector_type(N)));
  vec hi, lo;
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Splits two fp32 values into their bf16 hi parts (one packed conversion)
// and the bf16 lo parts of the remainders, each pair packed into a word
// (first value in the lower half).  A remainder x - hi(x) is exact in fp32
// (hi(x) is within a factor of two of x).
//
// The remainder comes from the bf16 dot product instruction straight from
// the packed word, x + (-1) * hi(x): the builtin selects the form that
// accumulates into x's register, one instruction per value, so x must die at
// the split (the state, which lives on, is first decayed into new
// registers; see acc_frag8_decay).  The selector words {-1, 0} and {0, -1} are passed through SGPRs:
// the compiler encodes the first as the inline constant -1.0, which the
// instruction does not read as that bf16 pair (the remainders of first
// values came out wrong); from a register both selectors are exact.
__device__ __forceinline__ float minus_hi(bf16x2 h, int half, float x) {
  uint32_t sel = half == 0 ? 0x0000bf80u : 0xbf800000u;   // bf16 -1 in the chosen half
  asm("" : "+s"(sel));
  return __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, sel), x, false);
}

__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  const bf16x2 h = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  hi = __builtin_bit_cast(uint32_t, h);
  const bf16x2 l = {static_cast<__bf16>(minus_hi(h, 0, a)), static_cast<__bf16>(minus_hi(h, 1, b))};
  lo = __builtin_bit_cast(uint32_t, l);
}

template <int PREC, int N>
__device__ __forceinline__ Frag<PREC, N> make_frag(const float (&x)[N]) {
  Frag<PREC, N> f;
  if constexpr (PREC == KDA_MATMUL_F32) {
#pragma unroll
    for (int j = 0; j < N; ++j) f.v[j] = x[j];
  } else {
    static_assert(N % 2 == 0, "split fragments hold pairs");
    uint32_t hi[N / 2], lo[N / 2];
#pragma unroll
    for (int j = 0; j < N / 2; ++j) split_pair(x[2 * j], x[2 * j + 1], hi[j], lo[j]);
    typedef typename Frag<PREC, N>::vec vec;
    f.hi = __builtin_bit_cast(vec, hi);
    f.lo = __builtin_bit_cast(vec, lo);
  }
  return f;
}

// A K = 16 bf16 operand widened to the K = 32 instruction's 8 values per
// lane, the upper four zero (the identity product of a 16-column slab).
// Every bf16 product here runs on the gfx950
// K = 32 instruction: with the older K = 16 bf16 instruction, results were
// observed to depend on the compiler's instruction schedule (wrong
// accumulator values in some schedules, right in others), so it is not used.
[[maybe_unused]] __device__ __forceinline__ bf16x8 widen(const bf16x4& x) {
  const bf16x4 z = {};
  return __builtin_shufflevector(x, z, 0, 1, 2, 3, 4, 5, 6, 7);
}

// acc += A B over the fragment's K indices.  A K = 16 split product runs as
// two K = 32 instructions with no zero padding: one operand carries hi in
// its first four K values and lo in its last four, the other carries its
// hi part twice, then its lo part twice, so the two instructions sum
// (a.hi + a.lo)(b.hi + b.lo), the lo * lo term included.  The duplicated
// operand costs register copies; DUP_A picks A for it when A is the one
// reused across calls.
template <int PREC, int N, bool DUP_A = false>
__device__ __forceinline__ void mma(f32x4& acc, const Frag<PREC, N>& a, const Frag<PREC, N>& b) {
  if constexpr (PREC == KDA_MATMUL_F32) {
#pragma unroll
    for (int j = 0; j < N; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
  } else if constexpr (N == 8) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
  } else if constexpr (DUP_A) {
    const bf16x8 bc = __builtin_shufflevector(b.hi, b.lo, 0, 1, 2, 3, 4, 5, 6, 7);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(a.hi, a.hi, 0, 1, 2, 3, 4, 5, 6, 7), bc, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(a.lo, a.lo, 0, 1, 2, 3, 4, 5, 6, 7), bc, acc, 0, 0, 0);
  } else {
    const bf16x8 ac = __builtin_shufflevector(a.hi, a.lo, 0, 1, 2, 3, 4, 5, 6, 7);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ac, __builtin_shufflevector(b.hi, b.hi, 0, 1, 2, 3, 4, 5, 6, 7), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ac, __builtin_shufflevector(b.lo, b.lo, 0, 1, 2, 3, 4, 5, 6, 7), acc, 0, 0, 0);
  }
}

// acc += A I_nt where I_nt is the identity restricted to value tile nt: the
// K = 4N indices (g, j) stand for the slab's columns N g + j, B[(g, j)][n] =
// [N g + j == 16 nt + n].  A bf16 value is exact in the hi part alone, so
// bf16 A enters the matrix instruction as loaded.
template <bool BF16, int N>
struct RunN;
template <int PREC, bool EXACT_BF16, int N>
__device__ __forceinline__ void mma_identity(f32x4& acc, const RunN<EXACT_BF16, N>& run, int nt, int n, int g) {
  float e[N];
#pragma unroll
  for (int j = 0; j < N; ++j) e[j] = N * g + j == 16 * nt + n ? 1.0f : 0.0f;
  if constexpr (PREC == KDA_MATMUL_SPLIT_BF16 && EXACT_BF16) {
    typedef typename Frag<PREC, N>::vec vec;
    const vec va = __builtin_bit_cast(vec, run.w);
    const Frag<PREC, N> fe = make_frag<PREC, N>(e);
    if constexpr (N == 8) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, fe.hi, acc, 0, 0, 0);
    else acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen(va), widen(fe.hi), acc, 0, 0, 0);
    return;
  }
  float a[N];
  run.unpack(a);
  if constexpr (PREC == KDA_MATMUL_F32) {
#pragma unroll
    for (int j = 0; j < N; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], e[j], acc, 0, 0, 0);
  } else {
    const Frag<PREC, N> fa = make_frag<PREC, N>(a);
    const Frag<PREC, N> fe = make_frag<PREC, N>(e);
    if constexpr (N == 8) {
      if constexpr (!EXACT_BF16) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa.lo, fe.hi, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa.hi, fe.hi, acc, 0, 0, 0);
    } else {
      if constexpr (!EXACT_BF16)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen(fa.lo), widen(fe.hi), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen(fa.hi), widen(fe.hi), acc, 0, 0, 0);
    }
  }
}

// Two state accumulator tiles as one K = 32 operand, and the same tiles
// decayed in that pass (row i of tile lo by elo[i], of tile hi by ehi[i]).
// The decayed values go to new registers, so the undecayed ones die at the
// split and their remainders come from the in-place dot product (one
// instruction each) instead of a widening shift or mask and a subtraction.
template <int PREC>
__device__ __forceinline__ Frag<PREC, 8> acc_frag8_decay(f32x4& lo, f32x4& hi, const f32x4& elo,
                                                         const f32x4& ehi) {
  const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  lo *= elo;
  hi *= ehi;
  // keeps the products here: sunk to the state update, they would keep the
  // undecayed values live past the split
  asm volatile("" : "+v"(lo), "+v"(hi));
  return make_frag<PREC, 8>(v);
}

template <int PREC>
__device__ __forceinline__ Frag<PREC, 4> acc_frag4(const f32x4& x) {
  const float v[4] = {x[0], x[1], x[2], x[3]};
  return make_frag<PREC, 4>(v);
}

// [16][DK] operand rows in LDS (Kt_raw, Qt_raw), stored already in the form
// the matrix instruction takes: fp32, or the bf16 hi and lo parts.  Rows
// are written 8 channels at a time and read as K = 32 slices in the order of
// two stacked accumulator tiles: value j of lane group g is channel
// 32s + 16 (j / 4) + 4g + j % 4.
//
// The LDS tables (this one, KupTable, ChunkShared) take a KERNEL parameter
// that differs between kernels, so no kernel shares their member functions
// with another.  A member function shared by several kernels is optimized
// once on its own, where `this` is a generic pointer, and only then inlined:
// the kernels then carried 64-bit generic address arithmetic for the table
// accesses (the 96-head prefill kernel spilled a register that way).
template <int PREC, int DK, int KERNEL>
struct RowTable;

template <int DK, int KERNEL>
struct RowTable<KDA_MATMUL_F32, DK, KERNEL> {
  static constexpr int P = DK + 4;
  float v[kChunk][P];
  template <int N>
  __device__ __forceinline__ void store(int t, int d0, const float (&x)[N]) {
#pragma unroll
    for (int i = 0; i < N; i += 4)
      *reinterpret_cast<f32x4*>(&v[t][d0 + i]) = f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]};
  }
  __device__ __forceinline__ Frag<KDA_MATMUL_F32, 8> frag8(int row, int s, int g) const {
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(&v[row][32 * s + 4 * g]);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(&v[row][32 * s + 16 + 4 * g]);
    Frag<KDA_MATMUL_F32, 8> f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f.v[j] = x0[j];
      f.v[4 + j] = x1[j];
    }
    return f;
  }
};

template <int DK, int KERNEL>
struct RowTable<KDA_MATMUL_SPLIT_BF16, DK, KERNEL> {
  static constexpr int P = DK + 8;
  __bf16 hi[kChunk][P];
  __bf16 lo[kChunk][P];
  template <int N>
  __device__ __forceinline__ void store(int t, int d0, const float (&x)[N]) {
    const Frag<KDA_MATMUL_SPLIT_BF16, N> f = make_frag<KDA_MATMUL_SPLIT_BF16, N>(x);
    typedef typename Frag<KDA_MATMUL_SPLIT_BF16, N>::vec vec;
    *reinterpret_cast<vec*>(&hi[t][d0]) = f.hi;
    *reinterpret_cast<vec*>(&lo[t][d0]) = f.lo;
  }
  __device__ __forceinline__ Frag<KDA_MATMUL_SPLIT_BF16, 8> frag8(int row, int s, int g) const {
    const bf16x4 h0 = *reinterpret_cast<const bf16x4*>(&hi[row][32 * s + 4 * g]);
    const bf16x4 h1 = *reinterpret_cast<const bf16x4*>(&hi[row][32 * s + 16 + 4 * g]);
    const bf16x4 l0 = *reinterpret_cast<const bf16x4*>(&lo[row][32 * s + 4 * g]);
    const bf16x4 l1 = *reinterpret_cast<const bf16x4*>(&lo[row][32 * s + 16 + 4 * g]);
    Frag<KDA_MATMUL_SPLIT_BF16, 8> f;
    f.hi = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
    f.lo = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
    return f;
  }
};

// Kup_raw^T [channel][token] in LDS, written two channels at a time by the
// lane that owns the token and read as K = 16 fragments of four
// consecutive tokens.  The split form keeps, per channel and group of four
// tokens, the four hi parts and then the four lo parts: one 16-byte read is
// the fragment as the matrix instruction takes it.
template <int PREC, int DK, int KERNEL>
struct KupTable;

template <int DK, int KERNEL>
struct KupTable<KDA_MATMUL_F32, DK, KERNEL> {
  float v[DK][kPT];
  __device__ __forceinline__ void store2(int d, int t, float x0, float x1) {
    v[d][t] = x0;
    v[d + 1][t] = x1;
  }
  __device__ __forceinline__ Frag<KDA_MATMUL_F32, 4> frag4(int row, int g) const {
    return acc_frag4<KDA_MATMUL_F32>(*reinterpret_cast<const f32x4*>(&v[row][4 * g]));
  }
};

template <int DK, int KERNEL>
struct KupTable<KDA_MATMUL_SPLIT_BF16, DK, KERNEL> {
  static constexpr int P = kChunk / 4 * 8 + 8;   // bf16 per channel row, padded
  __bf16 v[DK][P];
  // channels d and d + 1 of token t: one conversion for the two hi parts,
  // one for the two lo parts.  The packed words are passed through an empty
  // asm so that the compiler stores their upper halves as they are instead
  // of converting each value again into a lower half.
  __device__ __forceinline__ void store2(int d, int t, float x0, float x1) {
    const bf16x2 h = {static_cast<__bf16>(x0), static_cast<__bf16>(x1)};
    const bf16x2 l = {static_cast<__bf16>(minus_hi(h, 0, x0)), static_cast<__bf16>(minus_hi(h, 1, x1))};
    uint32_t hw = __builtin_bit_cast(uint32_t, h), lw = __builtin_bit_cast(uint32_t, l);
    asm("" : "+v"(hw), "+v"(lw));
    uint16_t* const r0 = reinterpret_cast<uint16_t*>(&v[d][8 * (t / 4) + t % 4]);
    uint16_t* const r1 = reinterpret_cast<uint16_t*>(&v[d + 1][8 * (t / 4) + t % 4]);
    r0[0] = static_cast<uint16_t>(hw);
    r1[0] = static_cast<uint16_t>(hw >> 16);
    r0[4] = static_cast<uint16_t>(lw);
    r1[4] = static_cast<uint16_t>(lw >> 16);
  }
  __device__ __forceinline__ Frag<KDA_MATMUL_SPLIT_BF16, 4> frag4(int row, int g) const {
    const bf16x8 w = *reinterpret_cast<const bf16x8*>(&v[row][8 * g]);
    Frag<KDA_MATMUL_SPLIT_BF16, 4> f;
    f.hi = __builtin_shufflevector(w, w, 0, 1, 2, 3);
    f.lo = __builtin_shufflevector(w, w, 4, 5, 6, 7);
    return f;
  }
};

// ---------------------------------------------------------------------------
// memory helpers
// ---------------------------------------------------------------------------

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* base, int64_t off) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[off]);
  else return static_cast<const float*>(base)[off];
}

// The state slab moves through a raw buffer resource spanning exactly the
// (slot, head) tile: a lane keeps one 32-bit byte offset and every access
// adds a constant, instead of a 64-bit address per element.
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_resource(void* tile, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(tile, static_cast<short>(0), bytes, kRawBufferWord3);
}

// N (1 or 4) consecutive state elements at byte offset voff + soff.
template <bool BF16, int N>
__device__ __forceinline__ void load_state(__amdgpu_buffer_rsrc_t r, int voff, int soff, float* x) {
  if constexpr (BF16 && N == 4) {
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    x[0] = bf16_to_f32(w.x & 0xffffu);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = bf16_to_f32(w.y & 0xffffu);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
  } else if constexpr (BF16) {
    x[0] = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
  } else if constexpr (N == 4) {
    const f32x4 w = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    x[0] = w.x;
    x[1] = w.y;
    x[2] = w.z;
    x[3] = w.w;
  } else {
    x[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));   // bits, not a conversion
  }
}

template <bool BF16, int N>
__device__ __forceinline__ void store_state(__amdgpu_buffer_rsrc_t r, int voff, int soff, const float* x) {
  if constexpr (BF16 && N == 4) {
    const u32x2 w = {f32x2_to_bf16x2_rne(x[0], x[1]), f32x2_to_bf16x2_rne(x[2], x[3])};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, voff, soff, 0);
  } else if constexpr (BF16) {
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(f32_to_bf16_rne(x[0])), r, voff, soff, 0);
  } else if constexpr (N == 4) {
    const f32x4 w = {x[0], x[1], x[2], x[3]};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), r, voff, soff, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x[0]), r, voff, soff, 0);
  }
}

template <bool BF16>
__device__ __forceinline__ void store_elem(void* base, int64_t off, float x) {
  if constexpr (BF16) static_cast<uint16_t*>(base)[off] = static_cast<uint16_t>(f32_to_bf16_rne(x));
  else static_cast<float*>(base)[off] = x;
}

// N (4 or 8) consecutive elements at an N-element aligned offset, kept in
// their storage form (bf16 pairs or fp32).
template <bool BF16, int N>
struct RunN {
  static constexpr int W = BF16 ? N / 2 : N;
  uint32_t w[W];
  // from a byte offset to a base pointer; with a uniform base and a 32-bit
  // offset the load takes the base from scalar registers and the offset from
  // one vector register (no 64-bit address arithmetic per lane)
  __device__ __forceinline__ void load(const char* base, uint32_t byte_off) {
    const char* b = base + byte_off;
    if constexpr (W == 2) {
      const u32x2 x = *reinterpret_cast<const u32x2*>(b);
      w[0] = x[0];
      w[1] = x[1];
    } else {
      const u32x4* p = reinterpret_cast<const u32x4*>(b);
#pragma unroll
      for (int i = 0; i < W / 4; ++i) {
        const u32x4 x = p[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[4 * i + j] = x[j];
      }
    }
  }
  __device__ __forceinline__ void unpack(float (&x)[N]) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if constexpr (BF16) x[i] = i % 2 == 0 ? bf16_to_f32(w[i / 2] & 0xffffu) : __uint_as_float(w[i / 2] & 0xffff0000u);
      else x[i] = __uint_as_float(w[i]);
    }
  }
};

// 4 consecutive output values of one token (bf16: the conversion
// instruction, round to nearest even).
// (a byte offset to a base pointer, as RunN::load)
template <bool BF16>
__device__ __forceinline__ void store4(char* base, uint32_t byte_off, const f32x4& x) {
  if constexpr (BF16) {
    bf16x4 p;
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = static_cast<__bf16>(x[i]);
    *reinterpret_cast<bf16x4*>(base + byte_off) = p;
  } else {
    *reinterpret_cast<f32x4*>(base + byte_off) = x;
  }
}

// DPP within each 16-lane row.
template <int CTRL, bool BOUND_ZERO>
__device__ __forceinline__ float dpp_row(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, BOUND_ZERO));
}
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast0 = 0x150;    // row_newbcast:s = 0x150 + s, lane s of the row to all
constexpr int kDppRowBcast15 = 0x15F;

__device__ __forceinline__ float exp2_f(float x) { return __builtin_amdgcn_exp2f(x); }

// inclusive prefix sums over the 16 lanes of each row, of N values at once
// (step by step across the values, so that consecutive DPP reads do not
// depend on each other)
template <int N>
__device__ __forceinline__ void row_scan_n(float (&x)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp_row<kDppRowShr1, true>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp_row<kDppRowShr2, true>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp_row<kDppRowShr4, true>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp_row<kDppRowShr8, true>(x[j]);
}

// inclusive prefix sum over the 16 lanes of each row
__device__ __forceinline__ float row_scan(float x) {
  x += dpp_row<kDppRowShr1, true>(x);
  x += dpp_row<kDppRowShr2, true>(x);
  x += dpp_row<kDppRowShr4, true>(x);
  x += dpp_row<kDppRowShr8, true>(x);
  return x;
}

// sum over the four lanes lane % 16 + 16 q, q = 0..3 (the other rows)
__device__ __forceinline__ float cross_row_sum(float x) {
  x = swap16_add(x, x);
  return swap32_add(x, x);
}

// Steps S.. of the row substitution for J columns of T = (I + L)^-1: lane
// (t, g) holds T[t][c_j] in tc[j], with column c_j the same for the 16
// lanes of its row, and -L[t][s] in nlt[s].  At step s row s is final:
// every lane adds -L[t][s] times row s's value, read from lane s of its
// 16-lane row by the DPP broadcast inside the multiply-add itself (the
// compiler would issue the broadcast as a move of its own).  Row 15 updates
// nothing.  A DPP read needs two wait states after the VALU write of its
// source, and the compiler does not see the DPP inside the assembly: each
// step opens with a two-cycle nop, whatever the compiler placed before it.
// (Within a step the J columns go in order, so a column written by the
// previous step is read J - 1 >= 3 instructions later anyway.)  Not
// volatile: the steps only order by their data, so the compiler may
// schedule independent work between them.
template <int S, int J>
__device__ __forceinline__ void solve_rows(float (&tc)[J], const float (&nlt)[kChunk]) {
  static_assert(J == 4, "one step updates four columns");
  if constexpr (S < kChunk - 1) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf"
        : "+v"(tc[0]), "+v"(tc[1]), "+v"(tc[2]), "+v"(tc[3]) : "v"(nlt[S]), "n"(S));
    solve_rows<S + 1, J>(tc, nlt);
  }
}

// ---------------------------------------------------------------------------
// LDS of one workgroup
// ---------------------------------------------------------------------------

// Sum of a token's NW per-wave partials (a row of NW floats padded to a
// multiple of four), started from the first partial: 0 + x is not folded
// away for floats, so a zero start would cost an addition.
template <int NW>
__device__ __forceinline__ float wave_sum(const float* row) {
  float s = 0.0f;
#pragma unroll
  for (int w4 = 0; w4 < NW; w4 += 4) {
    const f32x4 p4 = *reinterpret_cast<const f32x4*>(row + w4);
#pragma unroll
    for (int ww = 0; ww < 4 && w4 + ww < NW; ++ww) s = w4 + ww == 0 ? p4[0] : s + p4[ww];
  }
  return s;
}

// What a chunk's elementwise stage publishes (every wave for its channel
// group) and its products read (every wave for its slab).
template <int DK, int NW, int PREC, int KERNEL>
struct alignas(16) ChunkTables {
  static constexpr int NWP = (NW + 3) / 4 * 4;   // norm partials per token, padded
  RowTable<PREC, DK, KERNEL> kt;  // Kt_raw = k exp(Gamma)
  RowTable<PREC, DK, KERNEL> qt;  // Qt_raw = q exp(Gamma)
  KupTable<PREC, DK, KERNEL> kup; // Kup_raw^T [channel][token] = k exp(Gamma_last - Gamma)
  float egl[DK];                  // exp(Gamma_last)
  float beta[kChunk];
  float nq[kChunk][NWP];          // per-wave partial sums of q^2, k^2 [token][wave]
  float nk[kChunk][NWP];
  float pp[NW][kChunk][kPT];      // P_raw partial of wave w, transposed: [s][t]
  float rr[NW][kChunk][kPT];      // R_raw partial of wave w: [t][s]
};

// Private to each elementwise wave: the exact decay sums of its channel group
// (prefix sums of integer parts, of remainders).
template <int NW, int CGS>
struct ExactSums {
  float pg[NW][kChunk][CGS + 4];
  float ps[NW][kChunk][CGS + 4];
};

// Private to each products wave: its copy of -L, [t][s].
template <int NW>
struct NegL {
  float nl[NW][kChunk][kPT];
};

// Without the stage split, every wave runs both stages of a chunk: one set
// of tables, and the two scratch areas overlaid (the exact sums are used
// before the chunk's first barrier, -L between it and the last, never both).
// With it, the elementwise waves fill one set of tables while the products
// waves read the other, and the scratch areas are in use at the same time.
template <int DK, int NW, int PREC, int CGS, int KERNEL, bool SPLIT>
struct alignas(16) ChunkShared {
  ChunkTables<DK, NW, PREC, KERNEL> tab[1];
  union {
    ExactSums<NW, CGS> ex;
    NegL<NW> neg;
  };
};

template <int DK, int NW, int PREC, int CGS, int KERNEL>
struct alignas(16) ChunkShared<DK, NW, PREC, CGS, KERNEL, true> {
  ChunkTables<DK, NW, PREC, KERNEL> tab[2];
  ExactSums<NW, CGS> ex;
  NegL<NW> neg;
};

// Raw inputs of one chunk for one lane: per channel group pass, q, k and
// the gate pre-activation of token lane % 16 at a quarter of the group's
// channels; a quarter of the value slab's columns and the beta logit of that
// token.
template <int NP, bool QBF16, int CGS, int VC>
struct ChunkInputs {
  static constexpr int CPL = CGS / 4;
  RunN<QBF16, CPL> q[NP], k[NP];
  RunN<false, CPL> x[NP];
  RunN<QBF16, VC / 4> v;
  float bl;
};

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

// Per-token log2-decays of N channels, log2(e) g: the softplus form
// -exp(A_log) softplus(x + dt_bias), or the lower-bound form
// lb sigmoid(exp(A_log) (x + dt_bias)) = lb / (1 + exp(-z)) with
// exp(-z) = exp2(-z log2(e)); zero for a padding token.  The bias comes in
// the form the gate takes it: dt_bias for the softplus, -dt_bias exp(A_log)
// log2(e) for the lower bound (whose exponent is then one fused multiply-add
// of the pre-activation).  The softplus is
// taken in base 2, log2(e) softplus(z) = log2(e) max(z, 0) +
// log2(1 + 2^(-|z| log2(e))): the decay factor exp(g) only sees the
// absolute error of g, which here is about exp(A_log) * 1e-7 (the rounding
// of 1 + 2^(...)) at most, as for the softplus with the corrected log1p.
template <int N>
__device__ __forceinline__ void log2_decays(int gate_mode, float amp, float amp2, float lb2, bool live,
                                            const float (&x)[N], const float (&bias)[N], float (&G)[N]) {
  if (gate_mode == KDA_GATE_SOFTPLUS) {     // uniform branch
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const float z = x[j] + bias[j];
      const float l = __builtin_amdgcn_logf(1.0f + exp2_f(-kLog2e * fabsf(z)));   // log2
      G[j] = fmaf(-amp2, fmaxf(z, 0.0f), -amp * l);
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) G[j] = lb2 * __builtin_amdgcn_rcpf(1.0f + exp2_f(fmaf(-amp2, x[j], bias[j])));
  }
#pragma unroll
  for (int j = 0; j < N; ++j) G[j] = live ? G[j] : 0.0f;
}

// ---------------------------------------------------------------------------
// wide decay spans: hierarchical factoring of P and R
// ---------------------------------------------------------------------------
//
// For a chunk whose decay span is too wide for the one-product form, the
// lower triangle of P (and R) is split hierarchically.  Within every
// aligned block of 2h tokens (h = 8, 4, 2, 1), a pair t in the upper half
// and s in the lower half factors through the lower half's last token r:
// exp(Gamma_t - Gamma_s) = exp(Gamma_t - Gamma_r) exp(Gamma_r - Gamma_s),
// where the first exponent is the sum of the gates of t's half up to t
// (inclusive) and the second that of s's half after s: both factors are at
// most 1, and each exponent is a sum inside one half (a segmented scan over
// the lanes), so no large prefix cancels and an infinite decay only gives
// zeros.  One product per level covers all its pairs; its other entries are
// discarded.  The pairs left, inside the diagonal blocks of b = 16 >> tier
// tokens, take the midpoint factoring of their own block (exponents within
// +-span/2, which the tier choice bounds), or at b = 1 the plain diagonal
// sum.  The tier is the smallest whose diagonal blocks all span at most
// kSafeSpan, per wave (its own channel group).

constexpr int kDppQuad0000 = 0x00;   // quad_perm [0,0,0,0]
constexpr int kDppQuad0022 = 0xA0;   // quad_perm [0,0,2,2]
constexpr int kDppQuad1111 = 0x55;   // quad_perm [1,1,1,1]
constexpr int kDppQuad1133 = 0xF5;   // quad_perm [1,1,3,3]
constexpr int kDppQuad2222 = 0xAA;   // quad_perm [2,2,2,2]
constexpr int kDppQuad3333 = 0xFF;   // quad_perm [3,3,3,3]
constexpr int kDppRowShl1 = 0x101;
constexpr int kDppRowShl4 = 0x104;

// Every cross-lane move below runs on all lanes and only then is selected:
// written as `cond ? move(x) : 0` the compiler may issue the move under a
// partial exec mask, and a move that reads a disabled lane gets no value.

// Inclusive sums of x over the aligned blocks of 2, 4 and 8 lanes of each
// 16-lane row (lane n = token).
__device__ __forceinline__ void seg_prefix(float x, int n, float& f2, float& f4, float& f8) {
  const float y1 = dpp_row<kDppQuad0022, false>(x);
  f2 = x + ((n & 1) ? y1 : 0.0f);
  const float y2 = dpp_row<kDppQuad1111, false>(f2);
  f4 = f2 + ((n & 2) ? y2 : 0.0f);
  const float y4 = dpp_row<kDppRowShr4, true>(dpp_row<kDppQuad3333, false>(f4));
  f8 = f4 + ((n & 4) ? y4 : 0.0f);
}

// One step of the inclusive suffix sums within aligned blocks: from blocks
// of H / 2 lanes to blocks of H (H = 2, 4, 8).
template <int H>
__device__ __forceinline__ float seg_suffix_step(float r, int n) {
  float y;
  if constexpr (H == 2) y = dpp_row<kDppQuad1133, false>(r);
  else if constexpr (H == 4) y = dpp_row<kDppQuad2222, false>(r);
  else y = dpp_row<kDppRowShl4, true>(dpp_row<kDppQuad0000, false>(r));
  return r + ((n & (H / 2)) ? 0.0f : y);
}

// The entry (t, s) of a P or R^T accumulator element i at lane (n, g):
// t ^ s = (4g + i) ^ n in both layouts.
__device__ __forceinline__ int pair_xor(int n, int g, int i) { return (4 * g + i) ^ n; }

// Diagonal blocks of B tokens (B = 8, 4, 2): fb holds the inclusive sums of
// the log2-decays within each block; every factor lies within 2^(+-span/2).
template <int B, int PREC, int CPL>
__device__ __forceinline__ void wide_diagonal(f32x4& Pw, f32x4& Rw, const float (&fb)[CPL],
                                              const float (&k)[CPL], const float (&q)[CPL], int n, int g) {
  float kp[CPL], qp[CPL], ks[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    float end;   // the block's total: the sum at its last lane
    if constexpr (B == 8) {
      const float e15 = dpp_row<kDppRowBcast15, true>(fb[j]);
      const float e7 = dpp_row<kDppRowBcast0 + 7, true>(fb[j]);
      end = (n & 8) ? e15 : e7;
    } else if constexpr (B == 4) end = dpp_row<kDppQuad3333, false>(fb[j]);
    else end = dpp_row<kDppQuad1133, false>(fb[j]);
    const float ep = exp2_f(fmaf(-0.5f, end, fb[j]));
    kp[j] = k[j] * ep;
    qp[j] = q[j] * ep;
    ks[j] = k[j] * __builtin_amdgcn_rcpf(ep);
  }
  f32x4 Pd = {0.0f, 0.0f, 0.0f, 0.0f}, Rd = {0.0f, 0.0f, 0.0f, 0.0f};
  mma(Pd, make_frag<PREC, CPL>(kp), make_frag<PREC, CPL>(ks));
  mma(Rd, make_frag<PREC, CPL>(ks), make_frag<PREC, CPL>(qp));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool own = pair_xor(n, g, i) < B;
    Pw[i] = own ? Pd[i] : Pw[i];
    Rw[i] = own ? Rd[i] : Rw[i];
  }
}

// The exclusive suffix sums within aligned blocks of H lanes (the gates
// after s inside its block), from the inclusive ones rh.
template <int H, int CPL>
__device__ __forceinline__ void suffix_excl(float (&rx)[CPL], const float (&rh)[CPL], int n) {
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const float y = dpp_row<kDppRowShl1, true>(rh[j]);
    rx[j] = ((n + 1) & (H - 1)) ? y : 0.0f;
  }
}

// The level of half size H: fh holds the inclusive sums within aligned
// blocks of H lanes, rx the exclusive suffix sums within them (the lower
// half's exponents; zero at H = 1).
template <int H, int PREC, int CPL>
__device__ __forceinline__ void wide_level(f32x4& Pw, f32x4& Rw, const float (&fh)[CPL], const float (&rx)[CPL],
                                           const float (&k)[CPL], const float (&q)[CPL], int n, int g) {
  const bool up = (n & H) != 0;
  float aP[CPL], aR[CPL], bK[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const float f = exp2_f(up ? fh[j] : rx[j]);
    const float kf = k[j] * f;
    aP[j] = up ? kf : 0.0f;
    aR[j] = up ? q[j] * f : 0.0f;
    bK[j] = up ? 0.0f : kf;
  }
  f32x4 Pl = {0.0f, 0.0f, 0.0f, 0.0f}, Rl = {0.0f, 0.0f, 0.0f, 0.0f};
  const Frag<PREC, CPL> fb = make_frag<PREC, CPL>(bK);
  mma(Pl, make_frag<PREC, CPL>(aP), fb);
  mma(Rl, fb, make_frag<PREC, CPL>(aR));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int x = pair_xor(n, g, i);
    const bool own = x >= H && x < 2 * H;
    Pw[i] = own ? Pl[i] : Pw[i];
    Rw[i] = own ? Rl[i] : Rw[i];
  }
}

// ---------------------------------------------------------------------------
// tile order
// ---------------------------------------------------------------------------

// A float's bits as an integer ordered like the float (NaNs at the ends):
// comparisons of keys are a total order.
__device__ __forceinline__ int order_key(float x) {
  const int k = __float_as_int(x);
  return k ^ ((k >> 31) & 0x7fffffff);
}

// The value head of rank r when the HV heads are ordered by A_log, largest
// first (ties by head index).  Keys form a total order, so the map from
// rank to head is a permutation.  O(HV^2 / 64) per lane, once per wave.
__device__ __forceinline__ int head_by_decay_rank(const float* a_log, int HV, int r, int lane) {
  int result = 0;
  for (int base = 0; base < HV; base += kWave) {
    const int h = base + lane;
    const int kh = h < HV ? order_key(a_log[h]) : 0;
    int rank = 0;
    for (int b2 = 0; b2 < HV; b2 += kWave) {
      const int kv = b2 + lane < HV ? order_key(a_log[b2 + lane]) : 0;
      const int cnt = HV - b2 < kWave ? HV - b2 : kWave;
      for (int j = 0; j < cnt; ++j) {
        const int kj = __builtin_amdgcn_readlane(kv, j);
        rank += (kj > kh || (kj == kh && b2 + j < h)) ? 1 : 0;
      }
    }
    const unsigned long long hit = __ballot(h < HV && rank == r);
    if (hit != 0) result = base + __builtin_ctzll(hit);
  }
  return result;
}

// Under the softplus gate, heads are dispatched by decay rank when requests
// are long (64 tokens or more on average): a larger A_log means faster
// decay, wider chunk spans and more matrix products per chunk, so those
// tiles start first and the grid's tail holds the cheap ones (96-head
// batch of 8 x 2048 tokens: 1.48 -> 1.35 ms).  The lower-bound gate bounds
// every span, its tiles cost the same, and the request-major order keeps
// concurrent tiles on neighbouring rows of the token tensors (2% faster
// than head-major).  For short requests the ranking would cost more than
// it saves.
constexpr int kOrderMinTokens = 64;
constexpr int kOrderMaxHeads = 1024;

// Workgroups per (request, value head) tile: two with 16-column slabs.
constexpr int prefill_tile_groups(int vc) { return vc == kNarrowSlabCols ? 2 : 1; }

// With SPLIT (the stage split), a workgroup is twice as many waves: the
// first half runs the elementwise stage of chunk c + 1 while the second half
// runs the products of chunk c, the tables double-buffered between them, one
// barrier per chunk; the halves share the SIMDs, so each stage's waits are
// filled by the other's work.  At dv = 128 that is eight waves (at most 256
// registers per lane, two waves per SIMD) and 99 KiB of LDS: one workgroup
// per CU.  Without it, every wave runs both stages of a chunk in turn, with
// a barrier after each.
template <int DK, int DV, bool QBF16, bool SBF16, bool VFIRST, int PREC, int VC, bool SPLIT>
__global__ void __launch_bounds__(DV / VC / prefill_tile_groups(VC) * kWave * (SPLIT ? 2 : 1), 1)
kda_prefill_chunks(DecodeArgs a) {
  constexpr int NWG = prefill_tile_groups(VC);
  constexpr int NTV = VC / 16;           // value tiles per wave
  constexpr int VPL = VC / 4;            // value columns per lane in the V operand
  constexpr int NW = DV / VC / NWG;      // slabs per workgroup, and elementwise waves
  constexpr int CGS = kGroupChannels;
  constexpr int CPL = CGS / 4;           // channels per lane in the elementwise stage
  constexpr int NG = DK / CGS;           // channel groups
  constexpr int NP = (NG + NW - 1) / NW; // channel group passes per wave
  constexpr int MT = DK / 16;            // state row tiles
  constexpr int KS = DK / 32;            // K = 32 steps over the channels
  // the remaining template parameters, as the tables' per-kernel tag
  constexpr int KERNEL = (QBF16 ? 1 : 0) + (SBF16 ? 2 : 0) + (VFIRST ? 4 : 0) + 8 * VC + 1024 * DV +
                         (SPLIT ? 65536 : 0);
  using Shared = ChunkShared<DK, NW, PREC, CGS, KERNEL, SPLIT>;

  __shared__ Shared sh;

  const int lane = threadIdx.x % kWave;
  // The wave's role, from its index read into a scalar register: every
  // branch on it is uniform, so each wave executes exactly its own role's
  // code and barriers.
  const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
  const bool e_wave = !SPLIT || wid < NW;    // runs the elementwise stage
  const bool p_wave = !SPLIT || wid >= NW;   // runs the products
  const int w = SPLIT && wid >= NW ? wid - NW : wid;   // channel group / slab
  const int n = lane % 16;               // token / accumulator column
  const int g = lane / 16;               // channel quarter / accumulator row group

  // With the split, the stage that bounds a chunk issues first when both of
  // a SIMD's waves are ready: the products, but with 16-column slabs (half a
  // slab's products against the whole elementwise stage) under the softplus
  // gate (with its wide-span tiers) the elementwise stage.
  if constexpr (SPLIT) {
    const bool elementwise_first = VC == kNarrowSlabCols && a.gate_mode == KDA_GATE_SOFTPLUS;
    if (elementwise_first ? e_wave : p_wave) __builtin_amdgcn_s_setprio(1);
  }

  // the workgroup's tile, and its part of the tile's value columns
  const uint32_t tile_id = blockIdx.x / NWG;
  const int part = static_cast<int>(blockIdx.x % NWG);
  int b, hv;
  if (a.gate_mode == KDA_GATE_SOFTPLUS && a.HV > 1 && a.HV <= kOrderMaxHeads &&
      a.T / kOrderMinTokens >= a.B) {   // uniform
    b = static_cast<int>(tile_id % static_cast<uint32_t>(a.B));
    hv = head_by_decay_rank(a.a_log, a.HV, static_cast<int>(tile_id / static_cast<uint32_t>(a.B)), lane);
  } else {
    b = static_cast<int>(tile_id / static_cast<uint32_t>(a.HV));
    hv = static_cast<int>(tile_id) - b * a.HV;
  }
  const int h = hv / a.G;
  int t0 = a.cu_seqlens[b];
  int t1 = a.cu_seqlens[b + 1];
  t0 = t0 < 0 ? 0 : (t0 > a.T ? a.T : t0);
  t1 = t1 < t0 ? t0 : (t1 > a.T ? a.T : t1);
  if (t1 == t0) return;
  const int slot = a.state_indices[b];
  const int vcol0 = VC * (NW * part + w);

  if (slot < 0 || slot >= a.N) {   // skipped request: zero rows, no state access
    if (p_wave)
      for (int t = t0; t < t1; ++t)
        if (lane < VC) store_elem<QBF16>(a.out, (static_cast<int64_t>(t) * a.HV + hv) * DV + vcol0 + lane, 0.0f);
    return;
  }

  // ---- the state slab into the accumulators: S[mt][nt][i] is
  // S[16 mt + 4g + i][vcol0 + 16 nt + n]
  f32x4 S[MT][NTV];
  // Element (d, v) of the tile sits at v * DK + d (value-first) or d * DV + v
  // (key-first); with d = 16 mt + 4 g + i and v = vcol0 + 16 nt + n the
  // lane's part is lane_off, the rest a constant per (mt, nt, i).
  constexpr int kElem = SBF16 ? 2 : 4;
  char* const tile = static_cast<char*>(a.state_pool) +
                     (static_cast<int64_t>(slot) * a.HV + hv) * (DK * DV * kElem);
  const __amdgpu_buffer_rsrc_t st_res = tile_resource(tile, DK * DV * kElem);
  const int lane_off = (VFIRST ? (vcol0 + n) * DK + 4 * g : 4 * g * DV + vcol0 + n) * kElem;
  if (p_wave) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt) {
        if constexpr (VFIRST) {   // four consecutive keys: one access
          float x[4];
          load_state<SBF16, 4>(st_res, lane_off, (16 * nt * DK + 16 * mt) * kElem, x);
#pragma unroll
          for (int i = 0; i < 4; ++i) S[mt][nt][i] = x[i];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x;
            load_state<SBF16, 1>(st_res, lane_off, ((16 * mt + i) * DV + 16 * nt) * kElem, &x);
            S[mt][nt][i] = x;
          }
        }
      }
  }

  // channel groups of this wave: group w + NW p covers channels
  // [CGS (w + NW p), +CGS); this lane's CPL start at chan0[p]
  // gates are carried in base-2 units, G2 = G log2(e), so that every
  // exp(.) of them is one exp2 instruction
  const float amp = exp_f(a.a_log[hv]);
  const float amp2 = amp * kLog2e;
  const float lb2 = a.lower_bound * kLog2e;
  // the gate bias of the lane's channels, in the form log2_decays takes
  const bool lb_gate = a.gate_mode != KDA_GATE_SOFTPLUS;
  // Under the lower-bound gate a token's log-decay lies in [lower_bound, 0],
  // so a chunk spans at most -16 lower_bound: within kSafeSpan (with a margin
  // for rounding) no chunk needs the wide-span tiers, nor the check for them.
  const bool narrow_gate = lb_gate && -a.lower_bound * kChunk <= 0.99f * kSafeSpan;
  float dtb[NP][CPL];
  int chan0[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int gi = w + NW * p;
    chan0[p] = CGS * gi + CPL * g;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const float bj = gi < NG ? a.dt_bias[static_cast<int64_t>(hv) * DK + chan0[p] + j] : 0.0f;
      dtb[p][j] = lb_gate ? -amp2 * bj : bj;
    }
  }

  // Loads are unconditional (a token past the request's end reads the
  // request's last row and is zeroed where it is used), so the compiler can
  // count them exactly and never waits for more than the oldest in flight.
  // Without the split a wave loads its channels' q, k, gates and its slab's
  // v together; with it the elementwise waves load the former, the products
  // waves v.
  // The rows are addressed from the chunk's first row r0 (a uniform base)
  // plus the lane's row offset dr (a 32-bit byte offset).
  constexpr int kIn = QBF16 ? 2 : 4;   // bytes per q, k, v element
  auto load_inputs = [&](ChunkInputs<NP, QBF16, CGS, VC>& in, int c0) {
    const int r0 = c0 < t1 ? c0 : t1 - 1;
    const uint32_t dr = static_cast<uint32_t>(n < t1 - 1 - r0 ? n : t1 - 1 - r0);
    if (e_wave) {
      const char* const qb = static_cast<const char*>(a.q) + ((static_cast<int64_t>(r0) * a.H + h) * DK) * kIn;
      const char* const kb = static_cast<const char*>(a.k) + ((static_cast<int64_t>(r0) * a.H + h) * DK) * kIn;
      const char* const xb = reinterpret_cast<const char*>(a.raw_gate) + ((static_cast<int64_t>(r0) * a.HV + hv) * DK) * 4;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (NG % NW == 0 || w + NW * p < NG) {
          const uint32_t qk_off = (dr * static_cast<uint32_t>(a.H * DK) + chan0[p]) * kIn;
          in.q[p].load(qb, qk_off);
          in.k[p].load(kb, qk_off);
          in.x[p].load(xb, (dr * static_cast<uint32_t>(a.HV * DK) + chan0[p]) * 4);
        }
      }
      in.bl = a.beta_logits[(static_cast<int64_t>(r0) * a.HV + hv) + dr * static_cast<uint32_t>(a.HV)];
    }
    if (p_wave)
      in.v.load(static_cast<const char*>(a.v) + ((static_cast<int64_t>(r0) * a.HV + hv) * DV) * kIn,
                (dr * static_cast<uint32_t>(a.HV * DV) + vcol0 + VPL * g) * kIn);
  };

  // One input buffer: each chunk first takes its inputs out of it (q, k
  // and the gate unpacked, v and beta kept), then refills it with the next
  // chunk's, which stay in flight while this chunk is processed.
  ChunkInputs<NP, QBF16, CGS, VC> in;
  ChunkInputs<NP, QBF16, CGS, VC> in_v;   // with the split: the products waves' v
  load_inputs(SPLIT && p_wave ? in_v : in, t0);
  // every load so far (state, first inputs) completes here, outside the
  // loop, so the loop's waits only cover the previous chunk's prefetch
  __builtin_amdgcn_s_waitcnt(0);
  const int nchunks = (t1 - t0 + kChunk - 1) / kChunk;
  // iteration i runs the elementwise stage of chunk i (i + 1 with the
  // split, whose first iteration, i = -1, runs only that) and the products
  // of chunk i
  for (int i = SPLIT ? -1 : 0; i < nchunks; ++i) {
    const int ce = t0 + (SPLIT ? i + 1 : i) * kChunk;   // the elementwise stage's chunk
    RunN<QBF16, VPL> v_cur;
    if (e_wave && ce < t1) {   // uniform
      auto& tab = sh.tab[SPLIT ? (i + 1) & 1 : 0];
      const int c0 = ce;
      const int m = t1 - c0 < kChunk ? t1 - c0 : kChunk;
      const bool live = n < m;
      // This chunk's inputs leave the buffer (q and k widened, the gate
      // pre-activations turned into log2-decays) before it is refilled with
      // the next chunk's: the raw words are dead by then, so the refill
      // loads into the same registers instead of into new ones that the
      // end of the iteration would copy back.
      float qin[NP][CPL], kin[NP][CPL], gin[NP][CPL];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        float xin[CPL];
        in.q[p].unpack(qin[p]);
        in.k[p].unpack(kin[p]);
        in.x[p].unpack(xin);
        log2_decays<CPL>(a.gate_mode, amp, amp2, lb2, live, xin, dtb[p], gin[p]);
#pragma unroll
        for (int j = 0; j < CPL; ++j) asm volatile("" : "+v"(qin[p][j]), "+v"(kin[p][j]), "+v"(gin[p][j]));
      }
      if constexpr (!SPLIT) v_cur = in.v;
      const float bl_cur = in.bl;
      asm volatile("" : : "v"(bl_cur) : "memory");
      load_inputs(in, c0 + kChunk);   // past the end: reloads the last row, unused

      // ================= stage E: this wave's channels, lane = (token n, quarter g)
      float sq = 0.0f, sk = 0.0f;
      f32x4 Pp = {0.0f, 0.0f, 0.0f, 0.0f};   // P_raw partial (acc: rows t, column s)
      f32x4 Rp = {0.0f, 0.0f, 0.0f, 0.0f};   // R_raw^T partial (acc: rows s, column t)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (w + NW * p >= NG) continue;
        const float (&q)[CPL] = qin[p];
        const float (&k)[CPL] = kin[p];
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          sq = fmaf(q[j], q[j], sq);
          sk = fmaf(k[j], k[j], sk);
        }
        // G, GL: Gamma and Gamma_last of the lane's channels, times log2(e);
        // gr the per-token log2-decays themselves, for wide spans
        float G[CPL], GL[CPL], gr[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) G[j] = gr[j] = gin[p][j];
        row_scan_n<CPL>(G);
#pragma unroll
        for (int j = 0; j < CPL; ++j) GL[j] = dpp_row<kDppRowBcast15, true>(G[j]);
        bool wide = false;
        if (!narrow_gate) {   // uniform
          bool wide_lane = false;
#pragma unroll
          for (int j = 0; j < CPL; ++j) wide_lane |= !(-GL[j] <= kSafeSpan * kLog2e);
          wide = __any(wide_lane);
        }
        // Kt, Qt and exp(Gamma_last) of the lane's channels into the tables
        auto store_rows = [&](const float (&kt)[CPL], const float (&qt)[CPL], const float (&egl)[CPL]) {
          tab.kt.template store<CPL>(n, chan0[p], kt);
          tab.qt.template store<CPL>(n, chan0[p], qt);
          if (n == 0) {
#pragma unroll
            for (int j = 0; j < CPL; j += 4)
              *reinterpret_cast<f32x4*>(&tab.egl[chan0[p] + j]) = f32x4{egl[j], egl[j + 1], egl[j + 2], egl[j + 3]};
          }
        };
        // Kup's factor exp(Gamma_last - Gamma_s) is exactly 1 for the last
        // real token.  In a ragged chunk Gamma_last is read from lane 15,
        // whose prefix sum holds the same terms as lane m - 1's (the padding
        // adds zeros) added in another order, so the difference would be an
        // ulp of |Gamma| instead of 0.
        const bool last_real = n == m - 1;
        if (!wide) {   // uniform
          // This group's P and R parts as one product each, of Kp = k
          // exp(Gamma - c) and Ks = k exp(c - Gamma), c = Gamma_last / 2 (Qp
          // likewise).  Token 15's exp(Gamma - c) is exp(c), so the tables
          // take the same exponentials: Kt = Kp exp(c), Qt = Qp exp(c), Kup =
          // Ks exp(c), exp(Gamma_last) = exp(c)^2.
          float kp[CPL], qp[CPL], ks[CPL];
          {
            float ec[CPL], kt[CPL], qt[CPL], egl[CPL];
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
              const float ep = exp2_f(fmaf(-0.5f, GL[j], G[j]));
              ec[j] = dpp_row<kDppRowBcast15, true>(ep);
              kp[j] = k[j] * ep;
              qp[j] = q[j] * ep;
              ks[j] = k[j] * __builtin_amdgcn_rcpf(ep);
              kt[j] = kp[j] * ec[j];
              qt[j] = qp[j] * ec[j];
              egl[j] = ec[j] * ec[j];
            }
            store_rows(kt, qt, egl);
#pragma unroll
            for (int j = 0; j < CPL; j += 2)
              tab.kup.store2(chan0[p] + j, n, last_real ? k[j] : ks[j] * ec[j],
                             last_real ? k[j + 1] : ks[j + 1] * ec[j + 1]);
          }
          const Frag<PREC, CPL> fkp = make_frag<PREC, CPL>(kp);
          const Frag<PREC, CPL> fks = make_frag<PREC, CPL>(ks);
          const Frag<PREC, CPL> fqp = make_frag<PREC, CPL>(qp);
          mma(Pp, fkp, fks);    // P[t][s] = Kp[t] . Ks[s]
          mma(Rp, fks, fqp);    // R^T[s][t] = Ks[s] . Qp[t]
        } else {
          bool exact_lane = false;
#pragma unroll
          for (int j = 0; j < CPL; ++j) exact_lane |= !(-GL[j] <= kExactSpan);
          const bool exact = __any(exact_lane);
          float kt[CPL], qt[CPL], egl[CPL];
          if (!exact) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
              const float eg = exp2_f(G[j]);
              egl[j] = dpp_row<kDppRowBcast15, true>(eg);   // exp(Gamma_last), from token 15
              kt[j] = k[j] * eg;
              qt[j] = q[j] * eg;
            }
#pragma unroll
            for (int j = 0; j < CPL; j += 2)
              tab.kup.store2(chan0[p] + j, n, last_real ? k[j] : k[j] * exp2_f(GL[j] - G[j]),
                             last_real ? k[j + 1] : k[j + 1] * exp2_f(GL[j + 1] - G[j + 1]));
          } else {
            // Gamma again, as Gb + Gs: Gb the prefix sums of the gates' integer
            // parts (exact), Gs those of the remainders (at most 16 in
            // magnitude).  A difference Gamma_t - Gamma_s is then
            // an exact difference plus a small one, whatever the decays before
            // s: no cancellation against a large prefix, and no inf - inf.
            // The per-token gates go through this lane's table rows, four
            // channels at a time, so few values are live at once.
#pragma unroll
            for (int j = 0; j < CPL; j += 4)
              *reinterpret_cast<f32x4*>(&sh.ex.pg[w][n][CPL * g + j]) = f32x4{gr[j], gr[j + 1], gr[j + 2], gr[j + 3]};
#pragma unroll
            for (int j = 0; j < CPL; j += 4) {
              const f32x4 x4 = *reinterpret_cast<const f32x4*>(&sh.ex.pg[w][n][CPL * g + j]);
              f32x4 b4, r4;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float gj = fmaxf(x4[i], -kGateFloor);
                const float gb = kGateStep * ceilf(gj * (1.0f / kGateStep));
                b4[i] = row_scan(gb);
                r4[i] = row_scan(gj - gb);
              }
              *reinterpret_cast<f32x4*>(&sh.ex.pg[w][n][CPL * g + j]) = b4;
              *reinterpret_cast<f32x4*>(&sh.ex.ps[w][n][CPL * g + j]) = r4;
            }
            wave_lds_order();
#pragma unroll
            for (int j = 0; j < CPL; j += 4) {
              const f32x4 b4 = *reinterpret_cast<const f32x4*>(&sh.ex.pg[w][n][CPL * g + j]);
              const f32x4 r4 = *reinterpret_cast<const f32x4*>(&sh.ex.ps[w][n][CPL * g + j]);
              float kl[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float dlast = (dpp_row<kDppRowBcast15, true>(b4[i]) - b4[i]) +
                                    (dpp_row<kDppRowBcast15, true>(r4[i]) - r4[i]);
                const float eg = exp2_f(b4[i] + r4[i]);
                egl[j + i] = dpp_row<kDppRowBcast15, true>(eg);
                kt[j + i] = k[j + i] * eg;
                qt[j + i] = q[j + i] * eg;
                kl[i] = last_real ? k[j + i] : k[j + i] * exp2_f(dlast);
              }
              tab.kup.store2(chan0[p] + j, n, kl[0], kl[1]);
              tab.kup.store2(chan0[p] + j + 2, n, kl[2], kl[3]);
            }
          }
          store_rows(kt, qt, egl);
          // hierarchical factoring (see wide_level): the tier from the spans
          // of the aligned blocks of 8, 4 and 2 tokens.  The gates are <= 0,
          // so a block's most negative partial sum is its total: the minimum
          // over all lanes and channels is the widest block's span.
          float f2[CPL], f4[CPL], f8[CPL];
          float m8 = 0.0f, m4 = 0.0f, m2 = 0.0f;
#pragma unroll
          for (int j = 0; j < CPL; ++j) {
            seg_prefix(gr[j], n, f2[j], f4[j], f8[j]);
            m8 = fminf(m8, f8[j]);
            m4 = fminf(m4, f4[j]);
            m2 = fminf(m2, f2[j]);
          }
          constexpr float kSpan2 = kSafeSpan * kLog2e;
          const int tier = !__any(!(-m8 <= kSpan2)) ? 1 : !__any(!(-m4 <= kSpan2)) ? 2
                         : !__any(!(-m2 <= kSpan2)) ? 3 : 4;
          f32x4 Pw = {0.0f, 0.0f, 0.0f, 0.0f}, Rw = {0.0f, 0.0f, 0.0f, 0.0f};
          if (tier == 1) {
            // the common wide case: the halves' spans are bounded, so the
            // lower half's exponents may be taken as differences of its
            // prefix sums (no larger than the tier-0 exponents)
            wide_diagonal<8, PREC>(Pw, Rw, f8, k, q, n, g);
            float rx[CPL];
#pragma unroll
            for (int j = 0; j < CPL; ++j) rx[j] = dpp_row<kDppRowBcast0 + 7, true>(f8[j]) - f8[j];
            wide_level<8, PREC>(Pw, Rw, f8, rx, k, q, n, g);
          } else {
            if (tier == 2) wide_diagonal<4, PREC>(Pw, Rw, f4, k, q, n, g);
            else if (tier == 3) wide_diagonal<2, PREC>(Pw, Rw, f2, k, q, n, g);
            else {   // blocks of one token: R's diagonal is q_t . k_t (P's is unused)
              float qk = 0.0f;
#pragma unroll
              for (int j = 0; j < CPL; ++j) qk = fmaf(q[j], k[j], qk);
              qk = cross_row_sum(qk);
#pragma unroll
              for (int i = 0; i < 4; ++i) Rw[i] = pair_xor(n, g, i) == 0 ? qk : 0.0f;
            }
            // the lower halves' exponents from suffix sums within blocks of
            // 1, 2, 4, 8 in turn (exact for any span)
            float rs[CPL], rx[CPL];
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
              rs[j] = seg_suffix_step<2>(gr[j], n);
              rx[j] = 0.0f;
            }
            if (tier >= 4) wide_level<1, PREC>(Pw, Rw, gr, rx, k, q, n, g);
            if (tier >= 3) {
              suffix_excl<2>(rx, rs, n);
              wide_level<2, PREC>(Pw, Rw, f2, rx, k, q, n, g);
            }
#pragma unroll
            for (int j = 0; j < CPL; ++j) rs[j] = seg_suffix_step<4>(rs[j], n);
            suffix_excl<4>(rx, rs, n);
            wide_level<4, PREC>(Pw, Rw, f4, rx, k, q, n, g);
#pragma unroll
            for (int j = 0; j < CPL; ++j) rs[j] = seg_suffix_step<8>(rs[j], n);
            suffix_excl<8>(rx, rs, n);
            wide_level<8, PREC>(Pw, Rw, f8, rx, k, q, n, g);
          }
          Pp += Pw;
          Rp += Rw;
        }
      }
      // publish the partials
      sq = cross_row_sum(sq);
      sk = cross_row_sum(sk);
      if (g == 0) {
        tab.nq[n][w] = sq;
        tab.nk[n][w] = sk;
        if (w == 0) tab.beta[n] = live ? sigmoid_f(bl_cur) : 0.0f;
      }
      *reinterpret_cast<f32x4*>(&tab.pp[w][n][4 * g]) = Pp;   // pp[s = n][t = 4g + i]
      *reinterpret_cast<f32x4*>(&tab.rr[w][n][4 * g]) = Rp;   // rr[t = n][s = 4g + i]
    }
    if constexpr (!SPLIT) lds_barrier();

    if (p_wave && i >= 0) {   // uniform
      const auto& tab = sh.tab[SPLIT ? i & 1 : 0];
      const int c0 = t0 + i * kChunk;
      const int m = t1 - c0 < kChunk ? t1 - c0 : kChunk;
      const bool live = n < m;
      if constexpr (SPLIT) {
        // v of padding tokens zeroed in its storage words, before the
        // buffer is refilled (as in the elementwise stage)
#pragma unroll
        for (int j = 0; j < RunN<QBF16, VPL>::W; ++j) {
          v_cur.w[j] = live ? in_v.v.w[j] : 0u;
          asm volatile("" : "+v"(v_cur.w[j]));
        }
        asm volatile("" : : : "memory");
        load_inputs(in_v, c0 + kChunk);
      } else {
#pragma unroll
        for (int j = 0; j < RunN<QBF16, VPL>::W; ++j) v_cur.w[j] = live ? v_cur.w[j] : 0u;
      }
      // ================= per wave: norms, L, T, then the slab's products
      float rk[4], br[4];
      {
        const f32x4 bt = *reinterpret_cast<const f32x4*>(&tab.beta[4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          rk[i] = rsqrt_f(wave_sum<NW>(&tab.nk[4 * g + i][0]) + a.l2_eps);
          br[i] = bt[i] * rk[i];
        }
      }
      const float rkn = rsqrt_f(wave_sum<NW>(&tab.nk[n][0]) + a.l2_eps);
      const float rqn = a.scale * rsqrt_f(wave_sum<NW>(&tab.nq[n][0]) + a.l2_eps);
      // -L[t][s] for rows t = 4g + i, column s = n, into the wave's copy
      {
        f32x4 Pf = *reinterpret_cast<const f32x4*>(&tab.pp[0][n][4 * g]);
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) Pf += *reinterpret_cast<const f32x4*>(&tab.pp[ww][n][4 * g]);
        const float cs = rkn * tab.beta[n];
#pragma unroll
        for (int i = 0; i < 4; ++i) sh.neg.nl[w][4 * g + i][n] = n < 4 * g + i ? -(rk[i] * cs * Pf[i]) : 0.0f;
      }
      wave_lds_order();
      // T = (I + L)^-1 with lane (t = n, g) holding T[t][4g + j], the A operand
      // of T X: forward substitution over the rows, T[t][.] -= L[t][s] T[s][.]
      // for s = 0, 1, ...; L is zero on and above the diagonal, so the update
      // leaves rows t <= s unchanged.  (Every wave solves the whole of T: with
      // each wave solving a quarter of the columns and the quarters exchanged
      // through LDS, the extra barrier cost more than the saved instructions.)
      float tc[4];
      {
        float nlt[kChunk];
#pragma unroll
        for (int q4 = 0; q4 < kChunk / 4; ++q4) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sh.neg.nl[w][n][4 * q4]);
#pragma unroll
          for (int j = 0; j < 4; ++j) nlt[4 * q4 + j] = l4[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) tc[j] = n == 4 * g + j ? 1.0f : 0.0f;
        solve_rows<0, 4>(tc, nlt);
      }
      // R_raw as the B operand of R_raw^T: lane (t = n, g) holds R[t][4g + j]
      float rv[4];
      {
        f32x4 Rf = *reinterpret_cast<const f32x4*>(&tab.rr[0][n][4 * g]);
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) Rf += *reinterpret_cast<const f32x4*>(&tab.rr[ww][n][4 * g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) rv[j] = 4 * g + j <= n ? Rf[j] : 0.0f;
      }

      // X = V - diag(rk) Kt_raw S,  Y^T = S^T Qt_raw^T   (per value tile nt)
      f32x4 X[NTV], YT[NTV];
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt) X[nt] = YT[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const Frag<PREC, 8> fk = tab.kt.frag8(n, s, g);
        const Frag<PREC, 8> fq = tab.qt.frag8(n, s, g);
        // exp(Gamma_last) of the two tiles' rows: S = diag(exp(Gamma_last)) S
        // is applied here, on the way to the operands
        const f32x4 e0 = *reinterpret_cast<const f32x4*>(&tab.egl[32 * s + 4 * g]);
        const f32x4 e1 = *reinterpret_cast<const f32x4*>(&tab.egl[32 * s + 16 + 4 * g]);
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt) {
          const Frag<PREC, 8> fs = acc_frag8_decay<PREC>(S[2 * s][nt], S[2 * s + 1][nt], e0, e1);
          mma(X[nt], fk, fs);
          mma(YT[nt], fs, fq);
        }
      }
      {
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) X[nt][i] *= -rk[i];
          mma_identity<PREC, QBF16, VPL>(X[nt], v_cur, nt, n, g);
        }
      }

      // U = T X, U' = diag(beta rk) U, O^T = diag(rq)(Y^T + U'^T R_raw^T),
      // S = diag(exp(Gamma_last)) S + Kup_raw^T U'.  (The K = 16 products of
      // the chunk's own tokens stay in the matrix precision: on the fp32
      // instruction, whose operands need no split, they measured slower.)
      const Frag<PREC, 4> ft = make_frag<PREC, 4>(tc);
      const Frag<PREC, 4> fr = make_frag<PREC, 4>(rv);
      Frag<PREC, 4> fu[NTV];
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt) {
        f32x4 U = {0.0f, 0.0f, 0.0f, 0.0f};
        mma<PREC, 4, true>(U, ft, acc_frag4<PREC>(X[nt]));
#pragma unroll
        for (int i = 0; i < 4; ++i) U[i] *= br[i];
        fu[nt] = acc_frag4<PREC>(U);
        f32x4 OT = YT[nt];
        mma(OT, fu[nt], fr);
        if (live) {
#pragma unroll
          for (int i = 0; i < 4; ++i) OT[i] *= rqn;
          store4<QBF16>(static_cast<char*>(a.out) + ((static_cast<int64_t>(c0) * a.HV + hv) * DV) * kIn,
                        (n * static_cast<uint32_t>(a.HV * DV) + vcol0 + 16 * nt + 4 * g) * kIn, OT);
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const Frag<PREC, 4> fk = tab.kup.frag4(16 * mt + n, g);
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt) mma(S[mt][nt], fk, fu[nt]);
      }
    }
    lds_barrier();   // the tables of this iteration's products are rewritten next
  }

  // ---- the advanced state back to its slot
  if (p_wave) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt) {
        if constexpr (VFIRST) {
          const float x[4] = {S[mt][nt][0], S[mt][nt][1], S[mt][nt][2], S[mt][nt][3]};
          store_state<SBF16, 4>(st_res, lane_off, (16 * nt * DK + 16 * mt) * kElem, x);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = S[mt][nt][i];
            store_state<SBF16, 1>(st_res, lane_off, ((16 * mt + i) * DV + 16 * nt) * kElem, &x);
          }
        }
      }
  }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

// The launch's own status decides KDA_ERR_LAUNCH (hipGetLastError could
// also report an earlier, unrelated error of the calling thread).
template <int DK, int DV, bool QBF16, bool SBF16, bool VFIRST, int PREC, int VC, bool SPLIT>
int launch_one(const DecodeArgs& a, hipStream_t stream) {
  constexpr int NWG = prefill_tile_groups(VC);
  const int64_t grid = static_cast<int64_t>(a.B) * a.HV * NWG;
  void* kargs[] = {const_cast<DecodeArgs*>(&a)};
  const hipError_t rc = hipLaunchKernel(
      reinterpret_cast<const void*>(&kda_prefill_chunks<DK, DV, QBF16, SBF16, VFIRST, PREC, VC, SPLIT>),
      dim3(static_cast<uint32_t>(grid)), dim3(DV / VC / NWG * kWave * (SPLIT ? 2 : 1)), kargs, 0, stream);
  return rc == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

// dv = 128 batches take the stage split: with its bounding stage's waves
// prioritized, one eight-wave workgroup per CU beats two plain four-wave
// workgroups (eight 2048-token requests over 96 heads: 1132 -> 1087 us,
// softplus 1328 -> 1291 us; 384 tiles 719 -> 679 us; 1536 tiles, three
// full rounds of the plain form, 1096 -> 1105 us), and it spills less with
// fp32 q/k/v.  dv = 64 takes it while one round of it (two four-wave
// workgroups per CU) holds the batch: the plain two-wave workgroups fit four
// per CU and, at dk = dv = 64, hold 1024 tiles in one round (2048-token
// requests over 96 heads: 192 tiles 370 -> 204 us, 512 tiles 546 -> 321 us,
// 576 546 -> 549 us, 768 550 -> 565 us).  Up to 128 tiles each tile is two
// workgroups of 16-column slabs, so that twice as many CUs work (one 16
// 384-token prompt over 96 heads: 2.32 ms against 3.80 ms as one plain
// workgroup per tile at dv = 128; 1.49 ms against 2.91 ms at dv = 64).
constexpr int64_t kCUs = 256;   // MI355X
constexpr int64_t kNarrowMaxTiles = kCUs / 2;
constexpr int64_t kSplitMaxTiles64 = 2 * kCUs;

template <int DK, int DV, bool QBF16, bool SBF16, bool VFIRST, int PREC>
int pick_slab(const DecodeArgs& a, hipStream_t s) {
  const int64_t tiles = static_cast<int64_t>(a.B) * a.HV;
  if constexpr (DV == 32) {
    return launch_one<DK, DV, QBF16, SBF16, VFIRST, PREC, kSlabCols, false>(a, s);
  } else {
    if (tiles <= kNarrowMaxTiles) return launch_one<DK, DV, QBF16, SBF16, VFIRST, PREC, kNarrowSlabCols, true>(a, s);
    if constexpr (DV == 64)
      if (tiles > kSplitMaxTiles64) return launch_one<DK, DV, QBF16, SBF16, VFIRST, PREC, kSlabCols, false>(a, s);
    return launch_one<DK, DV, QBF16, SBF16, VFIRST, PREC, kSlabCols, true>(a, s);
  }
}

template <int DK, int DV, bool QBF16, bool SBF16, bool VFIRST>
int pick_prec(const DecodeArgs& a, int prec, hipStream_t s) {
  return prec == KDA_MATMUL_F32 ? pick_slab<DK, DV, QBF16, SBF16, VFIRST, KDA_MATMUL_F32>(a, s)
                                : pick_slab<DK, DV, QBF16, SBF16, VFIRST, KDA_MATMUL_SPLIT_BF16>(a, s);
}

template <int DK, int DV>
int pick_types(const DecodeArgs& a, bool qbf16, bool sbf16, bool vfirst, int prec, hipStream_t s) {
  if (qbf16) {
    if (sbf16) return vfirst ? pick_prec<DK, DV, true, true, true>(a, prec, s) : pick_prec<DK, DV, true, true, false>(a, prec, s);
    return vfirst ? pick_prec<DK, DV, true, false, true>(a, prec, s) : pick_prec<DK, DV, true, false, false>(a, prec, s);
  }
  if (sbf16) return vfirst ? pick_prec<DK, DV, false, true, true>(a, prec, s) : pick_prec<DK, DV, false, true, false>(a, prec, s);
  return vfirst ? pick_prec<DK, DV, false, false, true>(a, prec, s) : pick_prec<DK, DV, false, false, false>(a, prec, s);
}

template <int DK>
int pick_dv(const DecodeArgs& a, int dv, bool qbf16, bool sbf16, bool vfirst, int prec, hipStream_t s) {
  switch (dv) {
    case 32: return pick_types<DK, 32>(a, qbf16, sbf16, vfirst, prec, s);
    case 64: return pick_types<DK, 64>(a, qbf16, sbf16, vfirst, prec, s);
    case 128: return pick_types<DK, 128>(a, qbf16, sbf16, vfirst, prec, s);
    default: return KDA_ERR_UNSUPPORTED;
  }
}

}  // namespace

// This object's dk (the build compiles this file once per dk).
#ifdef KDA_PREFILL_DK
template <>
int launch_prefill_dk<KDA_PREFILL_DK>(const DecodeArgs& args, int dv, bool qkv_bf16, bool state_bf16,
                                      int state_layout, int matmul, hipStream_t stream) {
  return pick_dv<KDA_PREFILL_DK>(args, dv, qkv_bf16, state_bf16, state_layout == KDA_STATE_V_FIRST, matmul,
                                 stream);
}
#endif

}  // namespace kda
