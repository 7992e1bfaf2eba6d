// TTT-MLP forward on the gfx950 matrix cores: f(k) = W2 SiLU(W1 k), d = 64, hidden 256,
// mini-batch b = 16, causal, bf16 Q/K/V/Z, fp32 state.
//
// Method: inner 2-layer SiLU MLP (ViT3 news page, section 2) trained by mini-batch GD on
// 1/2 ||f(k) - v||^2 (wmrh.cn summary of Sun et al. 2024, section 1.2.2), z_t = f(q_t; W_t).
// For a chunk with rows K, Q, V (16 x 64), chunk-start weights W1 [256 x 64], W2 [64 x 256]:
//   U = K W1^T, A = SiLU(U), S = SiLU'(U), R = A W2^T - V,
//   dU = (R W2) * S                                   (gradient of the hidden layer)
//   W1 <- W1 - eta dU^T K,  W2 <- W2 - eta R^T A        (sum of the chunk's gradients)
// (with per-token rates, eta times a row of R or dU is that token's rate: "Fast weights"
// page, opening formula; wmrh.cn summary, section 2.2.3; with the negative dot-product loss
// -v^T f(k) of the ViT3 news page, section 2, R = -V)
// and, because every hidden pre-activation of a query is linear in W1 and the output is
// linear in W2, the causal outputs with the in-chunk updates are
//   U_q = Q W1^T - eta tril(Q K^T) dU,  A_q = SiLU(U_q),
//   Z   = A_q W2^T - eta tril(A_q A^T) R.
// This equals the per-token recurrence up to floating-point order.
//
// kPaper: the paper's TTT-MLP (wmrh.cn summary, section 2.2.1), f(x) = x + LN(W2 GELU(W1 x))
// with per-head LN gain and bias.  GELU (u Phi(u), exact) replaces SiLU; the state still
// changes only through R = dl/d(A W2^T), which is now the error k + LN(O) - v (or -v) passed
// back through the layer norm of each token's row of O; and Z = q + LN(Z_pre) with Z_pre
// the dual-form output above.  Both reductions already give a token's 64 outputs to 32
// consecutive lanes (two each), so the LN statistics are 32-lane shuffle sums there.
//
// Mapping.  One workgroup of 8 waves per (batch, head) chain, two per SIMD so that one
// wave's dependency stalls are filled by the other's work.  Wave w owns hidden units
// 32w .. 32w+31: its rows of W1 and columns of W2 live in its registers as fp32 MFMA
// accumulator tiles (W1^T tiles with input rows, W2^T tiles with hidden rows), 64 values per
// lane.  The forward pass contracts W2 over hidden units, which the W2^T tiles serve
// directly; the backward pass contracts it over outputs, so each chunk the wave also
// writes its chunk-start W2 in bf16 to LDS (rows: outputs) and reads the operand back with
// the transposing LDS read.  The only cross-wave sums, O = A W2^T and Z, go through LDS.
// Every product is one v_mfma_f32_16x16x32_bf16 per 16 x 16 x 32 block.  Products over the
// 16 tokens of a chunk use the same instruction with the upper half of one operand zero where
// they share an accumulator with K = 32 products, and v_mfma_f32_16x16x16_bf16 where the
// accumulator is theirs alone (the state updates, the transposes by I): an accumulator is
// only ever written by one of the two opcodes.

// Layout conventions (C layout of a 16 x 16 tile: lane (g, n) = (lane / 16, lane % 16)
// holds rows 4g + e, e = 0..3, of column n):
//   * input index j of W1^T tiles: tile jb = 2h + p, row m <-> j = 16 (m/4) + 2 (m%4) + 8h + p,
//     so that an operand over j matches the contiguous 16-byte row loads of K and Q;
//   * hidden (hh) and output (i) indices are natural: tile a, row m <-> 16 a + m.  The
//     contraction over a wave's 32 hidden units places tile 0 in slots 0..3 and tile 1 in
//     slots 4..7 of each lane (cat_op), so lane group g covers hidden 4 g + 0..3 and
//     16 + 4 g + 0..3 of the wave's slice;
//   * a contraction over the 64 outputs takes them in natural order, 32 h + 8 g + s.
#include "common.hpp"

namespace ttt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kD = 64;        // model dim d
constexpr int kH = 256;       // hidden width
constexpr int kB = 16;        // chunk
constexpr int kWaves = 8;     // hidden slices of 32
constexpr int kHT = kH / (16 * kWaves);  // hidden tiles per wave (2)
static_assert(kHT == 2, "the wave's hidden contraction is one K = 32 block");
constexpr int kTileBytes = kB * kD * 2;

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ bf16x8_t bf(const u32x4& x) { return __builtin_bit_cast(bf16x8_t, x); }
__device__ __forceinline__ bf16x8_t op4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 u = {a, b, c, d};
  return bf(u);
}
// operand over a tile pair: dword e = (x[e], y[e])
__device__ __forceinline__ bf16x8_t pair_op(const float4_t& x, const float4_t& y, float s = 1.0f) {
  return op4(pack_bf16(s * x[0], s * y[0]), pack_bf16(s * x[1], s * y[1]),
             pack_bf16(s * x[2], s * y[2]), pack_bf16(s * x[3], s * y[3]));
}
// operand over a tile pair: slots 0..3 = x[0..3], slots 4..7 = y[0..3]
__device__ __forceinline__ u32x4 cat_u(const float4_t& x, const float4_t& y) {
  const u32x4 u = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
  return u;
}
__device__ __forceinline__ bf16x8_t cat_op(const float4_t& x, const float4_t& y) { return bf(cat_u(x, y)); }
// K = 16 operand (4 values, contraction index 4 g + s) padded to the K = 32 layout
__device__ __forceinline__ bf16x8_t pad_op(const float4_t& x, float s = 1.0f) {
  return op4(pack_bf16(s * x[0], s * x[1]), pack_bf16(s * x[2], s * x[3]), 0u, 0u);
}
__device__ __forceinline__ float4_t mfma(const bf16x8_t& a, const bf16x8_t& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Products over the 16 tokens of a chunk whose accumulator no K = 32 product touches (the
// state updates, the transposes by I): one 16x16x16 MFMA on the K = 16 operand itself (the
// first two dwords of its padded form, same contraction index 4 g + s).
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4_t mfma16(const u32x2& a, const u32x2& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, a),
                                                    __builtin_bit_cast(bf16x4_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ u32x2 k16(const float4_t& x) {
  return u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
}
__device__ __forceinline__ bf16x8_t pad2(const u32x2& x) { return op4(x.x, x.y, 0u, 0u); }

__device__ __forceinline__ float sigmoid_f(float u) { return sigmoidf_(u); }

template <typename T>
__device__ __forceinline__ T lds_load(const lds_char* base, int byte) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(base + byte);
}
template <typename T>
__device__ __forceinline__ void lds_store(lds_char* base, int byte, T v) {
  *reinterpret_cast<__attribute__((address_space(3))) T*>(base + byte) = v;
}
// gfx950 transposing LDS read: within 16 lanes, lane i receives element i % 4 of the 8 bytes
// fetched by lane 4 s + i / 4 (s = 0..3).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ u32x2 lds_load_tr(const lds_char* base, int byte) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + byte)));
}
// Per-wave bf16 copy of W2 in LDS: row i (output), the wave's 32 hidden units in 8 units of
// 8 bytes (64-byte rows); unit u of row r sits at u ^ w2swz(r) with w2swz(r) the 3-bit
// reversal of (r / 2) % 8.  The 8-byte row writes (16 lanes, rows r .. r + 15, one unit)
// then cover all 16 bank pairs of a 128-byte window, and so do the transposing reads (rows
// 4k .. 4k + 3, units 4 a .. 4 a + 3): rows 4k and 4k + 2 differ by 4 in the swizzle, which
// moves the 4-unit block to the other half.
__device__ __forceinline__ int w2swz(int r) {
  const int m = (r >> 1) & 7;
  return ((m & 1) << 2) | (m & 2) | ((m >> 2) & 1);
}
__device__ __forceinline__ int w2off(int row, int unit) { return row * 64 + ((unit ^ w2swz(row)) * 8); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* base, int left) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, left > 0 ? left : 0,
                                           0x00020000);
}

// One chunk's token operands of a lane.
struct ChunkIn {
  u32x4 ka0, ka1;     // K[t = n][16 g + 0..7], K[n][16 g + 8..15]  (A operands over j)
  u32x4 qb0, qb1;     // Q[n][16 g + 0..15]                          (B operands over j)
  uint32_t kt[4][2];  // kt[e][h] = K[4 g + e][c0 + 8 h .. + 1], c0 = 16 (n / 4) + 2 (n % 4)
  uint32_t vv;        // V[t = tid / 32][2 (tid % 32) .. + 1]         (for R = O - V)
  uint32_t kv, qv;    // K and Q at the same place (residual of the LN model only)
  float et;           // rate factor of token tid / 32 (1 without per-token rates)
};

struct Offsets {
  int row;         // n * 128 + 32 g
  int kt[4];       // (4 g + e) * 128 + 2 c0
  int vv;          // (tid / 32) * 128 + 4 (tid % 32)
  int et;          // (tid / 32) * 4
};

template <bool kPaper>
__device__ __forceinline__ void load_chunk(ChunkIn& r, const char* q, const char* k, const char* v,
                                           const float* etok, int c, int seq_bytes, const Offsets& o) {
  const int off = c * kTileBytes;
  const __amdgpu_buffer_rsrc_t rq = chunk_rsrc(q + off, seq_bytes - off);
  const __amdgpu_buffer_rsrc_t rk = chunk_rsrc(k + off, seq_bytes - off);
  const __amdgpu_buffer_rsrc_t rv = chunk_rsrc(v + off, seq_bytes - off);
  r.ka0 = __builtin_amdgcn_raw_buffer_load_b128(rk, o.row, 0, 0);
  r.ka1 = __builtin_amdgcn_raw_buffer_load_b128(rk, o.row + 16, 0, 0);
  r.qb0 = __builtin_amdgcn_raw_buffer_load_b128(rq, o.row, 0, 0);
  r.qb1 = __builtin_amdgcn_raw_buffer_load_b128(rq, o.row + 16, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r.kt[e][0] = __builtin_amdgcn_raw_buffer_load_b32(rk, o.kt[e], 0, 0);
    r.kt[e][1] = __builtin_amdgcn_raw_buffer_load_b32(rk, o.kt[e] + 16, 0, 0);
  }
  r.vv = __builtin_amdgcn_raw_buffer_load_b32(rv, o.vv, 0, 0);
  r.kv = kPaper ? __builtin_amdgcn_raw_buffer_load_b32(rk, o.vv, 0, 0) : 0u;
  r.qv = kPaper ? __builtin_amdgcn_raw_buffer_load_b32(rq, o.vv, 0, 0) : 0u;
  r.et = 1.0f;
  if (etok) {  // uniform: per-token rate factors of the chunk, 4 bytes per token
    const int eoff = c * kB * 4;
    const __amdgpu_buffer_rsrc_t re = chunk_rsrc(etok + c * kB, (seq_bytes >> 5) - eoff);
    r.et = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(re, o.et, 0, 0));
  }
}

struct State {
  float4_t w1t[4][kHT];  // [jb][a]: W1^T tile, rows j (permuted, tile jb), cols hidden h0 + 16a + n
  float4_t w2t[kHT][4];  // [a][it]: W2^T tile, rows hidden h0 + 16a + m, cols output 16it + n
};

// LDS: per-wave partial sums of O^T and Z^T as [wave][t][i] fp32; -eta R = -eta (O - V) in
// bf16 twice, as [t][i] (rows of 144 bytes) for the row operands over outputs and as [i][t]
// (rows of 40 bytes) for the operands in the C layout; each wave's bf16 chunk-start W2
// (swizzled rows of 64 bytes).  The fp32 rows are padded to kRow = 68 floats (272 bytes,
// 16 mod 128), so the 16-byte accesses of 8 lanes to 8 consecutive rows, and 16 lanes of one
// row against 16 lanes 4 rows further, use distinct banks; the two bf16 row strides keep the
// 16-byte reads of 16 consecutive rows (36 dwords apart) and the 8-byte reads of 16
// consecutive rows (10 dwords apart) on distinct banks.
constexpr int kRow = kD + 4;
constexpr int kRRow = 72;  // bf16 per row of -eta R [t][i]
constexpr int kTRow = 20;  // bf16 per row of -eta R^T [i][t]
constexpr int kThreads = 64 * kWaves;
struct Lds {
  float opart[kWaves][kB][kRow];
  float zpart[kWaves][kB][kRow];
  uint16_t rr[kB][kRRow];
  uint16_t rt[kD][kTRow];
  uint32_t w2b[kWaves][kD][8 * kHT];
  float lnp[2][kD];  // the head's LN gain and bias (kPaper)
};

__device__ __forceinline__ void barrier() { __syncthreads(); }

// Phi(u), the standard normal CDF, and exp(-u^2 / 2), branch-free: erfc(x) for x >= 0 by
// Abramowitz and Stegun, Handbook of Mathematical Functions, formula 7.1.26
// (t = 1 / (1 + p x), erfc(x) = (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) e^{-x^2},
// |error| <= 1.5e-7) at x = |u| / sqrt 2, whose e^{-x^2} is the exp(-u^2 / 2) that the
// derivative of GELU needs as well.  Largest errors over [-12, 12] in float32: 3e-7 for Phi,
// 4e-7 for GELU and its derivative (far below the bf16 rounding of the operands).
__device__ __forceinline__ float phi_cdf(float u, float& ex) {
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f * 0.70710678118654752f, fabsf(u), 1.0f));
  float poly = __builtin_fmaf(t, 1.061405429f, -1.453152027f);
  poly = __builtin_fmaf(t, poly, 1.421413741f);
  poly = __builtin_fmaf(t, poly, -0.284496736f);
  poly = __builtin_fmaf(t, poly, 0.254829592f);
  ex = __expf(-0.5f * u * u);
  const float half_erfc = 0.5f * t * poly * ex;  // (1 - erf(|u| / sqrt 2)) / 2
  return u >= 0.0f ? 1.0f - half_erfc : half_erfc;
}

// the inner activation and its derivative: SiLU (u sigma(u)), or GELU (u Phi(u)) for kPaper
template <bool kPaper>
__device__ __forceinline__ void act_grad(float u, float& act, float& der) {
  if constexpr (kPaper) {
    float ex;
    const float ph = phi_cdf(u, ex);
    act = u * ph;
    der = __builtin_fmaf(u * 0.39894228040143268f, ex, ph);  // Phi(u) + u phi(u)
  } else {
    const float sg = sigmoid_f(u);
    act = u * sg;
    der = __builtin_fmaf(act, 1.0f - sg, sg);  // sg (1 + u (1 - sg))
  }
}
template <bool kPaper>
__device__ __forceinline__ float act_only(float u) {
  if constexpr (kPaper) {
    float ex;
    return u * phi_cdf(u, ex);
  }
  return u * sigmoid_f(u);
}

// Two sums over aligned groups of 32 lanes at once (every lane of the wave takes part).
// Within each row of 16 lanes: offsets 1 and 2 by DPP quad permutations, 4 and 8 by the DPP
// half-row and row mirrors (lane i with 7 - i, then with 15 - i: each pairs lanes holding
// disjoint partial sums), after which every lane of a row holds the row's sum; the two rows
// of a 32-lane group are then added from v_readlane of lanes 0, 16, 32 and 48.  Every lane
// of a group ends with the same bits.
typedef float float2_t __attribute__((ext_vector_type(2)));
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}
__device__ __forceinline__ float lane_f(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
__device__ __forceinline__ float2_t sum32x2(float2_t x) {
  const float a = row_sum16(x[0]), b = row_sum16(x[1]);
  const float a_lo = lane_f(a, 0) + lane_f(a, 16), a_hi = lane_f(a, 32) + lane_f(a, 48);
  const float b_lo = lane_f(b, 0) + lane_f(b, 16), b_hi = lane_f(b, 32) + lane_f(b, 48);
  const bool upper = (threadIdx.x & 32) != 0;
  return float2_t{upper ? a_hi : a_lo, upper ? b_hi : b_lo};
}

// Layer-norm statistics of a token's 64 outputs held two per lane by 32 consecutive lanes
// (mean and mean square in one pass: E[y^2] - mean^2 costs the variance a relative error of
// about 6e-8 (mean / std)^2 in fp32, below the bf16 resolution of the outputs unless the
// mean exceeds ~250 standard deviations)
struct Ln2 {
  float2_t xh;
  float rstd;
};
__device__ __forceinline__ Ln2 ln2_row(float2_t y, float eps) {
  const float2_t m = sum32x2(float2_t{y[0] + y[1], y[0] * y[0] + y[1] * y[1]}) * (1.0f / kD);
  const float var = fmaxf(m[1] - m[0] * m[0], 0.0f);
  const float rstd = 1.0f / sqrtf(var + eps);
  return {(y - m[0]) * rstd, rstd};
}

// kHist: the state recursion alone (no outputs), storing every chunk-start state as the
// bf16 values the products use: W1 rows [256][64] then W2 rows [64][256] (64 KB per chunk,
// chunk c of chain ch at hist + (ch nchunks + c) 64 KB), for the backward pass.
template <bool kDot, bool kPaper, bool kHist>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mlp_mfma_kernel(
    MlpArgs a, char* hist) {
  __shared__ __attribute__((aligned(16))) Lds sh;
  lds_char* opart = (lds_char*)(&sh.opart[0][0][0]);
  lds_char* zpart = (lds_char*)(&sh.zpart[0][0][0]);
  lds_char* rrb = (lds_char*)(&sh.rr[0][0]);
  lds_char* rtb = (lds_char*)(&sh.rt[0][0]);
  lds_char* w2lds = (lds_char*)(&sh.w2b[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)][0][0]);

  const int chain = blockIdx.x;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int bi = chain / a.H;
  const int hi = chain - bi * a.H;
  const int T = a.T;
  const int nchunks = (T + kB - 1) / kB;
  const int seq_bytes = T * kD * 2;
  const float eta = a.eta;

  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * kD;
  const char* q = reinterpret_cast<const char*>(static_cast<const bf16*>(a.q) + tok0);
  const char* k = reinterpret_cast<const char*>(static_cast<const bf16*>(a.k) + tok0);
  const char* v = reinterpret_cast<const char*>(static_cast<const bf16*>(a.v) + tok0);
  char* z = reinterpret_cast<char*>(static_cast<bf16*>(a.z) + tok0);
  const float* etok = a.eta_tok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
  const size_t hd = static_cast<size_t>(kH) * kD;
  const float* w1g = a.w1 + bi * a.w_batch_stride + static_cast<long long>(hi) * hd;
  const float* w2g = a.w2 + bi * a.w_batch_stride + static_cast<long long>(hi) * hd;
  const int h0 = 16 * kHT * wv;  // first hidden unit of this wave
  // the head's LN gain and bias into LDS (read by the reductions, after the first barrier)
  if (kPaper && tid < 2 * kD) sh.lnp[tid / kD][tid % kD] = (tid < kD ? a.ln_w : a.ln_b)[hi * kD + tid % kD];

  // ---- initial state ----
  State st;
#pragma unroll
  for (int aa = 0; aa < kHT; ++aa) {
    // W1^T tile (jb, aa): element e = W1[h0 + 16 aa + n][j], j = 16 g + 8 h + 2 e + p
    const float* wr = w1g + static_cast<size_t>(h0 + 16 * aa + n) * kD + 16 * g;
    const float4_t f0 = *reinterpret_cast<const float4_t*>(wr);
    const float4_t f1 = *reinterpret_cast<const float4_t*>(wr + 4);
    const float4_t f2 = *reinterpret_cast<const float4_t*>(wr + 8);
    const float4_t f3 = *reinterpret_cast<const float4_t*>(wr + 12);
    st.w1t[0][aa] = float4_t{f0[0], f0[2], f1[0], f1[2]};
    st.w1t[1][aa] = float4_t{f0[1], f0[3], f1[1], f1[3]};
    st.w1t[2][aa] = float4_t{f2[0], f2[2], f3[0], f3[2]};
    st.w1t[3][aa] = float4_t{f2[1], f2[3], f3[1], f3[3]};
  }
#pragma unroll
  for (int aa = 0; aa < kHT; ++aa)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      // W2^T tile (aa, it): element e = W2[16 it + n][h0 + 16 aa + 4 g + e]
      st.w2t[aa][it] = *reinterpret_cast<const float4_t*>(
          w2g + static_cast<size_t>(16 * it + n) * kH + h0 + 16 * aa + 4 * g);
    }

  // ---- constants ----
  const uint32_t one = 0x3F80u;  // bf16 1.0
  const u32x2 eye = {(4 * g + 0 == n ? one : 0u) | (4 * g + 1 == n ? one << 16 : 0u),
                     (4 * g + 2 == n ? one : 0u) | (4 * g + 3 == n ? one << 16 : 0u)};
  const bool keep[4] = {4 * g + 0 <= n, 4 * g + 1 <= n, 4 * g + 2 <= n, 4 * g + 3 <= n};
  Offsets o;
  o.row = n * 128 + 32 * g;
  const int c0 = 16 * (n >> 2) + 2 * (n & 3);
#pragma unroll
  for (int e = 0; e < 4; ++e) o.kt[e] = (4 * g + e) * 128 + 2 * c0;
  const int rt = tid >> 5;          // reduction role: row t and 2 outputs
  const int ri = 2 * (tid & 31);
  o.vv = rt * 128 + 2 * ri;
  o.et = rt * 4;
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const float2_t zero2 = {0.0f, 0.0f};
  uint32_t qv_prev = 0u;  // Q of the previous chunk at this thread's outputs (kPaper)
  constexpr uint32_t kLo = 0x05040100u, kHi = 0x07060302u;

  // Z of the previous chunk: reduce the per-wave partial sums and store (thread: row rt,
  // 2 outputs)
  auto reduce_store_z = [&](int c) {
    float2_t s2 = zero2;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s2 += lds_load<float2_t>(zpart, ((w * kB + rt) * kRow + ri) * 4);
    if constexpr (kPaper) {  // z = q + LN(z_pre)
      const float2_t lng = *reinterpret_cast<const float2_t*>(&sh.lnp[0][ri]);
      const float2_t lnb = *reinterpret_cast<const float2_t*>(&sh.lnp[1][ri]);
      const Ln2 st2 = ln2_row(s2, a.ln_eps);
      s2 = float2_t{__builtin_bit_cast(float, qv_prev << 16), __builtin_bit_cast(float, qv_prev & 0xFFFF0000u)} +
           lng * st2.xh + lnb;
    }
    const int off = c * kTileBytes;
    __builtin_amdgcn_raw_buffer_store_b32(pack_bf16(s2[0], s2[1]), chunk_rsrc(z + off, seq_bytes - off),
                                          o.vv, 0, 0);
  };

  // One chunk: its operands in cur, the next chunk's loaded into nxt.
  auto step = [&](const ChunkIn& cur, ChunkIn& nxt, int c) {
    load_chunk<kPaper>(nxt, q, k, v, etok, c + 1, seq_bytes, o);  // prefetch (zeros past the end)
    const bf16x8_t ka0 = bf(cur.ka0), ka1 = bf(cur.ka1), qb0 = bf(cur.qb0), qb1 = bf(cur.qb1);

    // bf16 copies of this wave's chunk-start state
    bf16x8_t w1b[2][kHT];  // [h][a]: operand over j (pairs of W1^T tiles 2h, 2h+1)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int aa = 0; aa < kHT; ++aa) w1b[h][aa] = pair_op(st.w1t[2 * h][aa], st.w1t[2 * h + 1][aa]);
    char* hc = nullptr;  // this chunk's stored state (kHist)
    if constexpr (kHist) {
      hc = hist + (static_cast<size_t>(chain) * nchunks + c) * (2 * kH * kD * 2);
      // lane: W1[h0 + 16 a + n][16 g + 8 h .. + 7]
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int aa = 0; aa < kHT; ++aa)
          *reinterpret_cast<u32x4*>(hc + ((h0 + 16 * aa + n) * kD + 16 * g + 8 * h) * 2) =
              __builtin_bit_cast(u32x4, w1b[h][aa]);
    }

    // U = K W1^T (rows t, hidden tile aa);  A = act(U), S = act'(U)
    float4_t act[kHT], sd[kHT];
#pragma unroll
    for (int aa = 0; aa < kHT; ++aa) {
      float4_t u = mfma(ka0, w1b[0][aa], zero);
      u = mfma(ka1, w1b[1][aa], u);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float av, dv;
        act_grad<kPaper>(u[e], av, dv);
        act[aa][e] = av;
        sd[aa][e] = dv;
      }
    }
    // A as K = 16 operands (rows t); A^T (rows hidden) by an MFMA with I
    u32x2 ab[kHT];
    float4_t actT[kHT];
#pragma unroll
    for (int aa = 0; aa < kHT; ++aa) {
      ab[aa] = k16(act[aa]);
      actT[aa] = mfma16(ab[aa], eye, zero);
    }

    // bf16 chunk-start W2 as A operands over the wave's hidden units (rows output
    // 16 it + n), written also to this wave's LDS copy (rows output, 4 consecutive hidden
    // units per 8 bytes)
    u32x4 w2op[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      w2op[it] = cat_u(st.w2t[0][it], st.w2t[1][it]);
      const int row = 16 * it + n;
      lds_store<u32x2>(w2lds, w2off(row, g), u32x2{w2op[it].x, w2op[it].y});
      lds_store<u32x2>(w2lds, w2off(row, 4 + g), u32x2{w2op[it].z, w2op[it].w});
      if constexpr (kHist) {  // W2[16 it + n][h0 + 4 g .. + 3] and [h0 + 16 + 4 g .. + 3]
        char* w2r = hc + kH * kD * 2 + (row * kH + h0 + 4 * g) * 2;
        *reinterpret_cast<u32x2*>(w2r) = u32x2{w2op[it].x, w2op[it].y};
        *reinterpret_cast<u32x2*>(w2r + 32) = u32x2{w2op[it].z, w2op[it].w};
      }
    }
    // O^T partial = W2 A^T (rows output, cols t): contraction over this wave's 32 hidden
    // (not needed with the dot-product loss, whose error term is -V, unless a layer norm
    // follows: its backward needs O)
    const bf16x8_t atb = cat_op(actT[0], actT[1]);  // B operand over hidden
    if (!kDot || kPaper) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const float4_t ot = mfma(bf(w2op[it]), atb, zero);
        lds_store<float4_t>(opart, ((wv * kB + n) * kRow + 16 * it + 4 * g) * 4, ot);
      }
    }
    barrier();
    // previous chunk's Z (its partials were written before this barrier)
    if (!kHist && c > 0) reduce_store_z(c - 1);
    // -eta_t R = -eta_t (sum of partials - V), to LDS in bf16 as [t][i] and [i][t]
    {
      float2_t s2 = zero2;
      if (!kDot || kPaper) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s2 += lds_load<float2_t>(opart, ((w * kB + rt) * kRow + ri) * 4);
      }
      const uint32_t vb = cur.vv;
      const float2_t vr = {__builtin_bit_cast(float, vb << 16), __builtin_bit_cast(float, vb & 0xFFFF0000u)};
      float2_t r2;  // dl/dO of this thread's two outputs
      if constexpr (kPaper) {
        // f = k + LN(O); the error f - v (or -v) back through the layer norm
        const float2_t lng = *reinterpret_cast<const float2_t*>(&sh.lnp[0][ri]);
        const float2_t lnb = *reinterpret_cast<const float2_t*>(&sh.lnp[1][ri]);
        const Ln2 st2 = ln2_row(s2, a.ln_eps);
        const float2_t kr = {__builtin_bit_cast(float, cur.kv << 16),
                             __builtin_bit_cast(float, cur.kv & 0xFFFF0000u)};
        const float2_t err = kDot ? -vr : kr + lng * st2.xh + lnb - vr;
        const float2_t gg = lng * err;
        const float2_t m = sum32x2(float2_t{gg[0] + gg[1], gg[0] * st2.xh[0] + gg[1] * st2.xh[1]}) * (1.0f / kD);
        r2 = st2.rstd * (gg - m[0] - st2.xh * m[1]);
      } else {
        r2 = s2 - vr;
      }
      const float nrate = -eta * cur.et;
      const uint32_t rp = pack_bf16(r2[0] * nrate, r2[1] * nrate);
      lds_store<uint32_t>(rrb, (rt * kRRow + ri) * 2, rp);
      lds_store<uint16_t>(rtb, (ri * kTRow + rt) * 2, static_cast<uint16_t>(rp));
      lds_store<uint16_t>(rtb, ((ri + 1) * kTRow + rt) * 2, static_cast<uint16_t>(rp >> 16));
    }
    barrier();

    // -eta R tiles as padded K = 16 operands in the C layout (rows t = 4 g + 0..3 of column
    // 16 it + n), and as row operands over outputs (m = t, k = outputs 32 h + 8 g + 0..7)
    u32x2 rb[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) rb[it] = lds_load<u32x2>(rtb, ((16 * it + n) * kTRow + 4 * g) * 2);
    bf16x8_t rrow[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) rrow[h] = bf(lds_load<u32x4>(rrb, (n * kRRow + 32 * h + 8 * g) * 2));
    // -eta dU = (-eta R W2) * S  (rows t, hidden tile aa), as a padded operand.  The B
    // operand W2[32 h + 8 g + s][h0 + 16 aa + n] comes from two transposing reads of the LDS
    // copy: lane 4 s' + q of group g fetches row 32 h + 8 g + 4 half + s', hidden
    // 16 aa + 4 q .. + 3 of the wave's slice.
    u32x2 dub[kHT];
#pragma unroll
    for (int aa = 0; aa < kHT; ++aa) {
      float4_t da = zero;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x2 lo = lds_load_tr(w2lds, w2off(32 * h + 8 * g + (n >> 2), 4 * aa + (n & 3)));
        const u32x2 hi2 = lds_load_tr(w2lds, w2off(32 * h + 8 * g + 4 + (n >> 2), 4 * aa + (n & 3)));
        const u32x4 w2k = {lo.x, lo.y, hi2.x, hi2.y};
        da = mfma(rrow[h], bf(w2k), da);
      }
      dub[aa] = k16(da * sd[aa]);
    }

    // ---- outputs (use the chunk-start state) ----
    if constexpr (!kHist) {
      // P^T = K Q^T with the causal mask s <= t, padded B operand
      float4_t pt = mfma(ka0, qb0, zero);
      pt = mfma(ka1, qb1, pt);
#pragma unroll
      for (int e = 0; e < 4; ++e) pt[e] = keep[e] ? pt[e] : 0.0f;
      const bf16x8_t ptb = pad_op(pt);
      // U_q^T = W1 Q^T - eta dU^T P^T (rows hidden tile aa, cols t);  A_q^T = act(U_q^T)
      float4_t aqT[kHT];
#pragma unroll
      for (int aa = 0; aa < kHT; ++aa) {
        float4_t u = mfma(w1b[0][aa], qb0, zero);
        u = mfma(w1b[1][aa], qb1, u);
        u = mfma(pad2(dub[aa]), ptb, u);
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = act_only<kPaper>(u[e]);
        aqT[aa] = u;
      }
      const bf16x8_t aqb = cat_op(aqT[0], aqT[1]);
      // G^T = A A_q^T (rows s, cols t) over this wave's hidden units, masked s <= t
      float4_t gt = mfma(atb, aqb, zero);
#pragma unroll
      for (int e = 0; e < 4; ++e) gt[e] = keep[e] ? gt[e] : 0.0f;
      const bf16x8_t gtb = pad_op(gt);
      // Z^T partial = W2 A_q^T + (-eta R)^T G^T (rows output tile it, cols t)
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        float4_t zt = mfma(bf(w2op[it]), aqb, zero);
        zt = mfma(pad2(rb[it]), gtb, zt);
        lds_store<float4_t>(zpart, ((wv * kB + n) * kRow + 16 * it + 4 * g) * 4, zt);
      }
    }

    // ---- state update (sum of the chunk's gradients) ----
    // W1^T += K^T (-eta dU): A = K^T gather for j tile jb, B = dU tile aa
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const int h = jb >> 1;
      const uint32_t sel = (jb & 1) ? kHi : kLo;
      const u32x2 kt = {__builtin_amdgcn_perm(cur.kt[1][h], cur.kt[0][h], sel),
                        __builtin_amdgcn_perm(cur.kt[3][h], cur.kt[2][h], sel)};
#pragma unroll
      for (int aa = 0; aa < kHT; ++aa) st.w1t[jb][aa] = mfma16(kt, dub[aa], st.w1t[jb][aa]);
    }
    // W2^T += A^T (-eta R): A-operand = A tile aa (rows t), B = -eta R tile it
#pragma unroll
    for (int aa = 0; aa < kHT; ++aa)
#pragma unroll
      for (int it = 0; it < 4; ++it) st.w2t[aa][it] = mfma16(ab[aa], rb[it], st.w2t[aa][it]);
    qv_prev = cur.qv;
  };

  // two operand buffers in turn (a copy of a buffer whose loads are in flight would wait
  // for them)
  ChunkIn ca, cb;
  load_chunk<kPaper>(ca, q, k, v, etok, 0, seq_bytes, o);
  int c = 0;
  for (; c + 1 < nchunks; c += 2) {
    step(ca, cb, c);
    step(cb, ca, c + 1);
  }
  if (c < nchunks) step(ca, cb, c);
  barrier();
  if (!kHist && nchunks > 0) reduce_store_z(nchunks - 1);

  // ---- final state ----
  if (a.w1_out) {
    float* o1 = a.w1_out + static_cast<size_t>(chain) * hd;
#pragma unroll
    for (int aa = 0; aa < kHT; ++aa) {
      float* wr = o1 + static_cast<size_t>(h0 + 16 * aa + n) * kD + 16 * g;
      *reinterpret_cast<float4_t*>(wr) =
          float4_t{st.w1t[0][aa][0], st.w1t[1][aa][0], st.w1t[0][aa][1], st.w1t[1][aa][1]};
      *reinterpret_cast<float4_t*>(wr + 4) =
          float4_t{st.w1t[0][aa][2], st.w1t[1][aa][2], st.w1t[0][aa][3], st.w1t[1][aa][3]};
      *reinterpret_cast<float4_t*>(wr + 8) =
          float4_t{st.w1t[2][aa][0], st.w1t[3][aa][0], st.w1t[2][aa][1], st.w1t[3][aa][1]};
      *reinterpret_cast<float4_t*>(wr + 12) =
          float4_t{st.w1t[2][aa][2], st.w1t[3][aa][2], st.w1t[2][aa][3], st.w1t[3][aa][3]};
    }
  }
  if (a.w2_out) {
    float* o2 = a.w2_out + static_cast<size_t>(chain) * hd;
#pragma unroll
    for (int aa = 0; aa < kHT; ++aa)
#pragma unroll
      for (int it = 0; it < 4; ++it)
        *reinterpret_cast<float4_t*>(o2 + static_cast<size_t>(16 * it + n) * kH + h0 + 16 * aa + 4 * g) =
            st.w2t[aa][it];
  }
}


// ---------------------------------------------------------------------------------------
// Two workgroups per chain.  The recursion (U, A, R, dU and the state updates) does not
// depend on the queries, so a chain's outputs can be formed on a second compute unit that
// replays the same state updates on a copy of its own:
//   * the recursion workgroup (blocks 0 .. npad-1) runs the chunk loop above without the
//     query products and hands each chunk's update operands to its partner: -eta dU and A
//     of every wave (bf16, in the lanes' operand layout) and -eta R, 18 KB per chunk, into
//     the caller's workspace;
//   * the output workgroup (block npad + chain, the same residue mod 8, so the same XCD)
//     waits for them, forms U_q, A_q and Z, and applies the same rank-16 updates with the
//     same MFMAs in the same order, so its state, and hence Z, is bit-identical to that of
//     the one-workgroup kernel.
// Hand-off protocol.  Each chain has three 64-bit words in its own 128-byte line, each
// (call tag << 32 | value): the recursion's progress (chunks whose operands are stored), and
// the compute-unit cluster (XCC) of each of the two workgroups.  The tag changes on every
// call, so a word left by an earlier call is never taken for this one.
//   * Both workgroups first post their XCC id with an agent-scope release.  The output
//     workgroup waits for the recursion's (the recursion has the lower block index, so it
//     is dispatched first and posts at once); the recursion never waits for its partner and
//     only looks, once per chunk, whether the partner's id has arrived.
//   * Operands of chunk c are stored at the top of chunk c + 1, before that chunk's
//     prefetch loads.  Every wave waits for its older vector-memory operations before the
//     first barrier of chunk c + 2 (vector memory operations complete in issue order), so
//     after that barrier wave 0 publishes "c + 1 chunks complete".
//   * On one XCC the two workgroups share its L2, so the progress word is written and read,
//     and the operands are read, at device scope past the per-CU cache (sc1), with no cache
//     write-back or invalidation.  Until the recursion has seen that its partner sits on the
//     same XCC, and whenever the two sit on different ones, it publishes with an agent-scope
//     release (L2 write-back) and the output workgroup reads with an agent-scope acquire.
//     Blocks with equal residues mod 8 land on one XCC under round-robin dispatch, which the
//     grid arranges; the check keeps the results right if that ever fails.
//   * The output workgroup loads a chunk's operands one chunk ahead, once the progress word
//     covers it; wave 0 reads the word one chunk early (without waiting) and spins only when
//     that reading falls short.  The spin is bounded: past the bound it fills the chain's
//     remaining outputs with NaN and leaves.
constexpr int kSlotBytes = kWaves * 2048 + 2048;  // one chunk's hand-off
constexpr int kFlagStride = 128;
constexpr int kSpinLimit = 1 << 20;
// debug switches (ttt_set_split_debug): the agent-scope protocol whatever the placement; a
// forced failure of the output workgroup's first wait with a bound of 64 polls
constexpr int kSplitFormal = 1;
constexpr int kSplitTestAbort = 2;
__device__ __forceinline__ unsigned long long xcc_id() {
  return static_cast<unsigned long long>(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15);  // HW_REG_XCC_ID
}
// vector-memory operations issued at the top of a chunk before its first barrier: at least
// 2 operand stores and 11 prefetch loads (K rows, K^T gathers, V)
constexpr int kTopOps = 13;
__host__ __device__ __forceinline__ size_t split_flag_bytes(int nchains) {
  return (static_cast<size_t>(nchains) * kFlagStride + 255) & ~static_cast<size_t>(255);
}

struct Hand {
  u32x4 du;  // -eta dU tiles 0, 1 of the wave (u32x2 each)
  u32x4 ab;  // A tiles 0, 1 of the wave
  u32x4 r0;  // -eta R tiles 0, 1
  u32x4 r1;  // -eta R tiles 2, 3
};

struct SplitLds {
  Lds base;
  int abort_flag;
  int same_xcc;
};

__device__ __forceinline__ void init_state(State& st, const float* w1g, const float* w2g, int h0, int g, int n) {
#pragma unroll
  for (int aa = 0; aa < kHT; ++aa) {
    const float* wr = w1g + static_cast<size_t>(h0 + 16 * aa + n) * kD + 16 * g;
    const float4_t f0 = *reinterpret_cast<const float4_t*>(wr);
    const float4_t f1 = *reinterpret_cast<const float4_t*>(wr + 4);
    const float4_t f2 = *reinterpret_cast<const float4_t*>(wr + 8);
    const float4_t f3 = *reinterpret_cast<const float4_t*>(wr + 12);
    st.w1t[0][aa] = float4_t{f0[0], f0[2], f1[0], f1[2]};
    st.w1t[1][aa] = float4_t{f0[1], f0[3], f1[1], f1[3]};
    st.w1t[2][aa] = float4_t{f2[0], f2[2], f3[0], f3[2]};
    st.w1t[3][aa] = float4_t{f2[1], f2[3], f3[1], f3[3]};
  }
#pragma unroll
  for (int aa = 0; aa < kHT; ++aa)
#pragma unroll
    for (int it = 0; it < 4; ++it)
      st.w2t[aa][it] = *reinterpret_cast<const float4_t*>(w2g + static_cast<size_t>(16 * it + n) * kH + h0 +
                                                          16 * aa + 4 * g);
}

// the state update of one chunk (shared by both workgroups: same operands, same order)
__device__ __forceinline__ void update_state(State& st, const uint32_t (&kt4)[4][2], const u32x2 (&dub)[kHT],
                                             const u32x2 (&ab)[kHT], const u32x2 (&rb)[4]) {
  constexpr uint32_t kLo = 0x05040100u, kHi = 0x07060302u;
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    const int h = jb >> 1;
    const uint32_t sel = (jb & 1) ? kHi : kLo;
    const u32x2 kt = {__builtin_amdgcn_perm(kt4[1][h], kt4[0][h], sel), __builtin_amdgcn_perm(kt4[3][h], kt4[2][h], sel)};
#pragma unroll
    for (int aa = 0; aa < kHT; ++aa) st.w1t[jb][aa] = mfma16(kt, dub[aa], st.w1t[jb][aa]);
  }
#pragma unroll
  for (int aa = 0; aa < kHT; ++aa)
#pragma unroll
    for (int it = 0; it < 4; ++it) st.w2t[aa][it] = mfma16(ab[aa], rb[it], st.w2t[aa][it]);
}

__device__ __forceinline__ void store_state(const State& st, float* o1, float* o2, int h0, int g, int n) {
  if (o1) {
#pragma unroll
    for (int aa = 0; aa < kHT; ++aa) {
      float* wr = o1 + static_cast<size_t>(h0 + 16 * aa + n) * kD + 16 * g;
      *reinterpret_cast<float4_t*>(wr) =
          float4_t{st.w1t[0][aa][0], st.w1t[1][aa][0], st.w1t[0][aa][1], st.w1t[1][aa][1]};
      *reinterpret_cast<float4_t*>(wr + 4) =
          float4_t{st.w1t[0][aa][2], st.w1t[1][aa][2], st.w1t[0][aa][3], st.w1t[1][aa][3]};
      *reinterpret_cast<float4_t*>(wr + 8) =
          float4_t{st.w1t[2][aa][0], st.w1t[3][aa][0], st.w1t[2][aa][1], st.w1t[3][aa][1]};
      *reinterpret_cast<float4_t*>(wr + 12) =
          float4_t{st.w1t[2][aa][2], st.w1t[3][aa][2], st.w1t[2][aa][3], st.w1t[3][aa][3]};
    }
  }
  if (o2) {
#pragma unroll
    for (int aa = 0; aa < kHT; ++aa)
#pragma unroll
      for (int it = 0; it < 4; ++it)
        *reinterpret_cast<float4_t*>(o2 + static_cast<size_t>(16 * it + n) * kH + h0 + 16 * aa + 4 * g) =
            st.w2t[aa][it];
  }
}

// K, V of one chunk for the recursion workgroup (the layout of ChunkIn, without Q)
struct MainIn {
  u32x4 ka0, ka1;
  uint32_t kt[4][2];
  uint32_t vv, kv;
  float et;
};
template <bool kPaper>
__device__ __forceinline__ void load_main(MainIn& r, const char* k, const char* v, const float* etok, int c,
                                          int seq_bytes, const Offsets& o) {
  const int off = c * kTileBytes;
  const __amdgpu_buffer_rsrc_t rk = chunk_rsrc(k + off, seq_bytes - off);
  const __amdgpu_buffer_rsrc_t rv = chunk_rsrc(v + off, seq_bytes - off);
  r.ka0 = __builtin_amdgcn_raw_buffer_load_b128(rk, o.row, 0, 0);
  r.ka1 = __builtin_amdgcn_raw_buffer_load_b128(rk, o.row + 16, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r.kt[e][0] = __builtin_amdgcn_raw_buffer_load_b32(rk, o.kt[e], 0, 0);
    r.kt[e][1] = __builtin_amdgcn_raw_buffer_load_b32(rk, o.kt[e] + 16, 0, 0);
  }
  r.vv = __builtin_amdgcn_raw_buffer_load_b32(rv, o.vv, 0, 0);
  r.kv = kPaper ? __builtin_amdgcn_raw_buffer_load_b32(rk, o.vv, 0, 0) : 0u;
  r.et = 1.0f;
  if (etok) {
    const int eoff = c * kB * 4;
    const __amdgpu_buffer_rsrc_t re = chunk_rsrc(etok + c * kB, (seq_bytes >> 5) - eoff);
    r.et = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(re, o.et, 0, 0));
  }
}

// Q, K of one chunk for the output workgroup
struct PartIn {
  u32x4 ka0, ka1, qb0, qb1;
  uint32_t kt[4][2];
  uint32_t qv;
};
template <bool kPaper>
__device__ __forceinline__ void load_part(PartIn& r, const char* q, const char* k, int c, int seq_bytes,
                                          const Offsets& o) {
  const int off = c * kTileBytes;
  const __amdgpu_buffer_rsrc_t rq = chunk_rsrc(q + off, seq_bytes - off);
  const __amdgpu_buffer_rsrc_t rk = chunk_rsrc(k + off, seq_bytes - off);
  r.ka0 = __builtin_amdgcn_raw_buffer_load_b128(rk, o.row, 0, 0);
  r.ka1 = __builtin_amdgcn_raw_buffer_load_b128(rk, o.row + 16, 0, 0);
  r.qb0 = __builtin_amdgcn_raw_buffer_load_b128(rq, o.row, 0, 0);
  r.qb1 = __builtin_amdgcn_raw_buffer_load_b128(rq, o.row + 16, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r.kt[e][0] = __builtin_amdgcn_raw_buffer_load_b32(rk, o.kt[e], 0, 0);
    r.kt[e][1] = __builtin_amdgcn_raw_buffer_load_b32(rk, o.kt[e] + 16, 0, 0);
  }
  r.qv = kPaper ? __builtin_amdgcn_raw_buffer_load_b32(rq, o.vv, 0, 0) : 0u;
}

__device__ __forceinline__ u32x2 lo2(const u32x4& x) { return u32x2{x.x, x.y}; }
__device__ __forceinline__ u32x2 hi2(const u32x4& x) { return u32x2{x.z, x.w}; }

template <bool kDot, bool kPaper>
__device__ __forceinline__ void split_recursion(const MlpArgs& a, SplitLds& sl, int chain, char* slots,
                                                unsigned long long* flag, unsigned long long tag, int dbg) {
  Lds& sh = sl.base;
  lds_char* opart = (lds_char*)(&sh.opart[0][0][0]);
  lds_char* rrb = (lds_char*)(&sh.rr[0][0]);
  lds_char* rtb = (lds_char*)(&sh.rt[0][0]);
  lds_char* w2lds = (lds_char*)(&sh.w2b[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)][0][0]);

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int bi = chain / a.H;
  const int hi = chain - bi * a.H;
  const int T = a.T;
  const int nchunks = (T + kB - 1) / kB;
  const int seq_bytes = T * kD * 2;
  const float eta = a.eta;
  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * kD;
  const char* k = reinterpret_cast<const char*>(static_cast<const bf16*>(a.k) + tok0);
  const char* v = reinterpret_cast<const char*>(static_cast<const bf16*>(a.v) + tok0);
  const float* etok = a.eta_tok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
  const size_t hd = static_cast<size_t>(kH) * kD;
  const float* w1g = a.w1 + bi * a.w_batch_stride + static_cast<long long>(hi) * hd;
  const float* w2g = a.w2 + bi * a.w_batch_stride + static_cast<long long>(hi) * hd;
  const int h0 = 16 * kHT * wv;
  if (kPaper && tid < 2 * kD) sh.lnp[tid / kD][tid % kD] = (tid < kD ? a.ln_w : a.ln_b)[hi * kD + tid % kD];

  State st;
  init_state(st, w1g, w2g, h0, g, n);
  const uint32_t one = 0x3F80u;
  const u32x2 eye = {(4 * g + 0 == n ? one : 0u) | (4 * g + 1 == n ? one << 16 : 0u),
                     (4 * g + 2 == n ? one : 0u) | (4 * g + 3 == n ? one << 16 : 0u)};
  Offsets o;
  o.row = n * 128 + 32 * g;
  const int c0 = 16 * (n >> 2) + 2 * (n & 3);
#pragma unroll
  for (int e = 0; e < 4; ++e) o.kt[e] = (4 * g + e) * 128 + 2 * c0;
  const int rt = tid >> 5;
  const int ri = 2 * (tid & 31);
  o.vv = rt * 128 + 2 * ri;
  o.et = rt * 4;
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const float2_t zero2 = {0.0f, 0.0f};

  // update operands of the previous chunk, stored at the top of the next one
  u32x2 pdub[kHT], pab[kHT], prb[4];
  unsigned long long* hello_own = flag + 1;
  const unsigned long long* hello_other = flag + 2;
  const unsigned long long xm = xcc_id();
  if (wv == 0 && lane == 0) __hip_atomic_store(hello_own, (tag << 32) | xm, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  // wave 0: 0 = partner's XCC not seen yet, 1 = same XCC, 2 = another XCC; the partner's word
  // is read one chunk before it is looked at
  int mode = (dbg & kSplitFormal) ? 2 : 0;
  unsigned long long other = 0;
  auto progress = [&](int count) {  // wave 0, after a barrier
    if (lane == 0) {
      const unsigned long long f = (tag << 32) | static_cast<unsigned long long>(count);
      if (mode == 1)
        __hip_atomic_store(flag, f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        __hip_atomic_store(flag, f, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  auto publish = [&](int c) {
    if (c >= 1) {
      char* slot = slots + static_cast<size_t>(c - 1) * kSlotBytes;
      *reinterpret_cast<u32x4*>(slot + wv * 2048 + lane * 16) = u32x4{pdub[0].x, pdub[0].y, pdub[1].x, pdub[1].y};
      *reinterpret_cast<u32x4*>(slot + wv * 2048 + 1024 + lane * 16) = u32x4{pab[0].x, pab[0].y, pab[1].x, pab[1].y};
      if (wv == 0) {
        *reinterpret_cast<u32x4*>(slot + kWaves * 2048 + lane * 16) = u32x4{prb[0].x, prb[0].y, prb[1].x, prb[1].y};
        *reinterpret_cast<u32x4*>(slot + kWaves * 2048 + 1024 + lane * 16) =
            u32x4{prb[2].x, prb[2].y, prb[3].x, prb[3].y};
      }
    }
  };

  auto step = [&](const MainIn& cur, MainIn& nxt, int c) {
    publish(c);
    load_main<kPaper>(nxt, k, v, etok, c + 1, seq_bytes, o);
    const bf16x8_t ka0 = bf(cur.ka0), ka1 = bf(cur.ka1);
    bf16x8_t w1b[2][kHT];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int aa = 0; aa < kHT; ++aa) w1b[h][aa] = pair_op(st.w1t[2 * h][aa], st.w1t[2 * h + 1][aa]);
    float4_t act[kHT], sd[kHT];
#pragma unroll
    for (int aa = 0; aa < kHT; ++aa) {
      float4_t u = mfma(ka0, w1b[0][aa], zero);
      u = mfma(ka1, w1b[1][aa], u);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float av, dv;
        act_grad<kPaper>(u[e], av, dv);
        act[aa][e] = av;
        sd[aa][e] = dv;
      }
    }
    u32x2 ab[kHT];
    float4_t actT[kHT];
#pragma unroll
    for (int aa = 0; aa < kHT; ++aa) {
      ab[aa] = k16(act[aa]);
      actT[aa] = mfma16(ab[aa], eye, zero);
    }
    u32x4 w2op[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      w2op[it] = cat_u(st.w2t[0][it], st.w2t[1][it]);
      const int row = 16 * it + n;
      lds_store<u32x2>(w2lds, w2off(row, g), u32x2{w2op[it].x, w2op[it].y});
      lds_store<u32x2>(w2lds, w2off(row, 4 + g), u32x2{w2op[it].z, w2op[it].w});
    }
    const bf16x8_t atb = cat_op(actT[0], actT[1]);
    if (!kDot || kPaper) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const float4_t ot = mfma(bf(w2op[it]), atb, zero);
        lds_store<float4_t>(opart, ((wv * kB + n) * kRow + 16 * it + 4 * g) * 4, ot);
      }
    }
    // every operation older than this chunk's top (the operands of chunk c - 2) is complete
    __builtin_amdgcn_s_waitcnt(0x0F70 | kTopOps);
    barrier();
    if (wv == 0) {
      if (mode == 0) {  // lane 0 read the partner's word one chunk ago (0 before that)
        const uint32_t oh = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(other >> 32));
        const uint32_t ol = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(other));
        if (oh == static_cast<uint32_t>(tag)) mode = (ol == static_cast<uint32_t>(xm)) ? 1 : 2;
        if (mode == 0 && lane == 0) other = __hip_atomic_load(hello_other, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (c >= 2) progress(c - 1);
    }
    {
      float2_t s2 = zero2;
      if (!kDot || kPaper) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s2 += lds_load<float2_t>(opart, ((w * kB + rt) * kRow + ri) * 4);
      }
      const uint32_t vb = cur.vv;
      const float2_t vr = {__builtin_bit_cast(float, vb << 16), __builtin_bit_cast(float, vb & 0xFFFF0000u)};
      float2_t r2;
      if constexpr (kPaper) {
        const float2_t lng = *reinterpret_cast<const float2_t*>(&sh.lnp[0][ri]);
        const float2_t lnb = *reinterpret_cast<const float2_t*>(&sh.lnp[1][ri]);
        const Ln2 st2 = ln2_row(s2, a.ln_eps);
        const float2_t kr = {__builtin_bit_cast(float, cur.kv << 16), __builtin_bit_cast(float, cur.kv & 0xFFFF0000u)};
        const float2_t err = kDot ? -vr : kr + lng * st2.xh + lnb - vr;
        const float2_t gg = lng * err;
        const float2_t m = sum32x2(float2_t{gg[0] + gg[1], gg[0] * st2.xh[0] + gg[1] * st2.xh[1]}) * (1.0f / kD);
        r2 = st2.rstd * (gg - m[0] - st2.xh * m[1]);
      } else {
        r2 = s2 - vr;
      }
      const float nrate = -eta * cur.et;
      const uint32_t rp = pack_bf16(r2[0] * nrate, r2[1] * nrate);
      lds_store<uint32_t>(rrb, (rt * kRRow + ri) * 2, rp);
      lds_store<uint16_t>(rtb, (ri * kTRow + rt) * 2, static_cast<uint16_t>(rp));
      lds_store<uint16_t>(rtb, ((ri + 1) * kTRow + rt) * 2, static_cast<uint16_t>(rp >> 16));
    }
    barrier();
    u32x2 rb[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) rb[it] = lds_load<u32x2>(rtb, ((16 * it + n) * kTRow + 4 * g) * 2);
    bf16x8_t rrow[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) rrow[h] = bf(lds_load<u32x4>(rrb, (n * kRRow + 32 * h + 8 * g) * 2));
    u32x2 dub[kHT];
#pragma unroll
    for (int aa = 0; aa < kHT; ++aa) {
      float4_t da = zero;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x2 lo = lds_load_tr(w2lds, w2off(32 * h + 8 * g + (n >> 2), 4 * aa + (n & 3)));
        const u32x2 hi2v = lds_load_tr(w2lds, w2off(32 * h + 8 * g + 4 + (n >> 2), 4 * aa + (n & 3)));
        const u32x4 w2k = {lo.x, lo.y, hi2v.x, hi2v.y};
        da = mfma(rrow[h], bf(w2k), da);
      }
      dub[aa] = k16(da * sd[aa]);
    }
    update_state(st, cur.kt, dub, ab, rb);
#pragma unroll
    for (int aa = 0; aa < kHT; ++aa) {
      pdub[aa] = dub[aa];
      pab[aa] = ab[aa];
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) prb[it] = rb[it];
  };

  MainIn ca, cb;
  load_main<kPaper>(ca, k, v, etok, 0, seq_bytes, o);
  int c = 0;
  for (; c + 1 < nchunks; c += 2) {
    step(ca, cb, c);
    step(cb, ca, c + 1);
  }
  if (c < nchunks) step(ca, cb, c);
  publish(nchunks);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every operand store of this wave is complete
  barrier();
  if (wv == 0) progress(nchunks);
  // final state (the output workgroup holds the same values; the recursion writes it)
  store_state(st, a.w1_out ? a.w1_out + static_cast<size_t>(chain) * hd : nullptr,
              a.w2_out ? a.w2_out + static_cast<size_t>(chain) * hd : nullptr, h0, g, n);
}

template <bool kPaper>
__device__ __forceinline__ void load_hand(Hand& hd, __amdgpu_buffer_rsrc_t rs, int c, int wv, int lane) {
  const int off = c * kSlotBytes;
  constexpr int kSc1 = 16;  // device scope: read at the XCC's L2, past the CU's cache
  hd.du = __builtin_amdgcn_raw_buffer_load_b128(rs, off + wv * 2048 + lane * 16, 0, kSc1);
  hd.ab = __builtin_amdgcn_raw_buffer_load_b128(rs, off + wv * 2048 + 1024 + lane * 16, 0, kSc1);
  hd.r0 = __builtin_amdgcn_raw_buffer_load_b128(rs, off + kWaves * 2048 + lane * 16, 0, kSc1);
  hd.r1 = __builtin_amdgcn_raw_buffer_load_b128(rs, off + kWaves * 2048 + 1024 + lane * 16, 0, kSc1);
}

template <bool kDot, bool kPaper>
__device__ __forceinline__ void split_outputs(const MlpArgs& a, SplitLds& sl, int chain, const char* slots,
                                              unsigned long long* flag, unsigned long long tag, int dbg) {
  // failure-path test: wait for a tag the recursion never writes, with a short bound
  const unsigned long long want_tag = (dbg & kSplitTestAbort) ? (tag ^ 1ull) : tag;
  const int spin_limit = (dbg & kSplitTestAbort) ? 64 : kSpinLimit;
  Lds& sh = sl.base;
  lds_char* zpart = (lds_char*)(&sh.zpart[0][0][0]);
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int bi = chain / a.H;
  const int hi = chain - bi * a.H;
  const int T = a.T;
  const int nchunks = (T + kB - 1) / kB;
  const int seq_bytes = T * kD * 2;
  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * kD;
  const char* q = reinterpret_cast<const char*>(static_cast<const bf16*>(a.q) + tok0);
  const char* k = reinterpret_cast<const char*>(static_cast<const bf16*>(a.k) + tok0);
  char* z = reinterpret_cast<char*>(static_cast<bf16*>(a.z) + tok0);
  const size_t hd = static_cast<size_t>(kH) * kD;
  const float* w1g = a.w1 + bi * a.w_batch_stride + static_cast<long long>(hi) * hd;
  const float* w2g = a.w2 + bi * a.w_batch_stride + static_cast<long long>(hi) * hd;
  const int h0 = 16 * kHT * wv;
  if (kPaper && tid < 2 * kD) sh.lnp[tid / kD][tid % kD] = (tid < kD ? a.ln_w : a.ln_b)[hi * kD + tid % kD];
  if (tid == 0) sl.abort_flag = 0;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(slots), 0, nchunks * kSlotBytes, 0x00020000);

  State st;
  init_state(st, w1g, w2g, h0, g, n);
  const uint32_t one = 0x3F80u;
  const u32x2 eye = {(4 * g + 0 == n ? one : 0u) | (4 * g + 1 == n ? one << 16 : 0u),
                     (4 * g + 2 == n ? one : 0u) | (4 * g + 3 == n ? one << 16 : 0u)};
  const bool keep[4] = {4 * g + 0 <= n, 4 * g + 1 <= n, 4 * g + 2 <= n, 4 * g + 3 <= n};
  Offsets o;
  o.row = n * 128 + 32 * g;
  const int c0 = 16 * (n >> 2) + 2 * (n & 3);
#pragma unroll
  for (int e = 0; e < 4; ++e) o.kt[e] = (4 * g + e) * 128 + 2 * c0;
  const int rt = tid >> 5;
  const int ri = 2 * (tid & 31);
  o.vv = rt * 128 + 2 * ri;
  o.et = rt * 4;
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const float2_t zero2 = {0.0f, 0.0f};

  // XCC ids: post this workgroup's, wait for the recursion's
  const unsigned long long xp = xcc_id();
  if (wv == 0 && lane == 0) {
    __hip_atomic_store(flag + 2, (tag << 32) | xp, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    int spins = 0;
    unsigned long long h = 0;
    for (;;) {
      h = __hip_atomic_load(flag + 1, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
      if ((h >> 32) == want_tag) break;
      if (++spins > spin_limit) {
        sl.abort_flag = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    sl.same_xcc = ((h >> 32) == want_tag && (h & 0xffffffffull) == xp && !(dbg & kSplitFormal)) ? 1 : 0;
  }
  // chunks known complete (wave 0 only); wait until at least `need` are.  `ahead` holds the
  // progress word as read one chunk earlier.
  int pub = 0;
  bool same = false;  // wave 0: set after the first barrier
  unsigned long long ahead = 0;
  auto wait_for = [&](int need) {
    if (wv == 0) {
      if (pub < need) {
        int got = pub;
        if (lane == 0) {
          unsigned long long f = ahead;
          int spins = 0;
          while (!((f >> 32) == tag && static_cast<int>(f & 0xffffffffu) >= need)) {
            if (++spins > spin_limit) {
              sl.abort_flag = 1;
              break;
            }
            __builtin_amdgcn_s_sleep(2);
            f = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          got = spins > spin_limit ? nchunks : static_cast<int>(f & 0xffffffffu);
          // across XCCs the progress word came with an agent-scope release: acquire it
          if (!same) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        pub = __builtin_amdgcn_readfirstlane(got);
      }
      if (lane == 0) ahead = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  uint32_t qv_prev = 0u;
  auto reduce_store_z = [&](int c) {
    float2_t s2 = zero2;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s2 += lds_load<float2_t>(zpart, ((w * kB + rt) * kRow + ri) * 4);
    if constexpr (kPaper) {
      const float2_t lng = *reinterpret_cast<const float2_t*>(&sh.lnp[0][ri]);
      const float2_t lnb = *reinterpret_cast<const float2_t*>(&sh.lnp[1][ri]);
      const Ln2 st2 = ln2_row(s2, a.ln_eps);
      s2 = float2_t{__builtin_bit_cast(float, qv_prev << 16), __builtin_bit_cast(float, qv_prev & 0xFFFF0000u)} +
           lng * st2.xh + lnb;
    }
    const int off = c * kTileBytes;
    __builtin_amdgcn_raw_buffer_store_b32(pack_bf16(s2[0], s2[1]), chunk_rsrc(z + off, seq_bytes - off), o.vv, 0,
                                          0);
  };

  int cdone = 0;  // chunks whose outputs are stored
  auto step = [&](const PartIn& cur, PartIn& nxt, const Hand& hc, Hand& hn, int c) -> bool {
    wait_for(c + 2 < nchunks ? c + 2 : nchunks);
    barrier();
    if (sl.abort_flag) return false;
    load_part<kPaper>(nxt, q, k, c + 1, seq_bytes, o);
    load_hand<kPaper>(hn, rs, c + 1, wv, lane);
    const bf16x8_t ka0 = bf(cur.ka0), ka1 = bf(cur.ka1), qb0 = bf(cur.qb0), qb1 = bf(cur.qb1);
    const u32x2 dub[kHT] = {lo2(hc.du), hi2(hc.du)};
    const u32x2 ab[kHT] = {lo2(hc.ab), hi2(hc.ab)};
    const u32x2 rb[4] = {lo2(hc.r0), hi2(hc.r0), lo2(hc.r1), hi2(hc.r1)};
    bf16x8_t w1b[2][kHT];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int aa = 0; aa < kHT; ++aa) w1b[h][aa] = pair_op(st.w1t[2 * h][aa], st.w1t[2 * h + 1][aa]);
    float4_t actT[kHT];
#pragma unroll
    for (int aa = 0; aa < kHT; ++aa) actT[aa] = mfma16(ab[aa], eye, zero);
    const bf16x8_t atb = cat_op(actT[0], actT[1]);
    float4_t pt = mfma(ka0, qb0, zero);
    pt = mfma(ka1, qb1, pt);
#pragma unroll
    for (int e = 0; e < 4; ++e) pt[e] = keep[e] ? pt[e] : 0.0f;
    const bf16x8_t ptb = pad_op(pt);
    float4_t aqT[kHT];
#pragma unroll
    for (int aa = 0; aa < kHT; ++aa) {
      float4_t u = mfma(w1b[0][aa], qb0, zero);
      u = mfma(w1b[1][aa], qb1, u);
      u = mfma(pad2(dub[aa]), ptb, u);
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = act_only<kPaper>(u[e]);
      aqT[aa] = u;
    }
    const bf16x8_t aqb = cat_op(aqT[0], aqT[1]);
    float4_t gt = mfma(atb, aqb, zero);
#pragma unroll
    for (int e = 0; e < 4; ++e) gt[e] = keep[e] ? gt[e] : 0.0f;
    const bf16x8_t gtb = pad_op(gt);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const bf16x8_t w2o = bf(cat_u(st.w2t[0][it], st.w2t[1][it]));
      float4_t zt = mfma(w2o, aqb, zero);
      zt = mfma(pad2(rb[it]), gtb, zt);
      lds_store<float4_t>(zpart, ((wv * kB + n) * kRow + 16 * it + 4 * g) * 4, zt);
    }
    barrier();
    qv_prev = cur.qv;
    reduce_store_z(c);
    cdone = c + 1;
    update_state(st, cur.kt, dub, ab, rb);
    return true;
  };

  PartIn ca, cb;
  Hand ha, hb;
  barrier();
  same = sl.same_xcc != 0;
  wait_for(nchunks > 0 ? 1 : 0);
  barrier();
  bool ok = sl.abort_flag == 0;
  if (ok) {
    load_part<kPaper>(ca, q, k, 0, seq_bytes, o);
    load_hand<kPaper>(ha, rs, 0, wv, lane);
    int c = 0;
    for (; ok && c + 1 < nchunks; c += 2) {
      ok = step(ca, cb, ha, hb, c);
      if (ok) ok = step(cb, ca, hb, ha, c + 1);
    }
    if (ok && c < nchunks) ok = step(ca, cb, ha, hb, c);
  }
  if (!ok) {  // the recursion never published: no outputs from here on
    const uint32_t nan2 = 0x7FC07FC0u;
    for (int c = cdone; c < nchunks; ++c) {
      const int off = c * kTileBytes;
      __builtin_amdgcn_raw_buffer_store_b32(nan2, chunk_rsrc(z + off, seq_bytes - off), o.vv, 0, 0);
    }
  }
}

template <bool kDot, bool kPaper>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mlp_split_kernel(
    MlpArgs a, char* ws, unsigned long long tag, int npad, int dbg) {
  __shared__ __attribute__((aligned(16))) SplitLds sl;
  const int nchains = a.B * a.H;
  const bool outputs = static_cast<int>(blockIdx.x) >= npad;
  const int chain = outputs ? static_cast<int>(blockIdx.x) - npad : static_cast<int>(blockIdx.x);
  if (chain >= nchains) return;
  const int nchunks = (a.T + kB - 1) / kB;
  unsigned long long* flag = reinterpret_cast<unsigned long long*>(ws + static_cast<size_t>(chain) * kFlagStride);
  char* slots = ws + split_flag_bytes(nchains) + static_cast<size_t>(chain) * nchunks * kSlotBytes;
  if (outputs)
    split_outputs<kDot, kPaper>(a, sl, chain, slots, flag, tag, dbg);
  else
    split_recursion<kDot, kPaper>(a, sl, chain, slots, flag, tag, dbg);
}

}  // namespace

bool mlp_fast_supported(const MlpArgs& a, bool bf16_io) {
  auto al = [](const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & (m - 1)) == 0; };
  const bool aligned = al(a.q, 16) && al(a.k, 16) && al(a.v, 16) && al(a.z, 16) && al(a.w1, 16) &&
                       al(a.w2, 16) && (a.w_batch_stride % 4) == 0 &&
                       (a.w1_out == nullptr || al(a.w1_out, 16)) &&
                       (a.w2_out == nullptr || al(a.w2_out, 16));
  const bool fits = static_cast<long long>(a.T) * kD * 2 + 4LL * kTileBytes < 0x7fffffffLL;
  return bf16_io && a.d == kD && a.dh == kH && a.chunk == kB && a.causal == 1 && a.T > 0 &&
         aligned && fits && (a.eta_tok == nullptr || al(a.eta_tok, 4));
}

hipError_t launch_mlp_fast(const MlpArgs& a, hipStream_t s) {
  const long long nchains = static_cast<long long>(a.B) * a.H;
  if (nchains > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(nchains)), block(kThreads);
  const bool paper = a.ln_w != nullptr;  // the paper's TTT-MLP: GELU, LN and residual
  if (paper && a.dot_loss)
    hipLaunchKernelGGL((mlp_mfma_kernel<true, true, false>), grid, block, 0, s, a, nullptr);
  else if (paper)
    hipLaunchKernelGGL((mlp_mfma_kernel<false, true, false>), grid, block, 0, s, a, nullptr);
  else if (a.dot_loss)
    hipLaunchKernelGGL((mlp_mfma_kernel<true, false, false>), grid, block, 0, s, a, nullptr);
  else
    hipLaunchKernelGGL((mlp_mfma_kernel<false, false, false>), grid, block, 0, s, a, nullptr);
  return hipGetLastError();
}

size_t mlp_split_workspace_bytes(const MlpArgs& a) {
  const long long nchains = static_cast<long long>(a.B) * a.H;
  const long long nchunks = (a.T + kB - 1) / kB;
  return split_flag_bytes(static_cast<int>(nchains)) + static_cast<size_t>(nchains * nchunks) * kSlotBytes;
}

bool mlp_split_supported(const MlpArgs& a, bool bf16_io) {
  const long long nchunks = (a.T + kB - 1) / kB;
  return mlp_fast_supported(a, bf16_io) && nchunks * kSlotBytes < 0x7fffffffLL &&
         static_cast<long long>(a.B) * a.H <= (0x7fffffffLL - 8) / 2;
}

hipError_t launch_mlp_split(const MlpArgs& a, void* ws, uint32_t tag, int dbg, hipStream_t s) {
  const int nchains = a.B * a.H;
  const int npad = (nchains + 7) & ~7;  // a chain's two workgroups share a residue mod 8
  const dim3 grid(static_cast<unsigned>(2 * npad)), block(kThreads);
  char* w = static_cast<char*>(ws);
  const unsigned long long t = tag;
  const bool paper = a.ln_w != nullptr;
  if (paper && a.dot_loss)
    hipLaunchKernelGGL((mlp_split_kernel<true, true>), grid, block, 0, s, a, w, t, npad, dbg);
  else if (paper)
    hipLaunchKernelGGL((mlp_split_kernel<false, true>), grid, block, 0, s, a, w, t, npad, dbg);
  else if (a.dot_loss)
    hipLaunchKernelGGL((mlp_split_kernel<true, false>), grid, block, 0, s, a, w, t, npad, dbg);
  else
    hipLaunchKernelGGL((mlp_split_kernel<false, false>), grid, block, 0, s, a, w, t, npad, dbg);
  return hipGetLastError();
}

hipError_t launch_mlp_fwd_hist(const MlpArgs& a, void* hist, hipStream_t s) {
  const long long nchains = static_cast<long long>(a.B) * a.H;
  if (nchains > 0x7fffffffLL || a.ln_w != nullptr || a.dot_loss || a.eta_tok != nullptr)
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(nchains)), block(kThreads);
  hipLaunchKernelGGL((mlp_mfma_kernel<false, false, true>), grid, block, 0, s, a, static_cast<char*>(hist));
  return hipGetLastError();
}

}  // namespace ttt
