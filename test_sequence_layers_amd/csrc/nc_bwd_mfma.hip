// Backward pass of the non-causal TTT layers on the gfx950 matrix cores, for one full-batch
// step (the linear inner model at the end of this file): f(k) = W2 SiLU(W1 k), d = 64,
// hidden 64, 16 to 256 tokens, bf16
// Q/K/V/dZ/dQ/dK/dV, fp32 states and state gradients, reconstruction or negative
// dot-product loss, scalar rate or per-token rate factors (with their gradient).
//
// The outer loop trains the projections, the initial state and the rates through the inner
// update (ViT3 news page, section 1: keys and values are learned end to end, one full-batch
// inner step, then every query reads the trained model; wmrh.cn summary of Sun et al. 2024,
// section 2.2 and 2.2.3).  Forward, over all N tokens (rows t), phi = SiLU, S = phi'(U):
//   U = K W1^T, A = phi(U), R = A W2^T - V (or -V), Rt = diag(e) R, Dm = Rt W2, dU = Dm * S,
//   G1 = dU^T K, G2 = Rt^T A, W1' = W1 - eta G1, W2' = W2 - eta G2,
//   Uq = Q W1'^T, Aq = phi(Uq), Z = Aq W2'^T.
// Reverse mode, our derivation of the chain rule (the same per-token formulas as the
// vector-ALU kernel, written over a tile of tokens):
//   queries:  dAq = dZ W2', dUq = dAq * phi'(Uq), dQ = dUq W1',
//             P1 = dW1_out + dUq^T Q,  P2 = dW2_out + dZ^T Aq,  S1 = -eta P1, S2 = -eta P2;
//   keys:     ddU = K S1^T, dDm = ddU * S, dRt = A S2^T + dDm W2^T, dR = diag(e) dRt,
//             de_t = <dRt_t, R_t>, dV = -dR,
//             dA = Rt S2 + dR W2 (the second term with the reconstruction loss only),
//             dUk = dA * S + ddU * Dm * phi''(U),  dK = dU S1 + dUk W1,
//             dW1 = P1 + dUk^T K,  dW2 = P2 + Rt^T dDm + dR^T A (the last term: reconstruction).
//
// Mapping.  One workgroup of four waves per (batch, head) chain; wave w takes the 16-token
// tiles w, w + 4, w + 8, w + 12.  Three passes over the tiles (keys, queries, keys again),
// each wave accumulating its share of a 64 x 64 sum in fp32 MFMA tiles; between passes the
// shares meet in LDS (each wave adds one row block of all four waves' shares into two padded
// fp32 matrices) and the workgroup forms the next pass's bf16 matrices there (W1', W2', then
// S1, S2).  The products with W1, W2 in pass 1 and with W1', W2' in pass 2 take each state as
// a sum of two bf16 parts (hi + lo): dq passes through the roundings of both, and with one
// part each its element-wise error reached 2.2e-2 of max|dq| over the 384 vision sequences
// (1.6e-2 with two; a numpy emulation of this kernel's rounding points reproduced both).
// Below 16 tokens the sums are too short to average the roundings out and the vector-ALU
// kernel serves.  Every per-tile quantity is
// formed transposed (rows: hidden or feature index, columns: tokens), so each lane holds
// four consecutive entries of one token and writes them as 8 bytes into a bf16 row-major
// tile in LDS; from there it is an operand over its columns (16-byte or paired 8-byte row
// reads) or over its tokens (the gfx950 transposing read).  A tile's inputs are loaded into
// registers one tile ahead, and its outputs stored one tile late, right after the wait for
// those loads: a global load issued while stores are in flight would make the wave wait for
// the stores as well.
//
// Layouts (v_mfma_f32_16x16x32_bf16; C layout: lane (g, x) = (lane / 16, lane % 16) holds
// rows 4 g + e, e = 0..3, of column x; both operands: lane (g, x) holds row x, k = 8 g + s):
//   * row operand over a matrix's columns: k = 32 kb + 8 g + s (one 16-byte read);
//   * permuted operands over an index of 64 (columns of a row-major matrix: two 8-byte
//     reads; rows of a matrix: two transposing reads): k = 8 g + s in block kb <->
//     32 kb + 16 (s / 4) + 4 g + s % 4;
//   * operands over the 16 tokens of a tile (transposing reads, upper half zero):
//     k = 8 g + s <-> token 4 g + s, s < 4.
// LDS rows of 128 bytes hold 16-byte pieces XOR-swizzled by row % 8.
#include <type_traits>

#include "common.hpp"

namespace ttt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) float lds_float;

constexpr int kD = 64;                    // features (and hidden units)
constexpr int kT = 16;                    // tokens per tile
constexpr int kRow = kD * 2;              // bytes per bf16 row
constexpr int kTileB = kT * kRow;         // one token tile
constexpr int kMatB = kD * kRow;          // one 64 x 64 bf16 matrix
constexpr int kWaves = 4;
constexpr int kMaxTokens = 256;
constexpr int kPerWave = kMaxTokens / kT / kWaves;
constexpr int kAccRow = kD + 4;           // fp32 accumulator rows, padded
// per-wave token tiles
constexpr int kIn1 = 0, kIn2 = kTileB, kA = 2 * kTileB, kRt = 3 * kTileB, kDU = 4 * kTileB,
              kDDm = 5 * kTileB, kDR = 6 * kTileB, kDUk = 7 * kTileB, kWaveB = 8 * kTileB;
// the workgroup's bf16 matrices: W1, W2 (all passes); the low parts of W1, W2 (pass 1), then of
// W1', W2' (pass 2); W1', W2' (pass 2), then S1, S2 (pass 3)
constexpr int kW1 = 0, kW2 = kMatB, kLo1 = 2 * kMatB, kLo2 = 3 * kMatB, kX1 = 4 * kMatB,
              kX2 = 5 * kMatB, kMatsB = 6 * kMatB;

struct NcBwdMfmaArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dz;
  const float* w1;  // [h][d]
  const float* w2;  // [d][h]
  long long w_batch_stride;
  const float* dw1_out;
  const float* dw2_out;
  const float* eta_tok;
  void* dq;
  void* dk;
  void* dv;
  float* dw1;
  float* dw2;
  float* deta_tok;
  int B, H, T;
  float eta;
};

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ bf16x8_t bf(const u32x4& x) { return __builtin_bit_cast(bf16x8_t, x); }
__device__ __forceinline__ bf16x8_t pad2(const u32x2& x) { return bf(u32x4{x.x, x.y, 0u, 0u}); }
__device__ __forceinline__ bf16x8_t join2(const u32x2& x, const u32x2& y) { return bf(u32x4{x.x, x.y, y.x, y.y}); }
__device__ __forceinline__ float4_t mfma(const bf16x8_t& a, const bf16x8_t& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4_t unpack4(const u32x2& x) {
  return float4_t{__builtin_bit_cast(float, x.x << 16), __builtin_bit_cast(float, x.x & 0xFFFF0000u),
                  __builtin_bit_cast(float, x.y << 16), __builtin_bit_cast(float, x.y & 0xFFFF0000u)};
}
__device__ __forceinline__ u32x2 pack4(const float4_t& x) { return u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])}; }
// x as hi + lo, both bf16 (about 16 significant bits together)
__device__ __forceinline__ void split4(const float4_t& x, u32x2& hi, u32x2& lo) {
  hi = pack4(x);
  lo = pack4(x - unpack4(hi));
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes > 0 ? bytes : 0, 0x00020000);
}
// byte offset of element (row, col) of a swizzled bf16 row-major tile, col % 4 == 0
__device__ __forceinline__ int sw(int row, int col) {
  return row * kRow + 16 * ((col >> 3) ^ (row & 7)) + 2 * (col & 7);
}
template <typename T>
__device__ __forceinline__ T lds_ld(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}
template <typename T>
__device__ __forceinline__ void lds_st(lds_char* p, T v) {
  *reinterpret_cast<__attribute__((address_space(3))) T*>(p) = v;
}
// transposing read: lane (g, x) fetches row `row` + (x / 4) offset as given, columns col .. + 3
// (col chosen per lane), and receives rows r0 + 0..3 of column c0(x / 4) + x % 4
__device__ __forceinline__ u32x2 tr(const lds_char* base, int row, int col) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + sw(row, col))));
}
__device__ __forceinline__ float phi2(float u, float sg) {  // SiLU''(u) = s (1 - s) (2 + u (1 - 2 s))
  return sg * (1.0f - sg) * (2.0f + u * (1.0f - 2.0f * sg));
}

// Operands of lane (g, x).
// rows r0 + x of M, k over its columns (natural order)
__device__ __forceinline__ bf16x8_t rowop(const lds_char* m, int r0, int kb, int g, int x) {
  return bf(lds_ld<u32x4>(m + sw(r0 + x, 32 * kb + 8 * g)));
}
// rows r0 + x of M, k over its columns (permuted order)
__device__ __forceinline__ bf16x8_t rowop_p(const lds_char* m, int r0, int kb, int g, int x) {
  return join2(lds_ld<u32x2>(m + sw(r0 + x, 32 * kb + 4 * g)), lds_ld<u32x2>(m + sw(r0 + x, 32 * kb + 16 + 4 * g)));
}
// columns c0 + x of M as rows, k over its rows (permuted order)
__device__ __forceinline__ bf16x8_t colop_p(const lds_char* m, int c0, int kb, int g, int x) {
  return join2(tr(m, 32 * kb + 4 * g + (x >> 2), c0 + 4 * (x & 3)),
               tr(m, 32 * kb + 16 + 4 * g + (x >> 2), c0 + 4 * (x & 3)));
}
// columns c0 + x of a token tile as rows, k over its 16 tokens
__device__ __forceinline__ bf16x8_t tokop(const lds_char* m, int c0, int g, int x) {
  return pad2(tr(m, 4 * g + (x >> 2), c0 + 4 * (x & 3)));
}
// C = sum over 64 of two row operands in natural order
__device__ __forceinline__ float4_t mm(const lds_char* a, int ra, const lds_char* b, int rb, int g, int x,
                                       float4_t c) {
  c = mfma(rowop(a, ra, 0, g, x), rowop(b, rb, 0, g, x), c);
  return mfma(rowop(a, ra, 1, g, x), rowop(b, rb, 1, g, x), c);
}
// C = sum over 64 of (columns c0 of a) and (rows rb of b), permuted order
__device__ __forceinline__ float4_t mm_t(const lds_char* a, int c0, const lds_char* b, int rb, int g, int x,
                                         float4_t c) {
  c = mfma(colop_p(a, c0, 0, g, x), rowop_p(b, rb, 0, g, x), c);
  return mfma(colop_p(a, c0, 1, g, x), rowop_p(b, rb, 1, g, x), c);
}

// One tile's two inputs (and rate factor) in registers: lane l holds 16 bytes of rows l / 8
// and 8 + l / 8, piece l % 8.
struct In {
  u32x4 a0, a1, b0, b1;
  float e;
};
template <bool kTok>
__device__ __forceinline__ In load_in(const char* pa, const char* pb, const float* etok, int tt, int T, int lane) {
  const int off = tt * kTileB, left = T * kRow - off;
  const __amdgpu_buffer_rsrc_t ra = rsrc(pa + off, left), rb = rsrc(pb + off, left);
  const int o0 = (lane >> 3) * kRow + 16 * (lane & 7);
  In r;
  r.a0 = __builtin_amdgcn_raw_buffer_load_b128(ra, o0, 0, 0);
  r.a1 = __builtin_amdgcn_raw_buffer_load_b128(ra, o0 + 8 * kRow, 0, 0);
  r.b0 = __builtin_amdgcn_raw_buffer_load_b128(rb, o0, 0, 0);
  r.b1 = __builtin_amdgcn_raw_buffer_load_b128(rb, o0 + 8 * kRow, 0, 0);
  r.e = 1.0f;
  if constexpr (kTok) {
    const __amdgpu_buffer_rsrc_t re = rsrc(etok + tt * kT, 4 * (T - tt * kT));
    r.e = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(re, 4 * (lane & 15), 0, 0));
  }
  return r;
}
__device__ __forceinline__ void put_in(const In& r, lds_char* ta, lds_char* tb, int lane) {
  const int row = lane >> 3, col = 8 * (lane & 7);
  lds_st<u32x4>(ta + sw(row, col), r.a0);
  lds_st<u32x4>(ta + sw(row + 8, col), r.a1);
  lds_st<u32x4>(tb + sw(row, col), r.b0);
  lds_st<u32x4>(tb + sw(row + 8, col), r.b1);
}

template <bool kTok, bool kDot>
__global__ __launch_bounds__(64 * kWaves) void mlp_nc_bwd_mfma_kernel(NcBwdMfmaArgs a) {
  __shared__ __attribute__((aligned(16))) char mats_mem[kMatsB];
  __shared__ __attribute__((aligned(16))) char tiles_mem[kWaves * kWaveB];
  __shared__ __attribute__((aligned(16))) float acc_mem[2 * kD * kAccRow];
  lds_char* mats = (lds_char*)(mats_mem);
  lds_char* my = (lds_char*)(tiles_mem) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * kWaveB;
  lds_float* acc1 = (lds_float*)(acc_mem);            // G1, then P1 (+ dW1), rows a, cols j
  lds_float* acc2 = (lds_float*)(acc_mem) + kD * kAccRow;  // G2, then P2 (+ dW2), rows i, cols a
  const int chain = blockIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 4, x = lane & 15;
  const int bi = chain / a.H, hi = chain - bi * a.H;
  const int T = a.T;
  const int ntiles = (T + kT - 1) / kT;
  const float eta = a.eta;
  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * kD;
  const char* q = reinterpret_cast<const char*>(static_cast<const bf16*>(a.q) + tok0);
  const char* k = reinterpret_cast<const char*>(static_cast<const bf16*>(a.k) + tok0);
  const char* v = reinterpret_cast<const char*>(static_cast<const bf16*>(a.v) + tok0);
  const char* dz = reinterpret_cast<const char*>(static_cast<const bf16*>(a.dz) + tok0);
  const char* dq = reinterpret_cast<const char*>(static_cast<bf16*>(a.dq) + tok0);
  const char* dk = reinterpret_cast<const char*>(static_cast<bf16*>(a.dk) + tok0);
  const char* dv = reinterpret_cast<const char*>(static_cast<bf16*>(a.dv) + tok0);
  const float* etok = kTok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
  float* detok = kTok && a.deta_tok ? a.deta_tok + static_cast<size_t>(chain) * T : nullptr;
  const size_t hd = static_cast<size_t>(kD) * kD;
  const float* w1g = a.w1 + bi * a.w_batch_stride + static_cast<long long>(hi) * hd;
  const float* w2g = a.w2 + bi * a.w_batch_stride + static_cast<long long>(hi) * hd;
  const float* up1 = a.dw1_out ? a.dw1_out + static_cast<size_t>(chain) * hd : nullptr;
  const float* up2 = a.dw2_out ? a.dw2_out + static_cast<size_t>(chain) * hd : nullptr;
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  constexpr int kPer = kD * kD / 4 / (64 * kWaves);  // float4 pieces of a matrix per thread

  // ---- W1, W2 as bf16 matrices; zero accumulators ----
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int p = tid + i * 64 * kWaves, r = p >> 4, c = 4 * (p & 15);
    u32x2 hi, lo;
    split4(*reinterpret_cast<const float4_t*>(w1g + r * kD + c), hi, lo);
    lds_st<u32x2>(mats + kW1 + sw(r, c), hi);
    lds_st<u32x2>(mats + kLo1 + sw(r, c), lo);
    split4(*reinterpret_cast<const float4_t*>(w2g + r * kD + c), hi, lo);
    lds_st<u32x2>(mats + kW2 + sw(r, c), hi);
    lds_st<u32x2>(mats + kLo2 + sw(r, c), lo);
    *reinterpret_cast<__attribute__((address_space(3))) float4_t*>(acc1 + r * kAccRow + c) = zero;
    *reinterpret_cast<__attribute__((address_space(3))) float4_t*>(acc2 + r * kAccRow + c) = zero;
  }
  __syncthreads();
  const lds_char* mW1 = mats + kW1;
  const lds_char* mW2 = mats + kW2;
  const lds_char* mLo1 = mats + kLo1;
  const lds_char* mLo2 = mats + kLo2;

  // U^T (rows a, cols t) of the keys in my + kIn1 from W1; A rows to my + kA; returns S^T,
  // and U^T in u
  // (kSplit: W1 and W2 as hi + lo parts, as in pass 1, whose sums form W1' and W2')
  auto fwd_a = [&](float4_t (&s)[4], float4_t (&u)[4], float4_t (&sg)[4], auto split_c) __attribute__((always_inline)) {
#pragma unroll
    for (int at = 0; at < 4; ++at) {
      u[at] = mm(mW1, 16 * at, my + kIn1, 0, g, x, zero);
      if constexpr (decltype(split_c)::value) u[at] = mm(mLo1, 16 * at, my + kIn1, 0, g, x, u[at]);
      float4_t act;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sg[at][e] = sigmoidf_(u[at][e]);
        act[e] = u[at][e] * sg[at][e];
        s[at][e] = sg[at][e] * (1.0f + u[at][e] * (1.0f - sg[at][e]));
      }
      lds_st<u32x2>(my + kA + sw(x, 16 * at + 4 * g), pack4(act));
    }
  };
  // R^T (rows i, cols t) = W2 A^T - V^T (or -V^T); Rt rows to my + kRt; returns R^T
  auto fwd_r = [&](float4_t (&r)[4], float et, auto split_c) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      r[it] = kDot ? zero : mm(mW2, 16 * it, my + kA, 0, g, x, zero);
      if constexpr (!kDot && decltype(split_c)::value) r[it] = mm(mLo2, 16 * it, my + kA, 0, g, x, r[it]);
      r[it] -= unpack4(lds_ld<u32x2>(my + kIn2 + sw(x, 16 * it + 4 * g)));
      lds_st<u32x2>(my + kRt + sw(x, 16 * it + 4 * g), pack4(r[it] * et));
    }
  };
  // Dm^T (rows a, cols t) = sum_i W2[i][a] Rt[t][i]; dU rows (Dm * S) to my + kDU
  auto fwd_du = [&](float4_t (&dm)[4], const float4_t (&s)[4], auto split_c) __attribute__((always_inline)) {
#pragma unroll
    for (int at = 0; at < 4; ++at) {
      dm[at] = mm_t(mW2, 16 * at, my + kRt, 0, g, x, zero);
      if constexpr (decltype(split_c)::value) dm[at] = mm_t(mLo2, 16 * at, my + kRt, 0, g, x, dm[at]);
      lds_st<u32x2>(my + kDU + sw(x, 16 * at + 4 * g), pack4(dm[at] * s[at]));
    }
  };
  // acc += the four waves' tiles (rows 16 rt + 4 g + e, cols 16 ct + x): each wave parks its
  // 16 tiles in its own token-tile area (free between passes), then wave w adds up row block
  // rt = w of all four into acc (rows 16 w .. 16 w + 15: no two waves write the same entry).
  // (LDS float atomics measured several times slower than the whole rest of the kernel.)
  auto reduce = [&](lds_float* accm, const float4_t (&t)[4][4]) __attribute__((always_inline)) {
    typedef __attribute__((address_space(3))) float4_t lds_f4;
#pragma unroll
    for (int f = 0; f < 16; ++f) reinterpret_cast<lds_f4*>(my)[f * 64 + lane] = t[f >> 2][f & 3];
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int f = 4 * wv + ct;
      float4_t sum = zero;
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2)
        sum += reinterpret_cast<const lds_f4*>((lds_char*)(tiles_mem) + w2 * kWaveB)[f * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) accm[(16 * wv + 4 * g + e) * kAccRow + 16 * ct + x] += sum[e];
    }
    __syncthreads();
  };

  // ================= pass 1 (keys): G1 = dU^T K, G2 = Rt^T A
  {
    float4_t g1[4][4], g2[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) g1[i][j] = g2[i][j] = zero;
    In cur = load_in<kTok>(k, v, etok, wv, T, lane);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int tt = wv + kWaves * i;
      // loads and LDS copies on every iteration: a load used on one path only would be sunk
      // next to its use, and the wave would wait for it there
      put_in(cur, my + kIn1, my + kIn2, lane);
      const In nxt = load_in<kTok>(k, v, etok, tt + kWaves, T, lane);
      __builtin_amdgcn_sched_barrier(0);
      if (tt < ntiles) {
      float4_t s[4], u[4], sg[4], r[4], dm[4];
      fwd_a(s, u, sg, std::true_type{});
      fwd_r(r, cur.e, std::true_type{});
      fwd_du(dm, s, std::true_type{});
      bf16x8_t kop[4];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) kop[jt] = tokop(my + kIn1, 16 * jt, g, x);
#pragma unroll
      for (int at = 0; at < 4; ++at) {
        const bf16x8_t dop = tokop(my + kDU, 16 * at, g, x);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) g1[at][jt] = mfma(dop, kop[jt], g1[at][jt]);
      }
      bf16x8_t aop[4];
#pragma unroll
      for (int at = 0; at < 4; ++at) aop[at] = tokop(my + kA, 16 * at, g, x);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const bf16x8_t rop = tokop(my + kRt, 16 * it, g, x);
#pragma unroll
        for (int at = 0; at < 4; ++at) g2[it][at] = mfma(rop, aop[at], g2[it][at]);
      }
      }
      cur = nxt;
    }
    reduce(acc1, g1);
    reduce(acc2, g2);
  }
  __syncthreads();
  // ---- W' = W - eta G (bf16 hi + lo); the accumulators restart from the upstream state
  // gradients ----
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int p = tid + i * 64 * kWaves, r = p >> 4, c = 4 * (p & 15);
    auto* a1 = reinterpret_cast<__attribute__((address_space(3))) float4_t*>(acc1 + r * kAccRow + c);
    auto* a2 = reinterpret_cast<__attribute__((address_space(3))) float4_t*>(acc2 + r * kAccRow + c);
    u32x2 hi, lo;
    split4(*reinterpret_cast<const float4_t*>(w1g + r * kD + c) - eta * *a1, hi, lo);
    lds_st<u32x2>(mats + kX1 + sw(r, c), hi);
    lds_st<u32x2>(mats + kLo1 + sw(r, c), lo);
    split4(*reinterpret_cast<const float4_t*>(w2g + r * kD + c) - eta * *a2, hi, lo);
    lds_st<u32x2>(mats + kX2 + sw(r, c), hi);
    lds_st<u32x2>(mats + kLo2 + sw(r, c), lo);
    *a1 = up1 ? *reinterpret_cast<const float4_t*>(up1 + r * kD + c) : zero;
    *a2 = up2 ? *reinterpret_cast<const float4_t*>(up2 + r * kD + c) : zero;
  }
  __syncthreads();

  // ================= pass 2 (queries): dQ, P1 += dUq^T Q, P2 += dZ^T Aq
  {
    const lds_char* mW1p = mats + kX1;
    const lds_char* mW2p = mats + kX2;
    float4_t p1[4][4], p2[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) p1[i][j] = p2[i][j] = zero;
    In cur = load_in<false>(q, dz, nullptr, wv, T, lane);
    u32x2 dqv[4];
    int pend = -1;  // the tile whose dQ is still to be stored
    auto store_dq = [&](int tt) __attribute__((always_inline)) {
      const __amdgpu_buffer_rsrc_t rd = rsrc(dq + tt * kTileB, T * kRow - tt * kTileB);
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
        __builtin_amdgcn_raw_buffer_store_b64(dqv[jt], rd, x * kRow + 2 * (16 * jt + 4 * g), 0, 0);
    };
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int tt = wv + kWaves * i;
      put_in(cur, my + kIn1, my + kIn2, lane);  // Q, dZ
      if (pend >= 0) store_dq(pend);
      pend = -1;
      const In nxt = load_in<false>(q, dz, nullptr, tt + kWaves, T, lane);
      __builtin_amdgcn_sched_barrier(0);
      if (tt < ntiles) {
      // Uq^T (rows a, cols t), Aq rows, Sq
      float4_t sq[4];
#pragma unroll
      for (int at = 0; at < 4; ++at) {
        const float4_t uq = mm(mLo1, 16 * at, my + kIn1, 0, g, x, mm(mW1p, 16 * at, my + kIn1, 0, g, x, zero));
        float4_t act;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sg = sigmoidf_(uq[e]);
          act[e] = uq[e] * sg;
          sq[at][e] = sg * (1.0f + uq[e] * (1.0f - sg));
        }
        lds_st<u32x2>(my + kA + sw(x, 16 * at + 4 * g), pack4(act));
      }
      // dAq^T (rows a) = sum_i W2'[i][a] dZ[t][i]; dUq rows
#pragma unroll
      for (int at = 0; at < 4; ++at) {
        const float4_t da = mm_t(mLo2, 16 * at, my + kIn2, 0, g, x, mm_t(mW2p, 16 * at, my + kIn2, 0, g, x, zero));
        lds_st<u32x2>(my + kDU + sw(x, 16 * at + 4 * g), pack4(da * sq[at]));
      }
      // dQ^T (rows j) = sum_a W1'[a][j] dUq[t][a]
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
        dqv[jt] = pack4(mm_t(mLo1, 16 * jt, my + kDU, 0, g, x, mm_t(mW1p, 16 * jt, my + kDU, 0, g, x, zero)));
      pend = tt;
      // P1 += dUq^T Q (rows a, cols j); P2 += dZ^T Aq (rows i, cols a)
      bf16x8_t qop[4], aop[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        qop[c] = tokop(my + kIn1, 16 * c, g, x);
        aop[c] = tokop(my + kA, 16 * c, g, x);
      }
#pragma unroll
      for (int at = 0; at < 4; ++at) {
        const bf16x8_t dop = tokop(my + kDU, 16 * at, g, x);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) p1[at][jt] = mfma(dop, qop[jt], p1[at][jt]);
      }
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const bf16x8_t zop = tokop(my + kIn2, 16 * it, g, x);
#pragma unroll
        for (int at = 0; at < 4; ++at) p2[it][at] = mfma(zop, aop[at], p2[it][at]);
      }
      }
      cur = nxt;
    }
    if (pend >= 0) store_dq(pend);
    reduce(acc1, p1);
    reduce(acc2, p2);
  }
  __syncthreads();
  // ---- S = -eta P (bf16); the accumulators keep P, the state gradients' first terms ----
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int p = tid + i * 64 * kWaves, r = p >> 4, c = 4 * (p & 15);
    const float4_t p1v = *reinterpret_cast<__attribute__((address_space(3))) float4_t*>(acc1 + r * kAccRow + c);
    const float4_t p2v = *reinterpret_cast<__attribute__((address_space(3))) float4_t*>(acc2 + r * kAccRow + c);
    lds_st<u32x2>(mats + kX1 + sw(r, c), pack4(-eta * p1v));
    lds_st<u32x2>(mats + kX2 + sw(r, c), pack4(-eta * p2v));
  }
  __syncthreads();

  // ================= pass 3 (keys): dK, dV, de, dW1 += dUk^T K, dW2 += Rt^T dDm + dR^T A
  {
    const lds_char* mS1 = mats + kX1;
    const lds_char* mS2 = mats + kX2;
    float4_t h1[4][4], h2[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) h1[i][j] = h2[i][j] = zero;
    In cur = load_in<kTok>(k, v, etok, wv, T, lane);
    u32x2 dkv[4], dvv[4];
    float dev = 0.0f;
    int pend = -1;
    auto store_out = [&](int tt) __attribute__((always_inline)) {
      const int off = tt * kTileB, left = T * kRow - off;
      const __amdgpu_buffer_rsrc_t rk = rsrc(dk + off, left), rv = rsrc(dv + off, left);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        __builtin_amdgcn_raw_buffer_store_b64(dkv[c], rk, x * kRow + 2 * (16 * c + 4 * g), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(dvv[c], rv, x * kRow + 2 * (16 * c + 4 * g), 0, 0);
      }
      if (kTok && detok) {  // the four lane groups store the same value
        const __amdgpu_buffer_rsrc_t re = rsrc(detok + tt * kT, 4 * (T - tt * kT));
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, dev), re, 4 * x, 0, 0);
      }
    };
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int tt = wv + kWaves * i;
      put_in(cur, my + kIn1, my + kIn2, lane);  // K, V
      if (pend >= 0) store_out(pend);
      pend = -1;
      const In nxt = load_in<kTok>(k, v, etok, tt + kWaves, T, lane);
      __builtin_amdgcn_sched_barrier(0);
      if (tt < ntiles) {
      const float et = cur.e;
      float4_t s[4], u[4], sg[4], r[4], dm[4];
      fwd_a(s, u, sg, std::false_type{});
      fwd_r(r, et, std::false_type{});
      fwd_du(dm, s, std::false_type{});
      // ddU^T (rows a, cols t) = sum_j S1[a][j] K[t][j]; dDm rows; ddU * Dm * phi''(U)
      float4_t sec[4];
#pragma unroll
      for (int at = 0; at < 4; ++at) {
        const float4_t ddu = mm(mS1, 16 * at, my + kIn1, 0, g, x, zero);
        lds_st<u32x2>(my + kDDm + sw(x, 16 * at + 4 * g), pack4(ddu * s[at]));
#pragma unroll
        for (int e = 0; e < 4; ++e) sec[at][e] = ddu[e] * dm[at][e] * phi2(u[at][e], sg[at][e]);
      }
      // dRt^T (rows i, cols t) = S2 A^T + W2 dDm^T; de; dR = e dRt; dV = -dR
      float dpart = 0.0f;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        float4_t drt = mm(mS2, 16 * it, my + kA, 0, g, x, zero);
        drt = mm(mW2, 16 * it, my + kDDm, 0, g, x, drt);
        if constexpr (kTok) {
#pragma unroll
          for (int e = 0; e < 4; ++e) dpart += drt[e] * r[it][e];
        }
        const float4_t dr = drt * et;
        dvv[it] = pack4(-dr);
        if constexpr (!kDot) lds_st<u32x2>(my + kDR + sw(x, 16 * it + 4 * g), pack4(dr));
      }
      if constexpr (kTok) {
        dpart += __shfl_xor(dpart, 16, 64);
        dpart += __shfl_xor(dpart, 32, 64);
        dev = dpart;
      }
      // dA^T (rows a, cols t) = sum_i S2[i][a] Rt[t][i] (+ sum_i W2[i][a] dR[t][i]); dUk rows
#pragma unroll
      for (int at = 0; at < 4; ++at) {
        float4_t da = mm_t(mS2, 16 * at, my + kRt, 0, g, x, zero);
        if constexpr (!kDot) da = mm_t(mW2, 16 * at, my + kDR, 0, g, x, da);
        lds_st<u32x2>(my + kDUk + sw(x, 16 * at + 4 * g), pack4(da * s[at] + sec[at]));
      }
      // dK^T (rows j, cols t) = sum_a S1[a][j] dU[t][a] + sum_a W1[a][j] dUk[t][a]
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        float4_t dkt = mm_t(mS1, 16 * jt, my + kDU, 0, g, x, zero);
        dkt = mm_t(mW1, 16 * jt, my + kDUk, 0, g, x, dkt);
        dkv[jt] = pack4(dkt);
      }
      pend = tt;
      // dW1 += dUk^T K (rows a, cols j); dW2 += Rt^T dDm + dR^T A (rows i, cols a)
      bf16x8_t kop[4], mop[4], aop[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        kop[c] = tokop(my + kIn1, 16 * c, g, x);
        mop[c] = tokop(my + kDDm, 16 * c, g, x);
        if constexpr (!kDot) aop[c] = tokop(my + kA, 16 * c, g, x);
      }
#pragma unroll
      for (int at = 0; at < 4; ++at) {
        const bf16x8_t uop = tokop(my + kDUk, 16 * at, g, x);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) h1[at][jt] = mfma(uop, kop[jt], h1[at][jt]);
      }
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const bf16x8_t rop = tokop(my + kRt, 16 * it, g, x);
#pragma unroll
        for (int at = 0; at < 4; ++at) h2[it][at] = mfma(rop, mop[at], h2[it][at]);
        if constexpr (!kDot) {
          const bf16x8_t dop = tokop(my + kDR, 16 * it, g, x);
#pragma unroll
          for (int at = 0; at < 4; ++at) h2[it][at] = mfma(dop, aop[at], h2[it][at]);
        }
      }
      }
      cur = nxt;
    }
    if (pend >= 0) store_out(pend);
    reduce(acc1, h1);
    reduce(acc2, h2);
  }
  __syncthreads();
  // ---- dW1 = P1 + dUk^T K, dW2 = P2 + Rt^T dDm + dR^T A ----
  float* dw1 = a.dw1 + static_cast<size_t>(chain) * hd;
  float* dw2 = a.dw2 + static_cast<size_t>(chain) * hd;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int p = tid + i * 64 * kWaves, r = p >> 4, c = 4 * (p & 15);
    *reinterpret_cast<float4_t*>(dw1 + r * kD + c) =
        *reinterpret_cast<__attribute__((address_space(3))) float4_t*>(acc1 + r * kAccRow + c);
    *reinterpret_cast<float4_t*>(dw2 + r * kD + c) =
        *reinterpret_cast<__attribute__((address_space(3))) float4_t*>(acc2 + r * kAccRow + c);
  }
}


// ---------------------------------------------------------------- linear inner model
// f(k) = W k, W [i][j] (64 x 64): with R = K W^T - V (or -V), Rt = diag(e) R, G = Rt^T K,
// W' = W - eta G and Z = Q W'^T, the reverse mode (the same per-token formulas as the
// vector-ALU kernel) is
//   queries:  dQ = dZ W',  P = dW_out + dZ^T Q,  S = -eta P;
//   keys:     dRt = K S^T, dR = diag(e) dRt, de_t = <dRt_t, R_t>, dV = -dR,
//             dK = Rt S (+ dR W),  dW = P (+ dR^T K)  (the terms in brackets: reconstruction
//             loss only).
// Same mapping as the MLP kernel: four waves, three passes over the tiles, W and W' as
// bf16 hi + lo parts in the products that form W' and dQ.
constexpr int kLW = 0, kLWlo = kMatB, kLX = 2 * kMatB, kLXlo = 3 * kMatB, kLMatsB = 4 * kMatB;

template <bool kTok, bool kDot>
__global__ __launch_bounds__(64 * kWaves) void linear_nc_bwd_mfma_kernel(NcBwdMfmaArgs a) {
  __shared__ __attribute__((aligned(16))) char mats_mem[kLMatsB];
  __shared__ __attribute__((aligned(16))) char tiles_mem[kWaves * kWaveB];
  __shared__ __attribute__((aligned(16))) float acc_mem[kD * kAccRow];
  lds_char* mats = (lds_char*)(mats_mem);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  lds_char* my = (lds_char*)(tiles_mem) + wv * kWaveB;
  lds_float* acc = (lds_float*)(acc_mem);  // G, then P (+ dW), rows i, cols j
  const int chain = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 4, x = lane & 15;
  const int bi = chain / a.H, hi = chain - bi * a.H;
  const int T = a.T;
  const int ntiles = (T + kT - 1) / kT;
  const float eta = a.eta;
  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * kD;
  const char* q = reinterpret_cast<const char*>(static_cast<const bf16*>(a.q) + tok0);
  const char* k = reinterpret_cast<const char*>(static_cast<const bf16*>(a.k) + tok0);
  const char* v = reinterpret_cast<const char*>(static_cast<const bf16*>(a.v) + tok0);
  const char* dz = reinterpret_cast<const char*>(static_cast<const bf16*>(a.dz) + tok0);
  const char* dq = reinterpret_cast<const char*>(static_cast<bf16*>(a.dq) + tok0);
  const char* dk = reinterpret_cast<const char*>(static_cast<bf16*>(a.dk) + tok0);
  const char* dv = reinterpret_cast<const char*>(static_cast<bf16*>(a.dv) + tok0);
  const float* etok = kTok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
  float* detok = kTok && a.deta_tok ? a.deta_tok + static_cast<size_t>(chain) * T : nullptr;
  const size_t dd = static_cast<size_t>(kD) * kD;
  const float* wg = a.w1 + bi * a.w_batch_stride + static_cast<long long>(hi) * dd;
  const float* up = a.dw1_out ? a.dw1_out + static_cast<size_t>(chain) * dd : nullptr;
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  constexpr int kPer = kD * kD / 4 / (64 * kWaves);
  typedef __attribute__((address_space(3))) float4_t lds_f4;

  // ---- W as bf16 hi + lo; zero the accumulator ----
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int p = tid + i * 64 * kWaves, r = p >> 4, c = 4 * (p & 15);
    u32x2 h, l;
    split4(*reinterpret_cast<const float4_t*>(wg + r * kD + c), h, l);
    lds_st<u32x2>(mats + kLW + sw(r, c), h);
    lds_st<u32x2>(mats + kLWlo + sw(r, c), l);
    *reinterpret_cast<lds_f4*>(acc + r * kAccRow + c) = zero;
  }
  __syncthreads();
  const lds_char* mW = mats + kLW;
  const lds_char* mWlo = mats + kLWlo;

  // acc += the four waves' tiles (rows 16 rt + 4 g + e, cols 16 ct + x); see the MLP kernel
  auto reduce = [&](const float4_t (&t)[4][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < 16; ++f) reinterpret_cast<lds_f4*>(my)[f * 64 + lane] = t[f >> 2][f & 3];
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int f = 4 * wv + ct;
      float4_t sum = zero;
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2)
        sum += reinterpret_cast<const lds_f4*>((lds_char*)(tiles_mem) + w2 * kWaveB)[f * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[(16 * wv + 4 * g + e) * kAccRow + 16 * ct + x] += sum[e];
    }
    __syncthreads();
  };
  // R^T (rows i, cols t) = W K^T - V^T (or -V^T); Rt rows to my + kRt
  auto fwd_r = [&](float4_t (&r)[4], float et, auto split_c) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      r[it] = zero;
      if constexpr (!kDot) {
        r[it] = mm(mW, 16 * it, my + kIn1, 0, g, x, zero);
        if constexpr (decltype(split_c)::value) r[it] = mm(mWlo, 16 * it, my + kIn1, 0, g, x, r[it]);
      }
      r[it] -= unpack4(lds_ld<u32x2>(my + kIn2 + sw(x, 16 * it + 4 * g)));
      lds_st<u32x2>(my + kRt + sw(x, 16 * it + 4 * g), pack4(r[it] * et));
    }
  };

  // ================= pass 1 (keys): G = Rt^T K
  {
    float4_t gs[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) gs[i][j] = zero;
    In cur = load_in<kTok>(k, v, etok, wv, T, lane);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int tt = wv + kWaves * i;
      put_in(cur, my + kIn1, my + kIn2, lane);
      const In nxt = load_in<kTok>(k, v, etok, tt + kWaves, T, lane);
      __builtin_amdgcn_sched_barrier(0);
      if (tt < ntiles) {
        float4_t r[4];
        fwd_r(r, cur.e, std::true_type{});
        bf16x8_t kop[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) kop[jt] = tokop(my + kIn1, 16 * jt, g, x);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const bf16x8_t rop = tokop(my + kRt, 16 * it, g, x);
#pragma unroll
          for (int jt = 0; jt < 4; ++jt) gs[it][jt] = mfma(rop, kop[jt], gs[it][jt]);
        }
      }
      cur = nxt;
    }
    reduce(gs);
  }
  // ---- W' = W - eta G (bf16 hi + lo); the accumulator restarts from the upstream gradient ----
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int p = tid + i * 64 * kWaves, r = p >> 4, c = 4 * (p & 15);
    auto* a1 = reinterpret_cast<lds_f4*>(acc + r * kAccRow + c);
    u32x2 h, l;
    split4(*reinterpret_cast<const float4_t*>(wg + r * kD + c) - eta * *a1, h, l);
    lds_st<u32x2>(mats + kLX + sw(r, c), h);
    lds_st<u32x2>(mats + kLXlo + sw(r, c), l);
    *a1 = up ? *reinterpret_cast<const float4_t*>(up + r * kD + c) : zero;
  }
  __syncthreads();

  // ================= pass 2 (queries): dQ = dZ W', P += dZ^T Q
  {
    const lds_char* mWp = mats + kLX;
    const lds_char* mWplo = mats + kLXlo;
    float4_t ps[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) ps[i][j] = zero;
    In cur = load_in<false>(q, dz, nullptr, wv, T, lane);
    u32x2 dqv[4];
    int pend = -1;
    auto store_dq = [&](int tt) __attribute__((always_inline)) {
      const __amdgpu_buffer_rsrc_t rd = rsrc(dq + tt * kTileB, T * kRow - tt * kTileB);
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
        __builtin_amdgcn_raw_buffer_store_b64(dqv[jt], rd, x * kRow + 2 * (16 * jt + 4 * g), 0, 0);
    };
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int tt = wv + kWaves * i;
      put_in(cur, my + kIn1, my + kIn2, lane);  // Q, dZ
      if (pend >= 0) store_dq(pend);
      pend = -1;
      const In nxt = load_in<false>(q, dz, nullptr, tt + kWaves, T, lane);
      __builtin_amdgcn_sched_barrier(0);
      if (tt < ntiles) {
        // dQ^T (rows j, cols t) = sum_i W'[i][j] dZ[t][i]
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
          dqv[jt] = pack4(mm_t(mWplo, 16 * jt, my + kIn2, 0, g, x, mm_t(mWp, 16 * jt, my + kIn2, 0, g, x, zero)));
        pend = tt;
        // P (rows i, cols j) += dZ^T Q
        bf16x8_t qop[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) qop[jt] = tokop(my + kIn1, 16 * jt, g, x);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const bf16x8_t zop = tokop(my + kIn2, 16 * it, g, x);
#pragma unroll
          for (int jt = 0; jt < 4; ++jt) ps[it][jt] = mfma(zop, qop[jt], ps[it][jt]);
        }
      }
      cur = nxt;
    }
    if (pend >= 0) store_dq(pend);
    reduce(ps);
  }
  // ---- S = -eta P (bf16); the accumulator keeps P ----
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int p = tid + i * 64 * kWaves, r = p >> 4, c = 4 * (p & 15);
    lds_st<u32x2>(mats + kLX + sw(r, c), pack4(-eta * *reinterpret_cast<lds_f4*>(acc + r * kAccRow + c)));
  }
  __syncthreads();

  // ================= pass 3 (keys): dK, dV, de, dW += dR^T K
  {
    const lds_char* mS = mats + kLX;
    float4_t hs[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) hs[i][j] = zero;
    In cur = load_in<kTok>(k, v, etok, wv, T, lane);
    u32x2 dkv[4], dvv[4];
    float dev = 0.0f;
    int pend = -1;
    auto store_out = [&](int tt) __attribute__((always_inline)) {
      const int off = tt * kTileB, left = T * kRow - off;
      const __amdgpu_buffer_rsrc_t rk = rsrc(dk + off, left), rv = rsrc(dv + off, left);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        __builtin_amdgcn_raw_buffer_store_b64(dkv[c], rk, x * kRow + 2 * (16 * c + 4 * g), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(dvv[c], rv, x * kRow + 2 * (16 * c + 4 * g), 0, 0);
      }
      if (kTok && detok) {  // the four lane groups store the same value
        const __amdgpu_buffer_rsrc_t re = rsrc(detok + tt * kT, 4 * (T - tt * kT));
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, dev), re, 4 * x, 0, 0);
      }
    };
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int tt = wv + kWaves * i;
      put_in(cur, my + kIn1, my + kIn2, lane);  // K, V
      if (pend >= 0) store_out(pend);
      pend = -1;
      const In nxt = load_in<kTok>(k, v, etok, tt + kWaves, T, lane);
      __builtin_amdgcn_sched_barrier(0);
      if (tt < ntiles) {
        const float et = cur.e;
        float4_t r[4];
        fwd_r(r, et, std::false_type{});
        // dRt^T (rows i, cols t) = sum_j S[i][j] K[t][j]; de; dR = e dRt; dV = -dR
        float dpart = 0.0f;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const float4_t drt = mm(mS, 16 * it, my + kIn1, 0, g, x, zero);
          if constexpr (kTok) {
#pragma unroll
            for (int e = 0; e < 4; ++e) dpart += drt[e] * r[it][e];
          }
          const float4_t dr = drt * et;
          dvv[it] = pack4(-dr);
          if constexpr (!kDot) lds_st<u32x2>(my + kDR + sw(x, 16 * it + 4 * g), pack4(dr));
        }
        if constexpr (kTok) {
          dpart += __shfl_xor(dpart, 16, 64);
          dpart += __shfl_xor(dpart, 32, 64);
          dev = dpart;
        }
        // dK^T (rows j, cols t) = sum_i S[i][j] Rt[t][i] (+ sum_i W[i][j] dR[t][i])
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          float4_t dkt = mm_t(mS, 16 * jt, my + kRt, 0, g, x, zero);
          if constexpr (!kDot) dkt = mm_t(mW, 16 * jt, my + kDR, 0, g, x, dkt);
          dkv[jt] = pack4(dkt);
        }
        pend = tt;
        // dW (rows i, cols j) += dR^T K
        if constexpr (!kDot) {
          bf16x8_t kop[4];
#pragma unroll
          for (int jt = 0; jt < 4; ++jt) kop[jt] = tokop(my + kIn1, 16 * jt, g, x);
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            const bf16x8_t dop = tokop(my + kDR, 16 * it, g, x);
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) hs[it][jt] = mfma(dop, kop[jt], hs[it][jt]);
          }
        }
      }
      cur = nxt;
    }
    if (pend >= 0) store_out(pend);
    reduce(hs);
  }
  // ---- dW0 = P + dR^T K ----
  float* dw0 = a.dw1 + static_cast<size_t>(chain) * dd;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int p = tid + i * 64 * kWaves, r = p >> 4, c = 4 * (p & 15);
    *reinterpret_cast<float4_t*>(dw0 + r * kD + c) = *reinterpret_cast<lds_f4*>(acc + r * kAccRow + c);
  }
}

}  // namespace

bool mlp_nc_bwd_mfma_supported(const void* q, const void* k, const void* v, const void* dz,
                               const float* w1, const float* w2, long long w_batch_stride,
                               const float* dw1_out, const float* dw2_out, const void* dq,
                               const void* dk, const void* dv, const float* dw1, const float* dw2,
                               int T, int d, int h, int chunk, int epochs, bool bf16_io) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool aligned = al(q) && al(k) && al(v) && al(dz) && al(dq) && al(dk) && al(dv) && al(w1) &&
                       al(w2) && al(dw1) && al(dw2) && (!dw1_out || al(dw1_out)) &&
                       (!dw2_out || al(dw2_out)) && (w_batch_stride % 4) == 0;
  // below one full tile the sums have too few terms to average out the bf16 operand
  // roundings (a single token's rank-1 update passes them on whole); the fp32 path serves those
  return bf16_io && d == kD && h == kD && T >= kT && T <= kMaxTokens && chunk >= T && epochs == 1 &&
         aligned;
}

bool linear_nc_bwd_mfma_supported(const void* q, const void* k, const void* v, const void* dz,
                                  const float* w0, long long w_batch_stride, const float* dw_out,
                                  const void* dq, const void* dk, const void* dv, const float* dw0,
                                  int T, int d, int chunk, int epochs, bool bf16_io) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool aligned = al(q) && al(k) && al(v) && al(dz) && al(dq) && al(dk) && al(dv) && al(w0) &&
                       al(dw0) && (!dw_out || al(dw_out)) && (w_batch_stride % 4) == 0;
  return bf16_io && d == kD && T >= kT && T <= kMaxTokens && chunk >= T && epochs == 1 && aligned;
}

hipError_t launch_linear_nc_bwd_mfma(const void* q, const void* k, const void* v, const void* dz,
                                     const float* w0, long long w_batch_stride, const float* dw_out,
                                     const float* eta_tok, void* dq, void* dk, void* dv, float* dw0,
                                     float* deta_tok, int B, int H, int T, float eta, int dot_loss,
                                     hipStream_t s) {
  const long long nchains = static_cast<long long>(B) * H;
  if (nchains > 0x7fffffffLL || T <= 0 || T > kMaxTokens) return hipErrorInvalidValue;
  NcBwdMfmaArgs a{q, k, v, dz, w0, nullptr, w_batch_stride, dw_out, nullptr, eta_tok, dq, dk, dv,
                  dw0, nullptr, deta_tok, B, H, T, eta};
  const dim3 grid(static_cast<unsigned>(nchains)), block(64 * kWaves);
  auto run = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, a);
    return hipGetLastError();
  };
  if (eta_tok && dot_loss) return run(linear_nc_bwd_mfma_kernel<true, true>);
  if (eta_tok) return run(linear_nc_bwd_mfma_kernel<true, false>);
  if (dot_loss) return run(linear_nc_bwd_mfma_kernel<false, true>);
  return run(linear_nc_bwd_mfma_kernel<false, false>);
}

hipError_t launch_mlp_nc_bwd_mfma(const void* q, const void* k, const void* v, const void* dz,
                                  const float* w1, const float* w2, long long w_batch_stride,
                                  const float* dw1_out, const float* dw2_out, const float* eta_tok,
                                  void* dq, void* dk, void* dv, float* dw1, float* dw2,
                                  float* deta_tok, int B, int H, int T, float eta, int dot_loss,
                                  hipStream_t s) {
  const long long nchains = static_cast<long long>(B) * H;
  if (nchains > 0x7fffffffLL || T <= 0 || T > kMaxTokens) return hipErrorInvalidValue;
  NcBwdMfmaArgs a{q, k, v, dz, w1, w2, w_batch_stride, dw1_out, dw2_out, eta_tok, dq, dk, dv,
                  dw1, dw2, deta_tok, B, H, T, eta};
  const dim3 grid(static_cast<unsigned>(nchains)), block(64 * kWaves);
  auto run = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, a);
    return hipGetLastError();
  };
  if (eta_tok && dot_loss) return run(mlp_nc_bwd_mfma_kernel<true, true>);
  if (eta_tok) return run(mlp_nc_bwd_mfma_kernel<true, false>);
  if (dot_loss) return run(mlp_nc_bwd_mfma_kernel<false, true>);
  return run(mlp_nc_bwd_mfma_kernel<false, false>);
}

}  // namespace ttt
