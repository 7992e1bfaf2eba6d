// Non-causal TTT-MLP forward on the gfx950 matrix cores: f(k) = W2 SiLU(W1 k), d = 64,
// hidden 64, bf16 Q/K/V/Z, fp32 state; one full-batch step, or several consecutive
// mini-batches and epochs.
//
// Method (ViT3 news page, section 1, inner training setup: the keys and values are a small
// training set, one full-batch gradient step, then the trained inner model is applied to
// every query; inner model: section 2, 2-layer SiLU MLP).  With U = K W1^T, A = SiLU(U),
// S = SiLU'(U), R = A W2^T - V and dU = (R W2) * S over all N tokens:
//   W1' = W1 - eta dU^T K,   W2' = W2 - eta R^T A,   Z = SiLU(Q W1'^T) W2'^T.
// With per-token rates each row t of R (and so of dU) is scaled by token t's rate factor
// ("Fast weights" page, opening formula; wmrh.cn summary, section 2.2.3).  With the
// negative dot-product loss -v^T f(k), the ViT3 page's own inner loss (section 2), R = -V.
// The same page (observation 2 and its figure on inner batch size and epochs) also splits
// the N pairs into consecutive mini-batches, one update each, and repeats the pass for
// several epochs: every step takes its gradients at the weights the previous step left.
//
// Mapping.  One workgroup of kNcWaves = 2 waves per (batch, head) chain; wave w takes the
// 16-token tiles w, w + 2, w + 4, ...  Pass 1 streams its tiles (the next tile's loads are
// issued before the current tile is computed) and accumulates the partial gradient sums
// G1^T = K^T dU and G2^T = A^T R in fp32 MFMA accumulator tiles, while W1, W2 stay fixed
// as bf16 operands (W2 in both orientations: the forward pass contracts it over hidden
// units, the backward pass over outputs).  The partial sums meet once in LDS: wave w adds
// up half of the tiles, forms W' = W - eta G there, and both waves read all of W1', W2'
// back (between steps through the LDS copy of the weights, which the next step's operands
// are built from).  Pass 2 streams the wave's query tiles.  With 768 waves for 384 chains every wave
// keeps a SIMD to itself.  Tokens past N (the last tile) read as zero and contribute
// nothing (no bias, SiLU(0) = 0); their outputs are not stored.  Layouts follow the causal MLP
// kernel: 16 x 16 C-layout tiles, the input index j permuted as j = 16 (m/4) + 2 (m%4) +
// 8h + p in W1^T tile 2h+p so that operands over j match 16-byte row loads of K and Q, and
// hidden / output indices natural.
#include "common.hpp"

namespace ttt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 64;
constexpr int kH = 64;
constexpr int kTile = 16;
constexpr int kRowBytes = kD * 2;  // one token row of K, V, Q or Z
constexpr int kTileBytes = kTile * kRowBytes;

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
__device__ __forceinline__ bf16x8_t pair_op(const float4_t& x, const float4_t& y) {
  return op4(pack_bf16(x[0], y[0]), pack_bf16(x[1], y[1]), pack_bf16(x[2], y[2]), pack_bf16(x[3], y[3]));
}
__device__ __forceinline__ bf16x8_t pad_op(const float4_t& x) {
  return op4(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), 0u, 0u);
}
__device__ __forceinline__ float4_t mfma(const bf16x8_t& a, const bf16x8_t& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float sigmoid_f(float u) { return sigmoidf_(u); }
__device__ __forceinline__ float bf_lo(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __builtin_bit_cast(float, x & 0xFFFF0000u); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int left) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, left > 0 ? left : 0,
                                           0x00020000);
}

// W1^T tiles [jb][a] (rows j permuted, cols hidden 16a + n) from W1 [hidden][d] fp32 with
// rows kWRow floats apart (the LDS copy)
__device__ __forceinline__ void load_w1t(float4_t (&w)[4][4], const float* w1, int g, int n) {
#pragma unroll
  for (int aa = 0; aa < 4; ++aa) {
    const float* wr = w1 + (16 * aa + n) * (kD + 4) + 16 * g;
    const float4_t f0 = *reinterpret_cast<const float4_t*>(wr);
    const float4_t f1 = *reinterpret_cast<const float4_t*>(wr + 4);
    const float4_t f2 = *reinterpret_cast<const float4_t*>(wr + 8);
    const float4_t f3 = *reinterpret_cast<const float4_t*>(wr + 12);
    w[0][aa] = float4_t{f0[0], f0[2], f1[0], f1[2]};
    w[1][aa] = float4_t{f0[1], f0[3], f1[1], f1[3]};
    w[2][aa] = float4_t{f2[0], f2[2], f3[0], f3[2]};
    w[3][aa] = float4_t{f2[1], f2[3], f3[1], f3[3]};
  }
}
// W2^T tiles [a][it] (rows hidden 16a + m, cols output 16it + n) from W2 [d][hidden] with
// rows kWRow floats apart (the LDS copy)
__device__ __forceinline__ void load_w2t(float4_t (&w)[4][4], const float* w2, int g, int n) {
#pragma unroll
  for (int aa = 0; aa < 4; ++aa)
#pragma unroll
    for (int it = 0; it < 4; ++it)
      w[aa][it] = *reinterpret_cast<const float4_t*>(w2 + (16 * it + n) * (kH + 4) + 16 * aa + 4 * g);
}

constexpr int kNcWaves = 2;

// One tile's key-side operands of a lane.
struct KvTile {
  u32x4 ka0, ka1;     // K[t = n][16 g + 0..7], K[n][16 g + 8..15]
  uint32_t kt[4][2];  // kt[e][h] = K[4 g + e][c0 + 8 h .. + 1]
  u32x2 vv[4];        // V[t = n][16 it + 4 g .. + 3]
  float et;           // rate factor of token n (1 without per-token rates)
};
template <bool kTok>
__device__ __forceinline__ void load_kv(KvTile& r, const char* k, const char* v, const float* etok, int tt,
                                        int seq_bytes, int row, const int (&kto)[4], int g, int n) {
  const int off = tt * kTileBytes;
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(k + off, seq_bytes - off);
  const __amdgpu_buffer_rsrc_t rv = tile_rsrc(v + off, seq_bytes - off);
  r.ka0 = __builtin_amdgcn_raw_buffer_load_b128(rk, row, 0, 0);
  r.ka1 = __builtin_amdgcn_raw_buffer_load_b128(rk, row + 16, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r.kt[e][0] = __builtin_amdgcn_raw_buffer_load_b32(rk, kto[e], 0, 0);
    r.kt[e][1] = __builtin_amdgcn_raw_buffer_load_b32(rk, kto[e] + 16, 0, 0);
  }
#pragma unroll
  for (int it = 0; it < 4; ++it)
    r.vv[it] = __builtin_amdgcn_raw_buffer_load_b64(rv, n * 128 + 2 * (16 * it + 4 * g), 0, 0);
  r.et = 1.0f;
  if (kTok) {  // 4 bytes per token, zero past the end
    const __amdgpu_buffer_rsrc_t re = tile_rsrc(etok + tt * kTile, (seq_bytes >> 5) - tt * kTile * 4);
    r.et = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(re, n * 4, 0, 0));
  }
}

// fp32 weight rows staged in LDS, padded to 68 floats so that the 16-byte reads of 16
// lanes in 16 consecutive rows spread over the banks
constexpr int kWRow = kD + 4;
// The tiles stream through register rings that are unrolled, with every load issued
// unconditionally (past the end of a step a tile reads zero and adds nothing) and scheduling
// barriers between the ring slots: a register copy of a tile still in flight, a load issued
// on one path only, or a product hoisted above another slot's loads would each make the
// wave wait for more loads than the tile it needs.
template <bool kDot, bool kTok>
__global__ __launch_bounds__(64 * kNcWaves) __attribute__((amdgpu_waves_per_eu(1, 1))) void mlp_nc_kernel(MlpArgs a) {
  // partial gradient tiles [wave][tile f][lane], then the trained tiles in [0][f][lane]
  __shared__ float4_t red[kNcWaves][16][64];
  // the head's initial W1 [hidden][d] and W2 [d][hidden], read from global memory once per
  // workgroup
  __shared__ __attribute__((aligned(16))) float wsh[2][kH][kWRow];
  const int chain = blockIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int bi = chain / a.H;
  const int hi = chain - bi * a.H;
  const int T = a.T;
  const int ntiles = (T + kTile - 1) / kTile;
  const int seq_bytes = T * kD * 2;
  const float eta = a.eta;

  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * kD;
  const char* q = reinterpret_cast<const char*>(static_cast<const bf16*>(a.q) + tok0);
  const char* k = reinterpret_cast<const char*>(static_cast<const bf16*>(a.k) + tok0);
  const char* v = reinterpret_cast<const char*>(static_cast<const bf16*>(a.v) + tok0);
  char* z = reinterpret_cast<char*>(static_cast<bf16*>(a.z) + tok0);
  const float* etok = kTok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
  const size_t hd = static_cast<size_t>(kH) * kD;
  const float* w1g = a.w1 + bi * a.w_batch_stride + static_cast<long long>(hi) * hd;
  const float* w2g = a.w2 + bi * a.w_batch_stride + static_cast<long long>(hi) * hd;

  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  constexpr uint32_t kLo = 0x05040100u, kHi = 0x07060302u;
  const uint32_t one = 0x3F80u;  // bf16 1.0
  const bf16x8_t eye = op4((4 * g + 0 == n ? one : 0u) | (4 * g + 1 == n ? one << 16 : 0u),
                           (4 * g + 2 == n ? one : 0u) | (4 * g + 3 == n ? one << 16 : 0u), 0u, 0u);
  const int row = n * 128 + 32 * g;  // K / Q operand rows (16 bytes at +0 and +16)
  const int c0 = 16 * (n >> 2) + 2 * (n & 3);
  int kto[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) kto[e] = (4 * g + e) * 128 + 2 * c0;

  // Training steps: `epochs` passes over the mini-batches [m0, m0 + b) of b = min(chunk, T)
  // tokens (the last one may be shorter).  A step streams only its own tokens: its tiles
  // are addressed from the mini-batch start and bounded by its end, so a tile's rows past
  // the mini-batch read as zero and add nothing to the sums.
  const int mb = min(a.chunk, T);
  const int nmb = (T + mb - 1) / mb;
  const int nsteps = nmb * a.epochs;
  int m0 = 0;                                // first token of the current step
  int ns = mb;                               // its tokens
  int ntl = (ns + kTile - 1) / kTile;        // its tiles

  // ring of four K/V tiles: slot x holds this wave's tile tt + x kNcWaves of the step
  constexpr int kRing = 4;
  KvTile ring[kRing];
  auto prefetch = [&](int start, int len) {  // this wave's first tiles of a step
    const char* ks = k + start * kRowBytes;
    const char* vs = v + start * kRowBytes;
    const float* es = kTok ? etok + start : nullptr;
#pragma unroll
    for (int x = 0; x < kRing; ++x) {
      load_kv<kTok>(ring[x], ks, vs, es, wv + x * kNcWaves, len * kRowBytes, row, kto, g, n);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  {
    // W1 and W2 (64 x 64 fp32 each) into LDS: thread x copies 16-byte pieces x, x + 128, ...
    // The global loads are issued before the first K/V tiles, so that the wait for them
    // leaves the tiles in flight.
    constexpr int kPer = kH * kD / 4 / (64 * kNcWaves);
    const int tid = threadIdx.x;
    float4_t wv4[2][kPer];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float* src = m ? w2g : w1g;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int x = tid + i * 64 * kNcWaves;
        wv4[m][i] = *reinterpret_cast<const float4_t*>(src + (x >> 4) * kD + (x & 15) * 4);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    prefetch(m0, ns);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int x = tid + i * 64 * kNcWaves;
        *reinterpret_cast<float4_t*>(&wsh[m][x >> 4][(x & 15) * 4]) = wv4[m][i];
      }
  }
  __syncthreads();
  float* w1l = &wsh[0][0][0];
  float* w2l = &wsh[1][0][0];

  bf16x8_t w1b[2][4];   // [h][a]: operand over j (B of K W1^T)
  bf16x8_t w2tb[2][4];  // [h][it]: operand over hidden (A of W2 A^T)
  bf16x8_t w2b[2][4];   // [h][a]: operand over outputs (B of R W2)
  // this wave's half of the W tiles, for W' = W - eta G after pass 1 (tile f = 4 x + y of
  // the [x][y] tile arrays, f in 8 w .. 8 w + 7)
  float4_t w1own[2][4], w2own[2][4];
  // ring of four query tiles for pass 2 (loaded while the last step's sums are reduced)
  u32x4 qa[kRing][2];
  auto load_q = [&](u32x4 (&dst)[2], int tt) {
    const int off = tt * kTileBytes;
    const __amdgpu_buffer_rsrc_t rq = tile_rsrc(q + off, seq_bytes - off);
    dst[0] = __builtin_amdgcn_raw_buffer_load_b128(rq, row, 0, 0);
    dst[1] = __builtin_amdgcn_raw_buffer_load_b128(rq, row + 16, 0, 0);
  };
  for (int step = 0;; ++step) {
    // ---- bf16 operands of the current weights (the LDS copy) ----
    {
      float4_t t[4][4];
      load_w1t(t, w1l, g, n);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int aa = 0; aa < 4; ++aa) w1b[h][aa] = pair_op(t[2 * h][aa], t[2 * h + 1][aa]);
      load_w2t(t, w2l, g, n);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int it = 0; it < 4; ++it) w2tb[h][it] = pair_op(t[2 * h][it], t[2 * h + 1][it]);
      // W2 tiles [it][a]: rows output 16it + m, cols hidden 16a + n
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int aa = 0; aa < 4; ++aa) {
          float4_t x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = w2l[(16 * it + 4 * g + e) * kWRow + 16 * aa + n];
          t[it][aa] = x;
        }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int aa = 0; aa < 4; ++aa) w2b[h][aa] = pair_op(t[2 * h][aa], t[2 * h + 1][aa]);
    }

    // ---- pass 1: partial gradient sums over this wave's tiles of the step ----
    float4_t g1t[4][4];  // sum of K^T dU, layout of W1^T
    float4_t g2t[4][4];  // sum of A^T R, layout of W2^T
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        g1t[i][j] = zero;
        g2t[i][j] = zero;
      }
    const char* ks = k + m0 * kRowBytes;
    const char* vs = v + m0 * kRowBytes;
    const float* es = kTok ? etok + m0 : nullptr;
    for (int tt0 = wv; tt0 < ntl; tt0 += kRing * kNcWaves) {
#pragma unroll
    for (int x = 0; x < kRing; ++x) {
    if (tt0 + x * kNcWaves < ntl) {
      const KvTile& cur = ring[x];
      const bf16x8_t ka0 = bf(cur.ka0), ka1 = bf(cur.ka1);
      // U = K W1^T (rows t); A = SiLU(U), S = SiLU'(U)
      float4_t act[4], sd[4];
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        float4_t u = mfma(ka0, w1b[0][aa], zero);
        u = mfma(ka1, w1b[1][aa], u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sg = sigmoid_f(u[e]);
          act[aa][e] = u[e] * sg;
          sd[aa][e] = sg * (1.0f + u[e] * (1.0f - sg));
        }
      }
      // A^T (rows hidden)
      float4_t actT[4];
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) actT[aa] = mfma(pad_op(act[aa]), eye, zero);
      const bf16x8_t atb0 = pair_op(actT[0], actT[1]), atb1 = pair_op(actT[2], actT[3]);
      // R^T = W2 A^T - V^T (rows output tile it, cols t), times the rate factor of token t
      // (its gradients carry its own rate)
      float4_t rT[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        float4_t o = zero;  // the dot-product loss's error term is -V alone
        if (!kDot) {
          o = mfma(w2tb[0][it], atb0, zero);
          o = mfma(w2tb[1][it], atb1, o);
        }
        o[0] -= bf_lo(cur.vv[it].x);
        o[1] -= bf_hi(cur.vv[it].x);
        o[2] -= bf_lo(cur.vv[it].y);
        o[3] -= bf_hi(cur.vv[it].y);
        rT[it] = o * cur.et;
      }
      // dU = (R W2) * S (rows t): A-operand R (m = t, k = output) from pairs of R^T tiles
      const bf16x8_t rrow0 = pair_op(rT[0], rT[1]), rrow1 = pair_op(rT[2], rT[3]);
      bf16x8_t dub[4];
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        float4_t da = mfma(rrow0, w2b[0][aa], zero);
        da = mfma(rrow1, w2b[1][aa], da);
        dub[aa] = pad_op(da * sd[aa]);
      }
      // R (rows t) from R^T by an MFMA with I, as padded operands
      bf16x8_t rb[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) rb[it] = pad_op(mfma(pad_op(rT[it]), eye, zero));
      // G1^T += K^T dU ; G2^T += A^T R
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const int h = jb >> 1;
        const uint32_t sel = (jb & 1) ? kHi : kLo;
        const bf16x8_t ktb = op4(__builtin_amdgcn_perm(cur.kt[1][h], cur.kt[0][h], sel),
                                 __builtin_amdgcn_perm(cur.kt[3][h], cur.kt[2][h], sel), 0u, 0u);
#pragma unroll
        for (int aa = 0; aa < 4; ++aa) g1t[jb][aa] = mfma(ktb, dub[aa], g1t[jb][aa]);
      }
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        const bf16x8_t ab = pad_op(act[aa]);
#pragma unroll
        for (int it = 0; it < 4; ++it) g2t[aa][it] = mfma(ab, rb[it], g2t[aa][it]);
      }
    }
    load_kv<kTok>(ring[x], ks, vs, es, tt0 + (x + kRing) * kNcWaves, ns * kRowBytes, row, kto, g, n);
    __builtin_amdgcn_sched_barrier(0);
    }
    }

    const bool last = step + 1 == nsteps;
    if (last) {
      // the queries of this wave's first tiles, loaded while the sums are reduced
#pragma unroll
      for (int x = 0; x < kRing; ++x) {
        load_q(qa[x], wv + x * kNcWaves);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // the next step's first tiles, loaded while the sums are reduced
      m0 = ((step + 1) % nmb) * mb;
      ns = min(mb, T - m0);
      ntl = (ns + kTile - 1) / kTile;
      prefetch(m0, ns);
    }

    // ---- W -= eta G: the partial sums meet in LDS; wave w reduces tiles 8 w .. 8 w + 7 ----
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      const float* wr = w1l + (16 * aa + n) * kWRow + 16 * g + 8 * wv;
      const float4_t f0 = *reinterpret_cast<const float4_t*>(wr);
      const float4_t f1 = *reinterpret_cast<const float4_t*>(wr + 4);
      w1own[0][aa] = float4_t{f0[0], f0[2], f1[0], f1[2]};
      w1own[1][aa] = float4_t{f0[1], f0[3], f1[1], f1[3]};
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int it = 0; it < 4; ++it)
        w2own[x][it] = *reinterpret_cast<const float4_t*>(w2l + (16 * it + n) * kWRow + 16 * (2 * wv + x) + 4 * g);
#pragma unroll
    for (int f = 0; f < 16; ++f) red[wv][f][lane] = g1t[f >> 2][f & 3];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int f = 8 * wv + i;
      float4_t sum = red[0][f][lane];
#pragma unroll
      for (int w = 1; w < kNcWaves; ++w) sum += red[w][f][lane];
      w1own[i >> 2][i & 3] -= eta * sum;
    }
    __syncthreads();  // every partial read before the W2 partials overwrite the slots
#pragma unroll
    for (int f = 0; f < 16; ++f) red[wv][f][lane] = g2t[f >> 2][f & 3];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int f = 8 * wv + i;
      float4_t sum = red[0][f][lane];
#pragma unroll
      for (int w = 1; w < kNcWaves; ++w) sum += red[w][f][lane];
      w2own[i >> 2][i & 3] -= eta * sum;
    }
    __syncthreads();  // every partial read before slot 0 is reused
    if (last) break;
    // the updated tiles back into the LDS copy, from which the next step builds its
    // operands (the inverse of the reads above; the two waves cover all 64 x 64 entries)
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      float* wr = w1l + (16 * aa + n) * kWRow + 16 * g + 8 * wv;
      const float4_t o0 = w1own[0][aa], o1 = w1own[1][aa];
      *reinterpret_cast<float4_t*>(wr) = float4_t{o0[0], o1[0], o0[1], o1[1]};
      *reinterpret_cast<float4_t*>(wr + 4) = float4_t{o0[2], o1[2], o0[3], o1[3]};
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int it = 0; it < 4; ++it)
        *reinterpret_cast<float4_t*>(w2l + (16 * it + n) * kWRow + 16 * (2 * wv + x) + 4 * g) = w2own[x][it];
    __syncthreads();
  }

  // ---- the trained tiles to both waves (and to w1_out / w2_out) ----
  bf16x8_t w1nb[2][4], w2nb[2][4];
  {
    float4_t t[4][4];
    // W1
#pragma unroll
    for (int i = 0; i < 8; ++i) red[0][8 * wv + i][lane] = w1own[i >> 2][i & 3];
    __syncthreads();
#pragma unroll
    for (int f = 0; f < 16; ++f) t[f >> 2][f & 3] = red[0][f][lane];
    if (a.w1_out && wv == 0) {
      float* o1 = a.w1_out + static_cast<size_t>(chain) * hd;
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        float* wr = o1 + (16 * aa + n) * kD + 16 * g;
        *reinterpret_cast<float4_t*>(wr) = float4_t{t[0][aa][0], t[1][aa][0], t[0][aa][1], t[1][aa][1]};
        *reinterpret_cast<float4_t*>(wr + 4) = float4_t{t[0][aa][2], t[1][aa][2], t[0][aa][3], t[1][aa][3]};
        *reinterpret_cast<float4_t*>(wr + 8) = float4_t{t[2][aa][0], t[3][aa][0], t[2][aa][1], t[3][aa][1]};
        *reinterpret_cast<float4_t*>(wr + 12) = float4_t{t[2][aa][2], t[3][aa][2], t[2][aa][3], t[3][aa][3]};
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) w1nb[h][aa] = pair_op(t[2 * h][aa], t[2 * h + 1][aa]);
    __syncthreads();  // every read of the W1 tiles before slot reuse
    // W2
#pragma unroll
    for (int i = 0; i < 8; ++i) red[0][8 * wv + i][lane] = w2own[i >> 2][i & 3];
    __syncthreads();
#pragma unroll
    for (int f = 0; f < 16; ++f) t[f >> 2][f & 3] = red[0][f][lane];
    if (a.w2_out && wv == 0) {
      float* o2 = a.w2_out + static_cast<size_t>(chain) * hd;
#pragma unroll
      for (int aa = 0; aa < 4; ++aa)
#pragma unroll
        for (int it = 0; it < 4; ++it)
          *reinterpret_cast<float4_t*>(o2 + (16 * it + n) * kH + 16 * aa + 4 * g) = t[aa][it];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int it = 0; it < 4; ++it) w2nb[h][it] = pair_op(t[2 * h][it], t[2 * h + 1][it]);
  }

  // ---- pass 2: Z^T = W2' SiLU(W1' Q^T) over this wave's tiles ----
  for (int tt0 = wv; tt0 < ntiles; tt0 += kRing * kNcWaves) {
#pragma unroll
    for (int x = 0; x < kRing; ++x) {
      const int tt = tt0 + x * kNcWaves;
      if (tt < ntiles) {
        const bf16x8_t qb0 = bf(qa[x][0]), qb1 = bf(qa[x][1]);
        float4_t aq[4];
#pragma unroll
        for (int aa = 0; aa < 4; ++aa) {
          float4_t u = mfma(w1nb[0][aa], qb0, zero);
          u = mfma(w1nb[1][aa], qb1, u);
#pragma unroll
          for (int e = 0; e < 4; ++e) u[e] = u[e] * sigmoid_f(u[e]);
          aq[aa] = u;
        }
        const bf16x8_t aqb0 = pair_op(aq[0], aq[1]), aqb1 = pair_op(aq[2], aq[3]);
        const int off = tt * kTileBytes;
        const __amdgpu_buffer_rsrc_t rz = tile_rsrc(z + off, seq_bytes - off);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          float4_t zt = mfma(w2nb[0][it], aqb0, zero);
          zt = mfma(w2nb[1][it], aqb1, zt);
          const u32x2 out = {pack_bf16(zt[0], zt[1]), pack_bf16(zt[2], zt[3])};
          __builtin_amdgcn_raw_buffer_store_b64(out, rz, n * 128 + 2 * (16 * it + 4 * g), 0, 0);
        }
      }
      load_q(qa[x], tt + kRing * kNcWaves);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

}  // namespace

bool mlp_nc_supported(const MlpArgs& a, bool bf16_io) {
  auto al = [](const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & (m - 1)) == 0; };
  const bool aligned = al(a.q, 16) && al(a.k, 16) && al(a.v, 16) && al(a.z, 16) && al(a.w1, 16) &&
                       al(a.w2, 16) && (a.w_batch_stride % 4) == 0 &&
                       (a.w1_out == nullptr || al(a.w1_out, 16)) &&
                       (a.w2_out == nullptr || al(a.w2_out, 16));
  const bool fits = static_cast<long long>(a.T) * kD * 2 + 2LL * kTileBytes < 0x7fffffffLL;
  return bf16_io && a.d == kD && a.dh == kH && a.causal == 0 && a.T > 0 && a.epochs >= 1 && a.ln_w == nullptr &&
         aligned && fits && (a.eta_tok == nullptr || al(a.eta_tok, 4));
}

hipError_t launch_mlp_nc(const MlpArgs& a, hipStream_t s) {
  const long long nchains = static_cast<long long>(a.B) * a.H;
  if (nchains > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(nchains)), block(64 * kNcWaves);
  if (a.dot_loss) {
    if (a.eta_tok)
      hipLaunchKernelGGL((mlp_nc_kernel<true, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((mlp_nc_kernel<true, false>), grid, block, 0, s, a);
  } else {
    if (a.eta_tok)
      hipLaunchKernelGGL((mlp_nc_kernel<false, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((mlp_nc_kernel<false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace ttt
