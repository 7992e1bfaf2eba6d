// Non-causal TTT-Linear forward on the gfx950 matrix cores: f(k) = W k, d = 64, bf16
// Q/K/V/Z, fp32 state; one full-batch step, or several consecutive mini-batches and epochs.
//
// Method (ViT3 news page, section 1, inner training setup: the keys and values are a small
// training set, trained on first, then the inner model is applied to every query; wmrh.cn
// summary of Sun et al. 2024, section 2.1.1: batch gradient descent on the linear model).
// With R = K W^T - V over the tokens of a step (rows t; each row scaled by its token's rate
// factor with per-token rates, "Fast weights" page, opening formula; R = -V with the
// negative dot-product loss of the blog page, section TTT / 如何理解):
//     W' = W - eta R^T K,   and after the last step   Z = Q W'^T.
// A step is one mini-batch of consecutive tokens (all of them for the full batch); an epoch
// is one pass over the mini-batches in order (ViT3 page, observation 2).
//
// Mapping.  One workgroup of kWaves = 4 waves per (batch, head) chain; wave w takes the
// 16-token tiles w, w + 4, w + 8, ... of a step, with loads issued two tiles ahead, and
// accumulates its partial G^T = K^T R in 16 fp32 accumulator tiles while W stays a fixed
// bf16 operand.  Per tile:
//   * R^T = W K^T - V^T (rows: outputs, columns: tokens), two K = 32 MFMAs per 16 outputs,
//     with the A operand W (16-byte pieces of its rows) and the B operand K (16-byte pieces
//     of the token rows), and V read as 8-byte row pieces straight into the accumulator
//     layout;
//   * R (rows: tokens) from R^T by an MFMA with I;
//   * G^T += K^T R, K = 16 token contractions with the upper operand half zero; the K^T
//     operand comes from 4-byte loads of two adjacent inputs of each token row.
// The partial sums meet once per step in LDS.  Wave w owns the output rows 16 w .. 16 w + 15
// of W (four fp32 tiles in registers): it adds the four partials of its tiles, applies
// W -= eta G, and publishes its updated tiles through LDS, from which every wave rebuilds
// the bf16 operands of all 64 x 64 entries.  Pass 2 streams the queries:
// Z^T = W' Q^T, stored as 8-byte row pieces.  Tokens past the end of a step read as zero
// and add nothing (R's row is zero); outputs past T are not stored.
//
// Layouts (16 x 16 C-layout tiles; lane (g, n) holds rows 4 g + e, column n): the input index
// j of a tile row m of tile jb = 2 h + p is j = 16 (m / 4) + 2 (m % 4) + 8 h + p, so that
// the pairs of tiles (2 h, 2 h + 1) interleaved are, lane for lane, the operand over
// j = 16 g + 8 h + 0..7 that matches a 16-byte load of a K or Q row; outputs are natural.
#include "common.hpp"

namespace ttt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 64;
constexpr int kTile = 16;
constexpr int kRowBytes = kD * 2;
constexpr int kTileBytes = kTile * kRowBytes;
constexpr int kWaves = 4;  // one per 16 output rows

__device__ __forceinline__ uint32_t pk(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ bf16x8_t as_bf(const u32x4& x) { return __builtin_bit_cast(bf16x8_t, x); }
__device__ __forceinline__ bf16x8_t words(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 u = {a, b, c, d};
  return as_bf(u);
}
// two C-layout tiles interleaved: slot 2 e + p of lane (g, n) = tile p's row 4 g + e
__device__ __forceinline__ bf16x8_t interleave(const float4_t& x, const float4_t& y) {
  return words(pk(x[0], y[0]), pk(x[1], y[1]), pk(x[2], y[2]), pk(x[3], y[3]));
}
// one C-layout tile as a K = 16 operand (slots 8 g + 0..3; the upper half zero)
__device__ __forceinline__ bf16x8_t half_op(const float4_t& x) { return words(pk(x[0], x[1]), pk(x[2], x[3]), 0u, 0u); }
__device__ __forceinline__ float4_t mma(const bf16x8_t& a, const bf16x8_t& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float lo_bf(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float hi_bf(uint32_t x) { return __builtin_bit_cast(float, x & 0xFFFF0000u); }

// Buffer resource from `base` over `left` bytes: loads past the end read zero, stores past
// it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int left) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, left > 0 ? left : 0,
                                           0x00020000);
}

// One tile's training operands of a lane.
struct Tile {
  u32x4 k0, k1;       // K[t = n][16 g .. + 7], K[n][16 g + 8 .. + 15]
  uint32_t kc[4][2];  // kc[e][h] = K[4 g + e][c0 + 8 h], K[4 g + e][c0 + 8 h + 1]
  u32x2 v[4];         // V[t = n][16 it + 4 g .. + 3], output tile it
  float e;            // rate factor of token n (1 without rates; 0 past the end)
};
template <bool kDot>
__device__ __forceinline__ void load_tile(Tile& r, const char* k, const char* v, const float* etok, int tt,
                                          int bytes, int row, const int (&kco)[4], int g, int n) {
  const int off = tt * kTileBytes;
  const __amdgpu_buffer_rsrc_t rk = rsrc(k + off, bytes - off);
  const __amdgpu_buffer_rsrc_t rv = rsrc(v + off, bytes - off);
  if (!kDot) {  // the dot-product loss's R = -V needs no K rows
    r.k0 = __builtin_amdgcn_raw_buffer_load_b128(rk, row, 0, 0);
    r.k1 = __builtin_amdgcn_raw_buffer_load_b128(rk, row + 16, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r.kc[e][0] = __builtin_amdgcn_raw_buffer_load_b32(rk, kco[e], 0, 0);
    r.kc[e][1] = __builtin_amdgcn_raw_buffer_load_b32(rk, kco[e] + 16, 0, 0);
  }
#pragma unroll
  for (int it = 0; it < 4; ++it)
    r.v[it] = __builtin_amdgcn_raw_buffer_load_b64(rv, n * kRowBytes + 2 * (16 * it + 4 * g), 0, 0);
  r.e = 1.0f;
  if (etok) {  // 4 bytes per token; `bytes` / 32 is the step's rate bytes
    const __amdgpu_buffer_rsrc_t re = rsrc(etok + tt * kTile, (bytes >> 5) - tt * kTile * 4);
    r.e = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(re, n * 4, 0, 0));
  }
}

template <bool kDot>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void linear_nc_kernel(LinearArgs a) {
  // [source wave][tile f = 4 jb + it][lane]: the partial sums, then (slot 0) the updated W
  __shared__ float4_t red[kWaves][16][64];
  const int chain = blockIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int bi = chain / a.H;
  const int hi = chain - bi * a.H;
  const int T = a.T;
  const int ntiles = (T + kTile - 1) / kTile;
  const int seq_bytes = T * kRowBytes;
  const float eta = a.eta;

  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * kD;
  const char* q = reinterpret_cast<const char*>(static_cast<const bf16*>(a.q) + tok0);
  const char* k = reinterpret_cast<const char*>(static_cast<const bf16*>(a.k) + tok0);
  const char* v = reinterpret_cast<const char*>(static_cast<const bf16*>(a.v) + tok0);
  char* z = reinterpret_cast<char*>(static_cast<bf16*>(a.z) + tok0);
  const float* etok = a.eta_tok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
  const float* w0 = a.w0 + bi * a.w0_batch_stride + static_cast<long long>(hi) * kD * kD;

  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  constexpr uint32_t kLo = 0x05040100u, kHi = 0x07060302u;  // low / high bf16 of two words
  const uint32_t one = 0x3F80u;                              // bf16 1.0
  const bf16x8_t eye = words((4 * g + 0 == n ? one : 0u) | (4 * g + 1 == n ? one << 16 : 0u),
                             (4 * g + 2 == n ? one : 0u) | (4 * g + 3 == n ? one << 16 : 0u), 0u, 0u);
  const int row = n * kRowBytes + 32 * g;  // K / Q row pieces (16 bytes at +0 and +16)
  const int c0 = 16 * (n >> 2) + 2 * (n & 3);
  int kco[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) kco[e] = (4 * g + e) * kRowBytes + 2 * c0;

  // Steps: `epochs` passes over the mini-batches [m0, m0 + mb) (the last may be shorter).
  const int mb = min(a.chunk, T);
  const int nmb = (T + mb - 1) / mb;
  const int nsteps = nmb * a.epochs;
  int m0 = 0, ns = mb, ntl = (mb + kTile - 1) / kTile;

  Tile cur, nx1, nx2;
  auto prefetch = [&](int start, int len, int tiles) {
    const char* ks = k + start * kRowBytes;
    const char* vs = v + start * kRowBytes;
    const float* es = etok ? etok + start : nullptr;
    if (wv < tiles) load_tile<kDot>(cur, ks, vs, es, wv, len * kRowBytes, row, kco, g, n);
    if (wv + kWaves < tiles) load_tile<kDot>(nx1, ks, vs, es, wv + kWaves, len * kRowBytes, row, kco, g, n);
  };
  prefetch(m0, ns, ntl);

  // This wave's fp32 tiles of W^T: wown[jb] = rows j of tile jb, columns = outputs 16 wv + n,
  // i.e. lane (g, n) reads row 16 wv + n of W at inputs 16 g .. 16 g + 15.
  float4_t wown[4];
  {
    const float* wr = w0 + (16 * wv + n) * kD + 16 * g;
    const float4_t f0 = *reinterpret_cast<const float4_t*>(wr);
    const float4_t f1 = *reinterpret_cast<const float4_t*>(wr + 4);
    const float4_t f2 = *reinterpret_cast<const float4_t*>(wr + 8);
    const float4_t f3 = *reinterpret_cast<const float4_t*>(wr + 12);
    wown[0] = float4_t{f0[0], f0[2], f1[0], f1[2]};
    wown[1] = float4_t{f0[1], f0[3], f1[1], f1[3]};
    wown[2] = float4_t{f2[0], f2[2], f3[0], f3[2]};
    wown[3] = float4_t{f2[1], f2[3], f3[1], f3[3]};
  }
  // bf16 operands of W over j: wb[h][it] (A of W K^T over j = 16 g + 8 h + 0..7)
  bf16x8_t wb[2][4];
  auto publish = [&]() {  // wown -> every wave's wb, through slot 0
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) red[0][4 * jb + wv][lane] = wown[jb];
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int it = 0; it < 4; ++it) wb[h][it] = interleave(red[0][4 * (2 * h) + it][lane], red[0][4 * (2 * h + 1) + it][lane]);
    __syncthreads();  // slot 0 read by all before its next use
  };
  publish();

  for (int step = 0;; ++step) {
    // ---- pass 1: partial G^T = K^T R over this wave's tiles of the step ----
    float4_t gt[4][4];  // [jb][it]
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int it = 0; it < 4; ++it) gt[jb][it] = zero;
    const char* ks = k + m0 * kRowBytes;
    const char* vs = v + m0 * kRowBytes;
    const float* es = etok ? etok + m0 : nullptr;
    for (int tt = wv; tt < ntl; tt += kWaves) {
      if (tt + 2 * kWaves < ntl) load_tile<kDot>(nx2, ks, vs, es, tt + 2 * kWaves, ns * kRowBytes, row, kco, g, n);
      // R^T = W K^T - V^T (rows outputs 16 it + 4 g + e, column token n), times token n's rate
      bf16x8_t rb[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        float4_t o = zero;
        if (!kDot) {
          o = mma(wb[0][it], as_bf(cur.k0), zero);
          o = mma(wb[1][it], as_bf(cur.k1), o);
        }
        o[0] -= lo_bf(cur.v[it].x);
        o[1] -= hi_bf(cur.v[it].x);
        o[2] -= lo_bf(cur.v[it].y);
        o[3] -= hi_bf(cur.v[it].y);
        o = o * cur.e;
        // R (rows tokens 4 g + e, column output 16 it + n) as a K = 16 operand over tokens
        rb[it] = half_op(mma(half_op(o), eye, zero));
      }
      // G^T[jb][it] += K^T R: A operand K^T (rows j of tile jb, tokens 4 g + e)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const int h = jb >> 1;
        const uint32_t sel = (jb & 1) ? kHi : kLo;
        const bf16x8_t kt = words(__builtin_amdgcn_perm(cur.kc[1][h], cur.kc[0][h], sel),
                                  __builtin_amdgcn_perm(cur.kc[3][h], cur.kc[2][h], sel), 0u, 0u);
#pragma unroll
        for (int it = 0; it < 4; ++it) gt[jb][it] = mma(kt, rb[it], gt[jb][it]);
      }
      cur = nx1;
      nx1 = nx2;
    }

    const bool last = step + 1 == nsteps;
    if (!last) {  // the next step's first tiles, loaded while the sums are reduced
      m0 = ((step + 1) % nmb) * mb;
      ns = min(mb, T - m0);
      ntl = (ns + kTile - 1) / kTile;
      prefetch(m0, ns, ntl);
    }

    // ---- W -= eta G: wave wv sums the partials of its tiles (jb, it = wv) ----
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int it = 0; it < 4; ++it) red[wv][4 * jb + it][lane] = gt[jb][it];
    __syncthreads();
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      float4_t sum = red[0][4 * jb + wv][lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) sum += red[w][4 * jb + wv][lane];
      wown[jb] -= eta * sum;
    }
    __syncthreads();  // every partial read before slot 0 is reused
    publish();
    if (last) break;
  }

  // ---- the final state (w_out: row 16 wv + n, inputs 16 g .. 16 g + 15) ----
  if (a.w_out) {
    float* wr = a.w_out + static_cast<size_t>(chain) * kD * kD + (16 * wv + n) * kD + 16 * g;
    const float4_t* t = wown;
    *reinterpret_cast<float4_t*>(wr) = float4_t{t[0][0], t[1][0], t[0][1], t[1][1]};
    *reinterpret_cast<float4_t*>(wr + 4) = float4_t{t[0][2], t[1][2], t[0][3], t[1][3]};
    *reinterpret_cast<float4_t*>(wr + 8) = float4_t{t[2][0], t[3][0], t[2][1], t[3][1]};
    *reinterpret_cast<float4_t*>(wr + 12) = float4_t{t[2][2], t[3][2], t[2][3], t[3][3]};
  }

  // ---- pass 2: Z^T = W' Q^T over this wave's tiles ----
  u32x4 qa0 = {0u, 0u, 0u, 0u}, qa1 = {0u, 0u, 0u, 0u};
  if (wv < ntiles) {
    const int off = wv * kTileBytes;
    const __amdgpu_buffer_rsrc_t rq = rsrc(q + off, seq_bytes - off);
    qa0 = __builtin_amdgcn_raw_buffer_load_b128(rq, row, 0, 0);
    qa1 = __builtin_amdgcn_raw_buffer_load_b128(rq, row + 16, 0, 0);
  }
  for (int tt = wv; tt < ntiles; tt += kWaves) {
    const bf16x8_t qb0 = as_bf(qa0), qb1 = as_bf(qa1);
    if (tt + kWaves < ntiles) {
      const int offn = (tt + kWaves) * kTileBytes;
      const __amdgpu_buffer_rsrc_t rqn = rsrc(q + offn, seq_bytes - offn);
      qa0 = __builtin_amdgcn_raw_buffer_load_b128(rqn, row, 0, 0);
      qa1 = __builtin_amdgcn_raw_buffer_load_b128(rqn, row + 16, 0, 0);
    }
    const int off = tt * kTileBytes;
    const __amdgpu_buffer_rsrc_t rz = rsrc(z + off, seq_bytes - off);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      float4_t zt = mma(wb[0][it], qb0, zero);
      zt = mma(wb[1][it], qb1, zt);
      const u32x2 out = {pk(zt[0], zt[1]), pk(zt[2], zt[3])};
      __builtin_amdgcn_raw_buffer_store_b64(out, rz, n * kRowBytes + 2 * (16 * it + 4 * g), 0, 0);
    }
  }
}

}  // namespace

bool linear_nc_supported(const LinearArgs& a, bool bf16_io) {
  auto al = [](const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & (m - 1)) == 0; };
  const bool aligned = al(a.q, 16) && al(a.k, 16) && al(a.v, 16) && al(a.z, 16) && al(a.w0, 16) &&
                       (a.w0_batch_stride % 4) == 0 && (a.w_out == nullptr || al(a.w_out, 16)) &&
                       (a.eta_tok == nullptr || al(a.eta_tok, 4));
  const bool fits = static_cast<long long>(a.T) * kRowBytes + 2LL * kTileBytes < 0x7fffffffLL;
  return bf16_io && a.d == kD && a.causal == 0 && a.T > 0 && a.chunk >= 1 && a.epochs >= 1 &&
         a.ln_w == nullptr && a.w_hist == nullptr && a.z != nullptr && aligned && fits;
}

hipError_t launch_linear_nc(const LinearArgs& a, hipStream_t s) {
  const long long nchains = static_cast<long long>(a.B) * a.H;
  if (nchains > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.dot_loss)
    hipLaunchKernelGGL(linear_nc_kernel<true>, dim3(static_cast<unsigned>(nchains)), dim3(64 * kWaves), 0, s, a);
  else
    hipLaunchKernelGGL(linear_nc_kernel<false>, dim3(static_cast<unsigned>(nchains)), dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
