// The paper's TTT-Linear on the gfx950 matrix cores: f(x) = x + LN(W x), d = 64, mini-batch
// b = 16, causal, bf16 Q/K/V/Z, fp32 state, per-head LN gain and bias.
//
// Method.  The wmrh.cn summary of Sun et al. 2024, section 2.2.1, always wraps the inner
// model as f(x) = x + LN(f_res(x)); trained by mini-batch GD on 1/2 ||f(k) - v||^2
// (section 1.2.2), or on -v^T f(k) (blog page, section TTT / 如何理解), with z_t = f(q_t; W_t).
// The state changes only through r = dl/d(W k): for a chunk with rows K, Q, V (16 x 64) and
// chunk-start weights W,
//   Y = K W^T,  E = K + LN(Y) - V (or -V),  R = rows of E passed back through the layer
//   norm of the rows of Y (R_t = rstd_t (g_t - mean(g_t) - xh_t mean(g_t xh_t)), g = gamma E),
//   W <- W - eta R^T K,
//   Z = Q + LN(Q W^T - eta tril(Q K^T) R)          (the dual form of the in-chunk updates)
// which equals the per-token recurrence up to floating-point order.  Per-token rates scale
// the rows of R.
//
// Mapping.  The layer norm couples all 64 outputs of a token, so one wave owns a whole
// (batch, head) chain and the state never leaves its registers: W^T as 16 fp32 accumulator
// tiles (64 VGPRs) plus a bf16 operand copy.  Every product is v_mfma_f32_16x16x32_bf16
// (C layout: lane (g, n) = (lane / 16, lane % 16) holds rows 4 g + e, e = 0..3, of column n;
// A operand: lane holds A[n][8 g + s]; B operand: B[8 g + s][n]).
//   * W^T tile (kb, hf, it): row m <-> input j = 32 kb + 8 (m / 4) + 4 hf + m % 4, column n
//     <-> output i = 16 it + n, so lane (g, n) holds W[16 it + n][32 kb + 8 g + 4 hf + e];
//     the two hf tiles side by side are, lane for lane, the B operand of Y = K W^T and the
//     A operand of Z^T = W Q^T over input block kb (with K and Q read as 16-byte rows).
//   * Y and R come out with tokens as rows, so a token's 64 outputs lie in one row of 16
//     lanes (four tiles): the LN sums are in-lane adds and a DPP row sum, with no LDS on the
//     serial chain.
//   * K - V (or -V) in the C layout comes from one MFMA per tile whose A operand holds K in
//     lane groups 0, 1 and V in groups 2, 3 (16-byte row loads) against a constant
//     selection B (+1 at k = n, -1 at k = n + 16).
//   * the K^T operand of the update (rows j in the tile order above, contraction over
//     tokens) is the C-layout product of K with a constant selection matrix;
//   * Z is formed transposed (rows outputs), so its LN sums cross the four lane groups (two
//     shuffles, off the serial chain) and each lane stores 4 consecutive outputs of one
//     token (8 bytes).
// With one wave per chain nothing else on the compute unit hides memory latency, so chunks
// stream kPre ahead into an LDS ring by direct-to-LDS loads (rows past T read as zero: a
// zero key adds nothing to the update, and the causal mask keeps padded tokens out of real
// outputs; their outputs are not stored).
#include "common.hpp"

namespace ttt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 64;
constexpr int kB = 16;
constexpr int kRowBytes = kD * 2;
constexpr int kTileBytes = kB * kRowBytes;

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
// slots 0..3 = x[0..3], slots 4..7 = y[0..3]
__device__ __forceinline__ bf16x8_t cat_op(const float4_t& x, const float4_t& y) {
  return op4(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]));
}
// a K = 16 operand (contraction index 4 g + s in slot s) padded to the K = 32 layout
__device__ __forceinline__ bf16x8_t pad_op(const float4_t& x) {
  return op4(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), 0u, 0u);
}
__device__ __forceinline__ float4_t mfma(const bf16x8_t& a, const bf16x8_t& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float bf_lo(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __builtin_bit_cast(float, x & 0xFFFF0000u); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* base, int left) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, left > 0 ? left : 0, 0x00020000);
}

// Sum over the 16 lanes of a DPP row (quad permutations, then half-row and row mirrors, each
// pairing lanes that hold disjoint partial sums); every lane of the row ends with the same
// bits.
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

// Three waves per chain: the chain wave runs the state recursion (R and the update) and
// hands each chunk's bf16 state operand and -eta R operand to the output wave, which forms
// that chunk's Z one step later; a loader wave fills an LDS ring of kRing chunk slots with
// direct-to-LDS buffer loads (rows past T read as zero).  Slot: Q, K, V tiles (16 rows of
// 128 bytes; the 16-byte pieces of row r are stored XOR-swizzled by r % 8, so that 16-byte
// reads of one piece from 8 consecutive rows fall on distinct banks), then the 16 rate
// factors.  (A separate loader keeps the compute waves free of pending LDS loads, before
// whose destination the compiler would otherwise make every LDS read wait.)
// Barrier b (b = 0 .. nchunks) publishes chunk b to the chain wave and chunk b - 1's handoff
// to the output wave, and frees the slot of chunk b - 2, which the loader then refills with
// chunk b - 2 + kRing.  Before barrier b the loads of chunk b are complete once at most
// kRing - 3 later chunks are outstanding (more before barrier 2: a smaller count then only
// waits longer).
constexpr int kRing = 8;
constexpr int kSlotQ = 0, kSlotK = kTileBytes, kSlotV = 2 * kTileBytes, kSlotE = 3 * kTileBytes;
constexpr int kSlotBytes = kSlotE + kB * 4;
template <bool kTok> struct Counts {
  static constexpr int kLoads = 6 + (kTok ? 1 : 0);
  static constexpr int kWait = (kRing - 3) * kLoads;
  static_assert(kWait < 64, "vmcnt is 6 bits");
};
// Handoff buffer (two, used in turn): the bf16 chunk-start state operands wop[kb][it] at
// 1024 (4 kb + it) + 16 lane, then the -eta R operands (first 8 bytes of each padded
// operand) at 8192 + 512 it + 8 lane: consecutive lanes write consecutive addresses.
constexpr int kHandR = 8 * 1024;
constexpr int kHandBytes = kHandR + 4 * 512;

// Workgroup barrier for LDS traffic only: this wave's LDS reads are complete, then both
// waves meet (the fence of __syncthreads() would also drain this wave's outstanding stores).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt unconstrained
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

typedef __attribute__((address_space(3))) char lds_char;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
template <typename T>
__device__ __forceinline__ T lds_load(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}
template <typename T>
__device__ __forceinline__ void lds_store(lds_char* p, const T& x) {
  *reinterpret_cast<__attribute__((address_space(3))) T*>(p) = x;
}

template <bool kTok, bool kDot>
__global__ __launch_bounds__(192) void linear_ln_mfma_kernel(LinearArgs a) {
  const int chain = blockIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // 0: chain, 1: output, 2: loader
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int bi = chain / a.H;
  const int hi = chain - bi * a.H;
  const int T = a.T;
  const int nchunks = (T + kB - 1) / kB;
  const int seq_bytes = T * kRowBytes;
  const float eta = a.eta;

  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * kD;
  const char* q = reinterpret_cast<const char*>(static_cast<const bf16*>(a.q) + tok0);
  const char* k = reinterpret_cast<const char*>(static_cast<const bf16*>(a.k) + tok0);
  const char* v = reinterpret_cast<const char*>(static_cast<const bf16*>(a.v) + tok0);
  char* z = reinterpret_cast<char*>(static_cast<bf16*>(a.z) + tok0);
  const float* etok = kTok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
  const float* w0 = a.w0 + bi * a.w0_batch_stride + static_cast<long long>(hi) * kD * kD;
  const float* gam = a.ln_w + hi * kD;
  const float* bet = a.ln_b + hi * kD;
  const float eps = a.ln_eps;
  using CT = Counts<kTok>;
  __shared__ __attribute__((aligned(16))) char ring_mem[kRing * kSlotBytes];
  __shared__ __attribute__((aligned(16))) char hand_mem[2 * kHandBytes];
  lds_char* ring = (lds_char*)(ring_mem);
  lds_char* hand = (lds_char*)(hand_mem);

  // ---- the state: W^T tiles [kb][hf][it] ----
  float4_t wt[2][2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const float* wr = w0 + (16 * it + n) * kD + 32 * kb + 8 * g;
      wt[kb][0][it] = *reinterpret_cast<const float4_t*>(wr);
      wt[kb][1][it] = *reinterpret_cast<const float4_t*>(wr + 4);
    }

  // ---- LN parameters: outputs 16 it + n (rows of R) in registers; the whole vectors in
  // LDS for the rows of Z^T (outputs 16 it + 4 g + e, read as float4 per tile) ----
  __shared__ __attribute__((aligned(16))) float lnp[2][kD];
  float gr[4], br[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    gr[it] = gam[16 * it + n];
    br[it] = bet[16 * it + n];
    lnp[0][16 * it + n] = gr[it];
    lnp[1][16 * it + n] = br[it];
  }
  __syncthreads();

  // ---- constant selection operands (bf16 +-1) ----
  const uint32_t one = 0x3F80u, mone = 0xBF80u;
  // K - V (or -V): B[k][n] = +1 at k = n (K half, not for the dot loss), -1 at k = n + 16
  uint32_t skv[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t w = 0u;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kk = 8 * g + 2 * p + h;
      const uint32_t val = (!kDot && kk == n) ? one : (kk == n + 16 ? mone : 0u);
      w |= val << (16 * h);
    }
    skv[p] = w;
  }
  const bf16x8_t sel_kv = op4(skv[0], skv[1], skv[2], skv[3]);
  // K^T rows in the W^T tile order: B[k][m] = 1 at k = 8 (m / 4) + 4 hf + m % 4
  bf16x8_t sel_t[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    uint32_t sw[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t w = 0u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kk = 8 * g + 2 * p + h;
        if (kk == 8 * (n >> 2) + 4 * hf + (n & 3)) w |= one << (16 * h);
      }
      sw[p] = w;
    }
    sel_t[hf] = op4(sw[0], sw[1], sw[2], sw[3]);
  }
  const bool keep[4] = {4 * g + 0 <= n, 4 * g + 1 <= n, 4 * g + 2 <= n, 4 * g + 3 <= n};
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};

  // ---- the ring: lane l of a half tile (rows 8 h .. 8 h + 7) fills physical piece l % 8 of
  // row 8 h + l / 8 with that row's logical piece (l % 8) ^ (row % 8) ----
  int gsrc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 8 * h + (lane >> 3);
    gsrc[h] = r * kRowBytes + 16 * ((lane & 7) ^ (r & 7));
  }
  const float* esrc = kTok ? etok : nullptr;
  auto issue = [&](int c) {  // chunk c into slot c % kRing (zeros past the end)
    const int off = c * kTileBytes;
    lds_char* dst = ring + (c % kRing) * kSlotBytes;
    const __amdgpu_buffer_rsrc_t rq = chunk_rsrc(q + off, seq_bytes - off);
    const __amdgpu_buffer_rsrc_t rk = chunk_rsrc(k + off, seq_bytes - off);
    const __amdgpu_buffer_rsrc_t rv = chunk_rsrc(v + off, seq_bytes - off);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, dst + kSlotQ + 1024 * h, 16, gsrc[h], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, dst + kSlotK + 1024 * h, 16, gsrc[h], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst + kSlotV + 1024 * h, 16, gsrc[h], 0, 0, 0);
    }
    if (kTok && lane < kB) {  // 4 bytes per token
      const __amdgpu_buffer_rsrc_t re = chunk_rsrc(esrc + c * kB, (seq_bytes >> 5) - c * kB * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(re, dst + kSlotE, 4, lane * 4, 0, 0, 0);
    }
  };
  if (wv == 2) {
    for (int c = 0; c < kRing; ++c) issue(c);
    for (int b = 0; b <= nchunks; ++b) {
      wait_vmcnt<CT::kWait>();
      lds_barrier();  // barrier b
      if (b >= 2) issue(b - 2 + kRing);
    }
    wait_vmcnt<0>();  // no load into LDS outlives the wave
    return;
  }

  // this lane's read offsets in a slot: piece P of row n sits at n * 128 + 16 (P ^ (n % 8))
  auto piece = [&](int p) { return n * kRowBytes + 16 * (p ^ (n & 7)); };

  // ---- output wave: Z of chunk c from its handoff ----
  if (wv == 1) {
    auto out_step = [&](int c) {
      const lds_char* sl = ring + (c % kRing) * kSlotBytes;
      const lds_char* hb = hand + (c & 1) * kHandBytes;
      bf16x8_t kop[2], qop[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        kop[kb] = bf(lds_load<u32x4>(sl + kSlotK + piece(4 * kb + g)));
        qop[kb] = bf(lds_load<u32x4>(sl + kSlotQ + piece(4 * kb + g)));
      }
      bf16x8_t wop[2][4], rb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int it = 0; it < 4; ++it) wop[kb][it] = bf(lds_load<u32x4>(hb + 1024 * (4 * kb + it) + 16 * lane));
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const u32x2 r = lds_load<u32x2>(hb + kHandR + 512 * it + 8 * lane);
        rb[it] = op4(r.x, r.y, 0u, 0u);
      }
      // Z^T (rows: outputs 16 it + 4 g + e; columns: tokens n)
      float4_t pt = mfma(kop[0], qop[0], zero);  // P^T = K Q^T, masked s <= t
      pt = mfma(kop[1], qop[1], pt);
#pragma unroll
      for (int e = 0; e < 4; ++e) pt[e] = keep[e] ? pt[e] : 0.0f;
      const bf16x8_t ptb = pad_op(pt);
      float4_t zt[4];
      float z1 = 0.0f, z2 = 0.0f;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        zt[it] = mfma(wop[0][it], qop[0], zero);
        zt[it] = mfma(wop[1][it], qop[1], zt[it]);
        zt[it] = mfma(rb[it], ptb, zt[it]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          z1 += zt[it][e];
          z2 += zt[it][e] * zt[it][e];
        }
      }
      // a token's 64 outputs: 16 in this lane, the rest in lanes n + 16, n + 32, n + 48
      z1 += __shfl_xor(z1, 16, 64);
      z2 += __shfl_xor(z2, 16, 64);
      z1 += __shfl_xor(z1, 32, 64);
      z2 += __shfl_xor(z2, 32, 64);
      const float mu = z1 * (1.0f / kD);
      const float rs = 1.0f / sqrtf(fmaxf(z2 * (1.0f / kD) - mu * mu, 0.0f) + eps);
      const int off = c * kTileBytes;
      const __amdgpu_buffer_rsrc_t rz = chunk_rsrc(z + off, seq_bytes - off);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const float4_t gz = *reinterpret_cast<const float4_t*>(&lnp[0][16 * it + 4 * g]);
        const float4_t bz = *reinterpret_cast<const float4_t*>(&lnp[1][16 * it + 4 * g]);
        const u32x2 qr = lds_load<u32x2>(sl + kSlotQ + piece(2 * it + (g >> 1)) + 8 * (g & 1));
        const float4_t o = float4_t{bf_lo(qr.x), bf_hi(qr.x), bf_lo(qr.y), bf_hi(qr.y)} +
                           gz * ((zt[it] - mu) * rs) + bz;
        const u32x2 out = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
        __builtin_amdgcn_raw_buffer_store_b64(out, rz, n * kRowBytes + 32 * it + 8 * g, 0, 0);
      }
    };
    lds_barrier();  // barrier 0
    for (int b = 1; b <= nchunks; ++b) {
      lds_barrier();  // barrier b: chunk b - 1's handoff is complete
      out_step(b - 1);
    }
    return;
  }

  // ---- chain wave: R, the handoff and the update of chunk c ----
  auto step = [&](int c) {
    const lds_char* sl = ring + (c % kRing) * kSlotBytes;
    lds_char* hb = hand + (c & 1) * kHandBytes;
    bf16x8_t kop[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) kop[kb] = bf(lds_load<u32x4>(sl + kSlotK + piece(4 * kb + g)));
    float4_t et = {1.0f, 1.0f, 1.0f, 1.0f};
    if (kTok) et = lds_load<float4_t>(sl + kSlotE + 16 * g);

    // bf16 chunk-start state (also handed to the output wave)
    bf16x8_t wop[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const u32x4 u = {pack_bf16(wt[kb][0][it][0], wt[kb][0][it][1]), pack_bf16(wt[kb][0][it][2], wt[kb][0][it][3]),
                         pack_bf16(wt[kb][1][it][0], wt[kb][1][it][1]), pack_bf16(wt[kb][1][it][2], wt[kb][1][it][3])};
        wop[kb][it] = bf(u);
        lds_store<u32x4>(hb + 1024 * (4 * kb + it) + 16 * lane, u);
      }

    // ---- R (rows: tokens 4 g + e; columns: outputs 16 it + n) ----
    float4_t y[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      y[it] = mfma(kop[0], wop[0][it], zero);
      y[it] = mfma(kop[1], wop[1][it], y[it]);
    }
    float4_t xh[4], err[4];
    float rstd[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        s1 += y[it][e];
        s2 += y[it][e] * y[it][e];
      }
      const float mu = row_sum16(s1) * (1.0f / kD);
      const float var = fmaxf(row_sum16(s2) * (1.0f / kD) - mu * mu, 0.0f);
      rstd[e] = 1.0f / sqrtf(var + eps);
#pragma unroll
      for (int it = 0; it < 4; ++it) xh[it][e] = (y[it][e] - mu) * rstd[e];
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      // K (lane groups 0, 1) or V (2, 3) of tile it, against the selection: K - V, or -V
      const u32x4 kvr = lds_load<u32x4>(sl + (g < 2 ? kSlotK : kSlotV) + piece(2 * it + (g & 1)));
      const float4_t kv = mfma(bf(kvr), sel_kv, zero);
      err[it] = kDot ? kv : kv + gr[it] * xh[it] + br[it];
    }
    bf16x8_t rb[4];  // -eta_t R as padded operands (also handed to the output wave)
    {
      float4_t m1 = zero, m2 = zero;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const float4_t gg = gr[it] * err[it];
        m1 += gg;
        m2 += gg * xh[it];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m1[e] = row_sum16(m1[e]) * (1.0f / kD);
        m2[e] = row_sum16(m2[e]) * (1.0f / kD);
      }
      const float4_t sc = float4_t{rstd[0], rstd[1], rstd[2], rstd[3]} * et * -eta;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const float4_t r = sc * (gr[it] * err[it] - m1 - xh[it] * m2);
        const u32x2 rp = {pack_bf16(r[0], r[1]), pack_bf16(r[2], r[3])};
        rb[it] = op4(rp.x, rp.y, 0u, 0u);
        lds_store<u32x2>(hb + kHandR + 512 * it + 8 * lane, rp);
      }
    }

    // ---- state update W^T += K^T (-eta R) ----
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const bf16x8_t ktb = pad_op(mfma(kop[kb], sel_t[hf], zero));
#pragma unroll
        for (int it = 0; it < 4; ++it) wt[kb][hf][it] = mfma(ktb, rb[it], wt[kb][hf][it]);
      }
  };

  for (int c = 0; c < nchunks; ++c) {
    lds_barrier();  // barrier c: chunk c is in its slot, the handoff buffer c % 2 is free
    step(c);
  }
  lds_barrier();  // barrier nchunks: the last handoff is complete

  if (a.w_out) {
    float* wo = a.w_out + static_cast<size_t>(chain) * kD * kD;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        float* wr = wo + (16 * it + n) * kD + 32 * kb + 8 * g;
        *reinterpret_cast<float4_t*>(wr) = wt[kb][0][it];
        *reinterpret_cast<float4_t*>(wr + 4) = wt[kb][1][it];
      }
  }
}

}  // namespace

bool linear_ln_mfma_supported(const LinearArgs& a, bool bf16_io) {
  auto al = [](const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & (m - 1)) == 0; };
  const bool aligned = al(a.q, 16) && al(a.k, 16) && al(a.v, 16) && al(a.z, 16) && al(a.w0, 16) &&
                       (a.w0_batch_stride % 4) == 0 && (a.w_out == nullptr || al(a.w_out, 16)) &&
                       al(a.ln_w, 16) && al(a.ln_b, 16) && (a.eta_tok == nullptr || al(a.eta_tok, 4));
  const bool fits = static_cast<long long>(a.T) * kRowBytes + 2LL * kTileBytes < 0x7fffffffLL;
  return bf16_io && a.ln_w != nullptr && a.d == kD && a.chunk == kB && a.causal == 1 && a.T > 0 &&
         a.z != nullptr && aligned && fits;
}

hipError_t launch_linear_ln_mfma(const LinearArgs& a, hipStream_t s) {
  const long long nchains = static_cast<long long>(a.B) * a.H;
  if (nchains > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(nchains)), block(192);  // chain, output and loader waves
  const bool tok = a.eta_tok != nullptr;
  if (tok && a.dot_loss)
    hipLaunchKernelGGL((linear_ln_mfma_kernel<true, true>), grid, block, 0, s, a);
  else if (tok)
    hipLaunchKernelGGL((linear_ln_mfma_kernel<true, false>), grid, block, 0, s, a);
  else if (a.dot_loss)
    hipLaunchKernelGGL((linear_ln_mfma_kernel<false, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((linear_ln_mfma_kernel<false, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
