// Backward pass of the causal TTT-Linear layer on the gfx950 matrix cores: d = 64, mini-batch
// b = 16, bf16 Q/K/V/dZ/dQ/dK/dV, fp32 dL/dW; reconstruction or negative dot-product loss,
// scalar rate or per-token rate factors (with their gradient).
//
// The outer loop trains the projections and the initial state through the inner updates
// (wmrh.cn summary of Sun et al. 2024, section 2.2; "Fast weights" page, opening
// paragraph).  For a chunk with W = W_c (R = K W^T - V, P = tril(Q K^T), Z = Q W^T - eta P R,
// W_{c+1} = W - eta R^T K) and G = dL/dW_{c+1}, our chain-rule derivation gives
//     dR = -eta (K G^T + P^T dZ),  dV = -dR,  dP = -eta tril(dZ R^T),
//     dQ = dZ W + dP K,  dK = -eta R G + dP^T Q + dR W,  dL/dW_c = G + dZ^T Q + dR^T K.
// With per-token rate factors e_t (token t's gradient at rate eta e_t; wmrh.cn summary,
// section 2.2.3) Rt = diag(e) R replaces R in Z and in the update; the lines above then hold
// for Rt (Rt in dP and in -eta Rt G, the dR line giving dRt), and dR = diag(e) dRt,
// de_t = <dRt_t, R_t>.  With the negative dot-product loss -v^T W k (ViT3 news page,
// section 2) R = -V, and the dR W term of dK and the dR^T K term of dL/dW_c drop out.
// Two kernels:
//   * linear_fwd_hist_kernel recomputes the forward chain (R and the update only) and stores
//     every chunk-start state W_c as bf16 rows [64][64] (the precision the forward products
//     use);
//   * linear_bwd_mfma_kernel walks the chunks from last to first with G in registers.
// Both run one compute wave per (batch, head) chain and a loader wave that streams the
// chunks into an LDS ring with direct-to-LDS loads (rows past T read as zero, which adds
// nothing anywhere: a zero key, value and upstream gradient; their gradients are not
// stored).
//
// Layouts (v_mfma_f32_16x16x32_bf16; C layout: lane (g, n) = (lane / 16, lane % 16) holds
// rows 4 g + e, e = 0..3, of column n; A operand: lane holds A[n][8 g + s]; B: B[8 g + s][n]):
//   * W^T and G^T as accumulator tiles [kb][hf][it]: row m <-> input j = 32 kb + 8 (m / 4) +
//     4 hf + m % 4, column n <-> output i = 16 it + n; the two hf tiles side by side are the
//     operand "rows i, contraction over input block kb" (lane: X[16 it + n][32 kb + 8 g ..]).
//   * Products over features read 16-byte rows of Q, K, dZ (lane: X[n][32 kb + 8 g ..]).
//   * Products over tokens take their operands from the gfx950 transposing LDS read
//     (ds_read_b64_tr_b16: within 16 lanes, lane i receives element i % 4 of the 8 bytes
//     fetched by lane 4 s + i / 4), fetching rows (tokens) 4 g + s.
//   * R, dR and the gradients are formed transposed (rows: features), so R^T and dR^T tiles
//     are directly the operands of products over outputs (two tiles 2 h, 2 h + 1 side by
//     side: k = 8 g + s' <-> i = 16 (2 h + s' / 4) + 4 g + s' % 4), and every lane stores 4
//     consecutive features of one token.
//   * The update of G^T puts both of its token sums into one K = 32 product: slots 0..3 hold
//     the dZ^T Q term's tokens, slots 4..7 the dR^T K term's.
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

constexpr int kD = 64;
constexpr int kB = 16;
constexpr int kRowBytes = kD * 2;
constexpr int kTileBytes = kB * kRowBytes;  // 16 token rows
constexpr int kStateBytes = kD * kRowBytes;  // 64 rows: a bf16 state

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ bf16x8_t bf(const u32x4& x) { return __builtin_bit_cast(bf16x8_t, x); }
__device__ __forceinline__ u32x4 cat_u(const float4_t& x, const float4_t& y) {
  const u32x4 u = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
  return u;
}
__device__ __forceinline__ bf16x8_t cat_op(const float4_t& x, const float4_t& y) { return bf(cat_u(x, y)); }
__device__ __forceinline__ bf16x8_t pad_op(const float4_t& x) {
  const u32x4 u = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), 0u, 0u};
  return bf(u);
}
__device__ __forceinline__ bf16x8_t pad2(const u32x2& x) {
  const u32x4 u = {x.x, x.y, 0u, 0u};
  return bf(u);
}
__device__ __forceinline__ bf16x8_t join2(const u32x2& x, const u32x2& y) {
  const u32x4 u = {x.x, x.y, y.x, y.y};
  return bf(u);
}
__device__ __forceinline__ float4_t mfma(const bf16x8_t& a, const bf16x8_t& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4_t unpack4(const u32x2& x) {
  return float4_t{__builtin_bit_cast(float, x.x << 16), __builtin_bit_cast(float, x.x & 0xFFFF0000u),
                  __builtin_bit_cast(float, x.y << 16), __builtin_bit_cast(float, x.y & 0xFFFF0000u)};
}
__device__ __forceinline__ u32x2 pack4(const float4_t& x) { return u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])}; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes > 0 ? bytes : 0, 0x00020000);
}

// Rows of 128 bytes in LDS with the 16-byte pieces of row r XOR-swizzled by r % 8.
__device__ __forceinline__ int sw(int row, int col) {  // byte offset of element (row, col), col % 4 == 0
  return row * kRowBytes + 16 * ((col >> 3) ^ (row & 7)) + 2 * (col & 7);
}
template <typename T>
__device__ __forceinline__ T lds_ld(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}
template <typename T>
__device__ __forceinline__ void lds_st(lds_char* p, T v) {
  *reinterpret_cast<__attribute__((address_space(3))) T*>(p) = v;
}
// Transposing read: lane (g, n) fetches row r0 + (n / 4), columns c0(n % 4) .. + 3, and
// receives rows r0 + 0..3 of column c0(n / 4) + n % 4.
__device__ __forceinline__ u32x2 tr(const lds_char* base, int row, int col) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + sw(row, col))));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Barrier for LDS traffic only (the fence of __syncthreads() would drain outstanding stores).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// Loader protocol shared by both kernels: step k reads slot k % R; barrier k publishes the
// chunk of step k and frees the slot of step k - 1, which the loader then refills with the
// chunk of step k - 1 + R.  Before barrier k the loads of step k are complete once at most
// R - 2 later steps (R - 1 before barrier 0) of kLoads loads each are outstanding.
template <int R, int kLoads, typename Issue>
__device__ __forceinline__ void loader_loop(int nsteps, Issue&& issue) {
  static_assert((R - 1) * kLoads < 64, "vmcnt is 6 bits");
  for (int k = 0; k < R; ++k) issue(k);
  for (int k = 0; k < nsteps; ++k) {
    if (k == 0)
      wait_vmcnt<(R - 1) * kLoads>();
    else
      wait_vmcnt<(R - 2) * kLoads>();
    lds_barrier();
    if (k >= 1) issue(k - 1 + R);
  }
  wait_vmcnt<0>();  // no load into LDS outlives the wave
}

// the lane's 1024-byte share of a tile of 8 rows: row 8 h + l / 8, physical piece l % 8 holds
// logical piece (l % 8) ^ (row % 8)
__device__ __forceinline__ int src_off(int h, int lane) {
  const int r = 8 * h + (lane >> 3);
  return r * kRowBytes + 16 * ((lane & 7) ^ (r & 7));
}

// ---------------------------------------------------------------- forward recompute
constexpr int kRingF = 8;
constexpr int kSlotFK = 0, kSlotFV = kTileBytes, kSlotFBytes = 2 * kTileBytes;

template <bool kTok, bool kDot>
__global__ __launch_bounds__(128) void linear_fwd_hist_kernel(LinearArgs a, bf16* whist) {
  __shared__ __attribute__((aligned(16))) char ring_mem[kRingF * kSlotFBytes];
  lds_char* ring = (lds_char*)(ring_mem);
  const int chain = blockIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, n = lane & 15;
  const int bi = chain / a.H, hi = chain - bi * a.H;
  const int T = a.T;
  const int nchunks = (T + kB - 1) / kB;
  const int seq_bytes = T * kRowBytes;
  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * kD;
  const char* k = reinterpret_cast<const char*>(static_cast<const bf16*>(a.k) + tok0);
  const char* v = reinterpret_cast<const char*>(static_cast<const bf16*>(a.v) + tok0);

  if (wv == 1) {
    const int s0 = src_off(0, lane), s1 = src_off(1, lane);
    loader_loop<kRingF, 4>(nchunks, [&](int c) {
      const int off = c * kTileBytes;
      lds_char* dst = ring + (c % kRingF) * kSlotFBytes;
      const __amdgpu_buffer_rsrc_t rk = rsrc(k + off, seq_bytes - off);
      const __amdgpu_buffer_rsrc_t rv = rsrc(v + off, seq_bytes - off);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, dst + kSlotFK, 16, s0, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, dst + kSlotFK + 1024, 16, s1, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst + kSlotFV, 16, s0, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst + kSlotFV + 1024, 16, s1, 0, 0, 0);
    });
    return;
  }

  const float eta = a.eta;
  const float* w0 = a.w0 + bi * a.w0_batch_stride + static_cast<long long>(hi) * kD * kD;
  float4_t wt[2][2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const float* wr = w0 + (16 * it + n) * kD + 32 * kb + 8 * g;
      wt[kb][0][it] = *reinterpret_cast<const float4_t*>(wr);
      wt[kb][1][it] = *reinterpret_cast<const float4_t*>(wr + 4);
    }
  bf16* wh = whist + static_cast<size_t>(chain) * nchunks * (kD * kD);
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // rate factors of tokens 4 g + 0..3 of chunk c (zero past T), loaded a chunk ahead
  const float* etok = kTok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
  auto load_e = [&](int c) {
    float4_t e = {1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (kTok) {
      const __amdgpu_buffer_rsrc_t re = rsrc(etok + c * kB, (T - c * kB) * 4);
#pragma unroll
      for (int x = 0; x < 4; ++x) e[x] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(re, (4 * g + x) * 4, 0, 0));
    }
    return e;
  };
  float4_t ecur = load_e(0);

  for (int c = 0; c < nchunks; ++c) {
    const float4_t enext = (kTok && c + 1 < nchunks) ? load_e(c + 1) : ecur;
    lds_barrier();
    const lds_char* sl = ring + (c % kRingF) * kSlotFBytes;
    // bf16 chunk-start state: the operand, and the stored copy (row 16 it + n, 8 inputs)
    bf16x8_t wop[2][4];
    char* out = reinterpret_cast<char*>(wh + static_cast<size_t>(c) * (kD * kD));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const u32x4 u = cat_u(wt[kb][0][it], wt[kb][1][it]);
        wop[kb][it] = bf(u);
        *reinterpret_cast<u32x4*>(out + (16 * it + n) * kRowBytes + (32 * kb + 8 * g) * 2) = u;
      }
    // R (rows: tokens 4 g + e; columns: outputs 16 it + n) = K W^T - V, times -eta
    bf16x8_t kop[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) kop[kb] = bf(lds_ld<u32x4>(sl + kSlotFK + sw(n, 32 * kb + 8 * g)));
    bf16x8_t rb[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      float4_t r = zero;
      if constexpr (!kDot) {
        r = mfma(kop[0], wop[0][it], zero);
        r = mfma(kop[1], wop[1][it], r);
      }
      // V in the C layout: tokens 4 g + e of column 16 it + n (a transposing read)
      r -= unpack4(tr(sl + kSlotFV, 4 * g + (n >> 2), 16 * it + 4 * (n & 3)));
      rb[it] = pad_op(r * (ecur * -eta));
    }
    // W^T += K^T (-eta R): K^T rows j in the tile order, tokens 4 g + s (transposing reads)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const bf16x8_t ktb = pad2(tr(sl + kSlotFK, 4 * g + (n >> 2), 32 * kb + 8 * (n & 3) + 4 * hf));
#pragma unroll
        for (int it = 0; it < 4; ++it) wt[kb][hf][it] = mfma(ktb, rb[it], wt[kb][hf][it]);
      }
    ecur = enext;
  }
}

// ---------------------------------------------------------------- reverse pass
constexpr int kRingB = 4;
constexpr int kSlotQ = 0, kSlotK = kTileBytes, kSlotV = 2 * kTileBytes, kSlotZ = 3 * kTileBytes;
constexpr int kSlotW = 4 * kTileBytes;
constexpr int kSlotBBytes = kSlotW + kStateBytes;

template <bool kTok, bool kDot>
__global__ __launch_bounds__(128) void linear_bwd_mfma_kernel(LinearBwdArgs a, const bf16* whist) {
  __shared__ __attribute__((aligned(16))) char ring_mem[kRingB * kSlotBBytes];
  __shared__ __attribute__((aligned(16))) char gcopy_mem[kStateBytes];  // bf16 G rows [i][j]
  __shared__ __attribute__((aligned(16))) char drs_mem[kTileBytes];     // bf16 dR rows [s][i]
  lds_char* ring = (lds_char*)(ring_mem);
  lds_char* gcp = (lds_char*)(gcopy_mem);
  lds_char* drs = (lds_char*)(drs_mem);
  const int chain = blockIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, n = lane & 15;
  const int T = a.T;
  const int nchunks = (T + kB - 1) / kB;
  const int seq_bytes = T * kRowBytes;
  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * kD;
  const char* q = reinterpret_cast<const char*>(static_cast<const bf16*>(a.q) + tok0);
  const char* k = reinterpret_cast<const char*>(static_cast<const bf16*>(a.k) + tok0);
  const char* v = reinterpret_cast<const char*>(static_cast<const bf16*>(a.v) + tok0);
  const char* dz = reinterpret_cast<const char*>(static_cast<const bf16*>(a.dz) + tok0);
  const char* wh = reinterpret_cast<const char*>(whist + static_cast<size_t>(chain) * nchunks * (kD * kD));

  if (wv == 1) {
    const int s0 = src_off(0, lane), s1 = src_off(1, lane);
    // step k handles chunk nchunks - 1 - k (steps past the first chunk load zeros)
    loader_loop<kRingB, 16>(nchunks, [&](int kk) {
      const int c = nchunks - 1 - kk;
      const int off = c * kTileBytes;
      const int left = c >= 0 ? seq_bytes - off : 0;
      lds_char* dst = ring + (kk % kRingB) * kSlotBBytes;
      const __amdgpu_buffer_rsrc_t rq = rsrc(q + (c >= 0 ? off : 0), left);
      const __amdgpu_buffer_rsrc_t rk = rsrc(k + (c >= 0 ? off : 0), left);
      const __amdgpu_buffer_rsrc_t rv = rsrc(v + (c >= 0 ? off : 0), left);
      const __amdgpu_buffer_rsrc_t rz = rsrc(dz + (c >= 0 ? off : 0), left);
      const __amdgpu_buffer_rsrc_t rw =
          rsrc(wh + (c >= 0 ? static_cast<size_t>(c) * kStateBytes : 0), c >= 0 ? kStateBytes : 0);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int so = h ? s1 : s0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, dst + kSlotQ + 1024 * h, 16, so, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, dst + kSlotK + 1024 * h, 16, so, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst + kSlotV + 1024 * h, 16, so, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, dst + kSlotZ + 1024 * h, 16, so, 0, 0, 0);
      }
#pragma unroll
      for (int h = 0; h < 8; ++h)  // the 64 rows of W_c, 8 per load
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, dst + kSlotW + 1024 * h, 16, src_off(h, lane), 0, 0, 0);
    });
    return;
  }

  const float eta = a.eta;
  // G^T tiles, from dL/dW_final (zeros without it)
  float4_t gt[2][2][4];
  const float* dwo = a.dw_out ? a.dw_out + static_cast<size_t>(chain) * kD * kD : nullptr;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const float4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
      const float* wr = dwo ? dwo + (16 * it + n) * kD + 32 * kb + 8 * g : nullptr;
      gt[kb][0][it] = dwo ? *reinterpret_cast<const float4_t*>(wr) : zero4;
      gt[kb][1][it] = dwo ? *reinterpret_cast<const float4_t*>(wr + 4) : zero4;
    }
  char* dq = reinterpret_cast<char*>(static_cast<bf16*>(a.dq) + tok0);
  char* dk = reinterpret_cast<char*>(static_cast<bf16*>(a.dk) + tok0);
  char* dv = reinterpret_cast<char*>(static_cast<bf16*>(a.dv) + tok0);
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // causal masks: P (rows t = 4 g + e, cols s = n) keeps s <= t; P^T (rows s, cols t) keeps s <= t
  bool keep_p[4], keep_t[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    keep_p[e] = n <= 4 * g + e;
    keep_t[e] = 4 * g + e <= n;
  }

  // the rate factor of token n of chunk c (zero past T), loaded a chunk ahead
  const float* etok = kTok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
  float* detok = kTok && a.deta_tok ? a.deta_tok + static_cast<size_t>(chain) * T : nullptr;
  auto load_e = [&](int c) {
    if constexpr (kTok)
      return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(etok + c * kB, (T - c * kB) * 4), n * 4, 0, 0));
    return 1.0f;
  };
  float ecur = load_e(nchunks - 1);

  for (int kk = 0; kk < nchunks; ++kk) {
    const int c = nchunks - 1 - kk;
    const float enext = (kTok && c > 0) ? load_e(c - 1) : ecur;
    lds_barrier();  // barrier kk: this step's chunk is in its slot
    const lds_char* sl = ring + (kk % kRingB) * kSlotBBytes;
    const lds_char* sq = sl + kSlotQ;
    const lds_char* sk = sl + kSlotK;
    const lds_char* sv = sl + kSlotV;
    const lds_char* sz = sl + kSlotZ;
    const lds_char* sw_ = sl + kSlotW;

    // ---- operands ----
    bf16x8_t kr[2], qr[2], zr[2];  // rows: X[n][32 kb + 8 g ..]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      kr[kb] = bf(lds_ld<u32x4>(sk + sw(n, 32 * kb + 8 * g)));
      qr[kb] = bf(lds_ld<u32x4>(sq + sw(n, 32 * kb + 8 * g)));
      zr[kb] = bf(lds_ld<u32x4>(sz + sw(n, 32 * kb + 8 * g)));
    }
    bf16x8_t wop[2][4], gop[2][4];  // rows i = 16 it + n, inputs 32 kb + 8 g ..
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        wop[kb][it] = bf(lds_ld<u32x4>(sw_ + sw(16 * it + n, 32 * kb + 8 * g)));
        const u32x4 gu = cat_u(gt[kb][0][it], gt[kb][1][it]);
        gop[kb][it] = bf(gu);
        lds_st<u32x4>(gcp + sw(16 * it + n, 32 * kb + 8 * g), gu);  // G rows for the G^T reads
      }
    u32x2 zq[4];  // dZ[n][16 it + 4 g .. + 3]
#pragma unroll
    for (int it = 0; it < 4; ++it) zq[it] = lds_ld<u32x2>(sz + sw(n, 16 * it + 4 * g));

    // ---- R^T (rows i = 16 it + 4 g + e, cols s = n) = W K^T - V^T ----
    float4_t rt[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      rt[it] = zero;
      if constexpr (!kDot) {
        rt[it] = mfma(wop[0][it], kr[0], zero);
        rt[it] = mfma(wop[1][it], kr[1], rt[it]);
      }
      rt[it] -= unpack4(lds_ld<u32x2>(sv + sw(n, 16 * it + 4 * g)));
    }
    bf16x8_t rtop[2], zcat[2];  // over outputs: tiles 2 h, 2 h + 1 side by side (Rt^T)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      rtop[h] = kTok ? cat_op(rt[2 * h] * ecur, rt[2 * h + 1] * ecur) : cat_op(rt[2 * h], rt[2 * h + 1]);
      zcat[h] = join2(zq[2 * h], zq[2 * h + 1]);
    }

    // ---- P, P^T (masked), dP = -eta tril(dZ R^T) (rows t), dP^T (rows s) ----
    float4_t pm = mfma(qr[0], kr[0], zero);
    pm = mfma(qr[1], kr[1], pm);
    float4_t dp = mfma(zcat[0], rtop[0], zero);
    dp = mfma(zcat[1], rtop[1], dp);
    float4_t dpt = mfma(rtop[0], zcat[0], zero);
    dpt = mfma(rtop[1], zcat[1], dpt);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pm[e] = keep_p[e] ? pm[e] : 0.0f;
      dp[e] = keep_p[e] ? -eta * dp[e] : 0.0f;
      dpt[e] = keep_t[e] ? -eta * dpt[e] : 0.0f;
    }
    const bf16x8_t pmb = pad_op(pm), dpb = pad_op(dp), dptb = pad_op(dpt);

    // ---- dR^T (rows i, cols s) = -eta (G K^T + dZ^T P) ----
    u32x2 ztr[4];  // dZ[4 g + s][16 it + n]: dZ^T rows i, tokens
#pragma unroll
    for (int it = 0; it < 4; ++it) ztr[it] = tr(sz, 4 * g + (n >> 2), 16 * it + 4 * (n & 3));
    float4_t drt[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      float4_t x = mfma(gop[0][it], kr[0], zero);
      x = mfma(gop[1][it], kr[1], x);
      x = mfma(pad2(ztr[it]), pmb, x);
      drt[it] = x * -eta;
    }
    if constexpr (kTok) {
      // de_n = <dRt_n, R_n>: this lane's 16 outputs, then the other three lane groups'
      float p = 0.0f;
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int e = 0; e < 4; ++e) p += drt[it][e] * rt[it][e];
      p += __shfl_xor(p, 16, 64);
      p += __shfl_xor(p, 32, 64);
      if (detok && g == 0)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, p), rsrc(detok + c * kB, (T - c * kB) * 4), n * 4, 0, 0);
#pragma unroll
      for (int it = 0; it < 4; ++it) drt[it] *= ecur;  // dR = diag(e) dRt
    }
    bf16x8_t drop[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) drop[h] = cat_op(drt[2 * h], drt[2 * h + 1]);

    // dV = -dR (lane: token n, outputs 16 it + 4 g ..), and dR rows [s][i] to LDS
    {
      const int off = c * kTileBytes;
      const __amdgpu_buffer_rsrc_t rdv = rsrc(dv + off, seq_bytes - off);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        __builtin_amdgcn_raw_buffer_store_b64(pack4(-drt[it]), rdv, n * kRowBytes + 32 * it + 8 * g, 0, 0);
        lds_st<u32x2>(drs + sw(n, 16 * it + 4 * g), pack4(drt[it]));
      }
    }

    // ---- dQ^T (rows j = 16 jt + 4 g + e, cols t) = W^T dZ^T + K^T dP^T;
    //      dK^T (rows j, cols s) = -eta G^T R^T + Q^T dP + W^T dR^T ----
    {
      const int off = c * kTileBytes;
      const __amdgpu_buffer_rsrc_t rdq = rsrc(dq + off, seq_bytes - off);
      const __amdgpu_buffer_rsrc_t rdk = rsrc(dk + off, seq_bytes - off);
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        float4_t xq = zero, xk = zero, xg = zero;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // W^T and G^T rows j = 16 jt + n, outputs i of tiles 2 h, 2 h + 1 (rows 4 g + s)
          const bf16x8_t wtr = join2(tr(sw_, 32 * h + 4 * g + (n >> 2), 16 * jt + 4 * (n & 3)),
                                     tr(sw_, 32 * h + 16 + 4 * g + (n >> 2), 16 * jt + 4 * (n & 3)));
          const bf16x8_t gtr = join2(tr(gcp, 32 * h + 4 * g + (n >> 2), 16 * jt + 4 * (n & 3)),
                                     tr(gcp, 32 * h + 16 + 4 * g + (n >> 2), 16 * jt + 4 * (n & 3)));
          xq = mfma(wtr, zcat[h], xq);
          if constexpr (!kDot) xk = mfma(wtr, drop[h], xk);
          xg = mfma(gtr, rtop[h], xg);
        }
        const bf16x8_t ktr = pad2(tr(sk, 4 * g + (n >> 2), 16 * jt + 4 * (n & 3)));
        const bf16x8_t qtr = pad2(tr(sq, 4 * g + (n >> 2), 16 * jt + 4 * (n & 3)));
        xq = mfma(ktr, dptb, xq);
        xk = mfma(qtr, dpb, xk);
        xk += -eta * xg;
        __builtin_amdgcn_raw_buffer_store_b64(pack4(xq), rdq, n * kRowBytes + 32 * jt + 8 * g, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(pack4(xk), rdk, n * kRowBytes + 32 * jt + 8 * g, 0, 0);
      }
    }

    // ---- G^T += Q^T dZ + K^T dR: slots 0..3 the dZ^T Q tokens, 4..7 the dR^T K tokens ----
    bf16x8_t bup[4];
#pragma unroll
    for (int it = 0; it < 4; ++it)
      bup[it] = join2(ztr[it], kDot ? u32x2{0u, 0u} : tr(drs, 4 * g + (n >> 2), 16 * it + 4 * (n & 3)));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int col = 32 * kb + 8 * (n & 3) + 4 * hf;
        const bf16x8_t aup = join2(tr(sq, 4 * g + (n >> 2), col), tr(sk, 4 * g + (n >> 2), col));
#pragma unroll
        for (int it = 0; it < 4; ++it) gt[kb][hf][it] = mfma(aup, bup[it], gt[kb][hf][it]);
      }
    ecur = enext;
  }

  float* dw0 = a.dw0 + static_cast<size_t>(chain) * kD * kD;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      float* wr = dw0 + (16 * it + n) * kD + 32 * kb + 8 * g;
      *reinterpret_cast<float4_t*>(wr) = gt[kb][0][it];
      *reinterpret_cast<float4_t*>(wr + 4) = gt[kb][1][it];
    }
}

}  // namespace

bool linear_bwd_mfma_supported(const LinearArgs& fwd, const LinearBwdArgs& a, bool bf16_io) {
  auto al = [](const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & (m - 1)) == 0; };
  // 16-byte vector accesses: token rows, dw0 / dw_out rows and the initial state's rows
  const bool aligned = al(a.q, 16) && al(a.k, 16) && al(a.v, 16) && al(a.dz, 16) && al(a.dq, 16) &&
                       al(a.dk, 16) && al(a.dv, 16) && al(a.dw0, 16) &&
                       (a.dw_out == nullptr || al(a.dw_out, 16)) && al(fwd.w0, 16) &&
                       (fwd.w0_batch_stride % 4) == 0;
  const bool fits = static_cast<long long>(a.T) * kRowBytes + 2LL * kTileBytes < 0x7fffffffLL;
  return bf16_io && a.d == kD && a.chunk == kB && a.T > 0 && aligned && fits;
}

size_t linear_bwd_mfma_workspace_bytes(const LinearBwdArgs& a) {
  const size_t nchunks = (static_cast<size_t>(a.T) + kB - 1) / kB;
  return static_cast<size_t>(a.B) * a.H * nchunks * kStateBytes;
}

hipError_t launch_linear_bwd_mfma(const LinearArgs& fwd, const LinearBwdArgs& a, void* workspace,
                                  hipStream_t s) {
  const long long nchains = static_cast<long long>(a.B) * a.H;
  if (nchains > 0x7fffffffLL) return hipErrorInvalidValue;
  bf16* whist = static_cast<bf16*>(workspace);
  const dim3 grid(static_cast<unsigned>(nchains)), block(128);  // compute wave + loader wave
  if ((fwd.eta_tok != nullptr) != (a.eta_tok != nullptr) || fwd.dot_loss != a.dot_loss)
    return hipErrorInvalidValue;
  const bf16* wc = static_cast<const bf16*>(whist);
  auto run = [&](auto fk, auto bk) {
    hipLaunchKernelGGL(fk, grid, block, 0, s, fwd, whist);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bk, grid, block, 0, s, a, wc);
    return hipGetLastError();
  };
  if (a.eta_tok && a.dot_loss)
    return run(linear_fwd_hist_kernel<true, true>, linear_bwd_mfma_kernel<true, true>);
  if (a.eta_tok) return run(linear_fwd_hist_kernel<true, false>, linear_bwd_mfma_kernel<true, false>);
  if (a.dot_loss) return run(linear_fwd_hist_kernel<false, true>, linear_bwd_mfma_kernel<false, true>);
  return run(linear_fwd_hist_kernel<false, false>, linear_bwd_mfma_kernel<false, false>);
}

}  // namespace ttt
