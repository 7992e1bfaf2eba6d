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

// Loader protocols.  Every loader wave issues kLoads loads per step, whatever the step (a step
// past the data loads zeros), so the vector-memory counter bounds the loads still in flight.
// Lag 1: step k reads slot k % R; barrier k publishes the chunk of step k and frees the slot
// of step k - 1, which the loader then refills with the chunk of step k - 1 + R.  Before
// barrier k the loads of step k are complete once at most R - 2 later steps (R - 1 before
// barrier 0) are outstanding.
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
// Lag 2 (a slot is read during two steps): nsteps + 1 barriers; barrier k publishes step k
// and frees the slot of step k - 2, refilled with step k - 2 + R.  Before barrier k, steps
// 0 .. R - 1 + max(0, k - 2) have been issued, so step k is complete once at most R - 1,
// R - 2, then R - 3 later steps are outstanding.
template <int R, int kLoads, typename Issue>
__device__ __forceinline__ void loader_loop_lag2(int nsteps, Issue&& issue) {
  static_assert(R >= 3 && (R - 1) * kLoads < 64, "ring depth / vmcnt");
  for (int k = 0; k < R; ++k) issue(k);
  for (int k = 0; k <= nsteps; ++k) {
    if (k == 0)
      wait_vmcnt<(R - 1) * kLoads>();
    else if (k == 1)
      wait_vmcnt<(R - 2) * kLoads>();
    else
      wait_vmcnt<(R - 3) * kLoads>();
    lds_barrier();
    if (k >= 2 && k < nsteps) issue(k - 2 + R);
  }
  wait_vmcnt<0>();
}

// the lane's 1024-byte share of a tile of 8 rows: row 8 h + l / 8, physical piece l % 8 holds
// logical piece (l % 8) ^ (row % 8)
__device__ __forceinline__ int src_off(int h, int lane) {
  const int r = 8 * h + (lane >> 3);
  return r * kRowBytes + 16 * ((lane & 7) ^ (r & 7));
}
__device__ __forceinline__ void load_lds(__amdgpu_buffer_rsrc_t r, lds_char* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
}
// 16 rate factors (4 bytes a lane; lanes past the range, and past T, read zero)
__device__ __forceinline__ void load_lds_e(const float* etok, int c, int T, lds_char* dst, int lane) {
  const bool live = c >= 0 && c * kB < T;
  const int cnt = live ? (T - c * kB < kB ? T - c * kB : kB) : 0;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(etok + (live ? c * kB : 0), 4 * cnt), dst, 4, 4 * lane, 0, 0, 0);
}
// the byte range of token tile c of a [T][64] bf16 sequence (empty outside 0 .. nchunks - 1)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* seq, int c, int nchunks, int seq_bytes) {
  const bool live = c >= 0 && c < nchunks;
  const int off = live ? c * kTileBytes : 0;
  return rsrc(seq + off, live ? seq_bytes - off : 0);
}

// Both kernels run four compute waves per chain: wave w owns the state rows (outputs)
// i = 16 w .. 16 w + 15.  The recursions W_{c+1} = W_c - eta Rt^T K and
// G_c = G_{c+1} + dZ^T Q + dR^T K act on each row of the state separately (R[:, i] needs
// only row i of W; dR[:, i] only row i of G), so the waves never exchange state.

// ---------------------------------------------------------------- forward recompute
// Each compute wave reads a step's operands from LDS one step ahead (into registers), so its
// recursion (state -> R -> update -> state) never waits on an LDS read.  Loader protocol for
// that: nsteps + 1 barriers; barrier k publishes steps 0 .. k + 1; the slot of step s is read
// before barrier max(s, 1), and after barrier k >= 1 the loader refills the slot of step
// k - 1 with step k - 1 + R.  Before barrier 0, steps 0 .. R - 1 have been issued, so steps
// 0 and 1 are complete once at most R - 2 later steps are outstanding; before barrier k >= 1,
// steps 0 .. R + k - 2, so steps up to k + 1 are complete once at most R - 3 are.
template <int R, int kLoads, typename Issue>
__device__ __forceinline__ void loader_loop_ahead1(int nsteps, Issue&& issue) {
  static_assert(R >= 4 && (R - 2) * kLoads < 64, "ring depth / vmcnt");
  for (int k = 0; k < R; ++k) issue(k);
  for (int k = 0; k <= nsteps; ++k) {
    if (k == 0)
      wait_vmcnt<(R - 2) * kLoads>();
    else
      wait_vmcnt<(R - 3) * kLoads>();
    lds_barrier();
    if (k >= 1) issue(k - 1 + R);
  }
  wait_vmcnt<0>();  // no load into LDS outlives the wave
}

template <int N>
using IC = std::integral_constant<int, N>;
constexpr int kWavesC = 4;
// The history pass is bound by its stores (8 KB of W_c per chunk and chain; one compute unit
// writes about 30 GB/s whatever the number of waves storing), so a chain's rows are split
// over kSplitF workgroups, each with kWavesC / kSplitF compute waves.
constexpr int kSplitF = 2;
constexpr int kWavesF = kWavesC / kSplitF;
constexpr int kRowsF = kD / kSplitF;     // state rows per workgroup
constexpr int kLoadWavesF = 2;           // one streams K, the other V
constexpr int kStoreWavesF = 2;          // each stores half of the workgroup's rows of W_c
constexpr int kRingF = 8;       // the compute loop unrolls by it
constexpr int kSlotFK = 0, kSlotFV = kTileBytes, kSlotFE = 2 * kTileBytes;
constexpr int kSlotFBytes = kSlotFE + 256;

template <bool kTok, bool kDot>
__global__ __launch_bounds__(64 * (kWavesF + kLoadWavesF + kStoreWavesF)) void linear_fwd_hist_kernel(LinearArgs a, bf16* whist) {
  __shared__ __attribute__((aligned(16))) char ring_mem[kRingF * kSlotFBytes];
  __shared__ __attribute__((aligned(16))) char stage_mem[2 * kStateBytes];  // bf16 W_c rows, by step parity
  lds_char* ring = (lds_char*)(ring_mem);
  lds_char* stage = (lds_char*)(stage_mem);
  // the kSplitF workgroups of a chain are b, b + 8, ...: the same XCD (workgroup id mod 8),
  // so its L2 serves the chain's K and V to all of them
  const int grp = blockIdx.x / (8 * kSplitF), within = blockIdx.x % (8 * kSplitF);
  const int chain = 8 * grp + within % 8, part = within / 8;
  if (chain >= a.B * a.H) return;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, n = lane & 15;
  const int bi = chain / a.H, hi = chain - bi * a.H;
  const int T = a.T;
  const int nchunks = (T + kB - 1) / kB;
  const int seq_bytes = T * kRowBytes;
  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * kD;

  char* wh = reinterpret_cast<char*>(whist + static_cast<size_t>(chain) * nchunks * (kD * kD));
  if (wv >= kWavesF + kLoadWavesF) {
    // store waves: after barrier c + 1, the workgroup's rows of W_c from the staging buffer
    // to HBM, 8 whole 128-byte rows per store (the compute waves' stores would stall their
    // recursion)
    const int sw_ = wv - kWavesF - kLoadWavesF;
    lds_barrier();  // barrier 0
    for (int c = 0; c < nchunks; ++c) {
      lds_barrier();  // barrier c + 1: W_c is in stage (c & 1)
      const lds_char* st = stage + (c & 1) * kStateBytes;
      const __amdgpu_buffer_rsrc_t rw = rsrc(wh + static_cast<size_t>(c) * kStateBytes, kStateBytes);
#pragma unroll
      for (int i = 0; i < kRowsF / (8 * kStoreWavesF); ++i) {
        const int row = kRowsF * part + (kRowsF / kStoreWavesF) * sw_ + 8 * i + (lane >> 3), piece = lane & 7;
        const u32x4 x = lds_ld<u32x4>(st + sw(row, 8 * piece));
        __builtin_amdgcn_raw_buffer_store_b128(x, rw, row * kRowBytes + 16 * piece, 0, 0);
      }
    }
    return;
  }
  if (wv >= kWavesF) {
    const int lw = wv - kWavesF;
    const char* src = reinterpret_cast<const char*>(static_cast<const bf16*>(lw == 0 ? a.k : a.v) + tok0);
    const int slot = lw == 0 ? kSlotFK : kSlotFV;
    const float* etok = kTok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
    const int s0 = src_off(0, lane), s1 = src_off(1, lane);
    loader_loop_ahead1<kRingF, kTok ? 3 : 2>(nchunks, [&](int c) {
      lds_char* dst = ring + (c % kRingF) * kSlotFBytes;
      const __amdgpu_buffer_rsrc_t r = tile_rsrc(src, c, nchunks, seq_bytes);
      load_lds(r, dst + slot, s0);
      load_lds(r, dst + slot + 1024, s1);
      if constexpr (kTok) load_lds_e(etok, c, T, dst + kSlotFE, lane);  // both waves, same bytes
    });
    return;
  }

  const int w = kWavesF * part + wv;  // this wave's state rows: 16 w .. 16 w + 15
  const float eta = a.eta;
  const float* w0 = a.w0 + bi * a.w0_batch_stride + static_cast<long long>(hi) * kD * kD;
  // W^T tiles of this wave's outputs i = 16 w + n: [kb][hf], rows j = 32 kb + 8 g + 4 hf + e
  float4_t wt[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const float* wr = w0 + (16 * w + n) * kD + 32 * kb + 8 * g;
    wt[kb][0] = *reinterpret_cast<const float4_t*>(wr);
    wt[kb][1] = *reinterpret_cast<const float4_t*>(wr + 4);
  }
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};

  struct Ops {
    bf16x8_t kop[2];  // K rows: K[n][32 kb + 8 g ..]
    u32x2 vt;         // V in the C layout: V[4 g + s][16 w + n]
    u32x2 kt[2][2];   // K^T rows j in the tile order, tokens 4 g + s
    float4_t sc;      // -eta e_t of tokens 4 g + 0..3
  };
  auto load = [&](auto slot_c) __attribute__((always_inline)) {
    const lds_char* sl = ring + static_cast<int>(slot_c) * kSlotFBytes;
    Ops o;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (!kDot) o.kop[kb] = bf(lds_ld<u32x4>(sl + kSlotFK + sw(n, 32 * kb + 8 * g)));
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) o.kt[kb][hf] = tr(sl + kSlotFK, 4 * g + (n >> 2), 32 * kb + 8 * (n & 3) + 4 * hf);
    }
    o.vt = tr(sl + kSlotFV, 4 * g + (n >> 2), 16 * w + 4 * (n & 3));
    o.sc = float4_t{-eta, -eta, -eta, -eta};
    if constexpr (kTok) o.sc *= lds_ld<float4_t>(sl + kSlotFE + 16 * g);
    return o;
  };
  // the work of step c; par = c & 1
  auto work = [&](const Ops& o, auto par_c) __attribute__((always_inline)) {
    // bf16 chunk-start rows: the operand (row 16 w + n, inputs 32 kb + 8 g ..), and the copy
    // for the store waves
    bf16x8_t wop[2];
    lds_char* st = stage + static_cast<int>(par_c) * kStateBytes;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u32x4 u = cat_u(wt[kb][0], wt[kb][1]);
      wop[kb] = bf(u);
      lds_st<u32x4>(st + sw(16 * w + n, 32 * kb + 8 * g), u);
    }
    // R (rows: tokens 4 g + e; columns: outputs 16 w + n) = K W^T - V, times -eta e_t
    float4_t r = zero;
    if constexpr (!kDot) {
      r = mfma(o.kop[0], wop[0], zero);
      r = mfma(o.kop[1], wop[1], r);
    }
    r -= unpack4(o.vt);
    const bf16x8_t rb = pad_op(r * o.sc);
    // W^T += K^T (-eta Rt)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) wt[kb][hf] = mfma(pad2(o.kt[kb][hf]), rb, wt[kb][hf]);
  };
  lds_barrier();  // barrier 0: steps 0 and 1 are in the ring
  Ops oa = load(IC<0>{});
  // step c: load step c + 1's operands, work on step c, barrier c + 1
  int c = 0;
  for (; c + kRingF <= nchunks; c += kRingF) {
    Ops ob = load(IC<1>{}); work(oa, IC<0>{}); lds_barrier();
    oa = load(IC<2>{}); work(ob, IC<1>{}); lds_barrier();
    ob = load(IC<3>{}); work(oa, IC<0>{}); lds_barrier();
    oa = load(IC<4>{}); work(ob, IC<1>{}); lds_barrier();
    ob = load(IC<5>{}); work(oa, IC<0>{}); lds_barrier();
    oa = load(IC<6>{}); work(ob, IC<1>{}); lds_barrier();
    ob = load(IC<7>{}); work(oa, IC<0>{}); lds_barrier();
    oa = load(IC<0>{}); work(ob, IC<1>{}); lds_barrier();
  }
  for (; c < nchunks; ++c) {
    const Ops ob = load((c + 1) % kRingF);
    work(oa, c & 1);
    lds_barrier();
    oa = ob;
  }
}

// ---------------------------------------------------------------- reverse pass
// Twelve waves per chain.  Between barriers k and k + 1:
//   recursion wave w (0..3), chunk c = nchunks - 1 - k, state rows 16 w .. 16 w + 15:
//     Rt^T and dR^T of those rows, dV, the update of G^T, and the rows' Rt, dR and G (bf16)
//     into LDS;
//   gradient wave w (4..7), chunk c + 1 (the previous step's), features j = 16 (w - 4) ..:
//     dP over all outputs, dQ^T and dK^T of those features, from the Rt, dR and G rows all
//     four recursion waves wrote during the previous step;
//   loader waves (8..11): the chunk of step k + 1 .. into the ring.
// Each SIMD runs one recursion and one gradient wave, so the gradient work fills the
// recursion's stalls.  The Rt / dR / G buffers alternate between steps; the ring slot of a
// step is read during two steps (lag-2 loader).
constexpr int kLoadWavesB = 4;
constexpr int kRingB = 6;  // even (buffer parity = slot parity); the loops unroll by it
constexpr int kSlotQ = 0, kSlotK = kTileBytes, kSlotV = 2 * kTileBytes, kSlotZ = 3 * kTileBytes;
constexpr int kSlotW = 4 * kTileBytes;
constexpr int kSlotE = kSlotW + kStateBytes;
constexpr int kSlotBBytes = kSlotE + 256;

template <bool kTok, bool kDot>
__global__ __launch_bounds__(64 * (2 * kWavesC + kLoadWavesB)) void linear_bwd_mfma_kernel(LinearBwdArgs a, const bf16* whist) {
  __shared__ __attribute__((aligned(16))) char ring_mem[kRingB * kSlotBBytes];
  __shared__ __attribute__((aligned(16))) char rt_mem[2 * kTileBytes];   // bf16 Rt rows [s][i]
  __shared__ __attribute__((aligned(16))) char dr_mem[2 * kTileBytes];   // bf16 dR rows [s][i]
  __shared__ __attribute__((aligned(16))) char g_mem[2 * kStateBytes];   // bf16 G rows [i][j]
  __shared__ __attribute__((aligned(16))) float de_mem[2 * kWavesC * kB];  // per-wave <dRt, R>
  lds_char* ring = (lds_char*)(ring_mem);
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
  const float* etok = kTok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;

  if (wv >= 2 * kWavesC) {
    // loader waves: 0 streams Q and K, 1 V and dZ, 2 and 3 half of W_c each; step k holds
    // chunk nchunks - 1 - k
    const int lw = wv - 2 * kWavesC;
    const char* wh = reinterpret_cast<const char*>(whist + static_cast<size_t>(chain) * nchunks * (kD * kD));
    const char* b0 = lw == 0 ? q : v;
    const char* b1 = lw == 0 ? k : dz;
    const int d0 = lw == 0 ? kSlotQ : kSlotV, d1 = lw == 0 ? kSlotK : kSlotZ;
    const int h0 = lw == 3 ? 4 : 0;
    const int s0 = src_off(0, lane), s1 = src_off(1, lane);
    loader_loop_lag2<kRingB, kTok ? 5 : 4>(nchunks, [&](int kk) {
      const int c = nchunks - 1 - kk;
      lds_char* dst = ring + (kk % kRingB) * kSlotBBytes;
      if (lw < 2) {
        const __amdgpu_buffer_rsrc_t r0 = tile_rsrc(b0, c, nchunks, seq_bytes);
        const __amdgpu_buffer_rsrc_t r1 = tile_rsrc(b1, c, nchunks, seq_bytes);
        load_lds(r0, dst + d0, s0);
        load_lds(r0, dst + d0 + 1024, s1);
        load_lds(r1, dst + d1, s0);
        load_lds(r1, dst + d1 + 1024, s1);
      } else {
        const bool live = c >= 0;
        const __amdgpu_buffer_rsrc_t rw =
            rsrc(wh + (live ? static_cast<size_t>(c) * kStateBytes : 0), live ? kStateBytes : 0);
#pragma unroll
        for (int h = 0; h < 4; ++h) load_lds(rw, dst + kSlotW + 1024 * (h0 + h), src_off(h0 + h, lane));
      }
      if constexpr (kTok) load_lds_e(etok, c, T, dst + kSlotE, lane);  // every loader, same bytes
    });
    return;
  }

  const float eta = a.eta;
  const char* dv = reinterpret_cast<const char*>(static_cast<bf16*>(a.dv) + tok0);
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // causal masks: P (rows t = 4 g + e, cols s = n) keeps s <= t; P^T (rows s, cols t) keeps s <= t
  bool keep_p[4], keep_t[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    keep_p[e] = n <= 4 * g + e;
    keep_t[e] = 4 * g + e <= n;
  }

  if (wv < kWavesC) {
    // ---------------- recursion wave: G^T tiles of the outputs i = 16 w + n, from
    // dL/dW_final (zeros without it)
    const int w = wv;
    float4_t gt[2][2];
    const float* dwo = a.dw_out ? a.dw_out + static_cast<size_t>(chain) * kD * kD : nullptr;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
      const float* wr = dwo ? dwo + (16 * w + n) * kD + 32 * kb + 8 * g : nullptr;
      gt[kb][0] = dwo ? *reinterpret_cast<const float4_t*>(wr) : zero4;
      gt[kb][1] = dwo ? *reinterpret_cast<const float4_t*>(wr + 4) : zero4;
    }
    // step kk (slot = kk % kRingB, passed as a constant in the unrolled loop so that every
    // LDS address is a loop-invariant register plus an immediate)
    auto step = [&](int kk, auto slot_c) __attribute__((always_inline)) {
      const int slot = slot_c;
      const int par = slot & 1;  // kRingB is even: the parity of kk
      lds_barrier();  // barrier kk: step kk's chunk is in its slot
      {
        const int c = nchunks - 1 - kk;
        const lds_char* sl = ring + slot * kSlotBBytes;
        const lds_char* sq = sl + kSlotQ;
        const lds_char* sk = sl + kSlotK;
        const lds_char* sz = sl + kSlotZ;
        lds_char* rtw = (lds_char*)(rt_mem) + par * kTileBytes;
        lds_char* drw = (lds_char*)(dr_mem) + par * kTileBytes;
        lds_char* gw = (lds_char*)(g_mem) + par * kStateBytes;

        bf16x8_t kr[2], qr[2], wop[2], gop[2];  // rows: K[n][..], Q[n][..], W[16 w + n][..], G[16 w + n][..]
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          kr[kb] = bf(lds_ld<u32x4>(sk + sw(n, 32 * kb + 8 * g)));
          qr[kb] = bf(lds_ld<u32x4>(sq + sw(n, 32 * kb + 8 * g)));
          wop[kb] = bf(lds_ld<u32x4>(sl + kSlotW + sw(16 * w + n, 32 * kb + 8 * g)));
          const u32x4 gu = cat_u(gt[kb][0], gt[kb][1]);
          gop[kb] = bf(gu);
          lds_st<u32x4>(gw + sw(16 * w + n, 32 * kb + 8 * g), gu);  // G rows for the G^T reads
        }
        // R^T (rows i = 16 w + 4 g + e, cols s = n) = W K^T - V^T
        float4_t rt = zero;
        if constexpr (!kDot) {
          rt = mfma(wop[0], kr[0], zero);
          rt = mfma(wop[1], kr[1], rt);
        }
        rt -= unpack4(lds_ld<u32x2>(sl + kSlotV + sw(n, 16 * w + 4 * g)));
        const float ecur = kTok ? lds_ld<float>(sl + kSlotE + 4 * n) : 1.0f;
        lds_st<u32x2>(rtw + sw(n, 16 * w + 4 * g), pack4(kTok ? rt * ecur : rt));
        // P = tril(Q K^T) (rows t = 4 g + e, cols s = n)
        float4_t pm = mfma(qr[0], kr[0], zero);
        pm = mfma(qr[1], kr[1], pm);
#pragma unroll
        for (int e = 0; e < 4; ++e) pm[e] = keep_p[e] ? pm[e] : 0.0f;
        // dR^T (rows i, cols s) = -eta (G K^T + dZ^T P)
        const u32x2 ztr = tr(sz, 4 * g + (n >> 2), 16 * w + 4 * (n & 3));  // dZ[4 g + s][16 w + n]
        float4_t drt = mfma(gop[0], kr[0], zero);
        drt = mfma(gop[1], kr[1], drt);
        drt = mfma(pad2(ztr), pad_op(pm), drt);
        drt *= -eta;
        if constexpr (kTok) {
          // this wave's share of de_s = <dRt_s, R_s>: its 16 outputs, over the four lane groups
          float p = 0.0f;
#pragma unroll
          for (int e = 0; e < 4; ++e) p += drt[e] * rt[e];
          p += __shfl_xor(p, 16, 64);
          p += __shfl_xor(p, 32, 64);
          lds_st<float>((lds_char*)(de_mem) + 4 * (par * kWavesC * kB + kB * w + n), p);
          drt *= ecur;  // dR = diag(e) dRt
        }
        // dV = -dR (token n, outputs 16 w + 4 g ..), dR rows to LDS
        __builtin_amdgcn_raw_buffer_store_b64(pack4(-drt), tile_rsrc(dv, c, nchunks, seq_bytes),
                                              n * kRowBytes + 32 * w + 8 * g, 0, 0);
        lds_st<u32x2>(drw + sw(n, 16 * w + 4 * g), pack4(drt));
        // G^T += Q^T dZ + K^T dR: slots 0..3 the dZ^T Q tokens, 4..7 the dR^T K tokens (dR
        // read back transposed from this wave's own rows)
        const bf16x8_t bup =
            join2(ztr, kDot ? u32x2{0u, 0u} : tr(drw, 4 * g + (n >> 2), 16 * w + 4 * (n & 3)));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int col = 32 * kb + 8 * (n & 3) + 4 * hf;
            const bf16x8_t aup = join2(tr(sq, 4 * g + (n >> 2), col), tr(sk, 4 * g + (n >> 2), col));
            gt[kb][hf] = mfma(aup, bup, gt[kb][hf]);
          }
      }
    };
    int kk = 0;
    for (; kk + kRingB <= nchunks; kk += kRingB) {
      step(kk, IC<0>{});
      step(kk + 1, IC<1>{});
      step(kk + 2, IC<2>{});
      step(kk + 3, IC<3>{});
      step(kk + 4, IC<4>{});
      step(kk + 5, IC<5>{});
    }
    for (; kk < nchunks; ++kk) step(kk, kk % kRingB);
    // the last step's G is dL/dW_0
    float* dw0 = a.dw0 + static_cast<size_t>(chain) * kD * kD;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float* wr = dw0 + (16 * w + n) * kD + 32 * kb + 8 * g;
      *reinterpret_cast<float4_t*>(wr) = gt[kb][0];
      *reinterpret_cast<float4_t*>(wr + 4) = gt[kb][1];
    }
    lds_barrier();  // barrier nchunks, for the gradient waves' last step
    return;
  }

  // ---------------- gradient wave: features j = 16 w + 4 g + e of the previous step's chunk
  const int w = wv - kWavesC;
  const char* dq = reinterpret_cast<const char*>(static_cast<bf16*>(a.dq) + tok0);
  const char* dk = reinterpret_cast<const char*>(static_cast<bf16*>(a.dk) + tok0);
  float* detok = kTok ? a.deta_tok : nullptr;
  if (detok) detok += static_cast<size_t>(chain) * T;
  // barrier kk (kk >= 1): step kk - 1's rows are in LDS; slot = (kk - 1) % kRingB, whose
  // parity is that of the buffers step kk - 1 wrote
  auto step = [&](int kk, auto slot_c) __attribute__((always_inline)) {
    const int slot = slot_c;
    const int par1 = slot & 1;
    lds_barrier();
    {
      const int c2 = nchunks - kk;  // the chunk of step kk - 1
      const lds_char* sl = ring + slot * kSlotBBytes;
      const lds_char* sq = sl + kSlotQ;
      const lds_char* sk = sl + kSlotK;
      const lds_char* sz = sl + kSlotZ;
      const lds_char* sw_ = sl + kSlotW;
      const lds_char* rtr = (lds_char*)(rt_mem) + par1 * kTileBytes;
      const lds_char* drr = (lds_char*)(dr_mem) + par1 * kTileBytes;
      const lds_char* gr = (lds_char*)(g_mem) + par1 * kStateBytes;
      // operands over outputs (tiles 2 h, 2 h + 1 side by side: k = 8 g + s' <->
      // i = 16 (2 h + s' / 4) + 4 g + s' % 4): dZ rows, Rt rows, dR rows of token n
      bf16x8_t zcat[2], rtop[2], drop[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        zcat[h] = join2(lds_ld<u32x2>(sz + sw(n, 32 * h + 4 * g)), lds_ld<u32x2>(sz + sw(n, 32 * h + 16 + 4 * g)));
        rtop[h] = join2(lds_ld<u32x2>(rtr + sw(n, 32 * h + 4 * g)), lds_ld<u32x2>(rtr + sw(n, 32 * h + 16 + 4 * g)));
        if constexpr (!kDot)
          drop[h] = join2(lds_ld<u32x2>(drr + sw(n, 32 * h + 4 * g)), lds_ld<u32x2>(drr + sw(n, 32 * h + 16 + 4 * g)));
      }
      // dP = -eta tril(dZ Rt^T) (rows t), dP^T (rows s)
      float4_t dp = mfma(zcat[0], rtop[0], zero);
      dp = mfma(zcat[1], rtop[1], dp);
      float4_t dpt = mfma(rtop[0], zcat[0], zero);
      dpt = mfma(rtop[1], zcat[1], dpt);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dp[e] = keep_p[e] ? -eta * dp[e] : 0.0f;
        dpt[e] = keep_t[e] ? -eta * dpt[e] : 0.0f;
      }
      // dQ^T (rows j, cols t) = W^T dZ^T + K^T dP^T;  dK^T (rows j, cols s) = -eta G^T Rt^T +
      // Q^T dP + W^T dR^T.  W^T and G^T rows j = 16 w + n over outputs i (transposing reads).
      float4_t xq = zero, xk = zero, xg = zero;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8_t wtr = join2(tr(sw_, 32 * h + 4 * g + (n >> 2), 16 * w + 4 * (n & 3)),
                                   tr(sw_, 32 * h + 16 + 4 * g + (n >> 2), 16 * w + 4 * (n & 3)));
        const bf16x8_t gtr = join2(tr(gr, 32 * h + 4 * g + (n >> 2), 16 * w + 4 * (n & 3)),
                                   tr(gr, 32 * h + 16 + 4 * g + (n >> 2), 16 * w + 4 * (n & 3)));
        xq = mfma(wtr, zcat[h], xq);
        if constexpr (!kDot) xk = mfma(wtr, drop[h], xk);
        xg = mfma(gtr, rtop[h], xg);
      }
      const bf16x8_t ktr = pad2(tr(sk, 4 * g + (n >> 2), 16 * w + 4 * (n & 3)));
      const bf16x8_t qtr = pad2(tr(sq, 4 * g + (n >> 2), 16 * w + 4 * (n & 3)));
      xq = mfma(ktr, pad_op(dpt), xq);
      xk = mfma(qtr, pad_op(dp), xk);
      xk += -eta * xg;
      __builtin_amdgcn_raw_buffer_store_b64(pack4(xq), tile_rsrc(dq, c2, nchunks, seq_bytes),
                                            n * kRowBytes + 32 * w + 8 * g, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b64(pack4(xk), tile_rsrc(dk, c2, nchunks, seq_bytes),
                                            n * kRowBytes + 32 * w + 8 * g, 0, 0);
      if constexpr (kTok) {
        // de of this chunk: the four recursion waves' shares, stored by gradient wave 0 (its
        // four lane groups write the same value)
        const lds_char* dsh = (lds_char*)(de_mem) + 4 * (par1 * kWavesC * kB + n);
        const float d = lds_ld<float>(dsh) + lds_ld<float>(dsh + 4 * kB) + lds_ld<float>(dsh + 8 * kB) +
                        lds_ld<float>(dsh + 12 * kB);
        const bool live = detok && w == 0;
        const int cnt = live ? (T - c2 * kB < kB ? T - c2 * kB : kB) : 0;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, d),
                                              rsrc(live ? detok + c2 * kB : detok, 4 * cnt), 4 * n, 0, 0);
      }
    }
  };
  lds_barrier();  // barrier 0
  int kk = 1;
  for (; kk + kRingB <= nchunks + 1; kk += kRingB) {
    step(kk, IC<0>{});
    step(kk + 1, IC<1>{});
    step(kk + 2, IC<2>{});
    step(kk + 3, IC<3>{});
    step(kk + 4, IC<4>{});
    step(kk + 5, IC<5>{});
  }
  for (; kk <= nchunks; ++kk) step(kk, (kk - 1) % kRingB);
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
  if (nchains > (1LL << 27)) return hipErrorInvalidValue;  // grids of at most 2^30 workgroups
  bf16* whist = static_cast<bf16*>(workspace);
  const dim3 grid(static_cast<unsigned>(nchains));
  const dim3 fgrid(static_cast<unsigned>((nchains + 7) / 8 * 8 * kSplitF));
  const dim3 fblock(64 * (kWavesF + kLoadWavesF + kStoreWavesF)), bblock(64 * (2 * kWavesC + kLoadWavesB));
  if ((fwd.eta_tok != nullptr) != (a.eta_tok != nullptr) || fwd.dot_loss != a.dot_loss)
    return hipErrorInvalidValue;
  const bf16* wc = static_cast<const bf16*>(whist);
  auto run = [&](auto fk, auto bk) {
    hipLaunchKernelGGL(fk, fgrid, fblock, 0, s, fwd, whist);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bk, grid, bblock, 0, s, a, wc);
    return hipGetLastError();
  };
  if (a.eta_tok && a.dot_loss)
    return run(linear_fwd_hist_kernel<true, true>, linear_bwd_mfma_kernel<true, true>);
  if (a.eta_tok) return run(linear_fwd_hist_kernel<true, false>, linear_bwd_mfma_kernel<true, false>);
  if (a.dot_loss) return run(linear_fwd_hist_kernel<false, true>, linear_bwd_mfma_kernel<false, true>);
  return run(linear_fwd_hist_kernel<false, false>, linear_bwd_mfma_kernel<false, false>);
}

}  // namespace ttt
