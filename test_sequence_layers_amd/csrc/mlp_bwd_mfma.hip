// Backward pass of the causal TTT-MLP layer on the gfx950 matrix cores: f(k) = W2 SiLU(W1 k),
// d = 64, hidden 256, mini-batch b = 16, bf16 Q/K/V/dZ/dQ/dK/dV, fp32 dL/dW1 and dL/dW2,
// reconstruction loss, scalar rate.
//
// The outer loop trains the projections and the initial states through the inner updates
// (wmrh.cn summary of Sun et al. 2024, section 2.2; "Fast weights" page, opening
// paragraph).  Forward chunk from W1, W2 (ViT3 news page, section 2, inner MLP; wmrh.cn
// summary, section 1.2.2, mini-batch rule), phi = SiLU, M = tril(Q K^T):
//   U = K W1^T, A = phi(U), R = A W2^T - V, Dm = R W2, dU = Dm * phi'(U),
//   Uq = Q W1^T - eta M dU, Aq = phi(Uq), N = tril(Aq A^T), Z = Aq W2^T - eta N R,
//   W1n = W1 - eta dU^T K,  W2n = W2 - eta R^T A.
// Reverse mode with G1 = dL/dW1n, G2 = dL/dW2n and dZ (our derivation of the chain rule):
//   Nb = -eta tril(dZ R^T),  dAq = dZ W2 + Nb A,  dUq = dAq * phi'(Uq),
//   Mb = -eta tril(dUq dU^T),  ddU = -eta M^T dUq - eta K G1^T,
//   dR = -eta N^T dZ - eta A G2^T + (ddU * phi'(U)) W2^T,  dV = -dR,
//   dA = Nb^T Aq - eta R G2 + dR W2,  dUk = dA * phi'(U) + ddU * Dm * phi''(U),
//   dQ = dUq W1 + Mb K,  dK = Mb^T Q - eta dU G1 + dUk W1,
//   G1 <- G1 + dUq^T Q + dUk^T K,  G2 <- G2 + dZ^T Aq + R^T (ddU * phi'(U)) + dR^T A.
// The chunk-start states come from the matrix-core forward kernel run in its history mode,
// which stores them as the bf16 values its products use (W1 rows [256][64], then W2 rows
// [64][256]: 64 KB per chunk); rows past T are zero everywhere and add nothing.
//
// Mapping.  One workgroup of 8 waves per (batch, head) chain walks the chunks from last to
// first:
//   * wave w owns hidden units 32 w .. 32 w + 31 and keeps its rows of G1 and columns of G2
//     in fp32 accumulator tiles;
//   * each wave loads its share of the next chunk's two states and Q, K, dZ tiles into the
//     other of two LDS buffers with direct-to-LDS loads;
//   * sums over hidden units: O = A W2^T is formed whole by waves 0..3 (one output tile
//     each) from the bf16 A^T operands all waves exchange through LDS; dR, dQ and dK, which
//     hold terms with the per-wave G slices, are summed from per-wave partial tiles in pairs
//     (waves 4..7 store, waves 0..3 add, then sum the four slots).  R and dR go to bf16 rows
//     in LDS.  Ten barriers per chunk.
//
// Layouts (v_mfma_f32_16x16x32_bf16; C layout: lane (g, n) = (lane / 16, lane % 16) holds
// rows 4 g + e, e = 0..3, of column n; A operand: lane holds A[n][8 g + s]; B: B[8 g + s][n]):
//   * every per-wave hidden-sized quantity X is held either as C-layout tiles with hidden
//     rows (X^T) or with token rows; a product with I converts one into the other;
//   * products over the wave's 32 hidden units take two X^T tiles side by side: k = 8 g + s
//     <-> hidden 16 (s / 4) + 4 g + s % 4 (W1 and W2 operands are read in that order);
//   * products over tokens take a token-row tile padded to K = 32 (k = 8 g + s, s < 4 <->
//     token 4 g + s), or the gfx950 transposing LDS read (ds_read_b64_tr_b16: within 16
//     lanes, lane i receives element i % 4 of the 8 bytes fetched by lane 4 s + i / 4) of a
//     row-major tile;
//   * products over features read 16-byte pieces of rows (k = 8 g + s <-> feature
//     32 h + 8 g + s), or, against tiles of G (C layout, 16 feature rows each), two 8-byte
//     reads (k <-> 32 h + 16 (s / 4) + 4 g + s % 4);
//   * G1 tiles: rows j = 16 jt + 4 g + e, columns hidden; G2 tiles: rows hidden, columns
//     i = 16 it + n.
// LDS rows (128 bytes for W1 and token tiles, 512 bytes for W2) hold 16-byte pieces XOR-
// swizzled in their low 3 bits by 2 (r % 4) + (r / 4) % 2, which keeps the transposing
// reads (4 rows by 32 bytes) and the 16-byte reads of 8 rows free of bank conflicts.
#include "common.hpp"

namespace ttt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kD = 64;
constexpr int kH = 256;
constexpr int kB = 16;
constexpr int kWaves = 8;  // hidden slices of 32
constexpr int kThreads = 64 * kWaves;
constexpr int kRow1 = kD * 2;  // bytes per row of W1 and of a token tile
constexpr int kRow2 = kH * 2;  // bytes per row of W2
constexpr int kW1Bytes = kH * kRow1;
constexpr int kHistBytes = kW1Bytes + kD * kRow2;  // one chunk's two states
constexpr int kTileBytes = kB * kRow1;
constexpr int kQ = 0, kK = kTileBytes, kZ = 2 * kTileBytes;
constexpr int kChunkBytes = 3 * kTileBytes;

// One chunk's inputs: its two states and its Q, K, dZ tiles.  The two buffers are separate
// LDS objects, so that the compiler can tell a read of one from the loads into the other.
struct Buf {
  char hist[kHistBytes];
  char chunk[kChunkBytes];
};
// Cross-wave sums: red[s][tile][lane], four slots of four C-layout tiles, lane-major (also
// the exchange of the waves' A^T operands, xch[wave][lane], in its first 8 KB).
struct Lds {
  float4_t red[4][4][64];
  char rb[kTileBytes];   // R, bf16 rows
  char drb[kTileBytes];  // dR, bf16 rows
};

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ bf16x8_t bf(const u32x4& x) { return __builtin_bit_cast(bf16x8_t, x); }
__device__ __forceinline__ u32x2 pack4(const float4_t& x, float s = 1.0f) {
  return u32x2{pack_bf16(s * x[0], s * x[1]), pack_bf16(s * x[2], s * x[3])};
}
__device__ __forceinline__ bf16x8_t join2(const u32x2& x, const u32x2& y) {
  const u32x4 u = {x.x, x.y, y.x, y.y};
  return bf(u);
}
__device__ __forceinline__ bf16x8_t pad2(const u32x2& x) {
  const u32x4 u = {x.x, x.y, 0u, 0u};
  return bf(u);
}
// two C-layout tiles side by side (slots 0..3, 4..7)
__device__ __forceinline__ bf16x8_t cat_op(const float4_t& x, const float4_t& y, float s = 1.0f) {
  return join2(pack4(x, s), pack4(y, s));
}
__device__ __forceinline__ float4_t mfma(const bf16x8_t& a, const bf16x8_t& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float bf_lo(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __builtin_bit_cast(float, x & 0xFFFF0000u); }

// SiLU and its first two derivatives: sigma (1 + u (1 - sigma)), sigma (1 - sigma) (2 + u (1 - 2 sigma))
__device__ __forceinline__ void silu3(float u, float& act, float& d1, float& d2) {
  const float sg = sigmoidf_(u);
  const float om = 1.0f - sg;
  act = u * sg;
  d1 = sg * __builtin_fmaf(u, om, 1.0f);
  d2 = sg * om * __builtin_fmaf(u, om - sg, 2.0f);
}
__device__ __forceinline__ void silu2(float u, float& act, float& d1) {
  const float sg = sigmoidf_(u);
  act = u * sg;
  d1 = sg * __builtin_fmaf(u, 1.0f - sg, 1.0f);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes > 0 ? bytes : 0, 0x00020000);
}

// 16 bytes per lane, global -> LDS (M0 = the wave's 1 KB destination block), issued from
// inline assembly so that the compiler's wait insertion does not see them (for the builtin
// it makes every LDS access it cannot prove disjoint, atomics included, wait for all
// outstanding loads); their completion is awaited explicitly (vmcnt) before the barrier that
// publishes them.  One wait state separates the M0 write from its use.
__device__ __forceinline__ u32x4 desc(const void* base, int bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return u32x4{static_cast<uint32_t>(p), static_cast<uint32_t>(p >> 32) & 0xFFFFu,
               static_cast<uint32_t>(bytes > 0 ? bytes : 0), 0x00020000u};
}
// (M0 is declared clobbered; this kernel has no other use of M0.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const u32x4& d, const lds_char* dst, int voff) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst));
  __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :
                   : "s"(m0), "v"(voff), "s"(d)
                   : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }
// byte offset of bf16 element (row, col) in LDS rows of kRowB bytes (col % 4 == 0)
template <int kRowB>
__device__ __forceinline__ int so(int row, int col) {
  return row * kRowB + (((col >> 3) ^ swz(row)) << 4) + 2 * (col & 7);
}
template <typename T>
__device__ __forceinline__ T lds_ld(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}
template <typename T>
__device__ __forceinline__ void lds_st(lds_char* p, T v) {
  *reinterpret_cast<__attribute__((address_space(3))) T*>(p) = v;
}
template <int kRowB>
__device__ __forceinline__ u32x4 rd16(const lds_char* b, int row, int col) {  // col % 8 == 0
  return lds_ld<u32x4>(b + so<kRowB>(row, col));
}
template <int kRowB>
__device__ __forceinline__ u32x2 rd8(const lds_char* b, int row, int col) {
  return lds_ld<u32x2>(b + so<kRowB>(row, col));
}
// transposing read: the lane fetches (row, col .. col + 3)
template <int kRowB>
__device__ __forceinline__ u32x2 trd(const lds_char* b, int row, int col) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + so<kRowB>(row, col))));
}

// Compiler-only fence: LDS values read before it are read again after it instead of being
// held in registers (register pressure).
__device__ __forceinline__ void reread() { __asm__ __volatile__("" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Barrier for LDS traffic only (the fence of __syncthreads() would drain outstanding stores);
// no instruction is scheduled across it (which keeps each phase's values out of the others'
// register budgets).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(kThreads) void mlp_bwd_mfma_kernel(MlpBwdArgs a, const char* hist) {
  __shared__ __attribute__((aligned(16))) Buf buf0;
  __shared__ __attribute__((aligned(16))) Buf buf1;
  __shared__ __attribute__((aligned(16))) Lds sh;
  lds_char* const rbl = (lds_char*)(&sh.rb[0]);
  lds_char* const drbl = (lds_char*)(&sh.drb[0]);

  const int chain = blockIdx.x;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g_ = lane >> 4;
  const int n_ = lane & 15;
  const int T = a.T;
  const int nchunks = (T + kB - 1) / kB;
  const int seq_bytes = T * kRow1;
  const float eta = a.eta;
  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * kD;
  const char* q = reinterpret_cast<const char*>(static_cast<const bf16*>(a.q) + tok0);
  const char* k = reinterpret_cast<const char*>(static_cast<const bf16*>(a.k) + tok0);
  const char* v = reinterpret_cast<const char*>(static_cast<const bf16*>(a.v) + tok0);
  const char* dz = reinterpret_cast<const char*>(static_cast<const bf16*>(a.dz) + tok0);
  char* dq = reinterpret_cast<char*>(static_cast<bf16*>(a.dq) + tok0);
  char* dk = reinterpret_cast<char*>(static_cast<bf16*>(a.dk) + tok0);
  char* dv = reinterpret_cast<char*>(static_cast<bf16*>(a.dv) + tok0);
  const char* hch = hist + static_cast<size_t>(chain) * nchunks * kHistBytes;


  const int h0 = 32 * wv;
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};

  // ---- G1, G2 (from the caller's gradients of the final states, or zero) ----
  const size_t hd = static_cast<size_t>(kH) * kD;
  float4_t g1t[4][2], g2t[2][4];
  {
    const float* i1 = a.dw1_out ? a.dw1_out + chain * hd : nullptr;
    const float* i2 = a.dw2_out ? a.dw2_out + chain * hd : nullptr;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int aa = 0; aa < 2; ++aa)
        g1t[jt][aa] = i1 ? *reinterpret_cast<const float4_t*>(i1 + (h0 + 16 * aa + n_) * kD + 16 * jt + 4 * g_) : zero;
#pragma unroll
    for (int aa = 0; aa < 2; ++aa)
#pragma unroll
      for (int it = 0; it < 4; ++it)
        g2t[aa][it] = i2 ? *reinterpret_cast<const float4_t*>(i2 + (16 * it + n_) * kH + h0 + 16 * aa + 4 * g_) : zero;
  }

  u32x4* const xch = reinterpret_cast<u32x4*>(&sh.red[0][0][0]);
  // Sum over the 8 waves of four C-layout tiles x (every wave calls it): waves 4..7 store,
  // waves 0..3 add their partner's and store; then slot s holds the sum of waves s, s + 4,
  // and wave w < 4 finishes tile w with sum4().
  // (lane indices below come from an opaque copy: recomputed, not held in registers)
  auto opaque_lane = [&]() {
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
    return ln;
  };
  auto reduce8 = [&](float4_t (&x)[4]) {
    const int ln = opaque_lane();
    if (wv >= 4) {
#pragma unroll
      for (int t = 0; t < 4; ++t) sh.red[wv - 4][t][ln] = x[t];
    }
    lds_barrier();
    if (wv < 4) {
#pragma unroll
      for (int t = 0; t < 4; ++t) sh.red[wv][t][ln] = x[t] + sh.red[wv][t][ln];
    }
    lds_barrier();
  };
  auto sum4 = [&]() {
    const int ln = opaque_lane();
    return sh.red[0][wv][ln] + sh.red[1][wv][ln] + sh.red[2][wv][ln] + sh.red[3][wv][ln];
  };

  // This wave's share of the loads of chunk c into buffer b: W1 rows 32 w .. 32 w + 31,
  // W2 rows 8 w .. 8 w + 7, and (waves 0..5) 8 rows of the Q, K or dZ tile, with direct-to-
  // LDS loads (1 KB each: lane l fills physical piece l % 8 of row l / 8, or piece l % 32 of
  // row l / 32 in W2, with the row's logical piece under the swizzle; rows past T read as
  // zero).
  auto issue = [&](Buf& b, int c) {
    // (offsets from an opaque copy of the lane index: recomputed here, not held in registers)
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
    const int r8 = ln >> 3;
    const int src8 = r8 * kRow1 + 16 * ((ln & 7) ^ swz(r8));
    const lds_char* hb = (const lds_char*)(&b.hist[0]);
    const u32x4 dh = desc(hch + static_cast<size_t>(c) * kHistBytes, kHistBytes);
#pragma unroll
    for (int m = 4 * wv; m < 4 * wv + 4; ++m) {
      dma16(dh, hb + 1024 * m, src8 + 1024 * m);
      const int row = 2 * m + (ln >> 5);
      dma16(dh, hb + kW1Bytes + 1024 * m, kW1Bytes + row * kRow2 + 16 * ((ln & 31) ^ swz(row)));
    }
    const int off = c * kTileBytes, m = wv & 1;
    const lds_char* cb = (const lds_char*)(&b.chunk[0]) + 1024 * m;
    if (wv < 2)
      dma16(desc(q + off, seq_bytes - off), cb + kQ, src8 + 1024 * m);
    else if (wv < 4)
      dma16(desc(k + off, seq_bytes - off), cb + kK, src8 + 1024 * m);
    else if (wv < 6)
      dma16(desc(dz + off, seq_bytes - off), cb + kZ, src8 + 1024 * m);
  };
  // V at this lane's place of output tile w % 4: V[n][16 (w % 4) + 4 g .. + 3]
  auto load_v = [&](int c) {
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
    const int off = c * kTileBytes;
    return __builtin_amdgcn_raw_buffer_load_b64(rsrc(v + off, seq_bytes - off), (ln & 15) * kRow1 + 32 * (wv & 3) + 8 * (ln >> 4), 0, 0);
  };

  // One chunk: its inputs in rd (V in vv), the next chunk's loads into wr (V into vv).
  auto run = [&](Buf& rd, Buf& wr, int c, u32x2& vv_io) {
    // the lane's coordinates, opaque to the compiler here: the many LDS offsets derived from
    // them are recomputed each chunk (a few ALU operations) instead of held in registers
    int g = g_, n = n_;
    __asm__ volatile("" : "+v"(g), "+v"(n));
    const uint32_t one = 0x3F80u;  // bf16 1.0
    const bf16x8_t eye = pad2(u32x2{(4 * g + 0 == n ? one : 0u) | (4 * g + 1 == n ? one << 16 : 0u),
                                    (4 * g + 2 == n ? one : 0u) | (4 * g + 3 == n ? one << 16 : 0u)});
    auto tp = [&](const float4_t& x) { return mfma(pad2(pack4(x)), eye, zero); };  // transpose of a tile
    // C-layout masks: keep = row 4 g + e <= column n; keepT = column n <= row 4 g + e
    bool keep[4], keepT[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      keep[e] = 4 * g + e <= n;
      keepT[e] = n <= 4 * g + e;
    }
    const lds_char* W1s = (const lds_char*)(&rd.hist[0]);
    const lds_char* W2s = W1s + kW1Bytes;
    const lds_char* Qs = (const lds_char*)(&rd.chunk[0]) + kQ;
    const lds_char* Ks = (const lds_char*)(&rd.chunk[0]) + kK;
    const lds_char* Zs = (const lds_char*)(&rd.chunk[0]) + kZ;
    const int off = c * kTileBytes;
    wait_vmcnt<0>();  // this wave's loads of chunk c
    lds_barrier();    // B0: chunk c is in rd; wr is free
    const u32x2 vv = vv_io;
    if (c > 0) {
      issue(wr, c - 1);
      vv_io = load_v(c - 1);
    }

    // ---- U^T = W1 K^T (rows hidden, cols t): A^T, phi'(U)^T, phi''(U)^T ----
    float4_t at[2], st[2], d2t[2];
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
      float4_t u = zero;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r = h0 + 16 * aa + n;
        const bf16x8_t w1 = join2(rd8<kRow1>(W1s, r, 32 * hh + 4 * g), rd8<kRow1>(W1s, r, 32 * hh + 16 + 4 * g));
        const bf16x8_t kj = join2(rd8<kRow1>(Ks, n, 32 * hh + 4 * g), rd8<kRow1>(Ks, n, 32 * hh + 16 + 4 * g));
        u = mfma(w1, kj, u);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x, y, w;
        silu3(u[e], x, y, w);
        at[aa][e] = x;
        st[aa][e] = y;
        d2t[aa][e] = w;
      }
    }
    const bf16x8_t atb = cat_op(at[0], at[1]);  // A rows t over hidden / A^T over hidden
    xch[wv * 64 + 16 * g + n] = __builtin_bit_cast(u32x4, atb);  // for O = A W2^T over all hidden units
    u32x2 ab[2];  // A with token rows (operand over tokens)
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) ab[aa] = pack4(tp(at[aa]));
    // P^T = K Q^T (rows s, cols t) and M = Q K^T (rows t, cols s), masked s <= t
    u32x2 ptb, mmb;
    {
      const u32x4 k0 = rd16<kRow1>(Ks, n, 8 * g), k1 = rd16<kRow1>(Ks, n, 32 + 8 * g);
      const u32x4 q0 = rd16<kRow1>(Qs, n, 8 * g), q1 = rd16<kRow1>(Qs, n, 32 + 8 * g);
      float4_t pt = mfma(bf(k1), bf(q1), mfma(bf(k0), bf(q0), zero));
      float4_t mm = mfma(bf(q1), bf(k1), mfma(bf(q0), bf(k0), zero));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pt[e] = keep[e] ? pt[e] : 0.0f;
        mm[e] = keepT[e] ? mm[e] : 0.0f;
      }
      ptb = pack4(pt);
      mmb = pack4(mm);
    }
    lds_barrier();  // B1

    // ---- waves 0..3: O^T tile w (rows i = 16 w + 4 g + e, cols t) = W2 A^T over all 256
    // hidden units (A^T operands of every wave); R = O - V to bf16 rows ----
    if (wv < 4) {
      float4_t x0 = zero, x1 = zero;
#pragma unroll
      for (int w = 0; w < kWaves; w += 2) {
        const int r = 16 * wv + n;
        x0 = mfma(join2(rd8<kRow2>(W2s, r, 32 * w + 4 * g), rd8<kRow2>(W2s, r, 32 * w + 16 + 4 * g)),
                  bf(xch[w * 64 + 16 * g + n]), x0);
        x1 = mfma(join2(rd8<kRow2>(W2s, r, 32 * w + 32 + 4 * g), rd8<kRow2>(W2s, r, 32 * w + 48 + 4 * g)),
                  bf(xch[(w + 1) * 64 + 16 * g + n]), x1);
      }
      const float4_t o = x0 + x1;
      const u32x2 rp = {pack_bf16(o[0] - bf_lo(vv.x), o[1] - bf_hi(vv.x)), pack_bf16(o[2] - bf_lo(vv.y), o[3] - bf_hi(vv.y))};
      lds_st<u32x2>(rbl + so<kRow1>(n, 16 * wv + 4 * g), rp);
    }
    lds_barrier();  // B2

    // ---- Dm^T = W2^T R^T; dU^T = Dm^T phi'; dd = Dm^T phi'' ----
    const u32x4 rn0 = rd16<kRow1>(rbl, n, 8 * g), rn1 = rd16<kRow1>(rbl, n, 32 + 8 * g);
    // W2 over outputs (32 h + 8 g + s), hidden columns h0 + 16 aa + n
    auto w2k = [&](int aa, int h) {
      const int col = h0 + 16 * aa + 4 * (n & 3);
      return join2(trd<kRow2>(W2s, 32 * h + 8 * g + (n >> 2), col), trd<kRow2>(W2s, 32 * h + 8 * g + 4 + (n >> 2), col));
    };
    float4_t dut[2], dd[2];
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
      const float4_t dm = mfma(w2k(aa, 1), bf(rn1), mfma(w2k(aa, 0), bf(rn0), zero));
      dut[aa] = dm * st[aa];
      dd[aa] = dm * d2t[aa];
    }
    const bf16x8_t duc = cat_op(dut[0], dut[1]);  // dU rows t over hidden / dU^T over hidden
    // ---- Uq (rows t) = Q W1^T - eta M dU;  Aq, phi'(Uq) ----
    float4_t aqt[2], sqt[2];
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
      float4_t u = mfma(pad2(ptb), pad2(pack4(tp(dut[aa]), -eta)), zero);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r = h0 + 16 * aa + n;
        const bf16x8_t w1 = join2(rd8<kRow1>(W1s, r, 32 * hh + 4 * g), rd8<kRow1>(W1s, r, 32 * hh + 16 + 4 * g));
        const bf16x8_t qj = join2(rd8<kRow1>(Qs, n, 32 * hh + 4 * g), rd8<kRow1>(Qs, n, 32 * hh + 16 + 4 * g));
        u = mfma(qj, w1, u);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x, y;
        silu2(u[e], x, y);
        aqt[aa][e] = x;
        sqt[aa][e] = y;
      }
    }
    u32x2 aqb[2];
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) aqb[aa] = pack4(aqt[aa]);
    const bf16x8_t aqc = cat_op(mfma(pad2(aqb[0]), eye, zero), mfma(pad2(aqb[1]), eye, zero));
    // N (rows t, cols s) = Aq A^T over this wave's hidden units, masked s <= t
    u32x2 nnb;
    {
      float4_t nn = mfma(aqc, atb, zero);
#pragma unroll
      for (int e = 0; e < 4; ++e) nn[e] = keepT[e] ? nn[e] : 0.0f;
      nnb = pack4(nn, -eta);  // operand -eta N^T (rows s over t)
    }
    // Nb^T (rows s, cols t) and Nb (rows t, cols s) = -eta tril(dZ R^T)
    reread();
    const u32x4 rn0b = rd16<kRow1>(rbl, n, 8 * g), rn1b = rd16<kRow1>(rbl, n, 32 + 8 * g);
    const u32x4 zn0 = rd16<kRow1>(Zs, n, 8 * g), zn1 = rd16<kRow1>(Zs, n, 32 + 8 * g);
    u32x2 nbtb, nbb;
    {
      float4_t nbt = mfma(bf(rn1b), bf(zn1), mfma(bf(rn0b), bf(zn0), zero));
      float4_t nb = mfma(bf(zn1), bf(rn1b), mfma(bf(zn0), bf(rn0b), zero));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        nbt[e] = keep[e] ? nbt[e] : 0.0f;
        nb[e] = keepT[e] ? nb[e] : 0.0f;
      }
      nbtb = pack4(nbt, -eta);
      nbb = pack4(nb, -eta);
    }
    // ---- dAq (rows t) = dZ W2 + Nb A;  dUq = dAq phi'(Uq) ----
    u32x2 duqb[2];
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
      float4_t x = mfma(pad2(nbtb), pad2(ab[aa]), zero);
      reread();
      x = mfma(bf(rd16<kRow1>(Zs, n, 8 * g)), w2k(aa, 0), x);
      x = mfma(bf(rd16<kRow1>(Zs, n, 32 + 8 * g)), w2k(aa, 1), x);
      duqb[aa] = pack4(x * sqt[aa]);
    }
    const bf16x8_t duqc = cat_op(mfma(pad2(duqb[0]), eye, zero), mfma(pad2(duqb[1]), eye, zero));
    // Mb (rows t, cols s) and Mb^T (rows s, cols t) over this wave's hidden units
    u32x2 mbb, mbtb;
    {
      float4_t mb = mfma(duqc, duc, zero);
      float4_t mbt = mfma(duc, duqc, zero);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mb[e] = keepT[e] ? mb[e] : 0.0f;
        mbt[e] = keep[e] ? mbt[e] : 0.0f;
      }
      mbb = pack4(mb, -eta);    // operand -eta Mb^T (rows s over t)
      mbtb = pack4(mbt, -eta);  // operand -eta Mb (rows t over s)
    }
    // ---- ddU^T (rows hidden, cols s) = -eta (dUq^T M + G1 K^T) ----
    float4_t dds[2], ddd[2];  // ddU phi'(U) and ddU Dm phi''(U), hidden rows
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
      float4_t x = mfma(pad2(duqb[aa]), pad2(mmb), zero);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const bf16x8_t kj = join2(rd8<kRow1>(Ks, n, 32 * hh + 4 * g), rd8<kRow1>(Ks, n, 32 * hh + 16 + 4 * g));
        x = mfma(cat_op(g1t[2 * hh][aa], g1t[2 * hh + 1][aa]), kj, x);
      }
      x = x * -eta;
      dds[aa] = x * st[aa];
      ddd[aa] = x * dd[aa];
    }
    const bf16x8_t ddsc = cat_op(dds[0], dds[1]);
    u32x2 ddsb[2];  // ddU phi'(U) with token rows
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) ddsb[aa] = pack4(tp(dds[aa]));
    // ---- dR^T (rows i, cols s) = -eta dZ^T N - eta G2 A^T + W2 (ddU phi')^T, summed ----
    {
      float4_t x[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = 16 * it + n;
        const bf16x8_t w2 = join2(rd8<kRow2>(W2s, r, h0 + 4 * g), rd8<kRow2>(W2s, r, h0 + 16 + 4 * g));
        const u32x2 ztr = trd<kRow1>(Zs, 4 * g + (n >> 2), 16 * it + 4 * (n & 3));
        x[it] = mfma(pad2(ztr), pad2(nnb), zero);
        x[it] = mfma(cat_op(g2t[0][it], g2t[1][it], -eta), atb, x[it]);
        x[it] = mfma(w2, ddsc, x[it]);
      }
      reduce8(x);
    }
    // ---- waves 0..3: dR[t][16 w + 4 g .. + 3] to bf16 rows; dV = -dR ----
    if (wv < 4) {
      const float4_t d4 = sum4();
      lds_st<u32x2>(drbl + so<kRow1>(n, 16 * wv + 4 * g), pack4(d4));
      __builtin_amdgcn_raw_buffer_store_b64(pack4(d4, -1.0f), rsrc(dv + off, seq_bytes - off),
                                            n * kRow1 + 32 * wv + 8 * g, 0, 0);
    }
    lds_barrier();  // dR rows complete

    // ---- dA^T (rows hidden, cols t) = Aq^T Nb - eta G2^T R^T + W2^T dR^T;  dUk^T ----
    const u32x4 drn0 = rd16<kRow1>(drbl, n, 8 * g), drn1 = rd16<kRow1>(drbl, n, 32 + 8 * g);
    float4_t dukt[2];
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
      float4_t x = mfma(pad2(aqb[aa]), pad2(nbb), zero);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8_t g2 = cat_op(tp(g2t[aa][2 * h]), tp(g2t[aa][2 * h + 1]), -eta);
        const bf16x8_t rj = join2(rd8<kRow1>(rbl, n, 32 * h + 4 * g), rd8<kRow1>(rbl, n, 32 * h + 16 + 4 * g));
        x = mfma(g2, rj, x);
      }
      x = mfma(w2k(aa, 0), bf(drn0), x);
      x = mfma(w2k(aa, 1), bf(drn1), x);
      dukt[aa] = x * st[aa] + ddd[aa];
    }
    const bf16x8_t dukc = cat_op(dukt[0], dukt[1]);
    u32x2 dukb[2];  // dUk with token rows
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) dukb[aa] = pack4(tp(dukt[aa]));
    // ---- G2^T += Aq^T dZ + (ddU phi')^T R + A^T dR (G2 has had its last use) ----
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int col = 16 * it + 4 * (n & 3);
      const u32x2 ztr = trd<kRow1>(Zs, 4 * g + (n >> 2), col);
      const u32x2 rtr = trd<kRow1>(rbl, 4 * g + (n >> 2), col);
      const u32x2 drtr = trd<kRow1>(drbl, 4 * g + (n >> 2), col);
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
        g2t[aa][it] = mfma(join2(aqb[aa], ddsb[aa]), join2(ztr, rtr), g2t[aa][it]);
        g2t[aa][it] = mfma(pad2(ab[aa]), pad2(drtr), g2t[aa][it]);
      }
    }
    // ---- dQ^T (rows j, cols t) = W1^T dUq^T + K^T Mb^T, summed; waves 0..3 store
    // dQ[t][16 w + 4 g .. + 3] ----
    {
      float4_t x[4];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int col = 16 * jt + 4 * (n & 3);
        const bf16x8_t w1h = join2(trd<kRow1>(W1s, h0 + 4 * g + (n >> 2), col), trd<kRow1>(W1s, h0 + 16 + 4 * g + (n >> 2), col));
        x[jt] = mfma(w1h, duqc, zero);
        x[jt] = mfma(pad2(trd<kRow1>(Ks, 4 * g + (n >> 2), col)), pad2(mbtb), x[jt]);
      }
      reduce8(x);
      if (wv < 4)
        __builtin_amdgcn_raw_buffer_store_b64(pack4(sum4()), rsrc(dq + off, seq_bytes - off), n * kRow1 + 32 * wv + 8 * g, 0, 0);
      lds_barrier();  // the dQ sums are read
    }
    // ---- dK^T (rows j, cols s) = Q^T Mb - eta G1^T dU^T + W1^T dUk^T (G1 before this
    // chunk's update), summed; waves 0..3 store dK ----
    {
      float4_t x[4];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int col = 16 * jt + 4 * (n & 3);
        const bf16x8_t w1h = join2(trd<kRow1>(W1s, h0 + 4 * g + (n >> 2), col), trd<kRow1>(W1s, h0 + 16 + 4 * g + (n >> 2), col));
        x[jt] = mfma(pad2(trd<kRow1>(Qs, 4 * g + (n >> 2), col)), pad2(mbb), zero);
        x[jt] = mfma(cat_op(tp(g1t[jt][0]), tp(g1t[jt][1]), -eta), duc, x[jt]);
        x[jt] = mfma(w1h, dukc, x[jt]);
        __builtin_amdgcn_sched_barrier(0);  // one tile at a time (register pressure)
      }
      reduce8(x);
      if (wv < 4)
        __builtin_amdgcn_raw_buffer_store_b64(pack4(sum4()), rsrc(dk + off, seq_bytes - off), n * kRow1 + 32 * wv + 8 * g, 0, 0);
    }
    // ---- G1^T += Q^T dUq + K^T dUk ----
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const int col = 16 * jt + 4 * (n & 3);
      const bf16x8_t qk = join2(trd<kRow1>(Qs, 4 * g + (n >> 2), col), trd<kRow1>(Ks, 4 * g + (n >> 2), col));
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) g1t[jt][aa] = mfma(qk, join2(duqb[aa], dukb[aa]), g1t[jt][aa]);
    }
  };

  issue(buf0, nchunks - 1);
  u32x2 vv = load_v(nchunks - 1);
  // chunks from last to first, alternating buffers (step s holds chunk nchunks - 1 - s in
  // buf0 for even s, buf1 for odd s)
  for (int s = 0; s < nchunks; s += 2) {
    run(buf0, buf1, nchunks - 1 - s, vv);
    if (s + 1 < nchunks) run(buf1, buf0, nchunks - 2 - s, vv);
  }

  // ---- dL/dW1, dL/dW2 of the initial states ----
  float* o1 = a.dw1 + chain * hd;
  float* o2 = a.dw2 + chain * hd;
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int aa = 0; aa < 2; ++aa)
      *reinterpret_cast<float4_t*>(o1 + (h0 + 16 * aa + n_) * kD + 16 * jt + 4 * g_) = g1t[jt][aa];
#pragma unroll
  for (int aa = 0; aa < 2; ++aa)
#pragma unroll
    for (int it = 0; it < 4; ++it)
      *reinterpret_cast<float4_t*>(o2 + (16 * it + n_) * kH + h0 + 16 * aa + 4 * g_) = g2t[aa][it];
}

}  // namespace

bool mlp_bwd_mfma_supported(const MlpBwdArgs& a, bool bf16_io) {
  auto al = [](const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & (m - 1)) == 0; };
  const bool aligned = al(a.q, 16) && al(a.k, 16) && al(a.v, 16) && al(a.dz, 16) && al(a.dq, 16) &&
                       al(a.dk, 16) && al(a.dv, 16) && al(a.dw1, 16) && al(a.dw2, 16) &&
                       (a.dw1_out == nullptr || al(a.dw1_out, 16)) && (a.dw2_out == nullptr || al(a.dw2_out, 16));
  const bool fits = static_cast<long long>(a.T) * kRow1 + 2LL * kTileBytes < 0x7fffffffLL;
  return bf16_io && a.d == kD && a.dh == kH && a.chunk == kB && a.T > 0 && aligned && fits;
}

size_t mlp_bwd_mfma_workspace_bytes(const MlpBwdArgs& a) {
  const size_t nchunks = (static_cast<size_t>(a.T) + kB - 1) / kB;
  return static_cast<size_t>(a.B) * a.H * nchunks * kHistBytes;
}

// The history run of the forward kernel must have written ws for the same inputs.
hipError_t launch_mlp_bwd_mfma(const MlpBwdArgs& a, const void* ws, hipStream_t s) {
  const long long nchains = static_cast<long long>(a.B) * a.H;
  if (nchains > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(nchains)), block(kThreads);
  hipLaunchKernelGGL(mlp_bwd_mfma_kernel, grid, block, 0, s, a, static_cast<const char*>(ws));
  return hipGetLastError();
}

}  // namespace ttt
