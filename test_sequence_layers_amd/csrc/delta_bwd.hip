// Backward pass of the delta rule (the causal TTT-Linear layer with one token per step) on the
// matrix cores, taken 16 tokens at a time in the exact chunked form: reconstruction or negative
// dot-product loss, scalar rate or per-token rate factors (with their gradient), d in
// {16, 32, 64}, fp32 or bf16 I/O, fp32 arithmetic throughout.  One workgroup of 1024 threads
// (16 waves) per (batch, head) chain.
//
// Forward ("Fast weights" page, section 1: W_t = W_{t-1} - eta e_t (W_{t-1} k_t - v_t) k_t^T,
// z_t = W_t q_t), for a chunk of b tokens from W (our derivation, exact algebra):
//   X = K W^T - V (or -V),  L = eta stril(K K^T) diag(e),  Tm = (I + L)^-1,  R = Tm X,
//   Rt = diag(e) R,  Z = Q W^T - eta tril(Q K^T) Rt,  W_next = W - eta Rt^T K.
// (With the dot-product loss the error term is -v whatever W is, so R = X = -V and L = 0.)
// Reverse mode, with G = dL/dW_next and dZ (our derivation of the chain rule):
//   dRt = -eta (K G^T + P^T dZ),  dP = -eta tril(dZ Rt^T)  (P = tril(Q K^T)),
//   dQ = dZ W + dP K,  dK = -eta Rt G + dP^T Q  (+ the terms below),  dL/dW = G + dZ^T Q,
//   dR = diag(e) dRt,  de_t = <dRt_t, R_t>,
//   through R = Tm X:  dX = Tm^T dR,  dL_ts = -(dX R^T)_ts for s < t,
//   through L_ts = eta (k_t . k_s) e_s:  dk_t += eta sum_{s<t} dL_ts e_s k_s,
//     dk_s += eta sum_{t>s} dL_ts e_s k_t,  de_s += eta sum_{t>s} dL_ts (k_t . k_s),
//   through X = K W^T - V:  dV = -dX,  dK += dX W,  dL/dW += dX^T K  (not with the dot loss).
// The kernel first runs the chunked forward, storing every chunk-start state in a workspace,
// then walks the chunks backwards.  Tm comes from the product formula
// (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8) (L is strictly lower triangular, so L^16 = 0).
//
// Every product is a sum of 16 x 16 tiles C = A B formed by v_mfma_f32_16x16x4_f32 from
// operands in LDS: A stored by rows and B stored transposed, so that both run along the
// contraction index k.  Lane (g, n) takes the k range [g K/4, (g + 1) K/4) of row n of A and
// of column n of B, 16-byte LDS reads, one MFMA per k (the four lane groups' ranges together
// cover k once); the tile comes out in the C layout (lane (g, n): rows 4 g + e, column n),
// from which a 16-byte write stores it transposed and four scalar writes store it by rows.
// W (forward) and G (reverse) stay in registers, one 16 x 16 tile per wave, and are copied to
// LDS by rows and transposed after each update.  Within a phase different waves form
// independent products; LDS-only barriers separate the phases.
#include "common.hpp"

namespace ttt {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kC = 16;           // tokens per chunk
constexpr int kP16 = kC + 4;     // row pitch (floats) of matrices with 16 columns

typedef float float4_t __attribute__((ext_vector_type(4)));

template <int D>
struct DeltaLds {  // float offsets in the dynamic LDS block; every region 16-byte aligned
  static constexpr int PD = D + 4;                     // row pitch of matrices with D columns
  static constexpr int kDD = D * PD, kTD = kC * PD, kDT = D * kP16, kTT = kC * kP16;
  static constexpr int W = 0, WT = W + kDD, G = WT + kDD, GT = G + kDD,
                       K = GT + kDD, Q = K + kTD, DZ = Q + kTD, V = DZ + kTD, R = V + kTD, RT = R + kTD,
                       DRT = RT + kTD, DX = DRT + kTD, RG = DX + kTD,
                       KT = RG + kTD, QT = KT + kDT, DZT = QT + kDT, XT = DZT + kDT, RTT = XT + kDT,
                       DRTR = RTT + kDT, DXT = DRTR + kDT,
                       KK = DXT + kDT, P = KK + kTT, PT = P + kTT, DP = PT + kTT, DPT = DP + kTT,
                       DL = DPT + kTT, M = DL + kTT, TM = M + kTT, TMT = TM + kTT, PW = TMT + kTT,
                       PWT = PW + kTT, ET = PWT + kTT, DE = ET + kC, TOTAL = DE + kC;
};

// C (16 x 16) = A B with A by rows (row pitch lda, rows n of the tile) and B transposed (row
// pitch ldb): lane (g, n) sums over k in [g KK/4, (g + 1) KK/4).
template <int KK>
__device__ __forceinline__ float4_t mm_tile(const float* A, int lda, const float* Bt, int ldb, int g, int n) {
  constexpr int kq = KK / 4;
  const float* ar = A + n * lda + g * kq;
  const float* br = Bt + n * ldb + g * kq;
  float4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < kq; s += 4) {
    const float4_t a4 = *reinterpret_cast<const float4_t*>(ar + s);
    const float4_t b4 = *reinterpret_cast<const float4_t*>(br + s);
#pragma unroll
    for (int u = 0; u < 4; ++u) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[u], b4[u], c, 0, 0, 0);
  }
  return c;
}
// C = X^T Y for 16 x 16 tiles X, Y held in the C layout (lane (g, n): rows 4 g + e of column
// n): with the lane's k range [4 g, 4 g + 4), element s of its X tile is the A operand
// X^T[n][4 g + s] and element s of its Y tile the B operand Y[4 g + s][n].  So with M kept
// together with its transpose, M N = mm_reg(M^T, N) and (M N)^T = mm_reg(N, M^T).
__device__ __forceinline__ float4_t mm_reg(const float4_t& x, const float4_t& y) {
  float4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(x[s], y[s], c, 0, 0, 0);
  return c;
}
// a C-layout tile to LDS: by rows (element (4 g + e, n) at M[(4 g + e) ld + n]) or transposed
// (at Mt[n ldt + 4 g + e], one 16-byte write)
__device__ __forceinline__ void put_rows(float* M, int ld, const float4_t& c, int g, int n) {
#pragma unroll
  for (int e = 0; e < 4; ++e) M[(4 * g + e) * ld + n] = c[e];
}
__device__ __forceinline__ void put_cols(float* Mt, int ldt, const float4_t& c, int g, int n) {
  *reinterpret_cast<float4_t*>(Mt + n * ldt + 4 * g) = c;
}
// x, hidden from the optimiser: per-lane LDS addresses derived from it are formed where they
// are used instead of being hoisted out of the chunk loops (dozens of them would not fit in
// the 128 registers a wave of a 1024-thread workgroup has)
__device__ __forceinline__ int opaque(int x) {
  __asm__ __volatile__("" : "+v"(x));
  return x;
}
// Loads and stores through buffer resources whose range ends at the chunk's last token:
// rows past it read as zero and their stores are dropped, with no branch around the access
// (a load behind a branch costs a wait for every outstanding memory operation where the
// paths join).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes > 0 ? bytes : 0, 0x00020000);
}
// element e of a 32-bit word of IO elements
template <typename IO> __device__ __forceinline__ float word_elem(uint32_t w, int e);
template <> __device__ __forceinline__ float word_elem<float>(uint32_t w, int) { return __builtin_bit_cast(float, w); }
template <> __device__ __forceinline__ float word_elem<bf16>(uint32_t w, int e) {
  return __builtin_bit_cast(float, e ? (w & 0xFFFF0000u) : (w << 16));
}
__device__ __forceinline__ void st_io(float x, __amdgpu_buffer_rsrc_t r, int off) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, off, 0, 0);
}
__device__ __forceinline__ void st_io(bf16 x, __amdgpu_buffer_rsrc_t r, int off) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, x), r, off, 0, 0);
}
// Workgroup barrier for LDS traffic: this wave's LDS accesses are complete, then all waves
// meet.  The sweeps exchange data between waves only through LDS; a __syncthreads() would
// also wait for every outstanding global load (the next chunk's prefetch) once stores are in
// flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt unconstrained
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}
// Every outstanding global access of this wave is complete.  Issued a phase after a step's
// stores and before the next loads: with loads and stores in flight together the compiler can
// only wait for all of them, so the prefetched loads are never behind pending stores.
__device__ __forceinline__ void drain_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), lgkmcnt/expcnt unconstrained
}
// the wave's own LDS traffic is complete (LDS communication inside one wave)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __asm__ __volatile__("" ::: "memory");
}

template <typename IO, int D>
__global__ __launch_bounds__(kThreads) void delta_bwd_kernel(LinearBwdArgs a, const float* w0,
                                                             long long w0_batch_stride, float* hist) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  using L = DeltaLds<D>;
  constexpr int PD = L::PD;
  constexpr int nT = D / 16;  // 16-column tiles of a D-wide matrix
  float* sW = lds + L::W;
  float* sWT = lds + L::WT;
  float* sG = lds + L::G;
  float* sGT = lds + L::GT;
  float* sK = lds + L::K;
  float* sQ = lds + L::Q;
  float* sDZ = lds + L::DZ;
  float* sV = lds + L::V;
  float* sR = lds + L::R;      // R = Tm X (without the rates)
  float* sRt = lds + L::RT;    // Rt = diag(e) R
  float* sDRt = lds + L::DRT;  // dRt
  float* sDX = lds + L::DX;
  float* sRG = lds + L::RG;    // -eta Rt G
  float* sKT = lds + L::KT;
  float* sQT = lds + L::QT;
  float* sDZT = lds + L::DZT;
  float* sXT = lds + L::XT;
  float* sRtT = lds + L::RTT;  // Rt^T (forward)
  float* sDRT = lds + L::DRTR; // dR^T
  float* sDXT = lds + L::DXT;
  float* sKk = lds + L::KK;
  float* sP = lds + L::P;
  float* sPT = lds + L::PT;
  float* sDP = lds + L::DP;
  float* sDPT = lds + L::DPT;
  float* sDL = lds + L::DL;
  float* sM = lds + L::M;
  float* sTm = lds + L::TM;
  float* sTmT = lds + L::TMT;
  float* sPw = lds + L::PW;
  float* sPwT = lds + L::PWT;
  float* et = lds + L::ET;
  float* de1 = lds + L::DE;

  const int tid0 = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid0 >> 6);
  const int chain = blockIdx.x;
  const int bi = chain / a.H, hi = chain - bi * a.H;
  const int T = a.T;
  const float eta = a.eta;
  const bool dot = a.dot_loss != 0;
  const int nchunks = (T + kC - 1) / kC;
  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * D;
  const IO* q = static_cast<const IO*>(a.q) + tok0;
  const IO* k = static_cast<const IO*>(a.k) + tok0;
  const IO* v = static_cast<const IO*>(a.v) + tok0;
  const IO* dz = static_cast<const IO*>(a.dz) + tok0;
  IO* dq = static_cast<IO*>(a.dq) + tok0;
  IO* dk = static_cast<IO*>(a.dk) + tok0;
  IO* dv = static_cast<IO*>(a.dv) + tok0;
  float* wh = hist + static_cast<size_t>(chain) * nchunks * (D * D + 2 * kC * kC);
  const float* etok = a.eta_tok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
  float* detok = a.deta_tok ? a.deta_tok + static_cast<size_t>(chain) * T : nullptr;
  const float* w0c = w0 + bi * w0_batch_stride + static_cast<long long>(hi) * D * D;

  // the wave's tile of the D x D state (W forward, G reverse): rows 16 (wv / nT), columns
  // 16 (wv % nT); waves past nT^2 own none
  const bool owner = wv < nT * nT;
  const int sr = 16 * (wv / nT), sc = 16 * (wv % nT);
  // the state tile to LDS, by rows (M) and transposed (Mt)
  auto put_state = [&](float* M, float* Mt, const float4_t& c, int g, int n) {
    put_rows(M + sr * PD + sc, PD, c, g, n);
    put_cols(Mt + sc * PD + sr, PD, c, g, n);
  };
  // the state tile from a D x D row-major global array
  auto get_state = [&](const float* src, int g, int n) {
    float4_t c;
#pragma unroll
    for (int e = 0; e < 4; ++e) c[e] = src[(sr + 4 * g + e) * D + sc + n];
    return c;
  };

  // The workspace holds per chunk the chunk-start state (D x D), Tm and K K^T (16 x 16 each),
  // written by the forward sweep and read by the reverse one.
  constexpr int kWs = D * D + 2 * kC * kC;
  // A chunk's inputs are loaded into registers one chunk ahead and written to LDS at the
  // start of its step, so the loads overlap the previous step's work.  Thread x takes 32-bit
  // word x % W (W words per token row) of rows 4 (x / W) .. + 3 of the 16 x D token tiles (K,
  // V; Q, dZ reverse; zero past the sequence), so that a transposed copy of a column is one
  // 16-byte LDS write (and the loads are whole registers, with no packing that would wait
  // for them at once); thread
  // x < D^2 / 4 does the same for the chunk-start state (reverse); thread x < 512 takes one
  // entry of Tm or K K^T (reverse), thread x < 16 the rate factor of token x.
  constexpr int kEpw = 4 / static_cast<int>(sizeof(IO));  // elements per 32-bit word
  constexpr int kWpr = D / kEpw;                           // words per token row
  constexpr int kTokQ = 4 * kWpr;
  constexpr int kWQ = D * D / 4;
  uint32_t pk[4], pq[4], pz[4], pv[4];
  float pw[4];
  float pt = 0.0f, pe = 0.0f;
  auto prefetch = [&](int c, bool rev, int tid) {
    const int c0 = c * kC, nn = min(kC, T - c0);
    const float* whc = wh + static_cast<size_t>(c) * kWs;
    // Every load is issued by every thread, with no branch (a join of paths makes the compiler
    // wait for loads still in flight): the ranges end at the valid data, so the threads past
    // it read zeros without a memory access.
    {
      const int w = tid % kWpr, t4 = tid / kWpr;  // t4 >= 4: past the chunk
      const size_t base = static_cast<size_t>(c0) * D;
      const int bytes = nn * D * static_cast<int>(sizeof(IO));
      const __amdgpu_buffer_rsrc_t rk = span(k + base, bytes), rv = span(v + base, bytes);
      const __amdgpu_buffer_rsrc_t rq = span(q + base, bytes), rz = span(dz + base, bytes);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int off = (4 * t4 + u) * D * static_cast<int>(sizeof(IO)) + 4 * w;
        pk[u] = __builtin_amdgcn_raw_buffer_load_b32(rk, off, 0, 0);
        pv[u] = __builtin_amdgcn_raw_buffer_load_b32(rv, off, 0, 0);
        if (rev) {
          pq[u] = __builtin_amdgcn_raw_buffer_load_b32(rq, off, 0, 0);
          pz[u] = __builtin_amdgcn_raw_buffer_load_b32(rz, off, 0, 0);
        }
      }
    }
    // the workspace: written by other waves in the forward sweep, read past the L1 cache
    // (threads past the state or the 512 entries of Tm and K K^T read values they do not use,
    // or zeros past the workspace chunk)
    const __amdgpu_buffer_rsrc_t rw = span(whc, kWs * 4);
    if (rev) {
      const int j = tid % D, i4 = tid / D;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        pw[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, ((4 * i4 + u) * D + j) * 4, 0, 1));
      pt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, (D * D + tid) * 4, 0, 1));
    }
    // always issued (an empty range without rates), resolved when it is written to LDS
    pe = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
        span(etok ? etok + c0 : nullptr, etok ? nn * 4 : 0), tid * 4, 0, 0));
  };
  auto put_tok = [&](const uint32_t (&src)[4], float* M, float* Mt, int w, int t4) {
#pragma unroll
    for (int e = 0; e < kEpw; ++e) {
      const int j = kEpw * w + e;
      float4_t x;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        x[u] = word_elem<IO>(src[u], e);
        M[(4 * t4 + u) * PD + j] = x[u];
      }
      if (Mt) *reinterpret_cast<float4_t*>(Mt + j * kP16 + 4 * t4) = x;
    }
  };
  auto put_prefetched = [&](bool rev, int tid, int nn) {
    if (tid < kTokQ) {
      const int w = tid % kWpr, t4 = tid / kWpr;
      put_tok(pk, sK, sKT, w, t4);
      put_tok(pv, sV, nullptr, w, t4);
      if (rev) {
        put_tok(pq, sQ, sQT, w, t4);
        put_tok(pz, sDZ, sDZT, w, t4);
      }
    }
    if (rev && tid < kWQ) {
      const int j = tid % D, i4 = tid / D;
#pragma unroll
      for (int u = 0; u < 4; ++u) sW[(4 * i4 + u) * PD + j] = pw[u];
      *reinterpret_cast<float4_t*>(sWT + j * PD + 4 * i4) = float4_t{pw[0], pw[1], pw[2], pw[3]};
    }
    if (rev && tid < 2 * kC * kC) {
      const int r = (tid >> 4) & 15, cc = tid & 15;
      if (tid < kC * kC) {
        sTm[r * kP16 + cc] = pt;
        sTmT[cc * kP16 + r] = pt;
      } else {
        sKk[r * kP16 + cc] = pt;
      }
    }
    if (tid < kC) et[tid] = etok ? pe : (tid < nn ? 1.0f : 0.0f);
  };

  // Tm = (I + L)^-1 by the product formula, on wave 0 alone and in registers (every matrix
  // with its transpose): Tm <- I - L, then for p = L^2, L^4, L^8 (squaring p each time)
  // Tm <- Tm + Tm p.  Writes Tm by rows.
  auto form_tm = [&](int g, int n) {
    if (wv != 0) return;
    float4_t p, pt, tm, tmt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * g + e, s = n;
      p[e] = (s < t && !dot) ? eta * sKk[t * kP16 + s] * et[s] : 0.0f;     // L[t][s]
      pt[e] = (t < s && !dot) ? eta * sKk[s * kP16 + t] * et[t] : 0.0f;    // L^T[t][s] = L[s][t]
      tm[e] = (t == s ? 1.0f : 0.0f) - p[e];
      tmt[e] = (t == s ? 1.0f : 0.0f) - pt[e];
    }
    if (!dot) {
#pragma unroll
      for (int step = 0; step < 3; ++step) {
        const float4_t p2 = mm_reg(pt, p);   // P P
        const float4_t p2t = mm_reg(p, pt);  // (P P)^T = P^T P^T
        tm += mm_reg(tmt, p2);               // Tm P2
        tmt += mm_reg(p2, tmt);              // (Tm P2)^T = P2^T Tm^T
        p = p2;
        pt = p2t;
      }
    }
    put_rows(sTm, kP16, tm, g, n);
  };

  // ======================= forward: chunk-start states into the workspace =================
  float4_t st = {0.0f, 0.0f, 0.0f, 0.0f};  // the wave's state tile
  if (owner) {
    const int lane = tid0 & 63;
    st = get_state(w0c, lane >> 4, lane & 15);
    put_rows(sW + sr * PD + sc, PD, st, lane >> 4, lane & 15);
  }
  prefetch(0, false, tid0);
  lds_barrier();
  for (int c = 0; c < nchunks; ++c) {
    const int c0 = c * kC, nn = min(kC, T - c0);
    const int tid = opaque(tid0);
    const int lane = tid & 63;
    const int g = lane >> 4, n = lane & 15;
    // F0: K (by rows and transposed), V and the rates of this chunk into LDS; W_c, and Tm and
    // K K^T of the previous chunk (still in LDS; none before chunk 0) to the workspace
    put_prefetched(false, tid, nn);
    for (int e = tid; e < D * D; e += kThreads) wh[static_cast<size_t>(c) * kWs + e] = sW[(e / D) * PD + e % D];
    if (tid >= kThreads / 2) {
      const int e = tid - kThreads / 2;
      const int r = (e >> 4) & 15, cc = e & 15;
      const __amdgpu_buffer_rsrc_t rt = span(wh + static_cast<size_t>(max(c - 1, 0)) * kWs + D * D, c > 0 ? 2 * kC * kC * 4 : 0);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, (e < kC * kC ? sTm : sKk)[r * kP16 + cc]), rt, e * 4, 0, 0);
    }
    lds_barrier();
    // F1: X = K W^T - V (waves 0 .. nT-1, transposed into XT); K K^T (wave nT)
    if (wv < nT) {
      float4_t x = {0.0f, 0.0f, 0.0f, 0.0f};
      if (!dot) x = mm_tile<D>(sK, PD, sW + 16 * wv * PD, PD, g, n);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] -= sV[(4 * g + e) * PD + 16 * wv + n];
      put_cols(sXT + 16 * wv * kP16, kP16, x, g, n);
    } else if (wv == nT) {
      put_rows(sKk, kP16, mm_tile<D>(sK, PD, sK, PD, g, n), g, n);
    }
    // the next chunk's inputs, once this step's stores are complete (the last chunk's again at
    // the end: every step issues the same loads and stores)
    drain_vmem();
    prefetch(min(c + 1, nchunks - 1), false, tid);
    lds_barrier();
    form_tm(g, n);
    lds_barrier();
    // F3: R = Tm X, Rt = e R, transposed into RtT (waves 0 .. nT-1)
    if (wv < nT) {
      float4_t r = mm_tile<kC>(sTm, kP16, sXT + 16 * wv * kP16, kP16, g, n);
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] *= et[4 * g + e];
      put_cols(sRtT + 16 * wv * kP16, kP16, r, g, n);
    }
    lds_barrier();
    // F4: W -= eta Rt^T K (the owners; contraction over the chunk's tokens)
    if (owner) {
      st -= eta * mm_tile<kC>(sRtT + sr * kP16, kP16, sKT + sc * kP16, kP16, g, n);
      put_rows(sW + sr * PD + sc, PD, st, g, n);
    }
    lds_barrier();
  }
  if (tid0 >= kThreads / 2) {  // Tm and K K^T of the last chunk
    const int e = tid0 - kThreads / 2;
    const int r = (e >> 4) & 15, cc = e & 15;
    wh[static_cast<size_t>(nchunks - 1) * kWs + D * D + e] = (e < kC * kC ? sTm : sKk)[r * kP16 + cc];
  }

  // ======================= reverse ========================================================
  __syncthreads();  // the forward sweep's workspace stores are complete before any read
  if (owner) {
    const int lane = tid0 & 63;
    st = a.dw_out ? get_state(a.dw_out + static_cast<size_t>(chain) * D * D, lane >> 4, lane & 15)
                  : float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    put_state(sG, sGT, st, lane >> 4, lane & 15);
  }
  prefetch(nchunks - 1, true, tid0);
  // A step's outputs (dq; dk and dv; the rates' gradient), stored at the start of the next
  // step by the waves that hold them (an empty range in the first step, which has no earlier
  // outputs); the loads of the next prefetch wait until they are complete.
  float4_t o1 = {0.0f, 0.0f, 0.0f, 0.0f}, o2 = {0.0f, 0.0f, 0.0f, 0.0f};
  int oc0 = 0, onn = 0;
  auto store_outputs = [&](int c0, int nn, int g, int n, int lane) {
    const size_t base = static_cast<size_t>(c0) * D;
    const int bytes = nn * D * static_cast<int>(sizeof(IO));
    const bool isq = wv >= 2 * nT + 2 && wv < 3 * nT + 2, isk = wv >= nT + 2 && wv < 2 * nT + 2;
    const int jt = isq || isk ? (wv - nT - 2) % nT : 0;
    if (isq) {
      const __amdgpu_buffer_rsrc_t rq = span(dq + base, bytes);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        st_io(from_f32<IO>(o1[e]), rq, ((4 * g + e) * D + 16 * jt + n) * static_cast<int>(sizeof(IO)));
    } else if (isk) {
      const __amdgpu_buffer_rsrc_t rk = span(dk + base, bytes), rv = span(dv + base, bytes);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int off = ((4 * g + e) * D + 16 * jt + n) * static_cast<int>(sizeof(IO));
        st_io(from_f32<IO>(o1[e]), rk, off);
        st_io(from_f32<IO>(o2[e]), rv, off);
      }
    } else if (wv == 1 && detok) {
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o1[0]), span(detok + c0, nn * 4), lane * 4, 0, 0);
    }
  };
  for (int c = nchunks - 1; c >= 0; --c) {
    const int c0 = c * kC, nn = min(kC, T - c0);
    const int tid = opaque(tid0);
    const int lane = tid & 63;
    const int g = lane >> 4, n = lane & 15;
    lds_barrier();  // the later chunk's reads are done; G of the later chunk is in LDS
    // R0: W_c by rows and transposed; K, Q, dZ (by rows and transposed), V, Tm, K K^T, the
    // rates into LDS; the earlier chunk's into registers
    put_prefetched(true, tid, nn);
    store_outputs(oc0, onn, g, n, lane);
    lds_barrier();
    // R1: X = K W^T - V (waves 0 .. nT-1); P = tril(Q K^T) (nT + 1);
    //     K G^T (nT + 2 ..), dZ W (2 nT + 2 ..), kept in registers; then, once the stores
    //     above are complete, the earlier chunk's inputs (chunk 0's again at the end)
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const int jt = wv < nT + 2 ? 0 : (wv - nT - 2) % nT;  // column tile of the kept product
    if (wv < nT) {
      float4_t x = {0.0f, 0.0f, 0.0f, 0.0f};
      if (!dot) x = mm_tile<D>(sK, PD, sW + 16 * wv * PD, PD, g, n);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] -= sV[(4 * g + e) * PD + 16 * wv + n];
      put_cols(sXT + 16 * wv * kP16, kP16, x, g, n);
    } else if (wv == nT + 1) {
      float4_t p = mm_tile<D>(sQ, PD, sK, PD, g, n);
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = n <= 4 * g + e ? p[e] : 0.0f;
      put_rows(sP, kP16, p, g, n);
      put_cols(sPT, kP16, p, g, n);
    } else if (wv < 2 * nT + 2) {
      acc = mm_tile<D>(sK, PD, sG + 16 * jt * PD, PD, g, n);  // K G^T, columns 16 jt ..
    } else if (wv < 3 * nT + 2) {
      acc = mm_tile<D>(sDZ, PD, sWT + 16 * jt * PD, PD, g, n);  // dZ W, columns 16 jt ..
    }
    drain_vmem();
    prefetch(max(c - 1, 0), true, tid);
    lds_barrier();
    // R2: dRt = -eta (K G^T + P^T dZ) (nT + 2 ..): by rows, and dR = e dRt transposed (Tm,
    //     by rows and transposed, and K K^T came from the workspace)
    if (wv >= nT + 2 && wv < 2 * nT + 2) {
      float4_t d = acc + mm_tile<kC>(sPT, kP16, sDZT + 16 * jt * kP16, kP16, g, n);
      d = -eta * d;
      put_rows(sDRt + 16 * jt, PD, d, g, n);
#pragma unroll
      for (int e = 0; e < 4; ++e) d[e] *= et[4 * g + e];
      put_cols(sDRT + 16 * jt * kP16, kP16, d, g, n);
    }
    lds_barrier();
    // R3: R = Tm X, Rt = e R by rows (waves 0 .. nT-1); dX = Tm^T dR by rows and transposed
    //     (waves nT .. 2 nT - 1)
    if (wv < nT) {
      float4_t r = mm_tile<kC>(sTm, kP16, sXT + 16 * wv * kP16, kP16, g, n);
      put_rows(sR + 16 * wv, PD, r, g, n);
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] *= et[4 * g + e];
      put_rows(sRt + 16 * wv, PD, r, g, n);
    } else if (wv < 2 * nT) {
      const int it = wv - nT;
      const float4_t x = mm_tile<kC>(sTmT, kP16, sDRT + 16 * it * kP16, kP16, g, n);
      put_rows(sDX + 16 * it, PD, x, g, n);
      put_cols(sDXT + 16 * it * kP16, kP16, x, g, n);
    }
    lds_barrier();
    // R4: dP = -eta tril(dZ Rt^T) (wave 0), dL = -stril(dX R^T) (wave 1), -eta Rt G (waves
    //     2 .. nT+1, to RG), dX W (kept, waves nT + 2 .. 2 nT + 1); the new G (owners, in
    //     registers); <dRt_t, R_t> (threads of wave 15)
    float4_t dxw = {0.0f, 0.0f, 0.0f, 0.0f};
    if (wv == 0) {
      float4_t p = mm_tile<D>(sDZ, PD, sRt, PD, g, n);
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = n <= 4 * g + e ? -eta * p[e] : 0.0f;
      put_rows(sDP, kP16, p, g, n);
      put_cols(sDPT, kP16, p, g, n);
    } else if (wv == 1) {
      float4_t l = {0.0f, 0.0f, 0.0f, 0.0f};
      if (!dot) l = mm_tile<D>(sDX, PD, sR, PD, g, n);
#pragma unroll
      for (int e = 0; e < 4; ++e) l[e] = n < 4 * g + e ? -l[e] : 0.0f;
      put_rows(sDL, kP16, l, g, n);
    } else if (wv < nT + 2) {
      const int it = wv - 2;
      put_rows(sRG + 16 * it, PD, -eta * mm_tile<D>(sRt, PD, sGT + 16 * it * PD, PD, g, n), g, n);
    } else if (wv < 2 * nT + 2) {
      if (!dot) dxw = mm_tile<D>(sDX, PD, sWT + 16 * jt * PD, PD, g, n);
    }
    if (wv == kWaves - 1 && lane < kC) {
      float s = 0.0f;
      for (int i = 0; i < D; ++i) s += sDRt[lane * PD + i] * sR[lane * PD + i];
      de1[lane] = s;
    }
    if (owner) {  // dL/dW_c = G + dZ^T Q + dX^T K
      st += mm_tile<kC>(sDZT + sr * kP16, kP16, sQT + sc * kP16, kP16, g, n);
      if (!dot) st += mm_tile<kC>(sDXT + sr * kP16, kP16, sKT + sc * kP16, kP16, g, n);
    }
    lds_barrier();
    // R5: M_ts = dL_ts e_s (s < t) + dL_st e_t (s > t) (wave 0); the rates' gradient
    //     de_s = <dRt_s, R_s> + eta sum_{t>s} dL_ts (k_t . k_s) (wave 1); the new G to LDS
    //     (owners: every read of the old G is done); dQ = dZ W + dP K (2 nT + 2 ..)
    if (wv == 0) {
      float4_t m;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 4 * g + e, s = n;
        m[e] = s < t ? sDL[t * kP16 + s] * et[s] : (s > t ? sDL[s * kP16 + t] * et[t] : 0.0f);
      }
      put_rows(sM, kP16, m, g, n);
    } else if (wv == 1) {
      if (detok) {
        const int s = lane & 15;
        float x = de1[s];
        for (int t = s + 1; t < nn; ++t) x += eta * sDL[t * kP16 + s] * sKk[t * kP16 + s];
        o1[0] = x;  // stored (lanes s < nn) with the chunk's other outputs
      }
    }
    if (owner) put_state(sG, sGT, st, g, n);
    if (wv >= 2 * nT + 2 && wv < 3 * nT + 2) o1 = acc + mm_tile<kC>(sDP, kP16, sKT + 16 * jt * kP16, kP16, g, n);
    lds_barrier();
    // R6: dK = dX W - eta Rt G + dP^T Q + eta M K; dV = -dX (waves nT + 2 .. 2 nT + 1)
    if (wv >= nT + 2 && wv < 2 * nT + 2) {
      float4_t kk = dxw + mm_tile<kC>(sDPT, kP16, sQT + 16 * jt * kP16, kP16, g, n);
      if (!dot) kk += eta * mm_tile<kC>(sM, kP16, sKT + 16 * jt * kP16, kP16, g, n);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 4 * g + e;
        o1[e] = kk[e] + sRG[t * PD + 16 * jt + n];
        o2[e] = -sDX[t * PD + 16 * jt + n];
      }
    }
    oc0 = c0;
    onn = nn;
  }
  {
    const int lane = tid0 & 63;
    store_outputs(oc0, onn, lane >> 4, lane & 15, lane);
  }
  lds_barrier();
  float* dw0 = a.dw0 + static_cast<size_t>(chain) * D * D;
  for (int e = tid0; e < D * D; e += kThreads) dw0[e] = sG[(e / D) * PD + e % D];
}

template <typename IO, int D>
hipError_t launch_one(const LinearBwdArgs& a, const float* w0, long long stride, float* hist, hipStream_t s) {
  const size_t lds = DeltaLds<D>::TOTAL * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&delta_bwd_kernel<IO, D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((delta_bwd_kernel<IO, D>), dim3(a.B * a.H), dim3(kThreads), lds, s, a, w0, stride, hist);
  return hipGetLastError();
}

template <typename IO>
hipError_t launch_d(const LinearBwdArgs& a, const float* w0, long long stride, float* hist, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_one<IO, 16>(a, w0, stride, hist, s);
    case 32: return launch_one<IO, 32>(a, w0, stride, hist, s);
    case 64: return launch_one<IO, 64>(a, w0, stride, hist, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t delta_bwd_workspace_bytes(const LinearBwdArgs& a) {
  const size_t nchunks = (static_cast<size_t>(a.T) + kC - 1) / kC;
  return static_cast<size_t>(a.B) * a.H * nchunks * (a.d * a.d + 2 * kC * kC) * sizeof(float);
}

hipError_t launch_delta_bwd(const LinearBwdArgs& a, const float* w0, long long w0_batch_stride, void* ws,
                            bool bf16_io, hipStream_t s) {
  if (a.T < 1) return hipErrorInvalidValue;
  float* hist = static_cast<float*>(ws);
  return bf16_io ? launch_d<bf16>(a, w0, w0_batch_stride, hist, s) : launch_d<float>(a, w0, w0_batch_stride, hist, s);
}

}  // namespace ttt
