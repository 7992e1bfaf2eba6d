// Backward pass of the non-causal TTT layers (linear and 2-layer SiLU MLP inner models) on the
// vector ALUs: one full-batch step, or consecutive mini-batches over several epochs, scalar
// or per-token rates, the reconstruction or the negative dot-product loss, d in {16, 32, 64},
// hidden width <= 256, fp32 or bf16 I/O.  One workgroup of 1024 threads per (batch, head)
// chain.
//
// The outer loop trains the projections, the initial state and the rates through the inner
// updates (wmrh.cn summary of Sun et al. 2024, section 2.2, and section 2.2.3 for the rate;
// "Fast weights" page, opening paragraph and section 2; ViT3 news page, section 1: the
// keys and values are learned end to end).  Forward (ViT3 page, section 1, observation 2):
// steps s = 1..S over mini-batches of tokens, W_s = W_{s-1} - eta sum_t e_t grad l_t(W_{s-1}),
// then z_t = f(q_t; W_S).  Reverse mode (our derivation of the chain rule):
//   * queries: with P = dL/dW_S (the upstream state gradient plus the output terms),
//     linear:  dq = W^T dz,  P += dz q^T;
//     MLP (u = W1 q, a = phi(u)):  da = W2^T dz, du = da * phi'(u), dq = W1^T du,
//          P2 += dz a^T,  P1 += du q^T;
//   * each step, last first, from its start weights W and P = dL/dW_s, with c = -eta (the
//     cotangent of the step's gradient sum is c P), every token independently:
//     linear (r = W k - v, or -v with the dot loss; rt = e r; G = sum rt k^T):
//          drt = c P k,  dk = c P^T rt,  dr = e drt,  de = <drt, r>,
//          dW += dr k^T,  dk += W^T dr  (these two only when r depends on W, k),  dv = -dr;
//     MLP (u = W1 k, a = phi(u), s = phi'(u), o = W2 a, r = o - v or -v, rt = e r,
//          da0 = W2^T rt, du0 = da0 * s; G1 = sum du0 k^T, G2 = sum rt a^T):
//          drt = c P2 a,  da = c P2^T rt,  ddu0 = c P1 k,  dk = c P1^T du0,
//          dda0 = ddu0 * s,  ds = ddu0 * da0,  dW2 += rt dda0^T,  drt += W2 dda0,
//          dr = e drt,  de = <drt, r>,  dv = -dr,
//          (reconstruction loss) dW2 += dr a^T,  da += W2^T dr,
//          du = da * phi'(u) + ds * phi''(u),  dW1 += du k^T,  dk += W1^T du;
//     then dL/dW_{s-1} = P + dW.
// The step-start states come from a forward pass in the same kernel that stores them in a
// workspace; dk, dv and the rates' gradient accumulate there in fp32 (a token is visited
// once per epoch) and are converted at the end.  P lives in the dw outputs (read by every
// thread during a step); dW accumulates in registers of the thread that owns each entry.
#include "common.hpp"

namespace ttt {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxH = 256;
constexpr int kMaxOwn = 16;  // state entries per thread per matrix (up to 256 x 64 / 1024)

__device__ __forceinline__ float d2silu(float u) {  // SiLU''(u) = s (1 - s) (2 + u (1 - 2 s))
  const float s = sigmoidf_(u);
  return s * (1.0f - s) * (2.0f + u * (1.0f - 2.0f * s));
}

struct NcBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dz;
  const float* w1;  // linear: W0 [d][d]; MLP: W1 [h][d]
  const float* w2;  // MLP: W2 [d][h]
  long long w_batch_stride;
  const float* dw1_out;  // upstream gradients of the final states or null
  const float* dw2_out;
  const float* eta_tok;
  void* dq;
  void* dk;
  void* dv;
  float* dw1;      // [B][H] x state 1
  float* dw2;      // [B][H] x state 2 (MLP)
  float* deta_tok; // [B][H][T] or null
  float* ws;       // per chain: (S + 1) states, dk and dv accumulators [T][d], de [T]
  int B, H, T, d, h, chunk, epochs;
  float eta;
  int dot_loss;
};

template <bool kMlp>
__host__ __device__ inline size_t state_floats(int d, int h) {
  return kMlp ? 2 * static_cast<size_t>(h) * d : static_cast<size_t>(d) * d;
}
template <bool kMlp>
__host__ __device__ inline size_t ws_floats(int d, int h, int T, int steps) {
  return (steps + 1) * state_floats<kMlp>(d, h) + 2 * static_cast<size_t>(T) * d + T;
}
__host__ __device__ inline int tile_tokens(int h) { return h <= 128 ? 16 : 8; }
// LDS floats of the token and hidden tiles, and of the padded copies of the step's state and
// of P (rows padded by one float against bank conflicts)
__host__ __device__ inline size_t tile_lds_floats(int d, int h) {
  const int tb = tile_tokens(h);
  return static_cast<size_t>(tb) * (7 * d + 1) + static_cast<size_t>(tb) * h * 10;
}
__host__ __device__ inline size_t mat_lds_floats(bool mlp, int d, int h) {
  return mlp ? 2 * (static_cast<size_t>(h) * (d + 1) + static_cast<size_t>(d) * (h + 1))
             : 2 * static_cast<size_t>(d) * (d + 1);
}

// A row-major matrix in global memory or a padded copy in LDS.
struct Mat {
  const float* p;
  int ld;
  __device__ __forceinline__ float operator()(int r, int c) const { return p[r * ld + c]; }
};

// kOwn: state entries per thread per matrix (4 for states of up to 4096 entries, else 16);
// kLds: the step's state and P are read from padded LDS copies (when they fit), else from
// global memory through the caches
template <typename IO, int D, bool kMlp, int kOwn, bool kLds>
__global__ __launch_bounds__(kThreads) void nc_bwd_kernel(NcBwdArgs a) {
  extern __shared__ float lds[];
  const int h = kMlp ? a.h : 0;
  const int TB = tile_tokens(h);
  // token tiles [TB][D]
  float* Ks = lds;
  float* Vs = Ks + TB * D;   // values, or dZ in the query pass
  float* Xs = Vs + TB * D;   // queries
  float* Rr = Xs + TB * D;   // r
  float* Rt = Rr + TB * D;   // rt = e r
  float* Dr = Rt + TB * D;   // drt, then dr
  float* Dk = Dr + TB * D;   // dk (or dq)
  float* Es = Dk + TB * D;   // rate factors [TB] (0 on padded rows)
  // hidden tiles [TB][h]
  float* Hu = Es + TB;
  float* Ha = Hu + TB * h;
  float* Hs = Ha + TB * h;    // phi'(u)
  float* Hda0 = Hs + TB * h;  // da0
  float* Hdu0 = Hda0 + TB * h;  // du0
  float* Hda = Hdu0 + TB * h;   // da
  float* Hddu = Hda + TB * h;   // ddu0
  float* Hdda = Hddu + TB * h;  // dda0
  float* Hds = Hdda + TB * h;   // ds
  float* Hdu = Hds + TB * h;    // du
  // padded copies: state 1 [rows1][D + 1] (W1 [h][D] or W [D][D]), state 2 [D][h + 1] (MLP),
  // then P1, P2 likewise
  const int rows1 = kMlp ? h : D;
  float* Ml = Hdu + TB * h;
  float* Wl1 = Ml;
  float* Wl2 = Wl1 + rows1 * (D + 1);
  float* Pl1 = Wl2 + (kMlp ? D * (h + 1) : 0);
  float* Pl2 = Pl1 + rows1 * (D + 1);

  const int tid = threadIdx.x;
  const int chain = blockIdx.x;
  const int bi = chain / a.H, hi = chain - bi * a.H;
  const int T = a.T;
  const float eta = a.eta, c = -a.eta;
  const int mb = min(a.chunk, T);
  const int nmb = (T + mb - 1) / mb;
  const int S = nmb * a.epochs;
  const size_t n1 = kMlp ? static_cast<size_t>(h) * D : static_cast<size_t>(D) * D;  // state 1 size
  const size_t n2 = kMlp ? static_cast<size_t>(D) * h : 0;                          // state 2 size
  const size_t sf = n1 + n2;
  const size_t tok0 = static_cast<size_t>(chain) * T * D;
  const IO* q = static_cast<const IO*>(a.q) + tok0;
  const IO* k = static_cast<const IO*>(a.k) + tok0;
  const IO* v = static_cast<const IO*>(a.v) + tok0;
  const IO* dz = static_cast<const IO*>(a.dz) + tok0;
  const float* etok = a.eta_tok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
  float* ws = a.ws + static_cast<size_t>(chain) * ws_floats<kMlp>(D, h, T, S);
  float* hist = ws;                        // (S + 1) states
  float* dkacc = ws + (S + 1) * sf;        // [T][D]
  float* dvacc = dkacc + static_cast<size_t>(T) * D;
  float* deacc = dvacc + static_cast<size_t>(T) * D;
  float* P1 = a.dw1 + static_cast<size_t>(chain) * n1;
  float* P2 = kMlp ? a.dw2 + static_cast<size_t>(chain) * n2 : nullptr;

  // initial state into hist[0]; accumulators to zero
  {
    const float* s1 = a.w1 + bi * a.w_batch_stride + static_cast<long long>(hi) * n1;
    const float* s2 = kMlp ? a.w2 + bi * a.w_batch_stride + static_cast<long long>(hi) * n2 : nullptr;
    for (size_t e = tid; e < n1; e += kThreads) hist[e] = s1[e];
    for (size_t e = tid; e < n2; e += kThreads) hist[n1 + e] = s2[e];
    for (size_t e = tid; e < 2 * static_cast<size_t>(T) * D + T; e += kThreads) dkacc[e] = 0.0f;
  }
  __syncthreads();

  auto load_rows = [&](float* dst, const IO* src, int t0, int n) {
    for (int e = tid; e < TB * D; e += kThreads) {
      const int t = e / D;
      dst[e] = t < n ? to_f32(src[static_cast<size_t>(t0 + t) * D + (e % D)]) : 0.0f;
    }
  };
  auto load_rates = [&](int t0, int n) {
    for (int t = tid; t < TB; t += kThreads) Es[t] = t < n ? (etok ? etok[t0 + t] : 1.0f) : 0.0f;
  };
  // the state at `src` (state 1 then state 2) as Mats, copied into LDS with kLds; ends
  // synchronised when it copies
  auto state_mats = [&](const float* src, float* l1, float* l2, Mat& m1, Mat& m2) {
    if (kLds) {
      for (size_t e = tid; e < n1; e += kThreads) l1[(e / D) * (D + 1) + e % D] = src[e];
      if (kMlp)
        for (size_t e = tid; e < n2; e += kThreads) l2[(e / h) * (h + 1) + e % h] = src[n1 + e];
      __syncthreads();
      m1 = Mat{l1, D + 1};
      m2 = Mat{l2, h + 1};
    } else {
      m1 = Mat{src, D};
      m2 = Mat{src + n1, h};
    }
  };

  // Shared per-tile forward of a training step from state W (W1 = W, W2 = W + n1):
  // Hu, Ha, Hs; Rr, Rt; Hda0, Hdu0 (MLP).  Ends synchronised.
  auto tile_forward = [&](const Mat& W1, const Mat& W2) {
    if (kMlp) {
      for (int e = tid; e < TB * h; e += kThreads) {
        const int t = e / h, j = e % h;
        float u = 0.0f;
        for (int i = 0; i < D; ++i) u += W1(j, i) * Ks[t * D + i];
        Hu[e] = u;
        Ha[e] = silu_(u);
        Hs[e] = dsilu_(u);
      }
      __syncthreads();
    }
    for (int e = tid; e < TB * D; e += kThreads) {
      const int t = e / D, i = e % D;
      float o = 0.0f;
      if (!a.dot_loss) {
        if (kMlp)
          for (int j = 0; j < h; ++j) o += W2(i, j) * Ha[t * h + j];
        else
          for (int j = 0; j < D; ++j) o += W1(i, j) * Ks[t * D + j];
      }
      const float r = o - Vs[e];
      Rr[e] = r;
      Rt[e] = Es[t] * r;
    }
    __syncthreads();
    if (kMlp) {
      for (int e = tid; e < TB * h; e += kThreads) {
        const int t = e / h, j = e % h;
        float da0 = 0.0f;
        for (int i = 0; i < D; ++i) da0 += W2(i, j) * Rt[t * D + i];
        Hda0[e] = da0;
        Hdu0[e] = da0 * Hs[e];
      }
      __syncthreads();
    }
  };

  float acc1[kOwn], acc2[kOwn];

  // ---- forward: every step, storing its start state ----
  for (int s = 0; s < S; ++s) {
    const int m0 = (s % nmb) * mb, ns = min(mb, T - m0);
    const float* W = hist + static_cast<size_t>(s) * sf;
    Mat Wm1, Wm2;
    state_mats(W, Wl1, Wl2, Wm1, Wm2);
#pragma unroll
    for (int m = 0; m < kOwn; ++m) acc1[m] = acc2[m] = 0.0f;
    for (int t0 = 0; t0 < ns; t0 += TB) {
      const int n = min(TB, ns - t0);
      load_rows(Ks, k, m0 + t0, n);
      load_rows(Vs, v, m0 + t0, n);
      load_rates(m0 + t0, n);
      __syncthreads();
      tile_forward(Wm1, Wm2);
      // G1 += du0 k^T (MLP) or G += rt k^T (linear); G2 += rt a^T
#pragma unroll
      for (int m = 0; m < kOwn; ++m) {
        const size_t e = tid + static_cast<size_t>(m) * kThreads;
        if (e < n1) {
          const int r = static_cast<int>(e / D), j = static_cast<int>(e % D);
          float x = 0.0f;
          for (int t = 0; t < n; ++t) x += (kMlp ? Hdu0[t * h + r] : Rt[t * D + r]) * Ks[t * D + j];
          acc1[m] += x;
        }
        if (kMlp && e < n2) {
          const int i = static_cast<int>(e / h), j = static_cast<int>(e % h);
          float x = 0.0f;
          for (int t = 0; t < n; ++t) x += Rt[t * D + i] * Ha[t * h + j];
          acc2[m] += x;
        }
      }
      __syncthreads();
    }
    float* Wn = hist + static_cast<size_t>(s + 1) * sf;
#pragma unroll
    for (int m = 0; m < kOwn; ++m) {
      const size_t e = tid + static_cast<size_t>(m) * kThreads;
      if (e < n1) Wn[e] = W[e] - eta * acc1[m];
      if (kMlp && e < n2) Wn[n1 + e] = W[n1 + e] - eta * acc2[m];
    }
    __syncthreads();
  }

  // ---- queries: dq and P = dL/dW_S ----
  {
    Mat W1, W2;
    state_mats(hist + static_cast<size_t>(S) * sf, Wl1, Wl2, W1, W2);
#pragma unroll
    for (int m = 0; m < kOwn; ++m) {
      const size_t e = tid + static_cast<size_t>(m) * kThreads;
      acc1[m] = (e < n1 && a.dw1_out) ? a.dw1_out[static_cast<size_t>(chain) * n1 + e] : 0.0f;
      acc2[m] = (kMlp && e < n2 && a.dw2_out) ? a.dw2_out[static_cast<size_t>(chain) * n2 + e] : 0.0f;
    }
    IO* dq = static_cast<IO*>(a.dq) + tok0;
    for (int t0 = 0; t0 < T; t0 += TB) {
      const int n = min(TB, T - t0);
      load_rows(Xs, q, t0, n);
      load_rows(Vs, dz, t0, n);
      __syncthreads();
      if (kMlp) {
        for (int e = tid; e < TB * h; e += kThreads) {
          const int t = e / h, j = e % h;
          float u = 0.0f, da = 0.0f;
          for (int i = 0; i < D; ++i) {
            u += W1(j, i) * Xs[t * D + i];
            da += W2(i, j) * Vs[t * D + i];
          }
          Ha[e] = silu_(u);
          Hdu[e] = da * dsilu_(u);
        }
        __syncthreads();
      }
      for (int e = tid; e < TB * D; e += kThreads) {
        const int t = e / D, j = e % D;
        if (t >= n) continue;
        float x = 0.0f;
        if (kMlp)
          for (int r = 0; r < h; ++r) x += W1(r, j) * Hdu[t * h + r];
        else
          for (int i = 0; i < D; ++i) x += W1(i, j) * Vs[t * D + i];
        dq[static_cast<size_t>(t0 + t) * D + j] = from_f32<IO>(x);
      }
#pragma unroll
      for (int m = 0; m < kOwn; ++m) {
        const size_t e = tid + static_cast<size_t>(m) * kThreads;
        if (e < n1) {  // MLP: P1 += du q^T; linear: P += dz q^T
          const int r = static_cast<int>(e / D), j = static_cast<int>(e % D);
          float x = 0.0f;
          for (int t = 0; t < n; ++t) x += (kMlp ? Hdu[t * h + r] : Vs[t * D + r]) * Xs[t * D + j];
          acc1[m] += x;
        }
        if (kMlp && e < n2) {  // P2 += dz a^T
          const int i = static_cast<int>(e / h), j = static_cast<int>(e % h);
          float x = 0.0f;
          for (int t = 0; t < n; ++t) x += Vs[t * D + i] * Ha[t * h + j];
          acc2[m] += x;
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int m = 0; m < kOwn; ++m) {
      const size_t e = tid + static_cast<size_t>(m) * kThreads;
      if (e < n1) P1[e] = acc1[m];
      if (kMlp && e < n2) P2[e] = acc2[m];
    }
    __syncthreads();
  }

  // ---- steps in reverse ----
  for (int s = S - 1; s >= 0; --s) {
    const int m0 = (s % nmb) * mb, ns = min(mb, T - m0);
    Mat W1, W2, Pm1, Pm2;
    state_mats(hist + static_cast<size_t>(s) * sf, Wl1, Wl2, W1, W2);
    if (kLds) {
      for (size_t e = tid; e < n1; e += kThreads) Pl1[(e / D) * (D + 1) + e % D] = P1[e];
      if (kMlp)
        for (size_t e = tid; e < n2; e += kThreads) Pl2[(e / h) * (h + 1) + e % h] = P2[e];
      __syncthreads();
      Pm1 = Mat{Pl1, D + 1};
      Pm2 = Mat{Pl2, h + 1};
    } else {
      Pm1 = Mat{P1, D};
      Pm2 = Mat{P2, h};
    }
#pragma unroll
    for (int m = 0; m < kOwn; ++m) acc1[m] = acc2[m] = 0.0f;
    for (int t0 = 0; t0 < ns; t0 += TB) {
      const int n = min(TB, ns - t0);
      load_rows(Ks, k, m0 + t0, n);
      load_rows(Vs, v, m0 + t0, n);
      load_rates(m0 + t0, n);
      __syncthreads();
      tile_forward(W1, W2);
      if (kMlp) {
        // da = c P2^T rt,  ddu0 = c P1 k,  dda0 = ddu0 s,  ds = ddu0 da0
        for (int e = tid; e < TB * h; e += kThreads) {
          const int t = e / h, j = e % h;
          float da = 0.0f, ddu = 0.0f;
          for (int i = 0; i < D; ++i) {
            da += Pm2(i, j) * Rt[t * D + i];
            ddu += Pm1(j, i) * Ks[t * D + i];
          }
          Hda[e] = c * da;
          Hddu[e] = c * ddu;
          Hdda[e] = c * ddu * Hs[e];
          Hds[e] = c * ddu * Hda0[e];
        }
        __syncthreads();
        // drt = c P2 a + W2 dda0;  dk = c P1^T du0
        for (int e = tid; e < TB * D; e += kThreads) {
          const int t = e / D, i = e % D;
          float x = 0.0f, y = 0.0f, z = 0.0f;
          for (int j = 0; j < h; ++j) {
            x += Pm2(i, j) * Ha[t * h + j];
            y += W2(i, j) * Hdda[t * h + j];
            z += Pm1(j, i) * Hdu0[t * h + j];
          }
          Dr[e] = c * x + y;
          Dk[e] = c * z;
        }
      } else {
        // drt = c P k;  dk = c P^T rt
        for (int e = tid; e < TB * D; e += kThreads) {
          const int t = e / D, i = e % D;
          float x = 0.0f, z = 0.0f;
          for (int j = 0; j < D; ++j) {
            x += Pm1(i, j) * Ks[t * D + j];
            z += Pm1(j, i) * Rt[t * D + j];
          }
          Dr[e] = c * x;
          Dk[e] = c * z;
        }
      }
      __syncthreads();
      // de = <drt, r> (one thread per token), then dr = e drt
      for (int t = tid; t < TB; t += kThreads) {
        float x = 0.0f;
        for (int i = 0; i < D; ++i) x += Dr[t * D + i] * Rr[t * D + i];
        if (t < n) deacc[m0 + t0 + t] += x;
      }
      __syncthreads();
      for (int e = tid; e < TB * D; e += kThreads) Dr[e] *= Es[e / D];
      __syncthreads();
      if (kMlp) {
        // da += W2^T dr (reconstruction loss);  du = da phi'(u) + ds phi''(u)
        for (int e = tid; e < TB * h; e += kThreads) {
          const int t = e / h, j = e % h;
          float x = Hda[e];
          if (!a.dot_loss)
            for (int i = 0; i < D; ++i) x += W2(i, j) * Dr[t * D + i];
          Hdu[e] = x * Hs[e] + Hds[e] * d2silu(Hu[e]);
        }
        __syncthreads();
      }
      // dk += W1^T du (MLP) or W^T dr (linear, reconstruction loss); dv = -dr
      for (int e = tid; e < TB * D; e += kThreads) {
        const int t = e / D, j = e % D;
        if (t >= n) continue;
        float x = Dk[e];
        if (kMlp)
          for (int r = 0; r < h; ++r) x += W1(r, j) * Hdu[t * h + r];
        else if (!a.dot_loss)
          for (int i = 0; i < D; ++i) x += W1(i, j) * Dr[t * D + i];
        const size_t o = static_cast<size_t>(m0 + t0 + t) * D + j;
        dkacc[o] += x;
        dvacc[o] -= Dr[e];
      }
      // dW1 += du k^T (MLP) or dW += dr k^T (linear, reconstruction loss);
      // dW2 += rt dda0^T + dr a^T (the second term with the reconstruction loss)
#pragma unroll
      for (int m = 0; m < kOwn; ++m) {
        const size_t e = tid + static_cast<size_t>(m) * kThreads;
        if (e < n1 && (kMlp || !a.dot_loss)) {
          const int r = static_cast<int>(e / D), j = static_cast<int>(e % D);
          float x = 0.0f;
          for (int t = 0; t < n; ++t) x += (kMlp ? Hdu[t * h + r] : Dr[t * D + r]) * Ks[t * D + j];
          acc1[m] += x;
        }
        if (kMlp && e < n2) {
          const int i = static_cast<int>(e / h), j = static_cast<int>(e % h);
          float x = 0.0f;
          for (int t = 0; t < n; ++t)
            x += Rt[t * D + i] * Hdda[t * h + j] + (a.dot_loss ? 0.0f : Dr[t * D + i] * Ha[t * h + j]);
          acc2[m] += x;
        }
      }
      __syncthreads();
    }
    // dL/dW_{s-1} = P + dW
#pragma unroll
    for (int m = 0; m < kOwn; ++m) {
      const size_t e = tid + static_cast<size_t>(m) * kThreads;
      if (e < n1) P1[e] += acc1[m];
      if (kMlp && e < n2) P2[e] += acc2[m];
    }
    __syncthreads();
  }

  // ---- outputs: dk, dv in the I/O dtype, the rates' gradient ----
  IO* dk = static_cast<IO*>(a.dk) + tok0;
  IO* dv = static_cast<IO*>(a.dv) + tok0;
  for (size_t e = tid; e < static_cast<size_t>(T) * D; e += kThreads) {
    dk[e] = from_f32<IO>(dkacc[e]);
    dv[e] = from_f32<IO>(dvacc[e]);
  }
  if (a.deta_tok)
    for (int t = tid; t < T; t += kThreads) a.deta_tok[static_cast<size_t>(chain) * T + t] = deacc[t];
}

template <typename IO, int D, bool kMlp, int kOwn, bool kLds>
hipError_t launch_lds(const NcBwdArgs& a, hipStream_t s) {
  const int h = kMlp ? a.h : 0;
  const size_t lds = (tile_lds_floats(D, h) + (kLds ? mat_lds_floats(kMlp, D, h) : 0)) * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&nc_bwd_kernel<IO, D, kMlp, kOwn, kLds>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((nc_bwd_kernel<IO, D, kMlp, kOwn, kLds>), dim3(a.B * a.H), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <typename IO, int D, bool kMlp, int kOwn>
hipError_t launch_own(const NcBwdArgs& a, hipStream_t s) {
  const int h = kMlp ? a.h : 0;
  if ((tile_lds_floats(D, h) + mat_lds_floats(kMlp, D, h)) * sizeof(float) <= 160 * 1024)
    return launch_lds<IO, D, kMlp, kOwn, true>(a, s);
  return launch_lds<IO, D, kMlp, kOwn, false>(a, s);
}

template <typename IO, int D, bool kMlp>
hipError_t launch_one(const NcBwdArgs& a, hipStream_t s) {
  const size_t n = static_cast<size_t>(kMlp ? a.h : D) * D;
  if (n <= 4 * static_cast<size_t>(kThreads)) return launch_own<IO, D, kMlp, 4>(a, s);
  return launch_own<IO, D, kMlp, kMaxOwn>(a, s);
}

template <typename IO, bool kMlp>
hipError_t launch_d(const NcBwdArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_one<IO, 16, kMlp>(a, s);
    case 32: return launch_one<IO, 32, kMlp>(a, s);
    case 64: return launch_one<IO, 64, kMlp>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t nc_bwd_workspace_floats(bool mlp, int B, int H, int T, int d, int h, int chunk, int epochs) {
  const int mb = chunk < T ? chunk : T;
  const int steps = ((T + mb - 1) / mb) * epochs;
  const size_t per = mlp ? ws_floats<true>(d, h, T, steps) : ws_floats<false>(d, h, T, steps);
  return static_cast<size_t>(B) * H * per;
}

hipError_t launch_nc_bwd(bool mlp, const void* q, const void* k, const void* v, const void* dz,
                         const float* w1, const float* w2, long long w_batch_stride,
                         const float* dw1_out, const float* dw2_out, const float* eta_tok,
                         void* dq, void* dk, void* dv, float* dw1, float* dw2, float* deta_tok,
                         float* ws, int B, int H, int T, int d, int h, int chunk, int epochs,
                         float eta, int dot_loss, bool bf16_io, hipStream_t s) {
  if (T < 1 || chunk < 1 || epochs < 1 || (mlp && (h < 1 || h > kMaxH)) ||
      static_cast<size_t>(mlp ? h : d) * d > static_cast<size_t>(kMaxOwn) * kThreads)
    return hipErrorInvalidValue;
  NcBwdArgs a{q, k, v, dz, w1, w2, w_batch_stride, dw1_out, dw2_out, eta_tok, dq, dk, dv, dw1, dw2,
              deta_tok, ws, B, H, T, d, h, chunk, epochs, eta, dot_loss};
  if (mlp) return bf16_io ? launch_d<bf16, true>(a, s) : launch_d<float, true>(a, s);
  return bf16_io ? launch_d<bf16, false>(a, s) : launch_d<float, false>(a, s);
}

}  // namespace ttt
