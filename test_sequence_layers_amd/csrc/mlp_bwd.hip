// Backward pass of the causal TTT-MLP layer on the vector ALUs: f(k) = W2 SiLU(W1 k),
// reconstruction loss or the negative dot-product loss (ViT3 news page, section 2), scalar
// rate or per-token rate factors, chunk <= 16, hidden width <= 256, d in {16, 32, 64}, fp32 or
// bf16 I/O.  One workgroup of 1024 threads per (batch, head) chain walks the chunks from last
// to first.
//
// The outer loop trains the projections and the initial states through the inner updates
// (wmrh.cn summary of Sun et al. 2024, section 2.2; "Fast weights" page, opening
// paragraph).  Forward chunk from W1, W2 (ViT3 news page, section 2, inner MLP; wmrh.cn
// summary, section 1.2.2, mini-batch rule), phi = SiLU, M = tril(Q K^T):
//   U = K W1^T, A = phi(U), R = A W2^T - V, Dm = R W2, dU = Dm * phi'(U),
//   W1n = W1 - eta dU^T K,  W2n = W2 - eta R^T A,
//   Uq = Q W1^T - eta M dU, Aq = phi(Uq), N = tril(Aq A^T), Z = Aq W2^T - eta N R.
// Reverse mode, with G1 = dL/dW1n, G2 = dL/dW2n from the later chunks and dZ (our
// derivation of the chain rule through these lines, last line first):
//   Nb = -eta tril(dZ R^T),  dAq = dZ W2 + Nb A,  dA = Nb^T Aq,  dR = -eta N^T dZ,
//   dUq = dAq * phi'(Uq),  Mb = -eta tril(dUq dU^T),  ddU = -eta M^T dUq - eta K G1^T,
//   dR += -eta A G2^T + (ddU * phi'(U)) W2^T,  dA += -eta R G2 + dR W2,
//   dUk = dA * phi'(U) + ddU * Dm * phi''(U),
//   dQ = dUq W1 + Mb K,  dK = Mb^T Q - eta dU G1 + dUk W1,  dV = -dR,
//   dL/dW1 = G1 + dUq^T Q + dUk^T K,  dL/dW2 = G2 + dZ^T Aq + R^T (ddU * phi'(U)) + dR^T A.
// With the dot-product loss R = -V depends on neither A nor W2, so the dR W2 term of dUk and
// the dR^T A term of dL/dW2 drop out (dV = -dR still holds).
// With per-token rate factors e (token t learns at eta e_t; wmrh.cn summary, section 2.2.3)
// every line above holds with Rt = diag(e) R in place of R, where R enters the update, the
// outputs and Dm (our derivation): the lines give dRt, and then dR = diag(e) dRt (the path
// through R = A W2^T - V: dV, dR W2, dR^T A) and de_t = <dRt_t, R_t>.
// G1 and G2 accumulate in the dw1 / dw2 outputs (read and written by the owning threads);
// the chunk-start states come from a forward recomputation that stores them (w_hist).
#include "common.hpp"

namespace ttt {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxB = 16;
constexpr int kMaxH = 256;

__device__ __forceinline__ float d2silu_(float u) {  // SiLU''(u) = s (1 - s) (2 + u (1 - 2 s))
  const float s = sigmoidf_(u);
  return s * (1.0f - s) * (2.0f + u * (1.0f - 2.0f * s));
}

template <int D>
struct BwdLds {  // float offsets in the dynamic LDS block for hidden width h (row stride h)
  static __host__ __device__ size_t tok(int i) { return static_cast<size_t>(i) * kMaxB * D; }  // 7 [b][D] + rates
  static __host__ __device__ size_t sq(int i) { return tok(8) + static_cast<size_t>(i) * kMaxB * kMaxB; }  // 4 [b][b]
  static __host__ __device__ size_t hid(int i, int h) { return sq(4) + static_cast<size_t>(i) * kMaxB * h; }  // 7 [b][h]
  static __host__ __device__ size_t total(int h) { return hid(7, h); }
};

template <typename IO, int D>
__global__ __launch_bounds__(kThreads) void mlp_bwd_generic_kernel(MlpBwdArgs a) {
  extern __shared__ float lds[];
  const int h = a.dh;
  float* Ks = lds + BwdLds<D>::tok(0);
  float* Qs = lds + BwdLds<D>::tok(1);
  float* Vs = lds + BwdLds<D>::tok(2);
  float* Zb = lds + BwdLds<D>::tok(3);   // dZ
  float* Rs = lds + BwdLds<D>::tok(4);   // Rt = diag(e) R
  float* Rb = lds + BwdLds<D>::tok(5);   // dRt, then dR
  float* Rr = lds + BwdLds<D>::tok(6);   // R (with per-token rates)
  float* Es = lds + BwdLds<D>::tok(7);   // rate factors [kMaxB] (1 without)
  float* Mm = lds + BwdLds<D>::sq(0);    // tril(Q K^T)
  float* Nn = lds + BwdLds<D>::sq(1);    // tril(Aq A^T)
  float* Nb = lds + BwdLds<D>::sq(2);
  float* Mb = lds + BwdLds<D>::sq(3);
  float* Hu = lds + BwdLds<D>::hid(0, h);   // U
  float* Ha = lds + BwdLds<D>::hid(1, h);   // A
  float* Hdu = lds + BwdLds<D>::hid(2, h);  // dU
  float* Haq = lds + BwdLds<D>::hid(3, h);  // Aq
  float* Huq = lds + BwdLds<D>::hid(4, h);  // Uq, then dUq
  float* Hda = lds + BwdLds<D>::hid(5, h);  // dA, then dUk
  float* Hdd = lds + BwdLds<D>::hid(6, h);  // ddU

  const int tid = threadIdx.x;
  const int chain = blockIdx.x;
  const int T = a.T;
  const float eta = a.eta;
  const int b = min(a.chunk, T);
  const int nchunks = (T + b - 1) / b;
  const size_t hd = static_cast<size_t>(h) * D;
  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * D;
  const IO* q = static_cast<const IO*>(a.q) + tok0;
  const IO* k = static_cast<const IO*>(a.k) + tok0;
  const IO* v = static_cast<const IO*>(a.v) + tok0;
  const IO* dz = static_cast<const IO*>(a.dz) + tok0;
  IO* dq = static_cast<IO*>(a.dq) + tok0;
  IO* dk = static_cast<IO*>(a.dk) + tok0;
  IO* dv = static_cast<IO*>(a.dv) + tok0;
  float* G1 = a.dw1 + static_cast<size_t>(chain) * hd;  // [h][D]
  float* G2 = a.dw2 + static_cast<size_t>(chain) * hd;  // [D][h]

  const float* etok = a.eta_tok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
  for (size_t e = tid; e < hd; e += kThreads) {
    G1[e] = a.dw1_out ? a.dw1_out[static_cast<size_t>(chain) * hd + e] : 0.0f;
    G2[e] = a.dw2_out ? a.dw2_out[static_cast<size_t>(chain) * hd + e] : 0.0f;
  }

  for (int c = nchunks - 1; c >= 0; --c) {
    const int c0 = c * b;
    const int n = min(b, T - c0);
    const float* W1 = a.w_hist + (static_cast<size_t>(chain) * nchunks + c) * 2 * hd;  // [h][D]
    const float* W2 = W1 + hd;                                                          // [D][h]
    __syncthreads();  // the previous chunk is done with every buffer; G1, G2 are complete
    for (int e = tid; e < kMaxB * D; e += kThreads) {
      const int t = e / D;
      const bool in = t < n;
      const size_t off = static_cast<size_t>(c0) * D + e;
      Ks[e] = in ? to_f32(k[off]) : 0.0f;
      Qs[e] = in ? to_f32(q[off]) : 0.0f;
      Vs[e] = in ? to_f32(v[off]) : 0.0f;
      Zb[e] = in ? to_f32(dz[off]) : 0.0f;
    }
    for (int t = tid; t < kMaxB; t += kThreads) Es[t] = (etok && t < n) ? etok[c0 + t] : 1.0f;
    __syncthreads();
    // U = K W1^T, A = phi(U);  M = tril(Q K^T)
    for (int e = tid; e < kMaxB * h; e += kThreads) {
      const int t = e / h, cc = e % h;
      float u = 0.0f;
      for (int j = 0; j < D; ++j) u += Ks[t * D + j] * W1[static_cast<size_t>(cc) * D + j];
      Hu[e] = u;
      Ha[e] = silu_(u);
    }
    for (int e = tid; e < kMaxB * kMaxB; e += kThreads) {
      const int t = e / kMaxB, s = e % kMaxB;
      float acc = 0.0f;
      if (s <= t && t < n)
        for (int j = 0; j < D; ++j) acc += Qs[t * D + j] * Ks[s * D + j];
      Mm[e] = acc;
    }
    __syncthreads();
    // R = A W2^T - V (zero on padded rows)
    for (int e = tid; e < kMaxB * D; e += kThreads) {
      const int t = e / D, i = e % D;
      float o = 0.0f;
      if (!a.dot_loss)
        for (int cc = 0; cc < h; ++cc) o += Ha[t * h + cc] * W2[static_cast<size_t>(i) * h + cc];
      const float r = t < n ? o - Vs[e] : 0.0f;
      Rr[e] = r;
      Rs[e] = Es[t] * r;
    }
    __syncthreads();
    // dU = (R W2) * phi'(U)
    for (int e = tid; e < kMaxB * h; e += kThreads) {
      const int t = e / h, cc = e % h;
      float dm = 0.0f;
      for (int i = 0; i < D; ++i) dm += Rs[t * D + i] * W2[static_cast<size_t>(i) * h + cc];
      Hdu[e] = dm * dsilu_(Hu[e]);
    }
    __syncthreads();
    // Uq = Q W1^T - eta M dU, Aq = phi(Uq)
    for (int e = tid; e < kMaxB * h; e += kThreads) {
      const int t = e / h, cc = e % h;
      float u = 0.0f;
      for (int j = 0; j < D; ++j) u += Qs[t * D + j] * W1[static_cast<size_t>(cc) * D + j];
      for (int s = 0; s <= t; ++s) u -= eta * Mm[t * kMaxB + s] * Hdu[s * h + cc];
      Huq[e] = u;
      Haq[e] = silu_(u);
    }
    __syncthreads();
    // N = tril(Aq A^T), Nb = -eta tril(dZ R^T)
    for (int e = tid; e < kMaxB * kMaxB; e += kThreads) {
      const int t = e / kMaxB, s = e % kMaxB;
      float nn = 0.0f, nb = 0.0f;
      if (s <= t && t < n) {
        for (int cc = 0; cc < h; ++cc) nn += Haq[t * h + cc] * Ha[s * h + cc];
        for (int i = 0; i < D; ++i) nb += Zb[t * D + i] * Rs[s * D + i];
      }
      Nn[e] = nn;
      Nb[e] = -eta * nb;
    }
    __syncthreads();
    // dUq = (dZ W2 + Nb A) * phi'(Uq);  dA = Nb^T Aq - eta R G2;  dR = -eta N^T dZ - eta A G2^T
    for (int e = tid; e < kMaxB * h; e += kThreads) {
      const int t = e / h, cc = e % h;
      float daq = 0.0f, da = 0.0f, rg = 0.0f;
      for (int i = 0; i < D; ++i) {
        daq += Zb[t * D + i] * W2[static_cast<size_t>(i) * h + cc];
        rg += Rs[t * D + i] * G2[static_cast<size_t>(i) * h + cc];
      }
      for (int s = 0; s < kMaxB; ++s) {
        daq += Nb[t * kMaxB + s] * Ha[s * h + cc];
        da += Nb[s * kMaxB + t] * Haq[s * h + cc];
      }
      Huq[e] = daq * dsilu_(Huq[e]);
      Hda[e] = da - eta * rg;
    }
    for (int e = tid; e < kMaxB * D; e += kThreads) {
      const int t = e / D, i = e % D;
      float acc = 0.0f, ag = 0.0f;
      for (int s = 0; s < kMaxB; ++s) acc += Nn[s * kMaxB + t] * Zb[s * D + i];
      for (int cc = 0; cc < h; ++cc) ag += Ha[t * h + cc] * G2[static_cast<size_t>(i) * h + cc];
      Rb[e] = -eta * (acc + ag);
    }
    __syncthreads();
    // Mb = -eta tril(dUq dU^T);  ddU = -eta (M^T dUq + K G1^T)
    for (int e = tid; e < kMaxB * kMaxB; e += kThreads) {
      const int t = e / kMaxB, s = e % kMaxB;
      float acc = 0.0f;
      if (s <= t && t < n)
        for (int cc = 0; cc < h; ++cc) acc += Huq[t * h + cc] * Hdu[s * h + cc];
      Mb[e] = -eta * acc;
    }
    for (int e = tid; e < kMaxB * h; e += kThreads) {
      const int t = e / h, cc = e % h;
      float acc = 0.0f;
      for (int s = 0; s < kMaxB; ++s) acc += Mm[s * kMaxB + t] * Huq[s * h + cc];
      for (int j = 0; j < D; ++j) acc += Ks[t * D + j] * G1[static_cast<size_t>(cc) * D + j];
      Hdd[e] = -eta * acc;
    }
    __syncthreads();
    // dR += (ddU * phi'(U)) W2^T  (then complete; dV = -dR)
    for (int e = tid; e < kMaxB * D; e += kThreads) {
      const int t = e / D, i = e % D;
      float acc = 0.0f;
      for (int cc = 0; cc < h; ++cc)
        acc += Hdd[t * h + cc] * dsilu_(Hu[t * h + cc]) * W2[static_cast<size_t>(i) * h + cc];
      Rb[e] += acc;  // dRt complete
    }
    __syncthreads();
    // de_t = <dRt_t, R_t>; dR = diag(e) dRt; dV = -dR
    if (a.deta_tok)
      for (int t = tid; t < n; t += kThreads) {
        float x = 0.0f;
        for (int i = 0; i < D; ++i) x += Rb[t * D + i] * Rr[t * D + i];
        a.deta_tok[static_cast<size_t>(chain) * T + c0 + t] = x;
      }
    __syncthreads();
    for (int e = tid; e < kMaxB * D; e += kThreads) {
      const int t = e / D, i = e % D;
      const float r = Es[t] * Rb[e];
      Rb[e] = r;
      if (t < n) dv[static_cast<size_t>(c0 + t) * D + i] = from_f32<IO>(-r);
    }
    __syncthreads();
    // dUk = (dA + dR W2) * phi'(U) + ddU * (R W2) * phi''(U)  (no dR W2 with the dot loss)
    for (int e = tid; e < kMaxB * h; e += kThreads) {
      const int t = e / h, cc = e % h;
      float rw = 0.0f, dm = 0.0f;
      for (int i = 0; i < D; ++i) {
        const float w = W2[static_cast<size_t>(i) * h + cc];
        rw += Rb[t * D + i] * w;
        dm += Rs[t * D + i] * w;
      }
      const float u = Hu[e];
      if (a.dot_loss) rw = 0.0f;
      Hda[e] = (Hda[e] + rw) * dsilu_(u) + Hdd[e] * dm * d2silu_(u);
    }
    __syncthreads();
    // dQ = dUq W1 + Mb K;  dK = Mb^T Q - eta dU G1 + dUk W1
    for (int e = tid; e < kMaxB * D; e += kThreads) {
      const int t = e / D, j = e % D;
      if (t >= n) continue;
      float aq = 0.0f, ak = 0.0f;
      for (int cc = 0; cc < h; ++cc) {
        const float w = W1[static_cast<size_t>(cc) * D + j];
        aq += Huq[t * h + cc] * w;
        ak += Hda[t * h + cc] * w - eta * Hdu[t * h + cc] * G1[static_cast<size_t>(cc) * D + j];
      }
      for (int s = 0; s < kMaxB; ++s) {
        aq += Mb[t * kMaxB + s] * Ks[s * D + j];
        ak += Mb[s * kMaxB + t] * Qs[s * D + j];
      }
      dq[static_cast<size_t>(c0 + t) * D + j] = from_f32<IO>(aq);
      dk[static_cast<size_t>(c0 + t) * D + j] = from_f32<IO>(ak);
    }
    __syncthreads();  // every read of G1, G2 of this chunk is done
    // G1 += dUq^T Q + dUk^T K;  G2 += dZ^T Aq + R^T (ddU * phi'(U)) + dR^T A (no dR^T A with
    // the dot loss)
    const float rterm = a.dot_loss ? 0.0f : 1.0f;
    for (size_t e = tid; e < hd; e += kThreads) {
      const int cc = static_cast<int>(e / D), j = static_cast<int>(e % D);
      float acc = 0.0f;
      for (int t = 0; t < n; ++t) acc += Huq[t * h + cc] * Qs[t * D + j] + Hda[t * h + cc] * Ks[t * D + j];
      G1[e] += acc;
    }
    for (size_t e = tid; e < hd; e += kThreads) {
      const int i = static_cast<int>(e / h), cc = static_cast<int>(e % h);
      float acc = 0.0f;
      for (int t = 0; t < n; ++t)
        acc += Zb[t * D + i] * Haq[t * h + cc] + Rs[t * D + i] * Hdd[t * h + cc] * dsilu_(Hu[t * h + cc]) +
               rterm * Rb[t * D + i] * Ha[t * h + cc];
      G2[e] += acc;
    }
  }
}

template <typename IO, int D>
hipError_t launch_one(const MlpBwdArgs& a, hipStream_t s) {
  const size_t lds = BwdLds<D>::total(a.dh) * sizeof(float);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&mlp_bwd_generic_kernel<IO, D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((mlp_bwd_generic_kernel<IO, D>), dim3(a.B * a.H), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <typename IO>
hipError_t launch_d(const MlpBwdArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_one<IO, 16>(a, s);
    case 32: return launch_one<IO, 32>(a, s);
    case 64: return launch_one<IO, 64>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_mlp_bwd_generic(const MlpBwdArgs& a, bool bf16_io, hipStream_t s) {
  if (a.chunk < 1 || a.T < 1 || min(a.chunk, a.T) > kMaxB || a.dh < 1 || a.dh > kMaxH)
    return hipErrorInvalidValue;
  return bf16_io ? launch_d<bf16>(a, s) : launch_d<float>(a, s);
}

}  // namespace ttt
