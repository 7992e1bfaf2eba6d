// Backward pass of the delta rule (the causal TTT-Linear layer with one token per step) on the
// vector ALUs, taken 16 tokens at a time in the exact chunked form: reconstruction or negative
// dot-product loss, scalar rate or per-token rate factors (with their gradient), d in
// {16, 32, 64}, fp32 or bf16 I/O.  One workgroup of 1024 threads per (batch, head) chain.
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
// then walks the chunks backwards with G in LDS.  Tm is formed per chunk from the product
// formula (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8) (L is strictly lower triangular, so
// L^16 = 0), one thread per entry for each of the six 16 x 16 products.
#include "common.hpp"

namespace ttt {
namespace {

constexpr int kThreads = 1024;
constexpr int kC = 16;  // tokens per chunk

template <int D>
struct DeltaLds {  // float offsets in the dynamic LDS block
  static constexpr int kM = D * (D + 1), kT = kC * (D + 1), kS = kC * (kC + 1);
  static constexpr int W = 0, G = kM, Q = 2 * kM, K = Q + kT, V = K + kT, DZ = V + kT, X = DZ + kT,
                       RT = X + kT, R0 = RT + kT, DR = R0 + kT, DX = DR + kT, KK = DX + kT, TM = KK + kS,
                       P = TM + kS, DP = P + kS, DL = DP + kS, L2 = DL + kS, L4 = L2 + kS,
                       ET = L4 + kS, TOTAL = ET + kC;
};

template <typename IO, int D>
__global__ __launch_bounds__(kThreads) void delta_bwd_kernel(LinearBwdArgs a, const float* w0,
                                                             long long w0_batch_stride, float* hist) {
  extern __shared__ float lds[];
  using L = DeltaLds<D>;
  constexpr int S = D + 1, SS = kC + 1;
  float* Wc = lds + L::W;
  float* G = lds + L::G;
  float* Qs = lds + L::Q;
  float* Ks = lds + L::K;
  float* Vs = lds + L::V;
  float* dZ = lds + L::DZ;
  float* Xs = lds + L::X;
  float* Rt = lds + L::RT;
  float* R0 = lds + L::R0;
  float* dR = lds + L::DR;
  float* dX = lds + L::DX;
  float* Kk = lds + L::KK;
  float* Tm = lds + L::TM;
  float* Ps = lds + L::P;
  float* dP = lds + L::DP;
  float* dL = lds + L::DL;
  float* M2 = lds + L::L2;  // scratch 16 x 16 matrices of the product formula
  float* M4 = lds + L::L4;
  float* et = lds + L::ET;

  const int tid = threadIdx.x;
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
  float* wh = hist + static_cast<size_t>(chain) * nchunks * D * D;
  const float* etok = a.eta_tok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
  float* detok = a.deta_tok ? a.deta_tok + static_cast<size_t>(chain) * T : nullptr;
  const float* w0c = w0 + bi * w0_batch_stride + static_cast<long long>(hi) * D * D;

  // the chunk's tokens, rates, X = K W^T - V, K K^T, Tm and R = Tm X (Rt = e R); ends synchronised
  auto chunk_forward = [&](int c0, int n, bool with_q) {
    for (int e = tid; e < kC * D; e += kThreads) {
      const int t = e / D, j = e % D;
      const bool in = t < n;
      const size_t off = static_cast<size_t>(c0 + t) * D + j;
      Ks[t * S + j] = in ? to_f32(k[off]) : 0.0f;
      Vs[t * S + j] = in ? to_f32(v[off]) : 0.0f;
      if (with_q) {
        Qs[t * S + j] = in ? to_f32(q[off]) : 0.0f;
        dZ[t * S + j] = in ? to_f32(dz[off]) : 0.0f;
      }
    }
    if (tid < kC) et[tid] = tid < n ? (etok ? etok[c0 + tid] : 1.0f) : 0.0f;
    __syncthreads();
    for (int e = tid; e < kC * D; e += kThreads) {
      const int t = e / D, i = e % D;
      float acc = 0.0f;
      if (!dot)
        for (int j = 0; j < D; ++j) acc += Wc[i * S + j] * Ks[t * S + j];
      Xs[t * S + i] = t < n ? acc - Vs[t * S + i] : 0.0f;
    }
    for (int e = tid; e < kC * kC; e += kThreads) {
      const int t = e / kC, s = e % kC;
      float acc = 0.0f, pq = 0.0f;
      if (t < n && s < n)
        for (int j = 0; j < D; ++j) acc += Ks[t * S + j] * Ks[s * S + j];
      if (with_q && s <= t && t < n)
        for (int j = 0; j < D; ++j) pq += Qs[t * S + j] * Ks[s * S + j];
      Kk[t * SS + s] = acc;
      if (with_q) Ps[t * SS + s] = pq;
    }
    __syncthreads();
    // Tm = (I + L)^-1, L_ts = eta (k_t . k_s) e_s (s < t; zero with the dot loss), by the
    // product formula: Tm <- I - L, then for p = L^2, L^4, L^8 (squaring p each time)
    // Tm <- Tm (I + p)
    const int rt = tid / kC, cs = tid % kC;  // the entry of threads 0 .. 255
    const bool ent = tid < kC * kC;
    if (ent) {
      const float l = (cs < rt && !dot) ? eta * Kk[rt * SS + cs] * et[cs] : 0.0f;
      M2[rt * SS + cs] = l;
      Tm[rt * SS + cs] = (rt == cs ? 1.0f : 0.0f) - l;
    }
    __syncthreads();
    float* pw = M2;  // the current power of L
    float* nx = M4;
    for (int step = 0; step < 3; ++step) {
      if (ent) {  // the next power, pw pw: L^2, L^4, L^8
        float sq = 0.0f;
        for (int u = 0; u < kC; ++u) sq += pw[rt * SS + u] * pw[u * SS + cs];
        nx[rt * SS + cs] = sq;
      }
      __syncthreads();
      float pr = 0.0f;  // Tm (I + nx) = Tm + Tm nx
      if (ent) {
        float x = 0.0f;
        for (int u = 0; u < kC; ++u) x += Tm[rt * SS + u] * nx[u * SS + cs];
        pr = Tm[rt * SS + cs] + x;
      }
      __syncthreads();
      if (ent) Tm[rt * SS + cs] = pr;
      __syncthreads();
      float* t = pw;
      pw = nx;
      nx = t;
    }
    for (int e = tid; e < kC * D; e += kThreads) {
      const int t = e / D, i = e % D;
      float acc = 0.0f;
      for (int s = 0; s <= t; ++s) acc += Tm[t * SS + s] * Xs[s * S + i];
      R0[t * S + i] = acc;
      Rt[t * S + i] = et[t] * acc;
    }
    __syncthreads();
  };

  // ---- forward: chunk-start states into the workspace ----
  for (int e = tid; e < D * D; e += kThreads) Wc[(e / D) * S + e % D] = w0c[e];
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int c0 = c * kC, n = min(kC, T - c0);
    for (int e = tid; e < D * D; e += kThreads) wh[static_cast<size_t>(c) * D * D + e] = Wc[(e / D) * S + e % D];
    chunk_forward(c0, n, false);
    // W -= eta Rt^T K
    for (int e = tid; e < D * D; e += kThreads) {
      const int i = e / D, j = e % D;
      float acc = 0.0f;
      for (int t = 0; t < n; ++t) acc += Rt[t * S + i] * Ks[t * S + j];
      Wc[i * S + j] -= eta * acc;
    }
    __syncthreads();
  }

  // ---- reverse ----
  for (int e = tid; e < D * D; e += kThreads)
    G[(e / D) * S + e % D] = a.dw_out ? a.dw_out[static_cast<size_t>(chain) * D * D + e] : 0.0f;
  for (int c = nchunks - 1; c >= 0; --c) {
    const int c0 = c * kC, n = min(kC, T - c0);
    __syncthreads();  // G of the later chunk is complete; the tiles are free
    for (int e = tid; e < D * D; e += kThreads) Wc[(e / D) * S + e % D] = wh[static_cast<size_t>(c) * D * D + e];
    __syncthreads();
    chunk_forward(c0, n, true);
    // dRt = -eta (K G^T + P^T dZ);  dP = -eta tril(dZ Rt^T)
    for (int e = tid; e < kC * D; e += kThreads) {
      const int t = e / D, i = e % D;
      float acc = 0.0f;
      for (int j = 0; j < D; ++j) acc += Ks[t * S + j] * G[i * S + j];
      for (int s = t; s < n; ++s) acc += Ps[s * SS + t] * dZ[s * S + i];
      dR[t * S + i] = t < n ? -eta * acc : 0.0f;
    }
    for (int e = tid; e < kC * kC; e += kThreads) {
      const int t = e / kC, s = e % kC;
      float acc = 0.0f;
      if (s <= t && t < n)
        for (int i = 0; i < D; ++i) acc += dZ[t * S + i] * Rt[s * S + i];
      dP[t * SS + s] = -eta * acc;
    }
    __syncthreads();
    // the rates' gradient, first part: <dRt, R>; then dR = diag(e) dRt
    if (tid < kC) {
      float acc = 0.0f;
      for (int i = 0; i < D; ++i) acc += dR[tid * S + i] * R0[tid * S + i];
      dL[tid * SS + kC] = acc;  // column kC of dL (unused by L) holds de_t for now
    }
    __syncthreads();
    for (int e = tid; e < kC * D; e += kThreads) dR[(e / D) * S + e % D] *= et[e / D];
    __syncthreads();
    // dX = Tm^T dR
    for (int e = tid; e < kC * D; e += kThreads) {
      const int s = e / D, i = e % D;
      float acc = 0.0f;
      for (int t = s; t < kC; ++t) acc += Tm[t * SS + s] * dR[t * S + i];
      dX[s * S + i] = s < n ? acc : 0.0f;
    }
    __syncthreads();
    // dL_ts = -(dX R^T)_ts for s < t (the cotangent of L)
    for (int e = tid; e < kC * kC; e += kThreads) {
      const int t = e / kC, s = e % kC;
      float acc = 0.0f;
      if (s < t && t < n && !dot)
        for (int i = 0; i < D; ++i) acc += dX[t * S + i] * R0[s * S + i];
      dL[t * SS + s] = -acc;
    }
    __syncthreads();
    // de_s: <dRt_s, R_s> + eta sum_{t>s} dL_ts (k_t . k_s)
    if (detok && tid < n) {
      const int s = tid;
      float acc = dL[s * SS + kC];
      for (int t = s + 1; t < n; ++t) acc += eta * dL[t * SS + s] * Kk[t * SS + s];
      detok[c0 + s] = acc;
    }
    // dQ = dZ W + dP K;  dK = -eta Rt G + dP^T Q + dX W + eta sum dL (e k);  dV = -dX
    for (int e = tid; e < kC * D; e += kThreads) {
      const int t = e / D, j = e % D;
      if (t >= n) continue;
      float aq = 0.0f, ak = 0.0f, rg = 0.0f;
      for (int i = 0; i < D; ++i) {
        aq += dZ[t * S + i] * Wc[i * S + j];
        if (!dot) ak += dX[t * S + i] * Wc[i * S + j];
        rg += Rt[t * S + i] * G[i * S + j];
      }
      for (int s = 0; s <= t; ++s) aq += dP[t * SS + s] * Ks[s * S + j];
      for (int s = t; s < n; ++s) ak += dP[s * SS + t] * Qs[s * S + j];
      float lk = 0.0f;
      for (int s = 0; s < t; ++s) lk += dL[t * SS + s] * et[s] * Ks[s * S + j];
      for (int u = t + 1; u < n; ++u) lk += dL[u * SS + t] * et[t] * Ks[u * S + j];
      const size_t off = static_cast<size_t>(c0 + t) * D + j;
      dq[off] = from_f32<IO>(aq);
      dk[off] = from_f32<IO>(ak - eta * rg + eta * lk);
      dv[off] = from_f32<IO>(-dX[t * S + j]);
    }
    __syncthreads();  // the old G is read above; now dL/dW_c = G + dZ^T Q + dX^T K
    for (int e = tid; e < D * D; e += kThreads) {
      const int i = e / D, j = e % D;
      float acc = 0.0f;
      for (int t = 0; t < n; ++t) acc += dZ[t * S + i] * Qs[t * S + j] + (dot ? 0.0f : dX[t * S + i] * Ks[t * S + j]);
      G[i * S + j] += acc;
    }
  }
  __syncthreads();
  float* dw0 = a.dw0 + static_cast<size_t>(chain) * D * D;
  for (int e = tid; e < D * D; e += kThreads) dw0[e] = G[(e / D) * S + e % D];
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
  return static_cast<size_t>(a.B) * a.H * nchunks * a.d * a.d * sizeof(float);
}

hipError_t launch_delta_bwd(const LinearBwdArgs& a, const float* w0, long long w0_batch_stride, void* ws,
                            bool bf16_io, hipStream_t s) {
  if (a.T < 1) return hipErrorInvalidValue;
  float* hist = static_cast<float*>(ws);
  return bf16_io ? launch_d<bf16>(a, w0, w0_batch_stride, hist, s) : launch_d<float>(a, w0, w0_batch_stride, hist, s);
}

}  // namespace ttt
