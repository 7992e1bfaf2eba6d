// Backward pass of the causal TTT-Linear layer on the vector ALUs (reconstruction loss,
// scalar rate or per-token rate factors, chunk <= 16, fp32 or bf16 I/O, d in {16, 32, 64}).  One workgroup of 1024
// threads (16 waves, four per SIMD, which hides the LDS latency of the short dot products)
// per (batch, head) chain walks the chunks from last to first.
//
// The outer loop trains the projections and the initial state through the inner updates
// (wmrh.cn summary of Sun et al. 2024, section 2.2; "Fast weights" page, opening
// paragraph), which needs the gradients of the layer's outputs with respect to its inputs.
// The forward chunk (wmrh.cn summary, section 1.2.2, mini-batch TTT), with W = W_c:
//     R = K W^T - V,   P = tril(Q K^T),   Z = Q W^T - eta P R,   W_{c+1} = W - eta R^T K.
// Reverse mode, with G = dL/dW_{c+1} coming from the later chunks (dL/dW_final for the last),
// our derivation of the chain rule through these four lines:
//     dR  = -eta (K G^T + P^T dZ)                      dV = -dR
//     dP  = -eta tril(dZ R^T)
//     dQ  = dZ W + dP K
//     dK  = -eta R G + dP^T Q + dR W
//     dL/dW_c = G + dZ^T Q + dR^T K
// With per-token rate factors e_t (token t's gradient taken with rate eta e_t; wmrh.cn
// summary, section 2.2.3) R is replaced by Rt = diag(e) R in Z and in the update; the lines
// above then give dRt (in place of dR, with Rt in dP and in -eta Rt G), and
//     dR = diag(e) dRt,   de_t = <dRt_t, R_t>.
// With the negative dot-product loss -v^T W k (ViT3 news page, section 2) R = -V depends on
// neither W nor K, and the dR W term of dK and the dR^T K term of dL/dW_c drop out.
// The chunk-start states W_c come from a forward recomputation that stores them
// (w_hist); the recursion in G is serial over the chunks, everything else is per chunk.
#include "common.hpp"

namespace ttt {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxB = 16;

template <typename IO, int D>
__global__ __launch_bounds__(kThreads) void linear_bwd_generic_kernel(LinearBwdArgs a) {
  __shared__ float Wc[D][D + 1];
  __shared__ float G[D][D + 1];
  __shared__ float Qs[kMaxB][D + 1];
  __shared__ float Ks[kMaxB][D + 1];
  __shared__ float Vs[kMaxB][D + 1];
  __shared__ float dZ[kMaxB][D + 1];
  __shared__ float Rs[kMaxB][D + 1];   // R, or diag(e) R with rate factors
  __shared__ float R0[kMaxB][D + 1];   // R (rate factors only)
  __shared__ float dR[kMaxB][D + 1];
  __shared__ float et[kMaxB];
  __shared__ float Ps[kMaxB][kMaxB + 1];
  __shared__ float dP[kMaxB][kMaxB + 1];

  const int tid = threadIdx.x;
  const int chain = blockIdx.x;
  const int T = a.T;
  const float eta = a.eta;
  const int b = min(a.chunk, T);
  const int nchunks = (T + b - 1) / b;
  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * D;
  const IO* q = static_cast<const IO*>(a.q) + tok0;
  const IO* k = static_cast<const IO*>(a.k) + tok0;
  const IO* v = static_cast<const IO*>(a.v) + tok0;
  const IO* dz = static_cast<const IO*>(a.dz) + tok0;
  IO* dq = static_cast<IO*>(a.dq) + tok0;
  IO* dk = static_cast<IO*>(a.dk) + tok0;
  IO* dv = static_cast<IO*>(a.dv) + tok0;
  const float* wh = a.w_hist + static_cast<size_t>(chain) * nchunks * D * D;
  const float* etok = a.eta_tok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
  float* detok = a.deta_tok ? a.deta_tok + static_cast<size_t>(chain) * T : nullptr;

  for (int e = tid; e < D * D; e += kThreads)
    G[e / D][e % D] = a.dw_out ? a.dw_out[static_cast<size_t>(chain) * D * D + e] : 0.0f;

  for (int c = nchunks - 1; c >= 0; --c) {
    const int c0 = c * b;
    const int n = min(b, T - c0);
    __syncthreads();  // G of the later chunk is complete; the previous chunk's tiles are free
    for (int e = tid; e < D * D; e += kThreads) Wc[e / D][e % D] = wh[static_cast<size_t>(c) * D * D + e];
    for (int e = tid; e < kMaxB * D; e += kThreads) {
      const int t = e / D, j = e % D;
      const bool in = t < n;
      const size_t off = static_cast<size_t>(c0 + t) * D + j;
      Qs[t][j] = in ? to_f32(q[off]) : 0.0f;
      Ks[t][j] = in ? to_f32(k[off]) : 0.0f;
      Vs[t][j] = in ? to_f32(v[off]) : 0.0f;
      dZ[t][j] = in ? to_f32(dz[off]) : 0.0f;
    }
    if (tid < kMaxB) et[tid] = etok && tid < n ? etok[c0 + tid] : 1.0f;
    __syncthreads();
    // forward quantities of the chunk: R = K W^T - V, P = tril(Q K^T)
    for (int e = tid; e < kMaxB * D; e += kThreads) {
      const int t = e / D, i = e % D;
      float acc = 0.0f;
#pragma unroll 16
      for (int j = 0; j < D; ++j) acc += Ks[t][j] * Wc[i][j];
      const float r = t < n ? (a.dot_loss ? 0.0f : acc) - Vs[t][i] : 0.0f;
      Rs[t][i] = et[t] * r;
      if (etok) R0[t][i] = r;
    }
    for (int e = tid; e < kMaxB * kMaxB; e += kThreads) {
      const int t = e / kMaxB, s = e % kMaxB;
      float acc = 0.0f;
      if (s <= t && t < n) {
#pragma unroll 16
        for (int j = 0; j < D; ++j) acc += Qs[t][j] * Ks[s][j];
      }
      Ps[t][s] = acc;
    }
    __syncthreads();
    // dR = -eta (K G^T + P^T dZ),  dP = -eta tril(dZ R^T)
    for (int e = tid; e < kMaxB * D; e += kThreads) {
      const int t = e / D, i = e % D;
      float acc = 0.0f;
#pragma unroll 16
      for (int j = 0; j < D; ++j) acc += Ks[t][j] * G[i][j];
      for (int s = t; s < n; ++s) acc += Ps[s][t] * dZ[s][i];
      dR[t][i] = t < n ? -eta * acc : 0.0f;
    }
    for (int e = tid; e < kMaxB * kMaxB; e += kThreads) {
      const int t = e / kMaxB, s = e % kMaxB;
      float acc = 0.0f;
      if (s <= t && t < n) {
#pragma unroll 16
        for (int i = 0; i < D; ++i) acc += dZ[t][i] * Rs[s][i];
      }
      dP[t][s] = -eta * acc;
    }
    __syncthreads();
    if (etok) {  // dR holds dRt: the factors' gradient, then dR = diag(e) dRt
      if (detok && tid < n) {
        float acc = 0.0f;
        for (int i = 0; i < D; ++i) acc += dR[tid][i] * R0[tid][i];
        detok[c0 + tid] = acc;
      }
      __syncthreads();
      for (int e = tid; e < kMaxB * D; e += kThreads) dR[e / D][e % D] *= et[e / D];
      __syncthreads();
    }
    // dQ = dZ W + dP K,  dK = -eta R G + dP^T Q + dR W,  dV = -dR
    for (int e = tid; e < kMaxB * D; e += kThreads) {
      const int t = e / D, j = e % D;
      if (t >= n) continue;
      float aq = 0.0f, ak = 0.0f, rg = 0.0f;
#pragma unroll 16
      for (int i = 0; i < D; ++i) {
        aq += dZ[t][i] * Wc[i][j];
        ak += dR[t][i] * Wc[i][j];
        rg += Rs[t][i] * G[i][j];
      }
      if (a.dot_loss) ak = 0.0f;  // R = -V does not depend on K: no dR W term
      for (int s = 0; s <= t; ++s) aq += dP[t][s] * Ks[s][j];
      for (int s = t; s < n; ++s) ak += dP[s][t] * Qs[s][j];
      const size_t off = static_cast<size_t>(c0 + t) * D + j;
      dq[off] = from_f32<IO>(aq);
      dk[off] = from_f32<IO>(ak - eta * rg);
      dv[off] = from_f32<IO>(-dR[t][j]);
    }
    __syncthreads();  // the old G is read above; now dL/dW_c = G + dZ^T Q + dR^T K
    for (int e = tid; e < D * D; e += kThreads) {
      const int i = e / D, j = e % D;
      float acc = 0.0f;
      for (int t = 0; t < n; ++t) acc += dZ[t][i] * Qs[t][j] + (a.dot_loss ? 0.0f : dR[t][i] * Ks[t][j]);
      G[i][j] += acc;
    }
  }
  __syncthreads();
  float* dw0 = a.dw0 + static_cast<size_t>(chain) * D * D;
  for (int e = tid; e < D * D; e += kThreads) dw0[e] = G[e / D][e % D];
}

template <typename IO>
hipError_t launch_d(const LinearBwdArgs& a, hipStream_t s) {
  const dim3 grid(a.B * a.H), block(kThreads);
  switch (a.d) {
    case 16: hipLaunchKernelGGL((linear_bwd_generic_kernel<IO, 16>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((linear_bwd_generic_kernel<IO, 32>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((linear_bwd_generic_kernel<IO, 64>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_bwd_generic(const LinearBwdArgs& a, bool bf16_io, hipStream_t s) {
  if (a.chunk < 1 || a.T < 1 || min(a.chunk, a.T) > kMaxB) return hipErrorInvalidValue;
  return bf16_io ? launch_d<bf16>(a, s) : launch_d<float>(a, s);
}

}  // namespace ttt
