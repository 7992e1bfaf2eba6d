// Generic TTT-Linear forward on the vector ALUs: any chunk size, causal or not, fp32 or
// bf16 I/O, d in {16, 32, 64}.  One workgroup of 1024 threads (16 waves, four per SIMD, so
// the LDS latency of the small dot products is hidden) per (batch, head) chain.
//
// Method: mini-batch gradient descent on 1/2 ||W k - v||^2 (gradient (W k - v) k^T,
// "Fast weights" page, section 1), or on the negative dot product -v^T W k (gradient
// -v k^T; blog page "TTT: Test-Time Training", section TTT / 如何理解); inside a chunk every gradient is taken at the
// chunk-start weights and W_t subtracts eta times the running sum (wmrh.cn summary of
// Sun et al. 2024, section 1.2.2); z_t = W_t q_t (blog page "TTT: Test-Time Training",
// general form).
//
// With per-token rates (eta_t = eta * eta_tok[t]; the "Fast weights" page writes the
// step with a per-step rate, and the wmrh.cn summary, section 2.2.3, makes it a function
// of the token) each token's gradient carries its own rate.
//
// The chunk is walked in sub-blocks of S = 16 tokens.  Two fp32 states live in LDS:
// Wc, the chunk-start weights every residual uses, and Wn, the weights after all earlier
// sub-blocks of the chunk.  For a sub-block with rate-scaled residuals
// R = diag(eta_t) (K Wc^T - V),
//   z_t = Wn q_t - sum_{s <= t in the sub-block} (q_t . k_s) r_s
//   Wn  -= R^T K,
// and at the end of a chunk Wc <- Wn.  This equals the per-token recurrence up to
// floating-point order.  With causal = 0 the training pass (repeated for `epochs` passes
// over the chunks, ViT3 news page, observation 2) writes no output and a second pass
// computes z_t = W_final q_t.
//
// kLN: the paper's instantiation f(x) = x + LN(W x) (wmrh.cn summary, section 2.2.1), LN with
// per-head gamma, beta.  The state still changes only through the residual rows (the
// gradient is r k^T with r = dl/d(W k)), so the dual form above is unchanged: the residual
// row is y = Wc k passed through LN and back, r = LN'(y)^T (k + LN(y) - v), and the output
// row is z = q + LN(Wn q - sum_s (q . k_s) r_s).  Each of the kSub x D elements of a
// sub-block belongs to one thread (kThreads >= kSub D), so a token's D features sit in D
// consecutive lanes and the LN statistics are shuffle sums inside that lane group.
#include "common.hpp"

namespace ttt {
namespace {

constexpr int kThreads = 1024;
constexpr int kSub = 16;

static_assert(kThreads >= kSub * 64, "one sub-block element per thread");

template <typename IO, int D, bool kLN>
__global__ __launch_bounds__(kThreads) void linear_generic_kernel(LinearArgs a) {
  __shared__ float Wc[D][D + 1];
  __shared__ float Wn[D][D + 1];
  __shared__ float Qs[kSub][D + 1];
  __shared__ float Ks[kSub][D + 1];
  __shared__ float Vs[kSub][D + 1];
  __shared__ float Rs[kSub][D + 1];
  __shared__ float Ps[kSub][kSub + 1];

  const int tid = threadIdx.x;
  const int chain = blockIdx.x;
  const int bi = chain / a.H;
  const int hi = chain - bi * a.H;
  const int T = a.T;
  const float eta = a.eta;
  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * D;
  const IO* q = static_cast<const IO*>(a.q) + tok0;
  const IO* k = static_cast<const IO*>(a.k) + tok0;
  const IO* v = static_cast<const IO*>(a.v) + tok0;
  IO* z = static_cast<IO*>(a.z) + tok0;
  const float* w0 = a.w0 + bi * a.w0_batch_stride + static_cast<long long>(hi) * D * D;
  const float* etok = a.eta_tok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
  // LN gain and bias of this thread's feature (the feature index of a sub-block element is
  // tid % D in every loop below)
  const float gam = kLN ? a.ln_w[hi * D + tid % D] : 0.0f;
  const float bet = kLN ? a.ln_b[hi * D + tid % D] : 0.0f;

  for (int e = tid; e < D * D; e += kThreads) {
    const float w = w0[e];
    Wc[e / D][e % D] = w;
    Wn[e / D][e % D] = w;
  }
  __syncthreads();

  const int b = T > 0 ? min(a.chunk, T) : 1;
  const int nchunks = (T + b - 1) / b;
  for (int step = 0; step < a.epochs * nchunks; ++step) {
    const int c0 = (step % nchunks) * b;
    const int cend = min(c0 + b, T);
    if (a.w_hist) {  // chunk-start state, for the backward pass
      float* wh = a.w_hist + (static_cast<size_t>(chain) * nchunks + c0 / b) * D * D;
      for (int e = tid; e < D * D; e += kThreads) wh[e] = Wc[e / D][e % D];
    }
    for (int s0 = c0; s0 < cend; s0 += kSub) {
      const int n = min(kSub, cend - s0);
      for (int e = tid; e < kSub * D; e += kThreads) {
        const int t = e / D, j = e % D;
        const bool in = t < n;
        const size_t off = static_cast<size_t>(s0 + t) * D + j;
        Qs[t][j] = in ? to_f32(q[off]) : 0.0f;
        Ks[t][j] = in ? to_f32(k[off]) : 0.0f;
        Vs[t][j] = in ? to_f32(v[off]) : 0.0f;
      }
      __syncthreads();
      // Rate-scaled residuals at the chunk-start weights, and the causal in-block scores.
      for (int e = tid; e < kSub * D; e += kThreads) {
        const int t = e / D, i = e % D;
        float acc = 0.0f;
#pragma unroll 16
        for (int j = 0; j < D; ++j) acc += Ks[t][j] * Wc[i][j];
        const float rate = t < n ? (etok ? eta * etok[s0 + t] : eta) : 0.0f;
        float err;  // dl/d(W k): f - v or -v, through the layer norm with kLN
        if constexpr (kLN) {
          const LnRow st = ln_row<D>(acc, a.ln_eps);
          const float f = Ks[t][i] + gam * st.xh + bet;
          err = ln_row_vjp<D>(st, gam, a.dot_loss ? -Vs[t][i] : f - Vs[t][i]);
        } else {
          err = a.dot_loss ? -Vs[t][i] : acc - Vs[t][i];
        }
        Rs[t][i] = t < n ? rate * err : 0.0f;
      }
      if (a.causal) {
        for (int e = tid; e < kSub * kSub; e += kThreads) {
          const int t = e / kSub, s = e % kSub;
          float acc = 0.0f;
          if (s <= t && t < n) {
#pragma unroll 16
            for (int j = 0; j < D; ++j) acc += Qs[t][j] * Ks[s][j];
          }
          Ps[t][s] = acc;
        }
      }
      __syncthreads();
      if (a.causal && a.z) {
        for (int e = tid; e < kSub * D; e += kThreads) {
          const int t = e / D, i = e % D;
          float acc = 0.0f;
#pragma unroll 16
          for (int j = 0; j < D; ++j) acc += Qs[t][j] * Wn[i][j];
          float corr = 0.0f;
          for (int s = 0; s <= t; ++s) corr += Ps[t][s] * Rs[s][i];
          float zt = acc - corr;
          if constexpr (kLN) zt = Qs[t][i] + gam * ln_row<D>(zt, a.ln_eps).xh + bet;
          if (t < n) z[static_cast<size_t>(s0 + t) * D + i] = from_f32<IO>(zt);
        }
        __syncthreads();
      }
      for (int e = tid; e < D * D; e += kThreads) {
        const int i = e / D, j = e % D;
        float acc = 0.0f;
        for (int t = 0; t < n; ++t) acc += Rs[t][i] * Ks[t][j];
        Wn[i][j] -= acc;
      }
      __syncthreads();
    }
    for (int e = tid; e < D * D; e += kThreads) Wc[e / D][e % D] = Wn[e / D][e % D];
    __syncthreads();
  }

  if (!a.causal && a.z) {
    for (int s0 = 0; s0 < T; s0 += kSub) {
      const int n = min(kSub, T - s0);
      for (int e = tid; e < kSub * D; e += kThreads) {
        const int t = e / D, j = e % D;
        Qs[t][j] = t < n ? to_f32(q[static_cast<size_t>(s0 + t) * D + j]) : 0.0f;
      }
      __syncthreads();
      for (int e = tid; e < kSub * D; e += kThreads) {
        const int t = e / D, i = e % D;
        float acc = 0.0f;
#pragma unroll 16
        for (int j = 0; j < D; ++j) acc += Qs[t][j] * Wn[i][j];
        if constexpr (kLN) acc = Qs[t][i] + gam * ln_row<D>(acc, a.ln_eps).xh + bet;
        if (t < n) z[static_cast<size_t>(s0 + t) * D + i] = from_f32<IO>(acc);
      }
      __syncthreads();
    }
  }

  if (a.w_out) {
    float* wo = a.w_out + static_cast<size_t>(chain) * D * D;
    for (int e = tid; e < D * D; e += kThreads) wo[e] = Wn[e / D][e % D];
  }
}

template <typename IO, bool kLN>
hipError_t launch_d(const LinearArgs& a, hipStream_t s) {
  const dim3 grid(a.B * a.H), block(kThreads);
  switch (a.d) {
    case 16: hipLaunchKernelGGL((linear_generic_kernel<IO, 16, kLN>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((linear_generic_kernel<IO, 32, kLN>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((linear_generic_kernel<IO, 64, kLN>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_generic(const LinearArgs& a, bool bf16_io, hipStream_t s) {
  if (a.ln_w) return bf16_io ? launch_d<bf16, true>(a, s) : launch_d<float, true>(a, s);
  return bf16_io ? launch_d<bf16, false>(a, s) : launch_d<float, false>(a, s);
}

}  // namespace ttt
