// Generic TTT-MLP forward on the vector ALUs: f(k) = W2 SiLU(W1 k) with hidden width dh,
// any chunk size, causal or not, fp32 or bf16 I/O, d in {16, 32, 64}, dh <= 512.
// One workgroup of 1024 threads (16 waves, four per SIMD, hiding LDS latency) per (batch,
// head) chain.
//
// Method: inner 2-layer SiLU MLP (ViT3 news page, section 2) trained by mini-batch GD on
// 1/2 ||f(k) - v||^2 (wmrh.cn summary of Sun et al. 2024, section 1.2.2), z_t = f(q_t; W_t),
// or on the negative dot product -v^T f(k) (ViT3 news page, section 2), whose error term is
// r = -v.  Per token, with u = W1 k, a = SiLU(u), r = W2 a - v:
//   dW2 = r a^T,   dW1 = ((W2^T r) * SiLU'(u)) k^T.
//
// With per-token rates (eta_t = eta * eta_tok[t]; "Fast weights" page, opening formula;
// wmrh.cn summary, section 2.2.3) each token's gradients carry its own rate: r and du
// below are scaled by eta_t.
//
// The chunk is walked in sub-blocks of S = 16 tokens.  The states are kept in a global
// workspace (4 dh d floats per chain): W1c/W2c, the chunk-start weights every gradient is
// taken at, and W1n/W2n, the weights after all earlier sub-blocks of the chunk.  For a
// sub-block, every hidden pre-activation of a query is linear in W1, so
//   u^q_t = W1n q_t - sum_{s<=t} (q_t . k_s) du_s,   a^q_t = SiLU(u^q_t),
//   z_t   = W2n a^q_t - sum_{s<=t} (a^q_t . a_s) r_s,
// then W1n -= dU^T K and W2n -= R^T A; at the end of a chunk W1c/W2c <- W1n/W2n.  The
// non-causal layer may repeat the pass over the chunks for several epochs (ViT3 news page,
// observation 2) before every query reads the final weights.
//
// kPaper: the paper's TTT-MLP, f(x) = x + LN(W2 GELU(W1 x)) (wmrh.cn summary, section 2.2.1),
// LN with per-head gamma, beta.  The dual form is unchanged with GELU in place of SiLU; the
// residual row r = dl/d(W2 a) passes the error k + LN(y) - v back through the layer norm of
// y = W2c a, and the output row is z = q + LN(y_q) with y_q the dual-form pre-LN output.
// Each of the kSub x D output elements of a sub-block belongs to one thread, so a token's D
// features sit in D consecutive lanes and the LN statistics are shuffle sums among them.
#include "common.hpp"

namespace ttt {
namespace {

constexpr int kThreads = 1024;
constexpr int kSub = 16;

template <int D>
struct MlpLds {
  // float offsets inside the dynamic LDS block, for hidden width h
  static __host__ __device__ size_t q() { return 0; }
  static __host__ __device__ size_t k() { return kSub * D; }
  static __host__ __device__ size_t v() { return 2 * kSub * D; }
  static __host__ __device__ size_t r() { return 3 * kSub * D; }
  static __host__ __device__ size_t p() { return 4 * kSub * D; }
  static __host__ __device__ size_t p2() { return 4 * kSub * D + kSub * kSub; }
  static __host__ __device__ size_t act(int) { return 4 * kSub * D + 2 * kSub * kSub; }
  static __host__ __device__ size_t du(int h) { return act(h) + static_cast<size_t>(kSub) * h; }
  static __host__ __device__ size_t aq(int h) { return du(h) + static_cast<size_t>(kSub) * h; }
  static __host__ __device__ size_t total(int h) { return aq(h) + static_cast<size_t>(kSub) * h; }
};

static_assert(kThreads >= kSub * 64, "one output element of a sub-block per thread");

template <bool kPaper>
__device__ __forceinline__ float act_(float u) { return kPaper ? gelu_(u) : silu_(u); }
template <bool kPaper>
__device__ __forceinline__ float dact_(float u) { return kPaper ? dgelu_(u) : dsilu_(u); }

template <typename IO, int D, bool kPaper>
__global__ __launch_bounds__(kThreads) void mlp_generic_kernel(MlpArgs a, float* ws) {
  extern __shared__ float lds[];
  const int h = a.dh;
  float* Qs = lds + MlpLds<D>::q();
  float* Ks = lds + MlpLds<D>::k();
  float* Vs = lds + MlpLds<D>::v();
  float* Rs = lds + MlpLds<D>::r();
  float* Ps = lds + MlpLds<D>::p();
  float* P2 = lds + MlpLds<D>::p2();
  float* Ab = lds + MlpLds<D>::act(h);   // [S][h] key activations a
  float* DU = lds + MlpLds<D>::du(h);    // [S][h] SiLU'(u), then du
  float* AQ = lds + MlpLds<D>::aq(h);    // [S][h] query activations

  const int tid = threadIdx.x;
  const int chain = blockIdx.x;
  const int bi = chain / a.H;
  const int hi = chain - bi * a.H;
  const int T = a.T;
  const float eta = a.eta;
  const size_t hd = static_cast<size_t>(h) * D;
  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * D;
  const IO* q = static_cast<const IO*>(a.q) + tok0;
  const IO* k = static_cast<const IO*>(a.k) + tok0;
  const IO* v = static_cast<const IO*>(a.v) + tok0;
  IO* z = static_cast<IO*>(a.z) + tok0;
  const float* w1i = a.w1 + bi * a.w_batch_stride + static_cast<long long>(hi) * hd;
  const float* w2i = a.w2 + bi * a.w_batch_stride + static_cast<long long>(hi) * hd;
  const float* etok = a.eta_tok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
  float* W1c = ws + static_cast<size_t>(chain) * 4 * hd;  // [h][D]
  float* W2c = W1c + hd;                                  // [D][h]
  float* W1n = W2c + hd;
  float* W2n = W1n + hd;
  // LN gain and bias of this thread's output feature (tid % D in every kSub x D loop)
  const float gam = kPaper ? a.ln_w[hi * D + tid % D] : 0.0f;
  const float bet = kPaper ? a.ln_b[hi * D + tid % D] : 0.0f;

  for (size_t e = tid; e < hd; e += kThreads) {
    const float x1 = w1i[e], x2 = w2i[e];
    W1c[e] = x1; W1n[e] = x1;
    W2c[e] = x2; W2n[e] = x2;
  }
  __syncthreads();

  const int b = T > 0 ? min(a.chunk, T) : 1;
  const int nchunks = (T + b - 1) / b;
  for (int step = 0; step < a.epochs * nchunks; ++step) {  // epochs > 1: non-causal only
    const int c0 = (step % nchunks) * b;
    if (a.w_hist) {  // chunk-start states, for the backward pass
      float* wh = a.w_hist + (static_cast<size_t>(chain) * nchunks + c0 / b) * 2 * hd;
      for (size_t e = tid; e < hd; e += kThreads) {
        wh[e] = W1c[e];
        wh[hd + e] = W2c[e];
      }
    }
    const int cend = min(c0 + b, T);
    for (int s0 = c0; s0 < cend; s0 += kSub) {
      const int n = min(kSub, cend - s0);
      for (int e = tid; e < kSub * D; e += kThreads) {
        const int t = e / D;
        const bool in = t < n;
        const size_t off = static_cast<size_t>(s0) * D + e;
        Qs[e] = in ? to_f32(q[off]) : 0.0f;
        Ks[e] = in ? to_f32(k[off]) : 0.0f;
        Vs[e] = in ? to_f32(v[off]) : 0.0f;
      }
      __syncthreads();
      // key forward, first layer: u = W1c k, a = act(u), keep act'(u)
      for (int e = tid; e < kSub * h; e += kThreads) {
        const int t = e / h, c = e % h;
        float u = 0.0f;
        for (int j = 0; j < D; ++j) u += Ks[t * D + j] * W1c[static_cast<size_t>(c) * D + j];
        const bool in = t < n;
        Ab[e] = in ? act_<kPaper>(u) : 0.0f;
        DU[e] = in ? dact_<kPaper>(u) : 0.0f;
      }
      __syncthreads();
      // second layer and rate-scaled residual: r = eta_t (W2c a - v)
      for (int e = tid; e < kSub * D; e += kThreads) {
        const int t = e / D, i = e % D;
        float o = 0.0f;
        for (int c = 0; c < h; ++c) o += Ab[t * h + c] * W2c[static_cast<size_t>(i) * h + c];
        const float rate = t < n ? (etok ? eta * etok[s0 + t] : eta) : 0.0f;
        float err;  // dl/d(W2 a): f - v or -v, through the layer norm with kPaper
        if constexpr (kPaper) {
          const LnRow st = ln_row<D>(o, a.ln_eps);
          const float f = Ks[e] + gam * st.xh + bet;
          err = ln_row_vjp<D>(st, gam, a.dot_loss ? -Vs[e] : f - Vs[e]);
        } else {
          err = a.dot_loss ? -Vs[e] : o - Vs[e];
        }
        Rs[e] = t < n ? rate * err : 0.0f;
      }
      __syncthreads();
      // backward to the hidden pre-activation: du = (W2c^T r) * act'(u)
      for (int e = tid; e < kSub * h; e += kThreads) {
        const int t = e / h, c = e % h;
        float g = 0.0f;
        for (int i = 0; i < D; ++i) g += Rs[t * D + i] * W2c[static_cast<size_t>(i) * h + c];
        DU[e] *= g;
      }
      if (a.causal) {
        for (int e = tid; e < kSub * kSub; e += kThreads) {
          const int t = e / kSub, s = e % kSub;
          float acc = 0.0f;
          if (s <= t && t < n)
            for (int j = 0; j < D; ++j) acc += Qs[t * D + j] * Ks[s * D + j];
          Ps[e] = acc;
        }
      }
      __syncthreads();
      if (a.causal && a.z) {  // outputs (skipped when only the states are wanted)
        // query hidden layer at W1_t (dual form of the in-block W1 updates)
        for (int e = tid; e < kSub * h; e += kThreads) {
          const int t = e / h, c = e % h;
          float u = 0.0f;
          for (int j = 0; j < D; ++j) u += Qs[t * D + j] * W1n[static_cast<size_t>(c) * D + j];
          float corr = 0.0f;
          for (int s = 0; s <= t && s < kSub; ++s) corr += Ps[t * kSub + s] * DU[s * h + c];
          AQ[e] = t < n ? act_<kPaper>(u - corr) : 0.0f;
        }
        __syncthreads();
        for (int e = tid; e < kSub * kSub; e += kThreads) {
          const int t = e / kSub, s = e % kSub;
          float acc = 0.0f;
          if (s <= t && t < n)
            for (int c = 0; c < h; ++c) acc += AQ[t * h + c] * Ab[s * h + c];
          P2[e] = acc;
        }
        __syncthreads();
        for (int e = tid; e < kSub * D; e += kThreads) {
          const int t = e / D, i = e % D;
          float o = 0.0f;
          for (int c = 0; c < h; ++c) o += AQ[t * h + c] * W2n[static_cast<size_t>(i) * h + c];
          float corr = 0.0f;
          for (int s = 0; s <= t; ++s) corr += P2[t * kSub + s] * Rs[s * D + i];
          float zt = o - corr;
          if constexpr (kPaper) zt = Qs[e] + gam * ln_row<D>(zt, a.ln_eps).xh + bet;
          if (t < n) z[static_cast<size_t>(s0 + t) * D + i] = from_f32<IO>(zt);
        }
        __syncthreads();
      }
      // W1n -= dU^T K ; W2n -= R^T A  (rates are in dU and R)
      for (size_t e = tid; e < hd; e += kThreads) {
        const int c = static_cast<int>(e / D), j = static_cast<int>(e % D);
        float acc = 0.0f;
        for (int t = 0; t < n; ++t) acc += DU[t * h + c] * Ks[t * D + j];
        W1n[e] -= acc;
      }
      for (size_t e = tid; e < hd; e += kThreads) {
        const int i = static_cast<int>(e / h), c = static_cast<int>(e % h);
        float acc = 0.0f;
        for (int t = 0; t < n; ++t) acc += Rs[t * D + i] * Ab[t * h + c];
        W2n[e] -= acc;
      }
      __syncthreads();
    }
    for (size_t e = tid; e < hd; e += kThreads) {
      W1c[e] = W1n[e];
      W2c[e] = W2n[e];
    }
    __syncthreads();
  }

  if (!a.causal && a.z) {
    for (int s0 = 0; s0 < T; s0 += kSub) {
      const int n = min(kSub, T - s0);
      for (int e = tid; e < kSub * D; e += kThreads) {
        const int t = e / D;
        Qs[e] = t < n ? to_f32(q[static_cast<size_t>(s0) * D + e]) : 0.0f;
      }
      __syncthreads();
      for (int e = tid; e < kSub * h; e += kThreads) {
        const int t = e / h, c = e % h;
        float u = 0.0f;
        for (int j = 0; j < D; ++j) u += Qs[t * D + j] * W1n[static_cast<size_t>(c) * D + j];
        AQ[e] = act_<kPaper>(u);
      }
      __syncthreads();
      for (int e = tid; e < kSub * D; e += kThreads) {
        const int t = e / D, i = e % D;
        float o = 0.0f;
        for (int c = 0; c < h; ++c) o += AQ[t * h + c] * W2n[static_cast<size_t>(i) * h + c];
        if constexpr (kPaper) o = Qs[e] + gam * ln_row<D>(o, a.ln_eps).xh + bet;
        if (t < n) z[static_cast<size_t>(s0 + t) * D + i] = from_f32<IO>(o);
      }
      __syncthreads();
    }
  }

  if (a.w1_out) {
    float* o = a.w1_out + static_cast<size_t>(chain) * hd;
    for (size_t e = tid; e < hd; e += kThreads) o[e] = W1n[e];
  }
  if (a.w2_out) {
    float* o = a.w2_out + static_cast<size_t>(chain) * hd;
    for (size_t e = tid; e < hd; e += kThreads) o[e] = W2n[e];
  }
}

template <typename IO, int D, bool kPaper>
hipError_t launch_one(const MlpArgs& a, float* ws, hipStream_t s) {
  const size_t lds = MlpLds<D>::total(a.dh) * sizeof(float);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&mlp_generic_kernel<IO, D, kPaper>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((mlp_generic_kernel<IO, D, kPaper>), dim3(a.B * a.H), dim3(kThreads), lds, s, a, ws);
  return hipGetLastError();
}

template <typename IO, bool kPaper>
hipError_t launch_d(const MlpArgs& a, float* ws, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_one<IO, 16, kPaper>(a, ws, s);
    case 32: return launch_one<IO, 32, kPaper>(a, ws, s);
    case 64: return launch_one<IO, 64, kPaper>(a, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t mlp_generic_workspace_floats(const MlpArgs& a) {
  return static_cast<size_t>(a.B) * a.H * 4 * static_cast<size_t>(a.dh) * a.d;
}

hipError_t launch_mlp_generic(const MlpArgs& a, bool bf16_io, float* ws, hipStream_t s) {
  if (a.ln_w) return bf16_io ? launch_d<bf16, true>(a, ws, s) : launch_d<float, true>(a, ws, s);
  return bf16_io ? launch_d<bf16, false>(a, ws, s) : launch_d<float, false>(a, ws, s);
}

}  // namespace ttt
