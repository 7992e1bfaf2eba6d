// Backward pass of the paper's causal TTT-Linear layer, f(x) = x + LN(W x) (wmrh.cn summary
// of Sun et al. 2024, section 2.2.1), on the vector ALUs: reconstruction or negative
// dot-product loss, scalar rate or per-token rate factors, chunk <= 16, d in {16, 32, 64},
// fp32 or bf16 I/O.  One workgroup of 1024 threads per (batch, head) chain walks the chunks
// from last to first; thread (t, i) holds feature i of token t of the chunk, so the layer
// norm's sums over a token's features are sums over D consecutive lanes.
//
// The outer loop trains q, k, v, the initial state, the rates and the layer norm's gain and
// bias through the inner updates (wmrh.cn summary, sections 2.2 and 2.2.3).  Forward chunk
// from W = W_c (LN(y) = gamma xh + beta, xh = (y - mean y) / s, s = sqrt(var y + eps);
// P_y(w) = w - mean(w) - xh mean(w xh) the projection of the layer norm's Jacobian):
//   Y_t = W k_t,  err_t = k_t + LN(Y_t) - v_t (or -v_t),  r_t = P_{Y_t}(gamma err_t) / s_t,
//   rt_t = e_t r_t,  Yq_t = W q_t - eta sum_{s<=t} (k_s . q_t) rt_s,  z_t = q_t + LN(Yq_t),
//   W_{c+1} = W - eta sum_s rt_s k_s^T.
// Reverse mode, with G = dL/dW_{c+1} and dz (our derivation of the chain rule):
//   a_t = P_{Yq_t}(gamma dz_t) / sq_t;  dgamma += dz xhq, dbeta += dz;  dq_t = dz_t + W^T a_t
//     + sum_{s<=t} dP_ts k_s with dP_ts = -eta a_t . rt_s;
//   drt_s = -eta (G k_s + sum_{t>=s} (k_s . q_t) a_t);  dk_s gets -eta G^T rt_s
//     + sum_{t>=s} dP_ts q_t;  dr_s = e_s drt_s, de_s = <drt_s, r_s>;
//   through r = P(gamma err) / s, with w = dr:  derr = gamma P(w) / s,  dgamma += err P(w) / s,
//     and the second-order term of the layer norm's Jacobian,
//     dY = -(xh <w, P(gg)> / D + mean(gg xh) P(w) + P(gg) <w, xh> / D) / s^2,  gg = gamma err;
//   through err = k + LN(Y) - v (reconstruction loss only):  dk += derr,  dv = -derr,
//     dY += P(gamma derr) / s,  dgamma += derr xh,  dbeta += derr  (dot loss: dv = -derr);
//   dk_s += W^T dY_s;  dL/dW_c = G + sum_t a_t q_t^T + sum_s dY_s k_s^T.
// The chunk-start states come from the forward recomputation on the generic kernel, which
// stores them (w_hist).
#include "common.hpp"

namespace ttt {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxB = 16;

template <int D>
struct LnBwdLds {  // float offsets in the dynamic LDS block
  static constexpr int kM = D * (D + 1);        // a D x D matrix, rows padded
  static constexpr int kT = kMaxB * (D + 1);    // a [kMaxB][D] token tile, rows padded
  static constexpr int kS = kMaxB * (kMaxB + 1);
  static constexpr int W = 0, G = kM, Q = 2 * kM, K = Q + kT, V = K + kT, DZ = V + kT, RT = DZ + kT,
                       R0 = RT + kT, XH = R0 + kT, ERR = XH + kT, A = ERR + kT, DRT = A + kT,
                       DERR = DRT + kT, DY = DERR + kT, DG = DY + kT, DB = DG + kT, P = DB + kT,
                       DP = P + kS, ET = DP + kS, GAM = ET + kMaxB, BET = GAM + D,
                       TOTAL = BET + D;
};

template <typename IO, int D>
__global__ __launch_bounds__(kThreads) void linear_ln_bwd_kernel(LinearBwdArgs a) {
  extern __shared__ float lds[];
  using L = LnBwdLds<D>;
  constexpr int S = D + 1;  // padded row stride
  float* Wc = lds + L::W;
  float* G = lds + L::G;
  float* Qs = lds + L::Q;
  float* Ks = lds + L::K;
  float* Vs = lds + L::V;
  float* dZ = lds + L::DZ;
  float* Rt = lds + L::RT;
  float* R0 = lds + L::R0;
  float* Xh = lds + L::XH;
  float* Er = lds + L::ERR;
  float* Aq = lds + L::A;
  float* dRt = lds + L::DRT;
  float* dEr = lds + L::DERR;
  float* dY = lds + L::DY;
  float* Dg = lds + L::DG;   // per-token contributions to dgamma
  float* Db = lds + L::DB;   // ... and to dbeta
  float* Ps = lds + L::P;
  float* dP = lds + L::DP;
  float* et = lds + L::ET;
  float* gam = lds + L::GAM;
  float* bet = lds + L::BET;

  const int tid = threadIdx.x;
  const int chain = blockIdx.x;
  const int hi = chain % a.H;
  const int T = a.T;
  const float eta = a.eta, eps = a.ln_eps;
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
  const bool mse = !a.dot_loss;

  // thread (t, i): feature i of token t (all threads of a wave active together: D divides 64)
  const bool own = tid < kMaxB * D;
  const int t = tid / D, i = tid % D;
  float dgam = 0.0f, dbet = 0.0f;  // this thread's share of dgamma_i, dbeta_i (threads t = 0)

  for (int e = tid; e < D * D; e += kThreads)
    G[(e / D) * S + e % D] = a.dw_out ? a.dw_out[static_cast<size_t>(chain) * D * D + e] : 0.0f;
  for (int e = tid; e < D; e += kThreads) {
    gam[e] = a.ln_w[hi * D + e];
    bet[e] = a.ln_b[hi * D + e];
  }

  for (int c = nchunks - 1; c >= 0; --c) {
    const int c0 = c * b;
    const int n = min(b, T - c0);
    __syncthreads();  // G of the later chunk is complete; the tiles are free
    for (int e = tid; e < D * D; e += kThreads) Wc[(e / D) * S + e % D] = wh[static_cast<size_t>(c) * D * D + e];
    if (own) {
      const bool in = t < n;
      const size_t off = static_cast<size_t>(c0 + t) * D + i;
      Qs[t * S + i] = in ? to_f32(q[off]) : 0.0f;
      Ks[t * S + i] = in ? to_f32(k[off]) : 0.0f;
      Vs[t * S + i] = in ? to_f32(v[off]) : 0.0f;
      dZ[t * S + i] = in ? to_f32(dz[off]) : 0.0f;
    }
    if (tid < kMaxB) et[tid] = tid < n ? (etok ? etok[c0 + tid] : 1.0f) : 0.0f;
    __syncthreads();
    // keys: Y, xh, err, r, rt;  P = tril(Q K^T)
    float xh = 0.0f, sk = 1.0f, err = 0.0f, r = 0.0f, bm = 0.0f;
    if (own) {
      float y = 0.0f;
      for (int j = 0; j < D; ++j) y += Wc[i * S + j] * Ks[t * S + j];
      const LnRow st = ln_row<D>(y, eps);
      xh = st.xh;
      sk = 1.0f / st.rstd;
      err = (mse ? Ks[t * S + i] + gam[i] * xh + bet[i] : 0.0f) - Vs[t * S + i];
      const float gg = gam[i] * err;
      const float m1 = group_sum<D>(gg) * (1.0f / D);
      bm = group_sum<D>(gg * xh) * (1.0f / D);
      r = t < n ? (gg - m1 - xh * bm) * st.rstd : 0.0f;
      Xh[t * S + i] = xh;
      Er[t * S + i] = err;
      R0[t * S + i] = r;
      Rt[t * S + i] = et[t] * r;
    }
    for (int e = tid; e < kMaxB * kMaxB; e += kThreads) {
      const int tt = e / kMaxB, s = e % kMaxB;
      float acc = 0.0f;
      if (s <= tt && tt < n)
        for (int j = 0; j < D; ++j) acc += Qs[tt * S + j] * Ks[s * S + j];
      Ps[tt * (kMaxB + 1) + s] = acc;
    }
    __syncthreads();
    // queries: Yq = W q - eta sum_{s<=t} P_ts rt_s; a = P_{Yq}(gamma dz) / sq
    if (own) {
      float yq = 0.0f;
      for (int j = 0; j < D; ++j) yq += Wc[i * S + j] * Qs[t * S + j];
      for (int s = 0; s <= t; ++s) yq -= eta * Ps[t * (kMaxB + 1) + s] * Rt[s * S + i];
      const LnRow st = ln_row<D>(yq, eps);
      const float g = dZ[t * S + i];
      const float gz = gam[i] * g;
      const float m1 = group_sum<D>(gz) * (1.0f / D);
      const float m2 = group_sum<D>(gz * st.xh) * (1.0f / D);
      Aq[t * S + i] = t < n ? (gz - m1 - st.xh * m2) * st.rstd : 0.0f;
      Dg[t * S + i] = t < n ? g * st.xh : 0.0f;
      Db[t * S + i] = g;
    }
    __syncthreads();
    // drt = -eta (G k + sum_{t'>=t} P_t't a_t');  dP_ts = -eta a_t . rt_s
    if (own) {
      float acc = 0.0f;
      for (int j = 0; j < D; ++j) acc += G[i * S + j] * Ks[t * S + j];
      for (int s = t; s < n; ++s) acc += Ps[s * (kMaxB + 1) + t] * Aq[s * S + i];
      dRt[t * S + i] = t < n ? -eta * acc : 0.0f;
    }
    for (int e = tid; e < kMaxB * kMaxB; e += kThreads) {
      const int tt = e / kMaxB, s = e % kMaxB;
      float acc = 0.0f;
      if (s <= tt && tt < n)
        for (int j = 0; j < D; ++j) acc += Aq[tt * S + j] * Rt[s * S + j];
      dP[tt * (kMaxB + 1) + s] = -eta * acc;
    }
    __syncthreads();
    // the rates' gradient; dr = e drt; back through r = P(gamma err) / s and err
    if (own) {
      const float drt = dRt[t * S + i];
      const float de = group_sum<D>(drt * r);
      if (detok && i == 0 && t < n) detok[c0 + t] = de;
      const float w = et[t] * drt;
      const float pw = w - group_sum<D>(w) * (1.0f / D) - xh * (group_sum<D>(w * xh) * (1.0f / D));
      const float gg = gam[i] * err;
      const float pgg = sk * r;  // P(gg)
      const float w_pgg = group_sum<D>(w * pgg) * (1.0f / D);
      const float w_xh = group_sum<D>(w * xh) * (1.0f / D);
      const float derr = gam[i] * pw / sk;
      float dy = -(xh * w_pgg + bm * pw + pgg * w_xh) / (sk * sk);
      float dgl = err * pw / sk;
      float dbl = 0.0f;
      if (mse) {  // err = k + LN(Y) - v
        const float u = gam[i] * derr;
        const float pu = u - group_sum<D>(u) * (1.0f / D) - xh * (group_sum<D>(u * xh) * (1.0f / D));
        dy += pu / sk;
        dgl += derr * xh;
        dbl += derr;
      }
      (void)gg;
      dEr[t * S + i] = t < n ? derr : 0.0f;
      dY[t * S + i] = t < n ? dy : 0.0f;
      if (t < n) {
        Dg[t * S + i] += dgl;
        Db[t * S + i] += dbl;
      }
    }
    __syncthreads();
    // dq = dz + W^T a + sum_{s<=t} dP_ts k_s;  dk = derr (reconstruction) + W^T dY - eta G^T rt
    // + sum_{t'>=t} dP_t't q_t';  dv = -derr
    if (own && t < n) {
      const int j = i;
      float aq = dZ[t * S + j], ak = mse ? dEr[t * S + j] : 0.0f;
      for (int ii = 0; ii < D; ++ii) {
        aq += Wc[ii * S + j] * Aq[t * S + ii];
        ak += Wc[ii * S + j] * dY[t * S + ii] - eta * G[ii * S + j] * Rt[t * S + ii];
      }
      for (int s = 0; s <= t; ++s) aq += dP[t * (kMaxB + 1) + s] * Ks[s * S + j];
      for (int s = t; s < n; ++s) ak += dP[s * (kMaxB + 1) + t] * Qs[s * S + j];
      const size_t off = static_cast<size_t>(c0 + t) * D + j;
      dq[off] = from_f32<IO>(aq);
      dk[off] = from_f32<IO>(ak);
      dv[off] = from_f32<IO>(-dEr[t * S + j]);
    }
    // the gain's and the bias's gradients (thread t = 0 of each feature)
    if (own && t == 0) {
      for (int s = 0; s < n; ++s) {
        dgam += Dg[s * S + i];
        dbet += Db[s * S + i];
      }
    }
    __syncthreads();  // the old G is read above; now dL/dW_c = G + sum a q^T + sum dY k^T
    for (int e = tid; e < D * D; e += kThreads) {
      const int ii = e / D, j = e % D;
      float acc = 0.0f;
      for (int s = 0; s < n; ++s) acc += Aq[s * S + ii] * Qs[s * S + j] + dY[s * S + ii] * Ks[s * S + j];
      G[ii * S + j] += acc;
    }
  }
  __syncthreads();
  float* dw0 = a.dw0 + static_cast<size_t>(chain) * D * D;
  for (int e = tid; e < D * D; e += kThreads) dw0[e] = G[(e / D) * S + e % D];
  if (own && t == 0) {
    a.dln_w[static_cast<size_t>(chain) * D + i] = dgam;
    a.dln_b[static_cast<size_t>(chain) * D + i] = dbet;
  }
}

template <typename IO, int D>
hipError_t launch_one(const LinearBwdArgs& a, hipStream_t s) {
  const size_t lds = LnBwdLds<D>::TOTAL * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&linear_ln_bwd_kernel<IO, D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((linear_ln_bwd_kernel<IO, D>), dim3(a.B * a.H), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <typename IO>
hipError_t launch_d(const LinearBwdArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_one<IO, 16>(a, s);
    case 32: return launch_one<IO, 32>(a, s);
    case 64: return launch_one<IO, 64>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_linear_ln_bwd(const LinearBwdArgs& a, bool bf16_io, hipStream_t s) {
  if (a.chunk < 1 || a.T < 1 || min(a.chunk, a.T) > kMaxB || !a.ln_w || !a.ln_b || !a.dln_w || !a.dln_b)
    return hipErrorInvalidValue;
  return bf16_io ? launch_d<bf16>(a, s) : launch_d<float>(a, s);
}

}  // namespace ttt
