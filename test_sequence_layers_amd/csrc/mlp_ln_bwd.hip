// Backward pass of the paper's causal TTT-MLP layer, f(x) = x + LN(W2 GELU(W1 x)) (wmrh.cn
// summary of Sun et al. 2024, section 2.2.1), on the vector ALUs: reconstruction or negative
// dot-product loss, scalar rate or per-token rate factors, chunk <= 16, hidden width <= 256,
// d in {16, 32, 64}, fp32 or bf16 I/O.  One workgroup of 1024 threads per (batch, head) chain
// walks the chunks from last to first.
//
// Forward chunk from W1, W2 (phi = GELU, LN(y) = gamma xh + beta, xh = (y - mean y) / s,
// s = sqrt(var y + eps), P_y(w) = w - mean(w) - xh mean(w xh)):
//   U = K W1^T, A = phi(U), Y = A W2^T, Err = K + LN(Y) - V (or -V),
//   R = P_Y(gamma Err) / s (row by row), Rt = diag(e) R, Dm = Rt W2, dU = Dm * phi'(U),
//   W1n = W1 - eta dU^T K,  W2n = W2 - eta Rt^T A,
//   Uq = Q W1^T - eta M dU (M = tril(Q K^T)), Aq = phi(Uq), N = tril(Aq A^T),
//   Yq = Aq W2^T - eta N Rt,  Z = Q + LN(Yq).
// Reverse mode (our derivation of the chain rule; the lines of the plain TTT-MLP backward with
// Rt in place of R and a = P_Yq(gamma dZ) / sq in place of dZ), with G1, G2 from the later
// chunks:
//   Nb = -eta tril(a Rt^T),  dAq = a W2 + Nb A,  dA = Nb^T Aq - eta Rt G2,
//   dRt = -eta (N^T a + A G2^T) + (ddU * phi'(U)) W2^T,  dUq = dAq * phi'(Uq),
//   Mb = -eta tril(dUq dU^T),  ddU = -eta (M^T dUq + K G1^T);
//   de = <dRt, R> (rows),  w = diag(e) dRt;  through R = P_Y(gamma Err) / s:
//     dErr = gamma P(w) / s,  dgamma += Err P(w) / s,
//     dY = -(xh <w, P(gg)> / D + mean(gg xh) P(w) + P(gg) <w, xh> / D) / s^2  (gg = gamma Err),
//   through Err = K + LN(Y) - V (reconstruction loss only): dK += dErr, dY += P(gamma dErr) / s,
//     dgamma += dErr xh, dbeta += dErr;  dV = -dErr;
//   dUk = (dA + dY W2) * phi'(U) + ddU * Dm * phi''(U),
//   dQ = dZ + dUq W1 + Mb K,  dK += Mb^T Q - eta dU G1 + dUk W1,
//   dL/dW1 = G1 + dUq^T Q + dUk^T K,  dL/dW2 = G2 + a^T Aq + Rt^T (ddU * phi'(U)) + dY^T A,
//   dgamma += sum dZ xhq,  dbeta += sum dZ.
// The chunk-start states come from the forward recomputation on the generic kernel, which
// stores them (w_hist); G1 and G2 accumulate in the dw1 / dw2 outputs.
#include "common.hpp"

namespace ttt {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxB = 16;
constexpr int kMaxH = 256;

__device__ __forceinline__ float gelu_pdf(float u) { return 0.39894228040143268f * __expf(-0.5f * u * u); }
__device__ __forceinline__ float d2gelu(float u) { return gelu_pdf(u) * (2.0f - u * u); }

template <int D>
struct LnMlpLds {  // float offsets in the dynamic LDS block for hidden width h
  static __host__ __device__ size_t tok(int i) { return static_cast<size_t>(i) * kMaxB * D; }  // 10 [b][D]
  static __host__ __device__ size_t small() { return tok(10); }  // Sk, Bm, Es [b]; Dg, Db [D]
  static __host__ __device__ size_t sq(int i) {
    return small() + 3 * kMaxB + 2 * D + static_cast<size_t>(i) * kMaxB * kMaxB;  // 4 [b][b]
  }
  static __host__ __device__ size_t hid(int i, int h) { return sq(4) + static_cast<size_t>(i) * kMaxB * h; }
  static __host__ __device__ size_t total(int h) { return hid(7, h); }
};

template <typename IO, int D>
__global__ __launch_bounds__(kThreads) void mlp_ln_bwd_kernel(MlpBwdArgs a) {
  extern __shared__ float lds[];
  using L = LnMlpLds<D>;
  const int h = a.dh;
  float* Ks = lds + L::tok(0);
  float* Qs = lds + L::tok(1);
  float* Er = lds + L::tok(2);   // V, then Err
  float* Zd = lds + L::tok(3);   // dZ
  float* Za = lds + L::tok(4);   // a = P_Yq(gamma dZ) / sq
  float* Rs = lds + L::tok(5);   // Rt = diag(e) R
  float* R0 = lds + L::tok(6);   // R
  float* Xh = lds + L::tok(7);   // xh of the keys' Y
  float* Rb = lds + L::tok(8);   // dRt, then dY
  float* De = lds + L::tok(9);   // dErr
  float* Sk = lds + L::small();  // s of the keys' Y
  float* Bm = Sk + kMaxB;        // mean(gg xh)
  float* Es = Bm + kMaxB;        // rate factors (0 on padded rows)
  float* Dg = Es + kMaxB;        // dgamma
  float* Db = Dg + D;            // dbeta
  float* Mm = lds + L::sq(0);
  float* Nn = lds + L::sq(1);
  float* Nb = lds + L::sq(2);
  float* Mb = lds + L::sq(3);
  float* Hu = lds + L::hid(0, h);   // U
  float* Ha = lds + L::hid(1, h);   // A
  float* Hdu = lds + L::hid(2, h);  // dU
  float* Haq = lds + L::hid(3, h);  // Aq
  float* Huq = lds + L::hid(4, h);  // Uq, then dUq
  float* Hda = lds + L::hid(5, h);  // dA, then dUk
  float* Hdd = lds + L::hid(6, h);  // ddU

  const int tid = threadIdx.x;
  const int chain = blockIdx.x;
  const int hi = chain % a.H;
  const int T = a.T;
  const float eta = a.eta, eps = a.ln_eps;
  const bool mse = !a.dot_loss;
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
  // thread (t, i): feature i of token t (a token's D features in D consecutive lanes)
  const bool own = tid < kMaxB * D;
  const int t = tid / D, i = tid % D;
  const float gam = own ? a.ln_w[hi * D + i] : 0.0f;
  const float bet = own ? a.ln_b[hi * D + i] : 0.0f;

  for (size_t e = tid; e < hd; e += kThreads) {
    G1[e] = a.dw1_out ? a.dw1_out[static_cast<size_t>(chain) * hd + e] : 0.0f;
    G2[e] = a.dw2_out ? a.dw2_out[static_cast<size_t>(chain) * hd + e] : 0.0f;
  }
  for (int e = tid; e < D; e += kThreads) Dg[e] = Db[e] = 0.0f;

  for (int c = nchunks - 1; c >= 0; --c) {
    const int c0 = c * b;
    const int n = min(b, T - c0);
    const float* W1 = a.w_hist + (static_cast<size_t>(chain) * nchunks + c) * 2 * hd;  // [h][D]
    const float* W2 = W1 + hd;                                                          // [D][h]
    const bool in = own && t < n;
    __syncthreads();  // the previous chunk is done with every buffer; G1, G2 are complete
    if (own) {
      const size_t off = static_cast<size_t>(c0 + t) * D + i;
      Ks[tid] = in ? to_f32(k[off]) : 0.0f;
      Qs[tid] = in ? to_f32(q[off]) : 0.0f;
      Er[tid] = in ? to_f32(v[off]) : 0.0f;
      Zd[tid] = in ? to_f32(dz[off]) : 0.0f;
    }
    if (tid < kMaxB) Es[tid] = tid < n ? (etok ? etok[c0 + tid] : 1.0f) : 0.0f;
    __syncthreads();
    // U = K W1^T, A = phi(U);  M = tril(Q K^T)
    for (int e = tid; e < kMaxB * h; e += kThreads) {
      const int tt = e / h, cc = e % h;
      float u = 0.0f;
      for (int j = 0; j < D; ++j) u += Ks[tt * D + j] * W1[static_cast<size_t>(cc) * D + j];
      Hu[e] = u;
      Ha[e] = gelu_(u);
    }
    for (int e = tid; e < kMaxB * kMaxB; e += kThreads) {
      const int tt = e / kMaxB, s = e % kMaxB;
      float acc = 0.0f;
      if (s <= tt && tt < n)
        for (int j = 0; j < D; ++j) acc += Qs[tt * D + j] * Ks[s * D + j];
      Mm[e] = acc;
    }
    __syncthreads();
    // Y = A W2^T, Err, R = P_Y(gamma Err) / s, Rt = e R
    if (own) {
      float y = 0.0f;
      for (int cc = 0; cc < h; ++cc) y += Ha[t * h + cc] * W2[static_cast<size_t>(i) * h + cc];
      const LnRow st = ln_row<D>(y, eps);
      const float err = (mse ? Ks[tid] + gam * st.xh + bet : 0.0f) - Er[tid];
      const float gg = gam * err;
      const float m1 = group_sum<D>(gg) * (1.0f / D);
      const float bm = group_sum<D>(gg * st.xh) * (1.0f / D);
      const float r = in ? (gg - m1 - st.xh * bm) * st.rstd : 0.0f;
      Er[tid] = err;
      Xh[tid] = st.xh;
      R0[tid] = r;
      Rs[tid] = Es[t] * r;
      if (i == 0) {
        Sk[t] = 1.0f / st.rstd;
        Bm[t] = bm;
      }
    }
    __syncthreads();
    // dU = (Rt W2) * phi'(U)
    for (int e = tid; e < kMaxB * h; e += kThreads) {
      const int tt = e / h, cc = e % h;
      float dm = 0.0f;
      for (int ii = 0; ii < D; ++ii) dm += Rs[tt * D + ii] * W2[static_cast<size_t>(ii) * h + cc];
      Hdu[e] = dm * dgelu_(Hu[e]);
    }
    __syncthreads();
    // Uq = Q W1^T - eta M dU, Aq = phi(Uq)
    for (int e = tid; e < kMaxB * h; e += kThreads) {
      const int tt = e / h, cc = e % h;
      float u = 0.0f;
      for (int j = 0; j < D; ++j) u += Qs[tt * D + j] * W1[static_cast<size_t>(cc) * D + j];
      for (int s = 0; s <= tt; ++s) u -= eta * Mm[tt * kMaxB + s] * Hdu[s * h + cc];
      Huq[e] = u;
      Haq[e] = gelu_(u);
    }
    __syncthreads();
    // N = tril(Aq A^T)
    for (int e = tid; e < kMaxB * kMaxB; e += kThreads) {
      const int tt = e / kMaxB, s = e % kMaxB;
      float nn = 0.0f;
      if (s <= tt && tt < n)
        for (int cc = 0; cc < h; ++cc) nn += Haq[tt * h + cc] * Ha[s * h + cc];
      Nn[e] = nn;
    }
    __syncthreads();
    // Yq = Aq W2^T - eta N Rt;  a = P_Yq(gamma dZ) / sq;  the output LN's gain / bias gradients
    if (own) {
      float y = 0.0f;
      for (int cc = 0; cc < h; ++cc) y += Haq[t * h + cc] * W2[static_cast<size_t>(i) * h + cc];
      for (int s = 0; s <= t; ++s) y -= eta * Nn[t * kMaxB + s] * Rs[s * D + i];
      const LnRow st = ln_row<D>(y, eps);
      const float g = Zd[tid];
      const float gz = gam * g;
      const float m1 = group_sum<D>(gz) * (1.0f / D);
      const float m2 = group_sum<D>(gz * st.xh) * (1.0f / D);
      Za[tid] = in ? (gz - m1 - st.xh * m2) * st.rstd : 0.0f;
      if (in) {
        atomicAdd(&Dg[i], g * st.xh);
        atomicAdd(&Db[i], g);
      }
    }
    __syncthreads();
    // Nb = -eta tril(a Rt^T)
    for (int e = tid; e < kMaxB * kMaxB; e += kThreads) {
      const int tt = e / kMaxB, s = e % kMaxB;
      float nb = 0.0f;
      if (s <= tt && tt < n)
        for (int ii = 0; ii < D; ++ii) nb += Za[tt * D + ii] * Rs[s * D + ii];
      Nb[e] = -eta * nb;
    }
    __syncthreads();
    // dUq = (a W2 + Nb A) * phi'(Uq);  dA = Nb^T Aq - eta Rt G2;  dRt = -eta (N^T a + A G2^T)
    for (int e = tid; e < kMaxB * h; e += kThreads) {
      const int tt = e / h, cc = e % h;
      float daq = 0.0f, da = 0.0f, rg = 0.0f;
      for (int ii = 0; ii < D; ++ii) {
        daq += Za[tt * D + ii] * W2[static_cast<size_t>(ii) * h + cc];
        rg += Rs[tt * D + ii] * G2[static_cast<size_t>(ii) * h + cc];
      }
      for (int s = 0; s < kMaxB; ++s) {
        daq += Nb[tt * kMaxB + s] * Ha[s * h + cc];
        da += Nb[s * kMaxB + tt] * Haq[s * h + cc];
      }
      Huq[e] = daq * dgelu_(Huq[e]);
      Hda[e] = da - eta * rg;
    }
    if (own) {
      float acc = 0.0f, ag = 0.0f;
      for (int s = 0; s < kMaxB; ++s) acc += Nn[s * kMaxB + t] * Za[s * D + i];
      for (int cc = 0; cc < h; ++cc) ag += Ha[t * h + cc] * G2[static_cast<size_t>(i) * h + cc];
      Rb[tid] = -eta * (acc + ag);
    }
    __syncthreads();
    // Mb = -eta tril(dUq dU^T);  ddU = -eta (M^T dUq + K G1^T)
    for (int e = tid; e < kMaxB * kMaxB; e += kThreads) {
      const int tt = e / kMaxB, s = e % kMaxB;
      float acc = 0.0f;
      if (s <= tt && tt < n)
        for (int cc = 0; cc < h; ++cc) acc += Huq[tt * h + cc] * Hdu[s * h + cc];
      Mb[e] = -eta * acc;
    }
    for (int e = tid; e < kMaxB * h; e += kThreads) {
      const int tt = e / h, cc = e % h;
      float acc = 0.0f;
      for (int s = 0; s < kMaxB; ++s) acc += Mm[s * kMaxB + tt] * Huq[s * h + cc];
      for (int j = 0; j < D; ++j) acc += Ks[tt * D + j] * G1[static_cast<size_t>(cc) * D + j];
      Hdd[e] = -eta * acc;
    }
    __syncthreads();
    // dRt += (ddU * phi'(U)) W2^T
    if (own) {
      float acc = 0.0f;
      for (int cc = 0; cc < h; ++cc)
        acc += Hdd[t * h + cc] * dgelu_(Hu[t * h + cc]) * W2[static_cast<size_t>(i) * h + cc];
      Rb[tid] += acc;
    }
    __syncthreads();
    // the rates' gradient; back through R = P_Y(gamma Err) / s and Err: dErr, dY; dV = -dErr
    if (own) {
      const float drt = Rb[tid];
      const float r = R0[tid], xh = Xh[tid], err = Er[tid];
      const float s = Sk[t], bm = Bm[t];
      const float de = group_sum<D>(drt * r);
      if (a.deta_tok && i == 0 && t < n) a.deta_tok[static_cast<size_t>(chain) * T + c0 + t] = de;
      const float w = Es[t] * drt;
      const float pw = w - group_sum<D>(w) * (1.0f / D) - xh * (group_sum<D>(w * xh) * (1.0f / D));
      const float pgg = s * r;
      const float w_pgg = group_sum<D>(w * pgg) * (1.0f / D);
      const float w_xh = group_sum<D>(w * xh) * (1.0f / D);
      const float derr = gam * pw / s;
      float dy = -(xh * w_pgg + bm * pw + pgg * w_xh) / (s * s);
      float dg = err * pw / s, db = 0.0f;
      if (mse) {
        const float u = gam * derr;
        const float pu = u - group_sum<D>(u) * (1.0f / D) - xh * (group_sum<D>(u * xh) * (1.0f / D));
        dy += pu / s;
        dg += derr * xh;
        db += derr;
      }
      Rb[tid] = in ? dy : 0.0f;
      De[tid] = in ? derr : 0.0f;
      if (in) {
        atomicAdd(&Dg[i], dg);
        atomicAdd(&Db[i], db);
        dv[static_cast<size_t>(c0 + t) * D + i] = from_f32<IO>(-derr);
      }
    }
    __syncthreads();
    // dUk = (dA + dY W2) * phi'(U) + ddU * (Rt W2) * phi''(U)
    for (int e = tid; e < kMaxB * h; e += kThreads) {
      const int tt = e / h, cc = e % h;
      float yw = 0.0f, dm = 0.0f;
      for (int ii = 0; ii < D; ++ii) {
        const float w = W2[static_cast<size_t>(ii) * h + cc];
        yw += Rb[tt * D + ii] * w;
        dm += Rs[tt * D + ii] * w;
      }
      const float u = Hu[e];
      Hda[e] = (Hda[e] + yw) * dgelu_(u) + Hdd[e] * dm * d2gelu(u);
    }
    __syncthreads();
    // dQ = dZ + dUq W1 + Mb K;  dK = dErr (reconstruction) + Mb^T Q - eta dU G1 + dUk W1
    if (in) {
      const int j = i;
      float aq = Zd[tid], ak = mse ? De[tid] : 0.0f;
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
    // G1 += dUq^T Q + dUk^T K;  G2 += a^T Aq + Rt^T (ddU * phi'(U)) + dY^T A
    for (size_t e = tid; e < hd; e += kThreads) {
      const int cc = static_cast<int>(e / D), j = static_cast<int>(e % D);
      float acc = 0.0f;
      for (int tt = 0; tt < n; ++tt) acc += Huq[tt * h + cc] * Qs[tt * D + j] + Hda[tt * h + cc] * Ks[tt * D + j];
      G1[e] += acc;
    }
    for (size_t e = tid; e < hd; e += kThreads) {
      const int ii = static_cast<int>(e / h), cc = static_cast<int>(e % h);
      float acc = 0.0f;
      for (int tt = 0; tt < n; ++tt)
        acc += Za[tt * D + ii] * Haq[tt * h + cc] + Rs[tt * D + ii] * Hdd[tt * h + cc] * dgelu_(Hu[tt * h + cc]) +
               Rb[tt * D + ii] * Ha[tt * h + cc];
      G2[e] += acc;
    }
  }
  __syncthreads();
  for (int e = tid; e < D; e += kThreads) {
    a.dln_w[static_cast<size_t>(chain) * D + e] = Dg[e];
    a.dln_b[static_cast<size_t>(chain) * D + e] = Db[e];
  }
}

template <typename IO, int D>
hipError_t launch_one(const MlpBwdArgs& a, hipStream_t s) {
  const size_t lds = LnMlpLds<D>::total(a.dh) * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&mlp_ln_bwd_kernel<IO, D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mlp_ln_bwd_kernel<IO, D>), dim3(a.B * a.H), dim3(kThreads), lds, s, a);
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

size_t mlp_ln_bwd_lds_bytes(int d, int dh) {
  switch (d) {
    case 16: return LnMlpLds<16>::total(dh) * sizeof(float);
    case 32: return LnMlpLds<32>::total(dh) * sizeof(float);
    default: return LnMlpLds<64>::total(dh) * sizeof(float);
  }
}

hipError_t launch_mlp_ln_bwd(const MlpBwdArgs& a, bool bf16_io, hipStream_t s) {
  if (a.chunk < 1 || a.T < 1 || min(a.chunk, a.T) > kMaxB || a.dh < 1 || a.dh > kMaxH || !a.ln_w ||
      !a.ln_b || !a.dln_w || !a.dln_b || mlp_ln_bwd_lds_bytes(a.d, a.dh) > 160 * 1024)
    return hipErrorInvalidValue;
  return bf16_io ? launch_d<bf16>(a, s) : launch_d<float>(a, s);
}

}  // namespace ttt
