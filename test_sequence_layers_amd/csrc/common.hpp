// Shared device/host helpers of libttt (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef __bf16 bf16;

// Element conversion for the two I/O dtypes.  float -> bf16 rounds to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// SiLU and its derivative, fp32.  sigma(u) = 1 / (1 + exp(-u)), with the hardware
// exponential and reciprocal (v_exp_f32, v_rcp_f32: about 1 ulp each) instead of an IEEE
// division; for large |u| the exponential saturates to 0 or inf and sigma to 1 or 0.
__device__ __forceinline__ float sigmoidf_(float u) { return __builtin_amdgcn_rcpf(1.0f + __expf(-u)); }
__device__ __forceinline__ float silu_(float u) { return u * sigmoidf_(u); }
__device__ __forceinline__ float dsilu_(float u) {
  const float s = sigmoidf_(u);
  return s * (1.0f + u * (1.0f - s));
}

// GELU(u) = u Phi(u) with the exact normal CDF Phi(u) = (1 + erf(u / sqrt 2)) / 2, and its
// derivative Phi(u) + u phi(u) (phi the standard normal density).
__device__ __forceinline__ float gelu_(float u) { return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f)); }
__device__ __forceinline__ float dgelu_(float u) {
  return 0.5f * (1.0f + erff(u * 0.70710678118654752f)) + u * 0.39894228040143268f * __expf(-0.5f * u * u);
}

// Sum over aligned groups of W consecutive lanes of a wave (W a power of two <= 64).  Every
// lane of the wave must take part.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Layer norm over the D features of a token held one per lane by D consecutive lanes:
// xh = (y - mean) / sqrt(var + eps) (biased variance) and rstd = 1 / sqrt(var + eps).
struct LnRow {
  float xh, rstd;
};
template <int D>
__device__ __forceinline__ LnRow ln_row(float y, float eps) {
  const float mu = group_sum<D>(y) * (1.0f / D);
  const float dy = y - mu;
  const float var = group_sum<D>(dy * dy) * (1.0f / D);
  const float rstd = 1.0f / sqrtf(var + eps);
  return {dy * rstd, rstd};
}
// dl/dy of LN(y) = gamma xh + beta given dl/dLN = g (chain rule through the mean and the
// variance): rstd (gg - mean(gg) - xh mean(gg xh)), gg = gamma g.
template <int D>
__device__ __forceinline__ float ln_row_vjp(const LnRow& s, float gamma, float g) {
  const float gg = gamma * g;
  const float m1 = group_sum<D>(gg) * (1.0f / D);
  const float m2 = group_sum<D>(gg * s.xh) * (1.0f / D);
  return s.rstd * (gg - m1 - s.xh * m2);
}

// Arguments of one forward call, as validated by the host API.
struct LinearArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* w0;
  long long w0_batch_stride;  // in floats
  void* z;
  float* w_out;
  int B, H, T, d, chunk, causal;
  float eta;
  const float* eta_tok;  // per-token rate factors [B][H][T] (rate eta * eta_tok[t]) or null
  int dot_loss;          // 1: loss -v^T f(k), error term -v; 0: 1/2 ||f(k) - v||^2
  float* w_hist;         // generic kernel only: chunk-start states [B][H][nchunks][d][d] or null
  int epochs = 1;        // passes over the chunks before the outputs (non-causal only)
  // the paper's inner model f(x) = x + LN(W x): per-head gamma, beta [H][d] (null: f = W x)
  const float* ln_w = nullptr;
  const float* ln_b = nullptr;
  float ln_eps = 0.0f;
};

// Backward pass of the causal TTT-Linear layer (reconstruction loss, scalar rate).
struct LinearBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dz;
  const float* dw_out;  // upstream gradient of the final state [B][H][d][d] or null
  const float* w_hist;  // chunk-start states [B][H][nchunks][d][d] (from the forward)
  void* dq;
  void* dk;
  void* dv;
  float* dw0;           // [B][H][d][d]
  int B, H, T, d, chunk;
  float eta;
  // per-token rate factors [B][H][T] (rate eta * eta_tok[t]) or null; their gradient
  // [B][H][T] (out) or null
  const float* eta_tok = nullptr;
  float* deta_tok = nullptr;
  int dot_loss = 0;  // 1: loss -v^T W k (R = -V)
  // the paper's inner model f(x) = x + LN(W x): per-head gamma, beta [H][d], eps, and their
  // gradients per sequence [B][H][d] (out)
  const float* ln_w = nullptr;
  const float* ln_b = nullptr;
  float ln_eps = 0.0f;
  float* dln_w = nullptr;
  float* dln_b = nullptr;
};

struct MlpArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* w1;
  const float* w2;
  long long w_batch_stride;  // in floats
  void* z;
  float* w1_out;
  float* w2_out;
  int B, H, T, d, dh, chunk, causal;
  float eta;
  const float* eta_tok;  // per-token rate factors [B][H][T] (rate eta * eta_tok[t]) or null
  int dot_loss;          // 1: loss -v^T f(k), error term -v; 0: 1/2 ||f(k) - v||^2
  int epochs = 1;        // passes over the chunks before the outputs (non-causal only)
  // the paper's TTT-MLP: f(x) = x + LN(W2 GELU(W1 x)), per-head gamma, beta [H][d]
  // (null: f = W2 SiLU(W1 x))
  const float* ln_w = nullptr;
  const float* ln_b = nullptr;
  float ln_eps = 0.0f;
  // generic kernel only: chunk-start states [B][H][nchunks][W1 (h d), W2 (d h)] or null
  float* w_hist = nullptr;
};

// Backward pass of the causal TTT-MLP layer (SiLU, reconstruction loss, scalar rate).
struct MlpBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dz;
  const float* dw1_out;  // upstream gradients of the final states [B][H][h][d], [B][H][d][h] or null
  const float* dw2_out;
  const float* w_hist;   // chunk-start states (from the forward)
  void* dq;
  void* dk;
  void* dv;
  float* dw1;            // [B][H][h][d]
  float* dw2;            // [B][H][d][h]
  int B, H, T, d, dh, chunk;
  float eta;
  int dot_loss = 0;      // 1: loss -v^T f(k), error term -v (vector-ALU path only)
  // per-token rate factors [B][H][T] (rate eta * eta_tok[t]) or null; their gradient
  // [B][H][T] (out) or null (vector-ALU path only)
  const float* eta_tok = nullptr;
  float* deta_tok = nullptr;
  // the paper's TTT-MLP x + LN(W2 GELU(W1 x)): per-head gamma, beta [H][d], eps, and their
  // gradients per sequence [B][H][d] (out)
  const float* ln_w = nullptr;
  const float* ln_b = nullptr;
  float ln_eps = 0.0f;
  float* dln_w = nullptr;
  float* dln_b = nullptr;
};

// Host-side launchers (return a hipError_t; argument checks are done by the caller).
hipError_t launch_linear_generic(const LinearArgs& a, bool bf16_io, hipStream_t s);
hipError_t launch_mlp_generic(const MlpArgs& a, bool bf16_io, float* workspace, hipStream_t s);
size_t mlp_generic_workspace_floats(const MlpArgs& a);

// Matrix-core paths for the shapes they are written for (the *_supported predicates say
// which); everything else runs on the generic kernels.
bool linear_mfma_supported(const LinearArgs& a, bool bf16_io);
hipError_t launch_linear_mfma(const LinearArgs& a, hipStream_t s);
bool linear_ln_mfma_supported(const LinearArgs& a, bool bf16_io);
hipError_t launch_linear_ln_mfma(const LinearArgs& a, hipStream_t s);
bool delta_fast_supported(const LinearArgs& a, bool bf16_io);
hipError_t launch_delta_fast(const LinearArgs& a, hipStream_t s);
bool mlp_fast_supported(const MlpArgs& a, bool bf16_io);
hipError_t launch_mlp_fast(const MlpArgs& a, hipStream_t s);
// the same layer on two workgroups per chain (recursion, outputs) with a caller workspace
bool mlp_split_supported(const MlpArgs& a, bool bf16_io);
size_t mlp_split_workspace_bytes(const MlpArgs& a);
hipError_t launch_mlp_split(const MlpArgs& a, void* ws, uint32_t tag, int dbg, hipStream_t s);
bool linear_nc_supported(const LinearArgs& a, bool bf16_io);
hipError_t launch_linear_nc(const LinearArgs& a, hipStream_t s);
bool mlp_nc_supported(const MlpArgs& a, bool bf16_io);
hipError_t launch_mlp_nc(const MlpArgs& a, hipStream_t s);

hipError_t launch_linear_bwd_generic(const LinearBwdArgs& a, bool bf16_io, hipStream_t s);
// backward of the delta rule (chunk 1), in the exact form 16 tokens at a time (vector ALUs;
// the kernel recomputes its own chunk-start states into the workspace)
size_t delta_bwd_workspace_bytes(const LinearBwdArgs& a);
hipError_t launch_delta_bwd(const LinearBwdArgs& a, const float* w0, long long w0_batch_stride, void* ws,
                            bool bf16_io, hipStream_t s);
// backward of the paper's TTT-Linear x + LN(W x) (vector ALUs; reads the chunk-start states
// in a.w_hist)
hipError_t launch_linear_ln_bwd(const LinearBwdArgs& a, bool bf16_io, hipStream_t s);
hipError_t launch_mlp_bwd_generic(const MlpBwdArgs& a, bool bf16_io, hipStream_t s);
// backward of the paper's TTT-MLP x + LN(W2 GELU(W1 x)) (vector ALUs; reads w_hist)
size_t mlp_ln_bwd_lds_bytes(int d, int dh);
hipError_t launch_mlp_ln_bwd(const MlpBwdArgs& a, bool bf16_io, hipStream_t s);
// matrix-core forward pass that stores the bf16 chunk-start states (64 KB per chunk), and
// the matrix-core backward pass reading them (d = 64, hidden 256, chunk 16, bf16)
hipError_t launch_mlp_fwd_hist(const MlpArgs& a, void* hist, hipStream_t s);
bool mlp_bwd_mfma_supported(const MlpBwdArgs& a, bool bf16_io);
size_t mlp_bwd_mfma_workspace_bytes(const MlpBwdArgs& a);
hipError_t launch_mlp_bwd_mfma(const MlpBwdArgs& a, const void* ws, hipStream_t s);
// matrix-core backward (bf16, d = 64, chunk 16): the forward recomputation (fwd: q, k, v, w0,
// w0_batch_stride, B, H, T, eta) stores the bf16 chunk-start states in the workspace
// fwd: the forward arguments (its initial state is read with 16-byte loads)
bool linear_bwd_mfma_supported(const LinearArgs& fwd, const LinearBwdArgs& a, bool bf16_io);
size_t linear_bwd_mfma_workspace_bytes(const LinearBwdArgs& a);
hipError_t launch_linear_bwd_mfma(const LinearArgs& fwd, const LinearBwdArgs& a, void* workspace,
                                  hipStream_t s);

// backward of the non-causal layers (vector ALUs; linear or SiLU MLP, any chunk / epochs)
size_t nc_bwd_workspace_floats(bool mlp, int B, int H, int T, int d, int h, int chunk, int epochs);
// matrix-core backward of the non-causal linear layer for one full-batch step (d = 64,
// 16 <= T <= 256, bf16 I/O); no workspace
bool linear_nc_bwd_mfma_supported(const void* q, const void* k, const void* v, const void* dz,
                                  const float* w0, long long w_batch_stride, const float* dw_out,
                                  const void* dq, const void* dk, const void* dv, const float* dw0,
                                  int T, int d, int chunk, int epochs, bool bf16_io);
hipError_t launch_linear_nc_bwd_mfma(const void* q, const void* k, const void* v, const void* dz,
                                     const float* w0, long long w_batch_stride, const float* dw_out,
                                     const float* eta_tok, void* dq, void* dk, void* dv, float* dw0,
                                     float* deta_tok, int B, int H, int T, float eta, int dot_loss,
                                     hipStream_t s);
// matrix-core backward of the non-causal MLP for one full-batch step (d = hidden = 64, T <= 256,
// bf16 I/O); no workspace
bool mlp_nc_bwd_mfma_supported(const void* q, const void* k, const void* v, const void* dz,
                               const float* w1, const float* w2, long long w_batch_stride,
                               const float* dw1_out, const float* dw2_out, const void* dq,
                               const void* dk, const void* dv, const float* dw1, const float* dw2,
                               int T, int d, int h, int chunk, int epochs, bool bf16_io);
hipError_t launch_mlp_nc_bwd_mfma(const void* q, const void* k, const void* v, const void* dz,
                                  const float* w1, const float* w2, long long w_batch_stride,
                                  const float* dw1_out, const float* dw2_out, const float* eta_tok,
                                  void* dq, void* dk, void* dv, float* dw1, float* dw2,
                                  float* deta_tok, int B, int H, int T, float eta, int dot_loss,
                                  hipStream_t s);
hipError_t launch_nc_bwd(bool mlp, const void* q, const void* k, const void* v, const void* dz,
                         const float* w1, const float* w2, long long w_batch_stride,
                         const float* dw1_out, const float* dw2_out, const float* eta_tok,
                         void* dq, void* dk, void* dv, float* dw1, float* dw2, float* deta_tok,
                         float* ws, int B, int H, int T, int d, int h, int chunk, int epochs,
                         float eta, int dot_loss, bool bf16_io, hipStream_t s);

// dst[b][h][:] = src + b * batch_stride + h * per_head (the state when T = 0); zeros when
// src is null.
hipError_t launch_copy_state(float* dst, const float* src, long long batch_stride, int B, int H,
                             size_t per_head, hipStream_t s);

// Debug check for non-finite outputs: one entry per output buffer (null or empty entries are
// skipped); host_flags[i] (kMaxCheckedOutputs entries) receives 1 if buffer i holds a NaN or
// an infinity.  Enqueues on s and then waits for s.
constexpr int kMaxCheckedOutputs = 8;
struct CheckedOutput {
  const char* name;
  const void* ptr;
  long long count;     // elements
  int bytes_per_elem;  // 2 (bf16) or 4 (float32)
};
hipError_t check_finite_outputs(const CheckedOutput* outs, int nouts, hipStream_t s,
                                unsigned int* host_flags);

}  // namespace ttt
