// C ABI of libttt: argument validation, kernel selection and error reporting.
// The functions are declared (with their argument conventions) in include/ttt.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <initializer_list>
#include <mutex>
#include <random>
#include <string>

#include "../../include/ttt.h"
#include "common.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(TTT_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool fits_int64(long long a, long long b, long long c, long long d) {
  const long long lim = (1LL << 62);
  long long x = a;
  for (long long m : {b, c, d}) {
    if (m != 0 && x > lim / m) return false;
    x *= m;
  }
  return true;
}

int check_common(const char* fn, const void* q, const void* k, const void* v, const void* z,
                 int B, int H, int T, int d, float eta, const float* eta_tok, int io_dtype) {
  if (B <= 0 || H <= 0 || d <= 0 || T < 0)
    return fail(TTT_E_INVALID, "%s: sizes must be positive (B=%d H=%d T=%d d=%d)", fn, B, H, T, d);
  if (io_dtype != TTT_F32 && io_dtype != TTT_BF16)
    return fail(TTT_E_INVALID, "%s: unknown io_dtype %d", fn, io_dtype);
  if (!std::isfinite(eta)) return fail(TTT_E_INVALID, "%s: eta must be finite", fn);
  if (eta_tok && (reinterpret_cast<uintptr_t>(eta_tok) & 3) != 0)
    return fail(TTT_E_INVALID, "%s: eta_tok must be 4-byte aligned", fn);
  if (T > 0 && (!q || !k || !v || !z))
    return fail(TTT_E_INVALID, "%s: q, k, v and z must be non-null", fn);
  if (!fits_int64(B, H, T > 0 ? T : 1, d))
    return fail(TTT_E_INVALID, "%s: B*H*T*d overflows", fn);
  if (static_cast<long long>(B) * H > 0x7fffffffLL)
    return fail(TTT_E_INVALID, "%s: B*H exceeds the grid limit", fn);
  return TTT_OK;
}

// Several epochs revisit every token, which only the non-causal layer may do (a causal
// output must not depend on later tokens).
int check_epochs(const char* fn, int epochs, int causal) {
  if (epochs < 1) return fail(TTT_E_INVALID, "%s: epochs must be >= 1 (got %d)", fn, epochs);
  if (causal == 1 && epochs != 1)
    return fail(TTT_E_INVALID, "%s: epochs > 1 needs causal = 0 (got %d)", fn, epochs);
  return TTT_OK;
}

// Per-call device workspace, allocated and released in stream order (hipMallocFromPoolAsync /
// hipFreeAsync on the caller's stream): the release is queued behind the kernels that use
// it, so concurrent calls on different streams never share a workspace and the host never
// waits.  The memory comes from a stream-ordered pool of the library's own, one per device,
// that keeps what it has allocated (no release threshold): the next call reuses those blocks
// instead of mapping fresh pages (a 100 MB workspace mapped per call cost more than the
// kernels using it).  The pool holds its largest working set until the process ends.
constexpr int kMaxDevices = 64;
std::mutex g_pool_mu;
hipMemPool_t g_pool[kMaxDevices] = {};

int workspace_pool(hipMemPool_t* out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(TTT_E_UNSUPPORTED, "workspace pool: device %d", dev);
  std::lock_guard<std::mutex> lock(g_pool_mu);
  if (!g_pool[dev]) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t p = nullptr;
    e = hipMemPoolCreate(&p, &props);
    if (e != hipSuccess) return hip_fail(e, "hipMemPoolCreate(workspace)");
    uint64_t keep = UINT64_MAX;
    e = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) {
      (void)hipMemPoolDestroy(p);
      return hip_fail(e, "hipMemPoolSetAttribute(workspace)");
    }
    g_pool[dev] = p;
  }
  *out = g_pool[dev];
  return TTT_OK;
}

struct StreamBuffer {
  void* ptr = nullptr;
  hipStream_t stream = nullptr;
  ~StreamBuffer() {
    if (ptr) (void)hipFreeAsync(ptr, stream);
  }
};

int get_workspace(size_t bytes, hipStream_t s, StreamBuffer* out) {
  out->stream = s;
  hipMemPool_t pool = nullptr;
  int rc = workspace_pool(&pool);
  if (rc != TTT_OK) return rc;
  hipError_t e = hipMallocFromPoolAsync(&out->ptr, bytes > 0 ? bytes : 1, pool, s);
  if (e != hipSuccess) {
    out->ptr = nullptr;
    return hip_fail(e, "hipMallocFromPoolAsync(workspace)");
  }
  return TTT_OK;
}

int copy_state(float* dst, const float* src, long long batch_stride, int B, int H,
               size_t per_head, hipStream_t s) {
  if (!dst) return TTT_OK;
  hipError_t e = ttt::launch_copy_state(dst, src, batch_stride, B, H, per_head, s);
  if (e != hipSuccess) return hip_fail(e, "state copy launch");
  return TTT_OK;
}

// Fixed scratch memory of the entry points that allocate nothing (ttt_linear_bwd_noalloc):
// a device array that every GPU the library runs on holds until the process ends.  Host
// code never passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol): it takes the device address once per device, with that device current, from
// hipGetSymbolAddress, and passes that.  Every call on one GPU shares the array, so calls
// that overlap on one GPU (different streams) race; a call writes every byte it reads.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

int scratch_ptr(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(TTT_E_UNSUPPORTED, "%s: device %d", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return TTT_OK;
}

// Shared by ttt_linear_fwd (f(x) = W x, ln_w null) and ttt_linear_ln_fwd (x + LN(W x)).
int linear_fwd(const char* fn, const void* q, const void* k, const void* v, const float* w0,
               long long w0_batch_stride, const float* ln_w, const float* ln_b, float ln_eps,
               void* z, float* w_out, int B, int H, int T, int d, int chunk, int causal,
               float eta, const float* eta_tok, int loss, int epochs, int io_dtype,
               ttt_stream_t stream) {
  int rc = check_common(fn, q, k, v, z, B, H, T, d, eta, eta_tok, io_dtype);
  if (rc != TTT_OK) return rc;
  if (loss != TTT_LOSS_MSE && loss != TTT_LOSS_DOT)
    return fail(TTT_E_INVALID, "%s: unknown loss %d", fn, loss);
  rc = check_epochs(fn, epochs, causal);
  if (rc != TTT_OK) return rc;
  if (!w0) return fail(TTT_E_INVALID, "%s: w0 must be non-null", fn);
  if (chunk < 1) return fail(TTT_E_INVALID, "%s: chunk must be >= 1 (got %d)", fn, chunk);
  if (causal != 0 && causal != 1)
    return fail(TTT_E_INVALID, "%s: causal must be 0 or 1", fn);
  if (w0_batch_stride < 0) return fail(TTT_E_INVALID, "%s: negative w0_batch_stride", fn);
  if (d != 16 && d != 32 && d != 64)
    return fail(TTT_E_UNSUPPORTED, "%s: d=%d not supported (16, 32, 64)", fn, d);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T == 0) return copy_state(w_out, w0, w0_batch_stride, B, H, static_cast<size_t>(d) * d, s);

  ttt::LinearArgs a{q, k, v, w0, w0_batch_stride, z, w_out, B, H, T, d, chunk, causal, eta, eta_tok,
                    loss == TTT_LOSS_DOT ? 1 : 0};
  a.epochs = epochs;
  a.ln_w = ln_w;
  a.ln_b = ln_b;
  a.ln_eps = ln_eps;
  const bool bf16 = io_dtype == TTT_BF16;
  hipError_t e;
  if (ttt::linear_mfma_supported(a, bf16))
    e = ttt::launch_linear_mfma(a, s);
  else if (ttt::linear_nc_supported(a, bf16))
    e = ttt::launch_linear_nc(a, s);
  else if (ttt::linear_ln_mfma_supported(a, bf16))
    e = ttt::launch_linear_ln_mfma(a, s);
  else
    e = ttt::launch_linear_generic(a, bf16, s);
  if (e != hipSuccess) return fail(TTT_E_HIP, "%s launch: %s", fn, hipGetErrorString(e));
  return TTT_OK;
}

int check_ln(const char* fn, const float* ln_w, const float* ln_b, float ln_eps) {
  if (!ln_w || !ln_b) return fail(TTT_E_INVALID, "%s: ln_weight and ln_bias must be non-null", fn);
  if (!std::isfinite(ln_eps) || !(ln_eps > 0.0f))
    return fail(TTT_E_INVALID, "%s: ln_eps must be finite and positive", fn);
  return TTT_OK;
}

// Tag of one two-workgroup MLP call: its hand-off flags carry it, so that a flag left in a
// reused workspace by an earlier call (of this process or, through the random start, of
// another) is not taken for this call's.  Never 0.
// Debug switches of the two-workgroup MLP kernel (ttt_set_split_debug).
std::atomic<int> g_split_debug{0};

uint32_t next_split_tag() {
  static std::atomic<uint32_t> counter{[] {
    std::random_device rd;
    return static_cast<uint32_t>(rd());
  }()};
  uint32_t t = 0;
  while (t == 0) t = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  return t;
}

// Shared by ttt_mlp_fwd (W2 SiLU(W1 x), ln_w null) and ttt_mlp_ln_fwd (x + LN(W2 GELU(W1 x)));
// the _ws forms pass a workspace for the two-workgroup kernel.
int mlp_fwd(const char* fn, const void* q, const void* k, const void* v, const float* w1,
            const float* w2, long long w_batch_stride, const float* ln_w, const float* ln_b,
            float ln_eps, void* z, float* w1_out, float* w2_out, int B, int H, int T, int d,
            int dh, int chunk, int causal, float eta, const float* eta_tok, int loss, int epochs,
            int io_dtype, ttt_stream_t stream, void* split_ws = nullptr, size_t split_ws_bytes = 0) {
  int rc = check_common(fn, q, k, v, z, B, H, T, d, eta, eta_tok, io_dtype);
  if (rc != TTT_OK) return rc;
  if (loss != TTT_LOSS_MSE && loss != TTT_LOSS_DOT)
    return fail(TTT_E_INVALID, "%s: unknown loss %d", fn, loss);
  rc = check_epochs(fn, epochs, causal);
  if (rc != TTT_OK) return rc;
  if (!w1 || !w2) return fail(TTT_E_INVALID, "%s: w1 and w2 must be non-null", fn);
  if (dh <= 0) return fail(TTT_E_INVALID, "%s: dh must be positive (got %d)", fn, dh);
  if (chunk < 1) return fail(TTT_E_INVALID, "%s: chunk must be >= 1 (got %d)", fn, chunk);
  if (causal != 0 && causal != 1) return fail(TTT_E_INVALID, "%s: causal must be 0 or 1", fn);
  if (w_batch_stride < 0) return fail(TTT_E_INVALID, "%s: negative w_batch_stride", fn);
  if (d != 16 && d != 32 && d != 64)
    return fail(TTT_E_UNSUPPORTED, "%s: d=%d not supported (16, 32, 64)", fn, d);
  if (dh > 512) return fail(TTT_E_UNSUPPORTED, "%s: dh=%d not supported (<= 512)", fn, dh);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t per = static_cast<size_t>(d) * dh;
  if (T == 0) {
    rc = copy_state(w1_out, w1, w_batch_stride, B, H, per, s);
    if (rc != TTT_OK) return rc;
    return copy_state(w2_out, w2, w_batch_stride, B, H, per, s);
  }
  ttt::MlpArgs a{q, k, v, w1, w2, w_batch_stride, z, w1_out, w2_out,
                 B, H, T, d, dh, chunk, causal, eta, eta_tok, loss == TTT_LOSS_DOT ? 1 : 0};
  a.epochs = epochs;
  a.ln_w = ln_w;
  a.ln_b = ln_b;
  a.ln_eps = ln_eps;
  const bool bf16 = io_dtype == TTT_BF16;
  hipError_t e;
  StreamBuffer ws;
  if (split_ws && ttt::mlp_split_supported(a, bf16)) {
    const size_t need = ttt::mlp_split_workspace_bytes(a);
    if (split_ws_bytes < need)
      return fail(TTT_E_INVALID, "%s: workspace of %zu bytes, this call needs %zu", fn, split_ws_bytes, need);
    if ((reinterpret_cast<uintptr_t>(split_ws) & 255) != 0)
      return fail(TTT_E_INVALID, "%s: workspace must be 256-byte aligned", fn);
    e = ttt::launch_mlp_split(a, split_ws, next_split_tag(), g_split_debug.load(std::memory_order_relaxed), s);
  } else if (ttt::mlp_fast_supported(a, bf16)) {
    e = ttt::launch_mlp_fast(a, s);
  } else if (ttt::mlp_nc_supported(a, bf16)) {
    e = ttt::launch_mlp_nc(a, s);
  } else {
    rc = get_workspace(ttt::mlp_generic_workspace_floats(a) * sizeof(float), s, &ws);
    if (rc != TTT_OK) return rc;
    e = ttt::launch_mlp_generic(a, bf16, static_cast<float*>(ws.ptr), s);
  }
  if (e != hipSuccess) return fail(TTT_E_HIP, "%s launch: %s", fn, hipGetErrorString(e));
  return TTT_OK;
}

// Shared by ttt_linear_bwd (stream-ordered workspace) and ttt_linear_bwd_noalloc (the
// library's fixed scratch array; no allocation).
int linear_bwd(const char* fn, const void* q, const void* k, const void* v, const float* w0,
               long long w0_batch_stride, const void* dz, const float* dw_out, void* dq, void* dk,
               void* dv, float* dw0, int B, int H, int T, int d, int chunk, float eta,
               const float* eta_tok, float* deta_tok, int loss, int io_dtype, ttt_stream_t stream,
               bool noalloc) {
  int rc = check_common(fn, q, k, v, dz, B, H, T, d, eta, eta_tok, io_dtype);
  if (rc != TTT_OK) return rc;
  if (loss != TTT_LOSS_MSE && loss != TTT_LOSS_DOT)
    return fail(TTT_E_INVALID, "%s: unknown loss %d", fn, loss);
  const int dot = loss == TTT_LOSS_DOT ? 1 : 0;
  if (deta_tok && !eta_tok) return fail(TTT_E_INVALID, "%s: deta_tok needs eta_tok", fn);
  if (deta_tok && (reinterpret_cast<uintptr_t>(deta_tok) & 3) != 0)
    return fail(TTT_E_INVALID, "%s: deta_tok must be 4-byte aligned", fn);
  if (!w0 || !dw0) return fail(TTT_E_INVALID, "%s: w0 and dw0 must be non-null", fn);
  if (T > 0 && (!dq || !dk || !dv))
    return fail(TTT_E_INVALID, "%s: dq, dk and dv must be non-null", fn);
  if (chunk < 1) return fail(TTT_E_INVALID, "%s: chunk must be >= 1 (got %d)", fn, chunk);
  if (w0_batch_stride < 0) return fail(TTT_E_INVALID, "%s: negative w0_batch_stride", fn);
  if (d != 16 && d != 32 && d != 64)
    return fail(TTT_E_UNSUPPORTED, "%s: d=%d not supported (16, 32, 64)", fn, d);
  if (T > 0 && (chunk < T ? chunk : T) > 16)
    return fail(TTT_E_UNSUPPORTED, "%s: chunks of more than 16 tokens not supported", fn);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t dd = static_cast<size_t>(d) * d;
  if (T == 0) return copy_state(dw0, dw_out, static_cast<long long>(H) * dd, B, H, dd, s);

  const bool bf16 = io_dtype == TTT_BF16;
  ttt::LinearArgs f{q, k, v, w0, w0_batch_stride, nullptr, nullptr, B, H, T, d, chunk, 1, eta,
                    eta_tok, dot, nullptr};
  ttt::LinearBwdArgs g{q, k, v, dz, dw_out, nullptr, dq, dk, dv, dw0,
                       B, H, T, d, chunk, eta, eta_tok, deta_tok, dot};
  const int b = chunk < T ? chunk : T;
  if (b == 1) {
    // the delta rule: its exact chunked form, 16 tokens per step, with float32 chunk-start
    // states every 16 tokens
    const size_t dneed = ttt::delta_bwd_workspace_bytes(g);
    StreamBuffer downed;
    void* dws = nullptr;
    if (noalloc) {
      if (dneed > kScratchBytes)
        return fail(TTT_E_UNSUPPORTED,
                    "%s: the state history needs %zu bytes, more than the %zu-byte scratch array",
                    fn, dneed, kScratchBytes);
      rc = scratch_ptr(fn, &dws);
      if (rc != TTT_OK) return rc;
    } else {
      rc = get_workspace(dneed, s, &downed);
      if (rc != TTT_OK) return rc;
      dws = downed.ptr;
    }
    hipError_t e = ttt::launch_delta_bwd(g, w0, w0_batch_stride, dws, bf16, s);
    if (e != hipSuccess) return hip_fail(e, "delta-rule backward launch");
    return TTT_OK;
  }
  // chunk-start states of the forward pass: bf16 on the matrix-core path (8 KB per chunk),
  // float32 on the vector-ALU path
  const bool mfma = ttt::linear_bwd_mfma_supported(f, g, bf16);
  const long long nchunks = (T + b - 1) / b;
  if (!fits_int64(B, H, nchunks, static_cast<long long>(dd) * 4))
    return fail(TTT_E_INVALID, "%s: state history overflows", fn);
  const size_t need = mfma ? ttt::linear_bwd_mfma_workspace_bytes(g)
                           : static_cast<size_t>(B) * H * nchunks * dd * sizeof(float);
  StreamBuffer owned;
  void* ws = nullptr;
  if (noalloc) {
    if (need > kScratchBytes)
      return fail(TTT_E_UNSUPPORTED,
                  "%s: the state history needs %zu bytes, more than the %zu-byte scratch array",
                  fn, need, kScratchBytes);
    rc = scratch_ptr(fn, &ws);
    if (rc != TTT_OK) return rc;
  } else {
    rc = get_workspace(need, s, &owned);
    if (rc != TTT_OK) return rc;
    ws = owned.ptr;
  }
  if (mfma) {
    hipError_t e = ttt::launch_linear_bwd_mfma(f, g, ws, s);
    if (e != hipSuccess) return hip_fail(e, "linear backward launch");
    return TTT_OK;
  }
  f.w_hist = static_cast<float*>(ws);
  hipError_t e = ttt::launch_linear_generic(f, bf16, s);
  if (e != hipSuccess) return hip_fail(e, "linear backward state launch");
  g.w_hist = static_cast<const float*>(ws);
  e = ttt::launch_linear_bwd_generic(g, bf16, s);
  if (e != hipSuccess) return hip_fail(e, "linear backward launch");
  return TTT_OK;
}

// ---- finite check of the outputs (debugging) ----
// -1: not yet read from the environment (TTT_CHECK_FINITE), else 0 / 1
std::atomic<int> g_check_finite{-1};

bool check_finite_on() {
  int v = g_check_finite.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* env = std::getenv("TTT_CHECK_FINITE");
    const int want = (env != nullptr && env[0] != '\0' && std::strcmp(env, "0") != 0) ? 1 : 0;
    g_check_finite.compare_exchange_strong(v, want, std::memory_order_relaxed);
    v = g_check_finite.load(std::memory_order_relaxed);
  }
  return v == 1;
}

using Out = ttt::CheckedOutput;

// rc of the call; when it is TTT_OK and the check is on, the call's outputs are scanned on
// its stream (which is then waited for) and TTT_E_NONFINITE names the first output holding
// a NaN or an infinity.
int finite_outputs(int rc, const char* fn, ttt_stream_t stream, std::initializer_list<Out> outs) {
  if (rc != TTT_OK || !check_finite_on()) return rc;
  unsigned int flags[ttt::kMaxCheckedOutputs] = {};
  const int n = static_cast<int>(outs.size());
  const hipError_t e = ttt::check_finite_outputs(outs.begin(), n, reinterpret_cast<hipStream_t>(stream), flags);
  if (e != hipSuccess) return fail(TTT_E_HIP, "%s finite check: %s", fn, hipGetErrorString(e));
  for (int i = 0; i < n; ++i)
    if (flags[i]) return fail(TTT_E_NONFINITE, "%s: non-finite values in %s", fn, outs.begin()[i].name);
  return TTT_OK;
}

// element counts: token tensors (none when T = 0, where they are left untouched) and states
long long tok(int B, int H, int T, int d) { return static_cast<long long>(B) * H * T * d; }
long long per_seq(int B, int H, long long n) { return static_cast<long long>(B) * H * n; }
int io_bytes(int io_dtype) { return io_dtype == TTT_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

int ttt_abi_version(void) { return 14; }

const char* ttt_last_error(void) { return g_last_error.c_str(); }

static int impl_delta_rule_fwd(const void* q, const void* k, const void* v, const float* w0,
                               long long w0_batch_stride, void* z, float* w_out, int B, int H, int T,
                               int d, float eta, const float* eta_tok, int io_dtype, ttt_stream_t stream) {
  g_last_error.clear();
  int rc = check_common("delta_rule_fwd", q, k, v, z, B, H, T, d, eta, eta_tok, io_dtype);
  if (rc != TTT_OK) return rc;
  if (!w0) return fail(TTT_E_INVALID, "delta_rule_fwd: w0 must be non-null");
  if (w0_batch_stride < 0) return fail(TTT_E_INVALID, "delta_rule_fwd: negative w0_batch_stride");
  if (d != 16 && d != 32 && d != 64)
    return fail(TTT_E_UNSUPPORTED, "delta_rule_fwd: d=%d not supported (16, 32, 64)", d);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T == 0) return copy_state(w_out, w0, w0_batch_stride, B, H, static_cast<size_t>(d) * d, s);

  ttt::LinearArgs a{q, k, v, w0, w0_batch_stride, z, w_out, B, H, T, d, 1, 1, eta, eta_tok, 0};
  const bool bf16 = io_dtype == TTT_BF16;
  hipError_t e;
  if (ttt::delta_fast_supported(a, bf16)) {
    e = ttt::launch_delta_fast(a, s);
  } else {
    e = ttt::launch_linear_generic(a, bf16, s);
  }
  if (e != hipSuccess) return hip_fail(e, "delta_rule_fwd launch");
  return TTT_OK;
}

static int impl_ttt_linear_bwd(const void* q, const void* k, const void* v, const float* w0,
                               long long w0_batch_stride, const void* dz, const float* dw_out, void* dq,
                               void* dk, void* dv, float* dw0, int B, int H, int T, int d, int chunk,
                               float eta, const float* eta_tok, float* deta_tok, int loss, int io_dtype,
                               ttt_stream_t stream) {
  g_last_error.clear();
  return linear_bwd("ttt_linear_bwd", q, k, v, w0, w0_batch_stride, dz, dw_out, dq, dk, dv, dw0, B,
                    H, T, d, chunk, eta, eta_tok, deta_tok, loss, io_dtype, stream, false);
}

static int impl_ttt_linear_bwd_noalloc(const void* q, const void* k, const void* v, const float* w0,
                                       long long w0_batch_stride, const void* dz, const float* dw_out,
                                       void* dq, void* dk, void* dv, float* dw0, int B, int H, int T, int d,
                                       int chunk, float eta, const float* eta_tok, float* deta_tok, int loss,
                                       int io_dtype, ttt_stream_t stream) {
  g_last_error.clear();
  return linear_bwd("ttt_linear_bwd_noalloc", q, k, v, w0, w0_batch_stride, dz, dw_out, dq, dk, dv,
                    dw0, B, H, T, d, chunk, eta, eta_tok, deta_tok, loss, io_dtype, stream, true);
}

static int impl_ttt_linear_ln_bwd(const void* q, const void* k, const void* v, const float* w0,
                                  long long w0_batch_stride, const float* ln_weight, const float* ln_bias,
                                  float ln_eps, const void* dz, const float* dw_out, void* dq, void* dk,
                                  void* dv, float* dw0, float* dln_weight, float* dln_bias, int B, int H,
                                  int T, int d, int chunk, float eta, const float* eta_tok, float* deta_tok,
                                  int loss, int io_dtype, ttt_stream_t stream) {
  g_last_error.clear();
  const char* fn = "ttt_linear_ln_bwd";
  int rc = check_ln(fn, ln_weight, ln_bias, ln_eps);
  if (rc != TTT_OK) return rc;
  rc = check_common(fn, q, k, v, dz, B, H, T, d, eta, eta_tok, io_dtype);
  if (rc != TTT_OK) return rc;
  if (loss != TTT_LOSS_MSE && loss != TTT_LOSS_DOT)
    return fail(TTT_E_INVALID, "%s: unknown loss %d", fn, loss);
  if (deta_tok && !eta_tok) return fail(TTT_E_INVALID, "%s: deta_tok needs eta_tok", fn);
  if (deta_tok && (reinterpret_cast<uintptr_t>(deta_tok) & 3) != 0)
    return fail(TTT_E_INVALID, "%s: deta_tok must be 4-byte aligned", fn);
  if (!w0 || !dw0 || !dln_weight || !dln_bias)
    return fail(TTT_E_INVALID, "%s: w0, dw0, dln_weight and dln_bias must be non-null", fn);
  if (T > 0 && (!dq || !dk || !dv))
    return fail(TTT_E_INVALID, "%s: dq, dk and dv must be non-null", fn);
  if (chunk < 1) return fail(TTT_E_INVALID, "%s: chunk must be >= 1 (got %d)", fn, chunk);
  if (w0_batch_stride < 0) return fail(TTT_E_INVALID, "%s: negative w0_batch_stride", fn);
  if (d != 16 && d != 32 && d != 64)
    return fail(TTT_E_UNSUPPORTED, "%s: d=%d not supported (16, 32, 64)", fn, d);
  if (T > 0 && (chunk < T ? chunk : T) > 16)
    return fail(TTT_E_UNSUPPORTED, "%s: chunks of more than 16 tokens not supported", fn);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t dd = static_cast<size_t>(d) * d;
  if (T == 0) {
    rc = copy_state(dw0, dw_out, static_cast<long long>(H) * dd, B, H, dd, s);
    if (rc != TTT_OK) return rc;
    rc = copy_state(dln_weight, nullptr, 0, B, H, static_cast<size_t>(d), s);
    if (rc != TTT_OK) return rc;
    return copy_state(dln_bias, nullptr, 0, B, H, static_cast<size_t>(d), s);
  }
  const int b = chunk < T ? chunk : T;
  const long long nchunks = (T + b - 1) / b;
  if (!fits_int64(B, H, nchunks, static_cast<long long>(dd) * 4))
    return fail(TTT_E_INVALID, "%s: state history overflows", fn);
  const bool bf16 = io_dtype == TTT_BF16;
  const int dot = loss == TTT_LOSS_DOT ? 1 : 0;
  StreamBuffer hist;
  rc = get_workspace(static_cast<size_t>(B) * H * nchunks * dd * sizeof(float), s, &hist);
  if (rc != TTT_OK) return rc;
  // the forward recomputation on the generic kernel, storing the chunk-start states
  ttt::LinearArgs f{q, k, v, w0, w0_batch_stride, nullptr, nullptr, B, H, T, d, chunk, 1, eta,
                    eta_tok, dot, static_cast<float*>(hist.ptr)};
  f.ln_w = ln_weight;
  f.ln_b = ln_bias;
  f.ln_eps = ln_eps;
  hipError_t e = ttt::launch_linear_generic(f, bf16, s);
  if (e != hipSuccess) return hip_fail(e, "ttt_linear_ln_bwd state launch");
  ttt::LinearBwdArgs g{q, k, v, dz, dw_out, static_cast<const float*>(hist.ptr), dq, dk, dv, dw0,
                       B, H, T, d, chunk, eta, eta_tok, deta_tok, dot};
  g.ln_w = ln_weight;
  g.ln_b = ln_bias;
  g.ln_eps = ln_eps;
  g.dln_w = dln_weight;
  g.dln_b = dln_bias;
  e = ttt::launch_linear_ln_bwd(g, bf16, s);
  if (e != hipSuccess) return hip_fail(e, "ttt_linear_ln_bwd launch");
  return TTT_OK;
}

static int impl_ttt_mlp_ln_bwd(const void* q, const void* k, const void* v, const float* w1, const float* w2,
                               long long w_batch_stride, const float* ln_weight, const float* ln_bias,
                               float ln_eps, const void* dz, const float* dw1_out, const float* dw2_out,
                               void* dq, void* dk, void* dv, float* dw1, float* dw2, float* dln_weight,
                               float* dln_bias, int B, int H, int T, int d, int dh, int chunk, float eta,
                               const float* eta_tok, float* deta_tok, int loss, int io_dtype,
                               ttt_stream_t stream) {
  g_last_error.clear();
  const char* fn = "ttt_mlp_ln_bwd";
  int rc = check_ln(fn, ln_weight, ln_bias, ln_eps);
  if (rc != TTT_OK) return rc;
  rc = check_common(fn, q, k, v, dz, B, H, T, d, eta, eta_tok, io_dtype);
  if (rc != TTT_OK) return rc;
  if (loss != TTT_LOSS_MSE && loss != TTT_LOSS_DOT)
    return fail(TTT_E_INVALID, "%s: unknown loss %d", fn, loss);
  if (deta_tok && !eta_tok) return fail(TTT_E_INVALID, "%s: deta_tok needs eta_tok", fn);
  if (deta_tok && (reinterpret_cast<uintptr_t>(deta_tok) & 3) != 0)
    return fail(TTT_E_INVALID, "%s: deta_tok must be 4-byte aligned", fn);
  if (!w1 || !w2 || !dw1 || !dw2 || !dln_weight || !dln_bias)
    return fail(TTT_E_INVALID, "%s: w1, w2, dw1, dw2, dln_weight and dln_bias must be non-null", fn);
  if (T > 0 && (!dq || !dk || !dv))
    return fail(TTT_E_INVALID, "%s: dq, dk and dv must be non-null", fn);
  if (dh <= 0) return fail(TTT_E_INVALID, "%s: dh must be positive (got %d)", fn, dh);
  if (chunk < 1) return fail(TTT_E_INVALID, "%s: chunk must be >= 1 (got %d)", fn, chunk);
  if (w_batch_stride < 0) return fail(TTT_E_INVALID, "%s: negative w_batch_stride", fn);
  if (d != 16 && d != 32 && d != 64)
    return fail(TTT_E_UNSUPPORTED, "%s: d=%d not supported (16, 32, 64)", fn, d);
  if (dh > 256) return fail(TTT_E_UNSUPPORTED, "%s: dh=%d not supported (<= 256)", fn, dh);
  if (T > 0 && (chunk < T ? chunk : T) > 16)
    return fail(TTT_E_UNSUPPORTED, "%s: chunks of more than 16 tokens not supported", fn);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t per = static_cast<size_t>(d) * dh;
  if (T == 0) {
    const long long st = static_cast<long long>(H) * static_cast<long long>(per);
    rc = copy_state(dw1, dw1_out, st, B, H, per, s);
    if (rc == TTT_OK) rc = copy_state(dw2, dw2_out, st, B, H, per, s);
    if (rc == TTT_OK) rc = copy_state(dln_weight, nullptr, 0, B, H, static_cast<size_t>(d), s);
    if (rc == TTT_OK) rc = copy_state(dln_bias, nullptr, 0, B, H, static_cast<size_t>(d), s);
    return rc;
  }
  const int b = chunk < T ? chunk : T;
  const long long nchunks = (T + b - 1) / b;
  if (!fits_int64(B, H, nchunks, 2LL * static_cast<long long>(per)))
    return fail(TTT_E_INVALID, "%s: state history overflows", fn);
  const bool bf16 = io_dtype == TTT_BF16;
  const int dot = loss == TTT_LOSS_DOT ? 1 : 0;
  // forward recomputation on the generic kernel, storing the chunk-start states
  ttt::MlpArgs f{q, k, v, w1, w2, w_batch_stride, nullptr, nullptr, nullptr,
                 B, H, T, d, dh, chunk, 1, eta, eta_tok, dot};
  f.ln_w = ln_weight;
  f.ln_b = ln_bias;
  f.ln_eps = ln_eps;
  StreamBuffer hist, fws;
  rc = get_workspace(static_cast<size_t>(B) * H * nchunks * 2 * per * sizeof(float), s, &hist);
  if (rc != TTT_OK) return rc;
  f.w_hist = static_cast<float*>(hist.ptr);
  rc = get_workspace(ttt::mlp_generic_workspace_floats(f) * sizeof(float), s, &fws);
  if (rc != TTT_OK) return rc;
  hipError_t e = ttt::launch_mlp_generic(f, bf16, static_cast<float*>(fws.ptr), s);
  if (e != hipSuccess) return hip_fail(e, "ttt_mlp_ln_bwd state launch");
  ttt::MlpBwdArgs g{q, k, v, dz, dw1_out, dw2_out, static_cast<const float*>(hist.ptr), dq, dk, dv,
                    dw1, dw2, B, H, T, d, dh, chunk, eta, dot, eta_tok, deta_tok};
  g.ln_w = ln_weight;
  g.ln_b = ln_bias;
  g.ln_eps = ln_eps;
  g.dln_w = dln_weight;
  g.dln_b = dln_bias;
  e = ttt::launch_mlp_ln_bwd(g, bf16, s);
  if (e != hipSuccess) return hip_fail(e, "ttt_mlp_ln_bwd launch");
  return TTT_OK;
}

// Shared by ttt_linear_nc_bwd (mlp false: w1 = w0, dw1 = dw0) and ttt_mlp_nc_bwd.
static int nc_bwd(const char* fn, bool mlp, const void* q, const void* k, const void* v, const float* w1,
                  const float* w2, long long w_batch_stride, const void* dz, const float* dw1_out,
                  const float* dw2_out, void* dq, void* dk, void* dv, float* dw1, float* dw2, int B,
                  int H, int T, int d, int dh, int chunk, int epochs, float eta, const float* eta_tok,
                  float* deta_tok, int loss, int io_dtype, ttt_stream_t stream) {
  int rc = check_common(fn, q, k, v, dz, B, H, T, d, eta, eta_tok, io_dtype);
  if (rc != TTT_OK) return rc;
  if (loss != TTT_LOSS_MSE && loss != TTT_LOSS_DOT)
    return fail(TTT_E_INVALID, "%s: unknown loss %d", fn, loss);
  rc = check_epochs(fn, epochs, 0);
  if (rc != TTT_OK) return rc;
  if (deta_tok && !eta_tok) return fail(TTT_E_INVALID, "%s: deta_tok needs eta_tok", fn);
  if (deta_tok && (reinterpret_cast<uintptr_t>(deta_tok) & 3) != 0)
    return fail(TTT_E_INVALID, "%s: deta_tok must be 4-byte aligned", fn);
  if (!w1 || !dw1 || (mlp && (!w2 || !dw2)))
    return fail(TTT_E_INVALID, "%s: the states and their gradients must be non-null", fn);
  if (T > 0 && (!dq || !dk || !dv))
    return fail(TTT_E_INVALID, "%s: dq, dk and dv must be non-null", fn);
  if (chunk < 1) return fail(TTT_E_INVALID, "%s: chunk must be >= 1 (got %d)", fn, chunk);
  if (w_batch_stride < 0) return fail(TTT_E_INVALID, "%s: negative state batch stride", fn);
  if (mlp && dh <= 0) return fail(TTT_E_INVALID, "%s: dh must be positive (got %d)", fn, dh);
  if (d != 16 && d != 32 && d != 64)
    return fail(TTT_E_UNSUPPORTED, "%s: d=%d not supported (16, 32, 64)", fn, d);
  if (mlp && dh > 256) return fail(TTT_E_UNSUPPORTED, "%s: dh=%d not supported (<= 256)", fn, dh);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t n1 = mlp ? static_cast<size_t>(dh) * d : static_cast<size_t>(d) * d;
  if (T == 0) {
    const long long st = static_cast<long long>(H) * static_cast<long long>(n1);
    rc = copy_state(dw1, dw1_out, st, B, H, n1, s);
    if (rc != TTT_OK || !mlp) return rc;
    return copy_state(dw2, dw2_out, st, B, H, n1, s);
  }
  if (!mlp && ttt::linear_nc_bwd_mfma_supported(q, k, v, dz, w1, w_batch_stride, dw1_out, dq, dk, dv,
                                                dw1, T, d, chunk, epochs, io_dtype == TTT_BF16)) {
    hipError_t e = ttt::launch_linear_nc_bwd_mfma(q, k, v, dz, w1, w_batch_stride, dw1_out, eta_tok,
                                                 dq, dk, dv, dw1, deta_tok, B, H, T, eta,
                                                 loss == TTT_LOSS_DOT ? 1 : 0, s);
    if (e != hipSuccess) return hip_fail(e, "non-causal backward launch");
    return TTT_OK;
  }
  if (mlp && ttt::mlp_nc_bwd_mfma_supported(q, k, v, dz, w1, w2, w_batch_stride, dw1_out, dw2_out, dq,
                                             dk, dv, dw1, dw2, T, d, dh, chunk, epochs,
                                             io_dtype == TTT_BF16)) {
    hipError_t e = ttt::launch_mlp_nc_bwd_mfma(q, k, v, dz, w1, w2, w_batch_stride, dw1_out, dw2_out,
                                              eta_tok, dq, dk, dv, dw1, dw2, deta_tok, B, H, T, eta,
                                              loss == TTT_LOSS_DOT ? 1 : 0, s);
    if (e != hipSuccess) return hip_fail(e, "non-causal backward launch");
    return TTT_OK;
  }
  const int b = chunk < T ? chunk : T;
  const long long steps = static_cast<long long>((T + b - 1) / b) * epochs;
  if (!fits_int64(B, H, steps + 2, 2LL * static_cast<long long>(n1) + 2LL * T * d + T) ||
      steps > 0x7fffffffLL)
    return fail(TTT_E_INVALID, "%s: workspace size overflows", fn);
  StreamBuffer ws;
  rc = get_workspace(ttt::nc_bwd_workspace_floats(mlp, B, H, T, d, dh, chunk, epochs) * sizeof(float),
                     s, &ws);
  if (rc != TTT_OK) return rc;
  hipError_t e = ttt::launch_nc_bwd(mlp, q, k, v, dz, w1, w2, w_batch_stride, dw1_out, dw2_out,
                                    eta_tok, dq, dk, dv, dw1, dw2, deta_tok,
                                    static_cast<float*>(ws.ptr), B, H, T, d, dh, chunk, epochs, eta,
                                    loss == TTT_LOSS_DOT ? 1 : 0, io_dtype == TTT_BF16, s);
  if (e != hipSuccess) return hip_fail(e, "non-causal backward launch");
  return TTT_OK;
}

static int impl_ttt_linear_nc_bwd(const void* q, const void* k, const void* v, const float* w0,
                                  long long w0_batch_stride, const void* dz, const float* dw_out, void* dq,
                                  void* dk, void* dv, float* dw0, int B, int H, int T, int d, int chunk,
                                  int epochs, float eta, const float* eta_tok, float* deta_tok, int loss,
                                  int io_dtype, ttt_stream_t stream) {
  g_last_error.clear();
  return nc_bwd("ttt_linear_nc_bwd", false, q, k, v, w0, nullptr, w0_batch_stride, dz, dw_out,
                nullptr, dq, dk, dv, dw0, nullptr, B, H, T, d, 0, chunk, epochs, eta, eta_tok,
                deta_tok, loss, io_dtype, stream);
}

static int impl_ttt_mlp_nc_bwd(const void* q, const void* k, const void* v, const float* w1, const float* w2,
                               long long w_batch_stride, const void* dz, const float* dw1_out,
                               const float* dw2_out, void* dq, void* dk, void* dv, float* dw1, float* dw2,
                               int B, int H, int T, int d, int dh, int chunk, int epochs, float eta,
                               const float* eta_tok, float* deta_tok, int loss, int io_dtype,
                               ttt_stream_t stream) {
  g_last_error.clear();
  return nc_bwd("ttt_mlp_nc_bwd", true, q, k, v, w1, w2, w_batch_stride, dz, dw1_out, dw2_out, dq,
                dk, dv, dw1, dw2, B, H, T, d, dh, chunk, epochs, eta, eta_tok, deta_tok, loss,
                io_dtype, stream);
}

static int impl_ttt_mlp_bwd(const void* q, const void* k, const void* v, const float* w1, const float* w2,
                            long long w_batch_stride, const void* dz, const float* dw1_out,
                            const float* dw2_out, void* dq, void* dk, void* dv, float* dw1, float* dw2, int B,
                            int H, int T, int d, int dh, int chunk, float eta, const float* eta_tok,
                            float* deta_tok, int loss, int io_dtype, ttt_stream_t stream) {
  g_last_error.clear();
  int rc = check_common("ttt_mlp_bwd", q, k, v, dz, B, H, T, d, eta, eta_tok, io_dtype);
  if (rc != TTT_OK) return rc;
  if (deta_tok && !eta_tok) return fail(TTT_E_INVALID, "ttt_mlp_bwd: deta_tok needs eta_tok");
  if (deta_tok && (reinterpret_cast<uintptr_t>(deta_tok) & 3) != 0)
    return fail(TTT_E_INVALID, "ttt_mlp_bwd: deta_tok must be 4-byte aligned");
  if (loss != TTT_LOSS_MSE && loss != TTT_LOSS_DOT)
    return fail(TTT_E_INVALID, "ttt_mlp_bwd: unknown loss %d", loss);
  if (!w1 || !w2 || !dw1 || !dw2)
    return fail(TTT_E_INVALID, "ttt_mlp_bwd: w1, w2, dw1 and dw2 must be non-null");
  if (T > 0 && (!dq || !dk || !dv))
    return fail(TTT_E_INVALID, "ttt_mlp_bwd: dq, dk and dv must be non-null");
  if (dh <= 0) return fail(TTT_E_INVALID, "ttt_mlp_bwd: dh must be positive (got %d)", dh);
  if (chunk < 1) return fail(TTT_E_INVALID, "ttt_mlp_bwd: chunk must be >= 1 (got %d)", chunk);
  if (w_batch_stride < 0) return fail(TTT_E_INVALID, "ttt_mlp_bwd: negative w_batch_stride");
  if (d != 16 && d != 32 && d != 64)
    return fail(TTT_E_UNSUPPORTED, "ttt_mlp_bwd: d=%d not supported (16, 32, 64)", d);
  if (dh > 256) return fail(TTT_E_UNSUPPORTED, "ttt_mlp_bwd: dh=%d not supported (<= 256)", dh);
  if (T > 0 && (chunk < T ? chunk : T) > 16)
    return fail(TTT_E_UNSUPPORTED, "ttt_mlp_bwd: chunks of more than 16 tokens not supported");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t per = static_cast<size_t>(d) * dh;
  if (T == 0) {
    const long long st = static_cast<long long>(H) * static_cast<long long>(per);
    rc = copy_state(dw1, dw1_out, st, B, H, per, s);
    if (rc != TTT_OK) return rc;
    return copy_state(dw2, dw2_out, st, B, H, per, s);
  }
  const int b = chunk < T ? chunk : T;
  const long long nchunks = (T + b - 1) / b;
  if (!fits_int64(B, H, nchunks, 2LL * static_cast<long long>(per)))
    return fail(TTT_E_INVALID, "ttt_mlp_bwd: state history overflows");
  const bool bf16 = io_dtype == TTT_BF16;
  const int dot = loss == TTT_LOSS_DOT ? 1 : 0;
  ttt::MlpBwdArgs g{q, k, v, dz, dw1_out, dw2_out, nullptr, dq, dk, dv,
                    dw1, dw2, B, H, T, d, dh, chunk, eta, dot, eta_tok, deta_tok};
  ttt::MlpArgs f{q, k, v, w1, w2, w_batch_stride, nullptr, nullptr, nullptr,
                 B, H, T, d, dh, chunk, 1, eta, eta_tok, dot};
  hipError_t e;
  if (!dot && !eta_tok && ttt::mlp_bwd_mfma_supported(g, bf16) && ttt::mlp_fast_supported(f, bf16)) {
    // matrix cores: the forward pass stores its bf16 chunk-start states, the backward pass
    // reads them
    StreamBuffer hist;
    rc = get_workspace(ttt::mlp_bwd_mfma_workspace_bytes(g), s, &hist);
    if (rc != TTT_OK) return rc;
    e = ttt::launch_mlp_fwd_hist(f, hist.ptr, s);
    if (e != hipSuccess) return hip_fail(e, "ttt_mlp_bwd state launch");
    e = ttt::launch_mlp_bwd_mfma(g, hist.ptr, s);
    if (e != hipSuccess) return hip_fail(e, "ttt_mlp_bwd launch");
    return TTT_OK;
  }
  // forward recomputation on the generic kernel, storing the chunk-start states
  StreamBuffer hist, fws;
  rc = get_workspace(static_cast<size_t>(B) * H * nchunks * 2 * per * sizeof(float), s, &hist);
  if (rc != TTT_OK) return rc;
  f.w_hist = static_cast<float*>(hist.ptr);
  rc = get_workspace(ttt::mlp_generic_workspace_floats(f) * sizeof(float), s, &fws);
  if (rc != TTT_OK) return rc;
  e = ttt::launch_mlp_generic(f, bf16, static_cast<float*>(fws.ptr), s);
  if (e != hipSuccess) return hip_fail(e, "ttt_mlp_bwd state launch");
  g.w_hist = static_cast<const float*>(hist.ptr);
  e = ttt::launch_mlp_bwd_generic(g, bf16, s);
  if (e != hipSuccess) return hip_fail(e, "ttt_mlp_bwd launch");
  return TTT_OK;
}

static int impl_ttt_linear_fwd(const void* q, const void* k, const void* v, const float* w0,
                               long long w0_batch_stride, void* z, float* w_out, int B, int H, int T,
                               int d, int chunk, int causal, float eta, const float* eta_tok, int loss,
                               int epochs, int io_dtype, ttt_stream_t stream) {
  g_last_error.clear();
  return linear_fwd("ttt_linear_fwd", q, k, v, w0, w0_batch_stride, nullptr, nullptr, 0.0f, z,
                    w_out, B, H, T, d, chunk, causal, eta, eta_tok, loss, epochs, io_dtype, stream);
}

static int impl_ttt_linear_ln_fwd(const void* q, const void* k, const void* v, const float* w0,
                                  long long w0_batch_stride, const float* ln_weight, const float* ln_bias,
                                  float ln_eps, void* z, float* w_out, int B, int H, int T, int d, int chunk,
                                  int causal, float eta, const float* eta_tok, int loss, int epochs,
                                  int io_dtype, ttt_stream_t stream) {
  g_last_error.clear();
  const int rc = check_ln("ttt_linear_ln_fwd", ln_weight, ln_bias, ln_eps);
  if (rc != TTT_OK) return rc;
  return linear_fwd("ttt_linear_ln_fwd", q, k, v, w0, w0_batch_stride, ln_weight, ln_bias, ln_eps,
                    z, w_out, B, H, T, d, chunk, causal, eta, eta_tok, loss, epochs, io_dtype,
                    stream);
}

static int impl_ttt_mlp_fwd(const void* q, const void* k, const void* v, const float* w1, const float* w2,
                            long long w_batch_stride, void* z, float* w1_out, float* w2_out, int B, int H,
                            int T, int d, int dh, int chunk, int causal, float eta, const float* eta_tok,
                            int loss, int epochs, int io_dtype, ttt_stream_t stream,
                            const char* fn = "ttt_mlp_fwd", void* ws = nullptr, size_t ws_bytes = 0) {
  g_last_error.clear();
  return mlp_fwd(fn, q, k, v, w1, w2, w_batch_stride, nullptr, nullptr, 0.0f, z,
                 w1_out, w2_out, B, H, T, d, dh, chunk, causal, eta, eta_tok, loss, epochs,
                 io_dtype, stream, ws, ws_bytes);
}

static int impl_ttt_mlp_ln_fwd(const void* q, const void* k, const void* v, const float* w1, const float* w2,
                               long long w_batch_stride, const float* ln_weight, const float* ln_bias,
                               float ln_eps, void* z, float* w1_out, float* w2_out, int B, int H, int T,
                               int d, int dh, int chunk, int causal, float eta, const float* eta_tok,
                               int loss, int epochs, int io_dtype, ttt_stream_t stream,
                               const char* fn = "ttt_mlp_ln_fwd", void* ws = nullptr, size_t ws_bytes = 0) {
  g_last_error.clear();
  const int rc = check_ln(fn, ln_weight, ln_bias, ln_eps);
  if (rc != TTT_OK) return rc;
  return mlp_fwd(fn, q, k, v, w1, w2, w_batch_stride, ln_weight, ln_bias, ln_eps,
                 z, w1_out, w2_out, B, H, T, d, dh, chunk, causal, eta, eta_tok, loss, epochs,
                 io_dtype, stream, ws, ws_bytes);
}

// ---- public entry points: the calls above, then the optional finite check ----

int ttt_set_check_finite(int on) {
  const int prev = check_finite_on() ? 1 : 0;
  g_check_finite.store(on ? 1 : 0, std::memory_order_relaxed);
  return prev;
}

int ttt_get_check_finite(void) { return check_finite_on() ? 1 : 0; }

int ttt_set_split_debug(int flags) {
  return g_split_debug.exchange(flags & (TTT_SPLIT_FORMAL | TTT_SPLIT_TEST_ABORT), std::memory_order_relaxed);
}

int ttt_linear_fwd(const void* q, const void* k, const void* v, const float* w0,
                   long long w0_batch_stride, void* z, float* w_out, int B, int H, int T, int d,
                   int chunk, int causal, float eta, const float* eta_tok, int loss, int epochs,
                   int io_dtype, ttt_stream_t stream) {
  const int rc = impl_ttt_linear_fwd(q, k, v, w0, w0_batch_stride, z, w_out, B, H, T, d, chunk,
                                     causal, eta, eta_tok, loss, epochs, io_dtype, stream);
  return finite_outputs(rc, "ttt_linear_fwd", stream,
                        {{"z", z, tok(B, H, T, d), io_bytes(io_dtype)},
                         {"w_out", w_out, per_seq(B, H, 1LL * d * d), 4}});
}

int ttt_linear_ln_fwd(const void* q, const void* k, const void* v, const float* w0,
                      long long w0_batch_stride, const float* ln_weight, const float* ln_bias,
                      float ln_eps, void* z, float* w_out, int B, int H, int T, int d, int chunk,
                      int causal, float eta, const float* eta_tok, int loss, int epochs,
                      int io_dtype, ttt_stream_t stream) {
  const int rc = impl_ttt_linear_ln_fwd(q, k, v, w0, w0_batch_stride, ln_weight, ln_bias, ln_eps,
                                        z, w_out, B, H, T, d, chunk, causal, eta, eta_tok, loss,
                                        epochs, io_dtype, stream);
  return finite_outputs(rc, "ttt_linear_ln_fwd", stream,
                        {{"z", z, tok(B, H, T, d), io_bytes(io_dtype)},
                         {"w_out", w_out, per_seq(B, H, 1LL * d * d), 4}});
}

int ttt_mlp_fwd(const void* q, const void* k, const void* v, const float* w1, const float* w2,
                long long w_batch_stride, void* z, float* w1_out, float* w2_out, int B, int H,
                int T, int d, int dh, int chunk, int causal, float eta, const float* eta_tok,
                int loss, int epochs, int io_dtype, ttt_stream_t stream) {
  const int rc = impl_ttt_mlp_fwd(q, k, v, w1, w2, w_batch_stride, z, w1_out, w2_out, B, H, T, d,
                                  dh, chunk, causal, eta, eta_tok, loss, epochs, io_dtype, stream);
  return finite_outputs(rc, "ttt_mlp_fwd", stream,
                        {{"z", z, tok(B, H, T, d), io_bytes(io_dtype)},
                         {"w1_out", w1_out, per_seq(B, H, 1LL * dh * d), 4},
                         {"w2_out", w2_out, per_seq(B, H, 1LL * d * dh), 4}});
}

int ttt_mlp_ln_fwd(const void* q, const void* k, const void* v, const float* w1, const float* w2,
                   long long w_batch_stride, const float* ln_weight, const float* ln_bias,
                   float ln_eps, void* z, float* w1_out, float* w2_out, int B, int H, int T,
                   int d, int dh, int chunk, int causal, float eta, const float* eta_tok,
                   int loss, int epochs, int io_dtype, ttt_stream_t stream) {
  const int rc = impl_ttt_mlp_ln_fwd(q, k, v, w1, w2, w_batch_stride, ln_weight, ln_bias, ln_eps,
                                     z, w1_out, w2_out, B, H, T, d, dh, chunk, causal, eta,
                                     eta_tok, loss, epochs, io_dtype, stream);
  return finite_outputs(rc, "ttt_mlp_ln_fwd", stream,
                        {{"z", z, tok(B, H, T, d), io_bytes(io_dtype)},
                         {"w1_out", w1_out, per_seq(B, H, 1LL * dh * d), 4},
                         {"w2_out", w2_out, per_seq(B, H, 1LL * d * dh), 4}});
}

size_t ttt_mlp_fwd_workspace_size(int B, int H, int T, int d, int dh, int chunk, int causal,
                                  int io_dtype) {
  if (B <= 0 || H <= 0 || T <= 0 || static_cast<long long>(B) * H > 0x7fffffffLL) return 0;
  ttt::MlpArgs a{};
  // shape-only query: aligned stand-in pointers, so that only the shape decides
  const void* p = reinterpret_cast<const void*>(uintptr_t(256));
  a.q = a.k = a.v = p;
  a.z = const_cast<void*>(p);
  a.w1 = a.w2 = static_cast<const float*>(p);
  a.B = B;
  a.H = H;
  a.T = T;
  a.d = d;
  a.dh = dh;
  a.chunk = chunk;
  a.causal = causal;
  if (!ttt::mlp_split_supported(a, io_dtype == TTT_BF16)) return 0;
  return ttt::mlp_split_workspace_bytes(a);
}

int ttt_mlp_fwd_ws(const void* q, const void* k, const void* v, const float* w1, const float* w2,
                   long long w_batch_stride, void* z, float* w1_out, float* w2_out, int B, int H,
                   int T, int d, int dh, int chunk, int causal, float eta, const float* eta_tok,
                   int loss, int epochs, int io_dtype, void* workspace, size_t workspace_bytes,
                   ttt_stream_t stream) {
  const int rc = impl_ttt_mlp_fwd(q, k, v, w1, w2, w_batch_stride, z, w1_out, w2_out, B, H, T, d,
                                  dh, chunk, causal, eta, eta_tok, loss, epochs, io_dtype, stream,
                                  "ttt_mlp_fwd_ws", workspace, workspace_bytes);
  return finite_outputs(rc, "ttt_mlp_fwd_ws", stream,
                        {{"z", z, tok(B, H, T, d), io_bytes(io_dtype)},
                         {"w1_out", w1_out, per_seq(B, H, 1LL * dh * d), 4},
                         {"w2_out", w2_out, per_seq(B, H, 1LL * d * dh), 4}});
}

int ttt_mlp_ln_fwd_ws(const void* q, const void* k, const void* v, const float* w1,
                      const float* w2, long long w_batch_stride, const float* ln_weight,
                      const float* ln_bias, float ln_eps, void* z, float* w1_out, float* w2_out,
                      int B, int H, int T, int d, int dh, int chunk, int causal, float eta,
                      const float* eta_tok, int loss, int epochs, int io_dtype, void* workspace,
                      size_t workspace_bytes, ttt_stream_t stream) {
  const int rc = impl_ttt_mlp_ln_fwd(q, k, v, w1, w2, w_batch_stride, ln_weight, ln_bias, ln_eps,
                                     z, w1_out, w2_out, B, H, T, d, dh, chunk, causal, eta,
                                     eta_tok, loss, epochs, io_dtype, stream, "ttt_mlp_ln_fwd_ws",
                                     workspace, workspace_bytes);
  return finite_outputs(rc, "ttt_mlp_ln_fwd_ws", stream,
                        {{"z", z, tok(B, H, T, d), io_bytes(io_dtype)},
                         {"w1_out", w1_out, per_seq(B, H, 1LL * dh * d), 4},
                         {"w2_out", w2_out, per_seq(B, H, 1LL * d * dh), 4}});
}

int delta_rule_fwd(const void* q, const void* k, const void* v, const float* w0,
                   long long w0_batch_stride, void* z, float* w_out, int B, int H, int T,
                   int d, float eta, const float* eta_tok, int io_dtype, ttt_stream_t stream) {
  const int rc = impl_delta_rule_fwd(q, k, v, w0, w0_batch_stride, z, w_out, B, H, T, d, eta,
                                     eta_tok, io_dtype, stream);
  return finite_outputs(rc, "delta_rule_fwd", stream,
                        {{"z", z, tok(B, H, T, d), io_bytes(io_dtype)},
                         {"w_out", w_out, per_seq(B, H, 1LL * d * d), 4}});
}

int ttt_linear_bwd(const void* q, const void* k, const void* v, const float* w0,
                   long long w0_batch_stride, const void* dz, const float* dw_out, void* dq,
                   void* dk, void* dv, float* dw0, int B, int H, int T, int d, int chunk,
                   float eta, const float* eta_tok, float* deta_tok, int loss, int io_dtype,
                   ttt_stream_t stream) {
  const int rc = impl_ttt_linear_bwd(q, k, v, w0, w0_batch_stride, dz, dw_out, dq, dk, dv, dw0, B,
                                     H, T, d, chunk, eta, eta_tok, deta_tok, loss, io_dtype, stream);
  const int ib = io_bytes(io_dtype);
  return finite_outputs(rc, "ttt_linear_bwd", stream,
                        {{"dq", dq, tok(B, H, T, d), ib}, {"dk", dk, tok(B, H, T, d), ib},
                         {"dv", dv, tok(B, H, T, d), ib}, {"dw0", dw0, per_seq(B, H, 1LL * d * d), 4},
                         {"deta_tok", deta_tok, tok(B, H, T, 1), 4}});
}

int ttt_linear_bwd_noalloc(const void* q, const void* k, const void* v, const float* w0,
                           long long w0_batch_stride, const void* dz, const float* dw_out,
                           void* dq, void* dk, void* dv, float* dw0, int B, int H, int T, int d,
                           int chunk, float eta, const float* eta_tok, float* deta_tok, int loss,
                           int io_dtype, ttt_stream_t stream) {
  const int rc = impl_ttt_linear_bwd_noalloc(q, k, v, w0, w0_batch_stride, dz, dw_out, dq, dk, dv,
                                             dw0, B, H, T, d, chunk, eta, eta_tok, deta_tok, loss,
                                             io_dtype, stream);
  const int ib = io_bytes(io_dtype);
  return finite_outputs(rc, "ttt_linear_bwd_noalloc", stream,
                        {{"dq", dq, tok(B, H, T, d), ib}, {"dk", dk, tok(B, H, T, d), ib},
                         {"dv", dv, tok(B, H, T, d), ib}, {"dw0", dw0, per_seq(B, H, 1LL * d * d), 4},
                         {"deta_tok", deta_tok, tok(B, H, T, 1), 4}});
}

int ttt_mlp_bwd(const void* q, const void* k, const void* v, const float* w1, const float* w2,
                long long w_batch_stride, const void* dz, const float* dw1_out,
                const float* dw2_out, void* dq, void* dk, void* dv, float* dw1, float* dw2, int B,
                int H, int T, int d, int dh, int chunk, float eta, const float* eta_tok,
                float* deta_tok, int loss, int io_dtype, ttt_stream_t stream) {
  const int rc = impl_ttt_mlp_bwd(q, k, v, w1, w2, w_batch_stride, dz, dw1_out, dw2_out, dq, dk,
                                  dv, dw1, dw2, B, H, T, d, dh, chunk, eta, eta_tok, deta_tok, loss,
                                  io_dtype, stream);
  const int ib = io_bytes(io_dtype);
  return finite_outputs(rc, "ttt_mlp_bwd", stream,
                        {{"dq", dq, tok(B, H, T, d), ib}, {"dk", dk, tok(B, H, T, d), ib},
                         {"dv", dv, tok(B, H, T, d), ib}, {"dw1", dw1, per_seq(B, H, 1LL * dh * d), 4},
                         {"dw2", dw2, per_seq(B, H, 1LL * d * dh), 4},
                         {"deta_tok", deta_tok, tok(B, H, T, 1), 4}});
}

int ttt_linear_ln_bwd(const void* q, const void* k, const void* v, const float* w0,
                      long long w0_batch_stride, const float* ln_weight, const float* ln_bias,
                      float ln_eps, const void* dz, const float* dw_out, void* dq, void* dk,
                      void* dv, float* dw0, float* dln_weight, float* dln_bias, int B, int H,
                      int T, int d, int chunk, float eta, const float* eta_tok, float* deta_tok,
                      int loss, int io_dtype, ttt_stream_t stream) {
  const int rc = impl_ttt_linear_ln_bwd(q, k, v, w0, w0_batch_stride, ln_weight, ln_bias, ln_eps,
                                        dz, dw_out, dq, dk, dv, dw0, dln_weight, dln_bias, B, H, T,
                                        d, chunk, eta, eta_tok, deta_tok, loss, io_dtype, stream);
  const int ib = io_bytes(io_dtype);
  return finite_outputs(rc, "ttt_linear_ln_bwd", stream,
                        {{"dq", dq, tok(B, H, T, d), ib}, {"dk", dk, tok(B, H, T, d), ib},
                         {"dv", dv, tok(B, H, T, d), ib}, {"dw0", dw0, per_seq(B, H, 1LL * d * d), 4},
                         {"dln_weight", dln_weight, per_seq(B, H, d), 4},
                         {"dln_bias", dln_bias, per_seq(B, H, d), 4},
                         {"deta_tok", deta_tok, tok(B, H, T, 1), 4}});
}

int ttt_mlp_ln_bwd(const void* q, const void* k, const void* v, const float* w1, const float* w2,
                   long long w_batch_stride, const float* ln_weight, const float* ln_bias,
                   float ln_eps, const void* dz, const float* dw1_out, const float* dw2_out,
                   void* dq, void* dk, void* dv, float* dw1, float* dw2, float* dln_weight,
                   float* dln_bias, int B, int H, int T, int d, int dh, int chunk, float eta,
                   const float* eta_tok, float* deta_tok, int loss, int io_dtype,
                   ttt_stream_t stream) {
  const int rc = impl_ttt_mlp_ln_bwd(q, k, v, w1, w2, w_batch_stride, ln_weight, ln_bias, ln_eps,
                                     dz, dw1_out, dw2_out, dq, dk, dv, dw1, dw2, dln_weight,
                                     dln_bias, B, H, T, d, dh, chunk, eta, eta_tok, deta_tok, loss,
                                     io_dtype, stream);
  const int ib = io_bytes(io_dtype);
  return finite_outputs(rc, "ttt_mlp_ln_bwd", stream,
                        {{"dq", dq, tok(B, H, T, d), ib}, {"dk", dk, tok(B, H, T, d), ib},
                         {"dv", dv, tok(B, H, T, d), ib}, {"dw1", dw1, per_seq(B, H, 1LL * dh * d), 4},
                         {"dw2", dw2, per_seq(B, H, 1LL * d * dh), 4},
                         {"dln_weight", dln_weight, per_seq(B, H, d), 4},
                         {"dln_bias", dln_bias, per_seq(B, H, d), 4},
                         {"deta_tok", deta_tok, tok(B, H, T, 1), 4}});
}

int ttt_linear_nc_bwd(const void* q, const void* k, const void* v, const float* w0,
                      long long w0_batch_stride, const void* dz, const float* dw_out, void* dq,
                      void* dk, void* dv, float* dw0, int B, int H, int T, int d, int chunk,
                      int epochs, float eta, const float* eta_tok, float* deta_tok, int loss,
                      int io_dtype, ttt_stream_t stream) {
  const int rc = impl_ttt_linear_nc_bwd(q, k, v, w0, w0_batch_stride, dz, dw_out, dq, dk, dv, dw0,
                                        B, H, T, d, chunk, epochs, eta, eta_tok, deta_tok, loss,
                                        io_dtype, stream);
  const int ib = io_bytes(io_dtype);
  return finite_outputs(rc, "ttt_linear_nc_bwd", stream,
                        {{"dq", dq, tok(B, H, T, d), ib}, {"dk", dk, tok(B, H, T, d), ib},
                         {"dv", dv, tok(B, H, T, d), ib}, {"dw0", dw0, per_seq(B, H, 1LL * d * d), 4},
                         {"deta_tok", deta_tok, tok(B, H, T, 1), 4}});
}

int ttt_mlp_nc_bwd(const void* q, const void* k, const void* v, const float* w1, const float* w2,
                   long long w_batch_stride, const void* dz, const float* dw1_out,
                   const float* dw2_out, void* dq, void* dk, void* dv, float* dw1, float* dw2,
                   int B, int H, int T, int d, int dh, int chunk, int epochs, float eta,
                   const float* eta_tok, float* deta_tok, int loss, int io_dtype,
                   ttt_stream_t stream) {
  const int rc = impl_ttt_mlp_nc_bwd(q, k, v, w1, w2, w_batch_stride, dz, dw1_out, dw2_out, dq, dk,
                                     dv, dw1, dw2, B, H, T, d, dh, chunk, epochs, eta, eta_tok,
                                     deta_tok, loss, io_dtype, stream);
  const int ib = io_bytes(io_dtype);
  return finite_outputs(rc, "ttt_mlp_nc_bwd", stream,
                        {{"dq", dq, tok(B, H, T, d), ib}, {"dk", dk, tok(B, H, T, d), ib},
                         {"dv", dv, tok(B, H, T, d), ib}, {"dw1", dw1, per_seq(B, H, 1LL * dh * d), 4},
                         {"dw2", dw2, per_seq(B, H, 1LL * d * dh), 4},
                         {"deta_tok", deta_tok, tok(B, H, T, 1), 4}});
}

}  // extern "C"
