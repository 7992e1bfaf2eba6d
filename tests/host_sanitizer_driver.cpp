// Host-side driver of the C ABI for a sanitizer build (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code of ttt_api.cpp): every call below has an
// argument the library must reject before any HIP call, so it runs without a GPU.  Each
// rejection must return the documented status and leave a message naming the function; the
// calls also run on several threads at once, since the message buffer is per thread.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "../include/ttt.h"

namespace {
alignas(256) unsigned char buf[1 << 16];
void* P = buf;               // a stand-in pointer (validation never dereferences it)
float* F = reinterpret_cast<float*>(buf);
const float* misaligned = reinterpret_cast<const float*>(buf + 1);
int failures = 0;

void expect(int got, int want, const char* fn, const char* what) {
  const char* msg = ttt_last_error();
  if (got != want || msg == nullptr || std::strstr(msg, fn) == nullptr) {
    std::printf("FAIL %s (%s): status %d (want %d), message \"%s\"\n", fn, what, got, want,
                msg ? msg : "(null)");
    ++failures;
  }
}

void run_all() {
  const float nan = std::nanf("");
  // forward passes
  expect(ttt_linear_fwd(nullptr, P, P, F, 0, P, nullptr, 1, 1, 16, 64, 16, 1, 0.1f, nullptr, 0, 1, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_linear_fwd", "null q");
  expect(ttt_linear_fwd(P, P, P, F, 0, P, nullptr, 0, 1, 16, 64, 16, 1, 0.1f, nullptr, 0, 1, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_linear_fwd", "B = 0");
  expect(ttt_linear_fwd(P, P, P, F, 0, P, nullptr, 1, 1, 16, 64, 0, 1, 0.1f, nullptr, 0, 1, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_linear_fwd", "chunk = 0");
  expect(ttt_linear_fwd(P, P, P, F, 0, P, nullptr, 1, 1, 16, 64, 16, 1, nan, nullptr, 0, 1, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_linear_fwd", "eta NaN");
  expect(ttt_linear_fwd(P, P, P, F, 0, P, nullptr, 1, 1, 16, 64, 16, 1, 0.1f, nullptr, 0, 1, 7, nullptr),
         TTT_E_INVALID, "ttt_linear_fwd", "dtype");
  expect(ttt_linear_fwd(P, P, P, F, 0, P, nullptr, 1, 1, 16, 64, 16, 1, 0.1f, nullptr, 5, 1, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_linear_fwd", "loss");
  expect(ttt_linear_fwd(P, P, P, F, 0, P, nullptr, 1, 1, 16, 64, 16, 1, 0.1f, nullptr, 0, 2, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_linear_fwd", "epochs > 1 causal");
  expect(ttt_linear_fwd(P, P, P, F, 0, P, nullptr, 1, 1, 16, 64, 16, 1, 0.1f, misaligned, 0, 1, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_linear_fwd", "misaligned eta_tok");
  expect(ttt_linear_fwd(P, P, P, F, 0, P, nullptr, 1, 1, 16, 48, 16, 1, 0.1f, nullptr, 0, 1, TTT_BF16, nullptr),
         TTT_E_UNSUPPORTED, "ttt_linear_fwd", "d = 48");
  expect(ttt_mlp_fwd(P, P, P, F, F, 0, P, nullptr, nullptr, 1, 1, 16, 64, 0, 16, 1, 0.1f, nullptr, 0, 1, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_mlp_fwd", "dh = 0");
  expect(ttt_mlp_fwd(P, P, P, F, F, 0, P, nullptr, nullptr, 1, 1, 16, 64, 4096, 16, 1, 0.1f, nullptr, 0, 1, TTT_BF16, nullptr),
         TTT_E_UNSUPPORTED, "ttt_mlp_fwd", "dh = 4096");
  {
    // the two-workgroup MLP entry points: a workspace one byte short, then a misaligned one
    const size_t need = ttt_mlp_fwd_workspace_size(2, 3, 40, 64, 256, 16, 1, TTT_BF16);
    if (need == 0) {
      std::printf("FAIL ttt_mlp_fwd_workspace_size: 0 for the d 64 shape\n");
      ++failures;
    }
    void* ws = reinterpret_cast<void*>(uintptr_t(0x10000));
    void* ws_mis = reinterpret_cast<void*>(uintptr_t(0x10010));
    expect(ttt_mlp_fwd_ws(P, P, P, F, F, 0, P, nullptr, nullptr, 2, 3, 40, 64, 256, 16, 1, 0.1f, nullptr, 0, 1,
                          TTT_BF16, ws, need - 1, nullptr),
           TTT_E_INVALID, "ttt_mlp_fwd_ws", "small workspace");
    expect(ttt_mlp_fwd_ws(P, P, P, F, F, 0, P, nullptr, nullptr, 2, 3, 40, 64, 256, 16, 1, 0.1f, nullptr, 0, 1,
                          TTT_BF16, ws_mis, need, nullptr),
           TTT_E_INVALID, "ttt_mlp_fwd_ws", "misaligned workspace");
    expect(ttt_mlp_ln_fwd_ws(P, P, P, F, F, 0, F, F, 0.0f, P, nullptr, nullptr, 2, 3, 40, 64, 256, 16, 1, 0.1f,
                             nullptr, 0, 1, TTT_BF16, ws, need, nullptr),
           TTT_E_INVALID, "ttt_mlp_ln_fwd_ws", "ln_eps 0");
  }
  if (ttt_set_split_debug(TTT_SPLIT_FORMAL) != 0 || ttt_set_split_debug(0) != TTT_SPLIT_FORMAL) {
    std::printf("FAIL ttt_set_split_debug: previous flags\n");
    ++failures;
  }
  expect(ttt_linear_ln_fwd(P, P, P, F, 0, nullptr, F, 1e-6f, P, nullptr, 1, 1, 16, 64, 16, 1, 0.1f, nullptr, 0, 1, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_linear_ln_fwd", "null ln weight");
  expect(ttt_mlp_ln_fwd(P, P, P, F, F, 0, F, F, 1e-6f, P, nullptr, nullptr, -1, 1, 16, 64, 256, 16, 1, 0.1f, nullptr, 0, 1, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_mlp_ln_fwd", "B < 0");
  expect(delta_rule_fwd(P, nullptr, P, F, 0, P, nullptr, 1, 1, 16, 64, 0.5f, nullptr, TTT_BF16, nullptr),
         TTT_E_INVALID, "delta_rule_fwd", "null k");
  // backward passes
  expect(ttt_linear_bwd(P, P, P, F, 0, P, nullptr, nullptr, P, P, F, 1, 1, 16, 64, 16, 0.1f, nullptr, nullptr, 0, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_linear_bwd", "null dq");
  expect(ttt_linear_bwd(P, P, P, F, 0, P, nullptr, P, P, P, F, 1, 1, 16, 64, 16, 0.1f, nullptr, F, 0, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_linear_bwd", "deta_tok without eta_tok");
  expect(ttt_linear_bwd_noalloc(P, P, P, F, 0, P, nullptr, P, P, P, F, 1, 1, 16, 64, 0, 0.1f, nullptr, nullptr, 0, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_linear_bwd_noalloc", "chunk = 0");
  expect(ttt_mlp_bwd(P, P, P, F, F, 0, P, nullptr, nullptr, P, P, P, F, nullptr, 1, 1, 16, 64, 256, 16, 0.1f, nullptr, nullptr, 0, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_mlp_bwd", "null dw2");
  expect(ttt_linear_ln_bwd(P, P, P, F, 0, F, F, 1e-6f, P, nullptr, P, P, P, F, nullptr, F, 1, 1, 16, 64, 16, 0.1f, nullptr, nullptr, 0, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_linear_ln_bwd", "null dln weight");
  expect(ttt_mlp_ln_bwd(P, P, P, F, F, 0, F, F, 1e-6f, P, nullptr, nullptr, P, P, P, F, F, F, F, 1, 1, 16, 64, 256, 16, 0.1f, nullptr, nullptr, 9, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_mlp_ln_bwd", "loss");
  expect(ttt_linear_nc_bwd(P, P, P, F, 0, P, nullptr, P, P, P, F, 1, 1, 16, 64, 16, 0, 0.1f, nullptr, nullptr, 0, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_linear_nc_bwd", "epochs = 0");
  expect(ttt_mlp_nc_bwd(P, P, P, F, F, -4, P, nullptr, nullptr, P, P, P, F, F, 1, 1, 16, 64, 64, 16, 1, 0.1f, nullptr, nullptr, 0, TTT_BF16, nullptr),
         TTT_E_INVALID, "ttt_mlp_nc_bwd", "negative batch stride");
}
}  // namespace

int main() {
  if (ttt_abi_version() <= 0) {
    std::printf("FAIL ttt_abi_version\n");
    return 1;
  }
  run_all();
  // the finite-check switch: invalid calls are still rejected before any GPU work
  const int prev = ttt_set_check_finite(1);
  if (ttt_get_check_finite() != 1) {
    std::printf("FAIL ttt_get_check_finite after ttt_set_check_finite(1)\n");
    ++failures;
  }
  run_all();
  if (ttt_set_check_finite(prev) != 1) {
    std::printf("FAIL ttt_set_check_finite did not return the previous setting\n");
    ++failures;
  }
  std::vector<std::thread> pool;
  for (int t = 0; t < 4; ++t) pool.emplace_back(run_all);
  for (auto& th : pool) th.join();
  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "OK", failures);
  return failures ? 1 : 0;
}
