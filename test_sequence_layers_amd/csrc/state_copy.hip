// Copies initial states to the final-state output (used when a call has no tokens), or
// zero-fills it when there is no source.
#include "common.hpp"

namespace ttt {
namespace {

__global__ void copy_state_kernel(float* dst, const float* src, long long batch_stride, int H,
                                  size_t per_head) {
  const int chain = blockIdx.x;
  const int bi = chain / H, hi = chain - bi * H;
  const float* s = src ? src + bi * batch_stride + static_cast<long long>(hi) * per_head : nullptr;
  float* d = dst + static_cast<size_t>(chain) * per_head;
  for (size_t e = threadIdx.x; e < per_head; e += blockDim.x)
    d[e] = s ? s[e] : 0.0f;
}

}  // namespace

hipError_t launch_copy_state(float* dst, const float* src, long long batch_stride, int B, int H,
                             size_t per_head, hipStream_t s) {
  hipLaunchKernelGGL(copy_state_kernel, dim3(B * H), dim3(256), 0, s, dst, src, batch_stride, H,
                     per_head);
  return hipGetLastError();
}

}  // namespace ttt
