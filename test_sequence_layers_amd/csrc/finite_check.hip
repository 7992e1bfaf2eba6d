// Debug check of a call's outputs for non-finite values (NaN, +inf, -inf), run when the
// library's finite check is switched on.  One flag per output buffer, in a file-scope device
// array (each GPU holds its own copy); the flags are cleared by a kernel on the call's
// stream, every element whose exponent bits are all ones sets its buffer's flag with a plain
// store (all writers store the same value), and the host reads the flags back after the
// stream has drained.  Calls with the check on share the flags of their GPU, so two such
// calls that overlap on one GPU can report each other's outputs; the check is meant for
// debugging, one stream at a time.
#include "common.hpp"

namespace ttt {
namespace {

static __device__ __align__(64) unsigned int nonfinite_flags[kMaxCheckedOutputs];

__global__ void clear_flags_kernel(unsigned int* flags, int n) {
  if (static_cast<int>(threadIdx.x) < n) flags[threadIdx.x] = 0u;
}

// 16-bit elements (bf16): exponent bits 0x7F80; 32-bit (float32): 0x7F800000
template <typename U, U kExp>
__global__ void scan_kernel(const U* p, long long n, unsigned int* flag) {
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  bool bad = false;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    bad |= (p[i] & kExp) == kExp;
  if (bad) *flag = 1u;
}

}  // namespace

hipError_t check_finite_outputs(const CheckedOutput* outs, int nouts, hipStream_t s,
                                unsigned int* host_flags) {
  if (nouts < 0 || nouts > kMaxCheckedOutputs) return hipErrorInvalidValue;
  void* dev = nullptr;
  hipError_t e = hipGetSymbolAddress(&dev, HIP_SYMBOL(nonfinite_flags));
  if (e != hipSuccess) return e;
  unsigned int* flags = static_cast<unsigned int*>(dev);
  hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(64), 0, s, flags, kMaxCheckedOutputs);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int i = 0; i < nouts; ++i) {
    const CheckedOutput& o = outs[i];
    if (o.ptr == nullptr || o.count <= 0) continue;
    const long long blocks = (o.count + 255) / 256;
    const dim3 grid(static_cast<unsigned>(blocks < 2048 ? blocks : 2048)), block(256);
    if (o.bytes_per_elem == 2)
      hipLaunchKernelGGL((scan_kernel<uint16_t, 0x7F80u>), grid, block, 0, s,
                         static_cast<const uint16_t*>(o.ptr), o.count, flags + i);
    else
      hipLaunchKernelGGL((scan_kernel<uint32_t, 0x7F800000u>), grid, block, 0, s,
                         static_cast<const uint32_t*>(o.ptr), o.count, flags + i);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  e = hipMemcpyAsync(host_flags, flags, kMaxCheckedOutputs * sizeof(unsigned int), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

}  // namespace ttt
