// Relative RoPE: rotate a [n_tokens][H][D] tensor by cache-relative frame
// positions ("fused Triton RoPE", hysenlabs.com, "NVFP4, sequence parallel
// and the async decode path"; relative RoPE, refft.com, question "How do
// KV-cache relative RoPE and TriAttention work together ...").
//
// One thread per 8 consecutive elements of one (token, head) row
// (rope_unit).  Memory-bound: 2 or 4 bytes read and 2 or 4 written per
// element.
#include "rope_unit.hpp"

namespace fp4kv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void rope_kernel(RopeParams p) {
  const long long n = rope_units(p);
  for (long long u = (long long)blockIdx.x * kThreads + threadIdx.x; u < n;
       u += (long long)gridDim.x * kThreads)
    rope_unit(p, u);
}

}  // namespace

hipError_t launch_rope(const RopeParams &p, hipStream_t s) {
  const long long n = rope_units(p);
  long long blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(rope_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace fp4kv
