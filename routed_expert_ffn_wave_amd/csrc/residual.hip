// Merge of the cold-expert residual into the layer output: out += residual on the device.
//
// The pairs whose expert is not resident are computed on the host cores (residual_host.cpp: the
// pages' engine runs cold experts on the CPU beside the GPU, FreeToken walk-through section 五);
// this kernel adds their per-token sum into the output of the device layer, fp32 or bf16.
#include "ft_device.h"
#include "ft_kernels.h"

namespace ftk {
namespace {

__global__ __launch_bounds__(256) void residual_add_kernel(void* out, const float* __restrict__ res, long long n,
                                                           bool out_bf16) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    if (out_bf16) {
      uint16_t* o = (uint16_t*)out;
      const float v = __uint_as_float((uint32_t)o[i] << 16) + res[i];
      uint32_t u = __float_as_uint(v);
      u = ((u & 0x7fffffffu) > 0x7f800000u) ? (u | 0x00400000u) : u + 0x7fffu + ((u >> 16) & 1u);
      o[i] = (uint16_t)(u >> 16);
    } else {
      ((float*)out)[i] += res[i];
    }
  }
}

}  // namespace

hipError_t launch_residual_add(void* out, const float* res, long long n, bool out_bf16, hipStream_t s) {
  if (n == 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(residual_add_kernel, dim3((unsigned)blocks), dim3(256), 0, s, out, res, n, out_bf16);
  return hipGetLastError();
}

}  // namespace ftk
