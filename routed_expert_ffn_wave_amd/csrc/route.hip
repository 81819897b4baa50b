// Router top-k with renormalised softmax weights (route_tokens in ft_route.h): four tokens per
// wave (one per 16-lane row) up to E = 256 and k = 16, else one token per wave.
#include "ft_device.h"
#include "ft_kernels.h"
#include "ft_route.h"

namespace ftk {

template <int VPL>  // values per lane of the one-token-per-wave path
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                    int32_t* __restrict__ ids, float* __restrict__ w) {
  route_tokens<VPL>(logits, T, E, k, blockIdx.x * 4 + (threadIdx.x >> 6), gridDim.x * 4,
                    [&](int t, int j, int e, float wt) {
                      ids[(size_t)t * k + j] = e;
                      w[(size_t)t * k + j] = wt;
                    });
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  dim3 grid((T + (route_by_rows(E, k) ? 15 : 3)) / (route_by_rows(E, k) ? 16 : 4)), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (E <= 128)
    hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (E <= 256)
    hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (E <= 512)
    hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, s, logits, T, E, k, ids, w);
  else
    hipLaunchKernelGGL(route_kernel<16>, grid, block, 0, s, logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace ftk
