// Layout transform between raster order and the blocked layout (SPADE
// arXiv 2608.03335, 3.3: rearrange into blocks; restore the original
// layout).  One workgroup per (batch*head, block): the block's box is
// decoded once, then 256 threads move its rows in 16-byte pieces.
#include <hip/hip_runtime.h>

#include "vsa_device.h"
#include "vsa_kernels.h"

namespace vsa {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <bool INVERSE>
__global__ __launch_bounds__(256) void permute_kernel(const uint8_t* __restrict__ src,
                                                      uint8_t* __restrict__ dst, DGeo g, int P,
                                                      int row_bytes) {
  const int bh = blockIdx.y, j = blockIdx.x;
  const Box b = block_box(g, j);
  const int nj = b.n();
  TokenMap map;
  map.init(g, b);
  const int pieces = row_bytes / 16;
  const size_t raster_base = (size_t)bh * g.N * row_bytes;
  const size_t blocked_base = ((size_t)bh * g.NB + j) * P * row_bytes;
  const int rows = INVERSE ? nj : P;
  for (int idx = threadIdx.x; idx < rows * pieces; idx += 256) {
    const int u = idx / pieces, part = idx - u * pieces;
    const size_t boff = blocked_base + (size_t)u * row_bytes + part * 16;
    if (INVERSE) {
      const size_t roff = raster_base + (size_t)map(u) * row_bytes + part * 16;
      *reinterpret_cast<u32x4_t*>(dst + roff) = *reinterpret_cast<const u32x4_t*>(src + boff);
    } else {
      u32x4_t val = u32x4_t{0u, 0u, 0u, 0u};
      if (u < nj) {
        const size_t roff = raster_base + (size_t)map(u) * row_bytes + part * 16;
        val = *reinterpret_cast<const u32x4_t*>(src + roff);
      }
      *reinterpret_cast<u32x4_t*>(dst + boff) = val;
    }
  }
}

hipError_t launch_permute(const void* x, void* xb, int elt, int D, const DGeo& g, int BH, int P,
                          bool inverse, hipStream_t st) {
  dim3 grid(g.NB, BH), block(256);
  const int row_bytes = D * elt;
  if (inverse)
    hipLaunchKernelGGL(permute_kernel<true>, grid, block, 0, st, (const uint8_t*)xb, (uint8_t*)x, g, P, row_bytes);
  else
    hipLaunchKernelGGL(permute_kernel<false>, grid, block, 0, st, (const uint8_t*)x, (uint8_t*)xb, g, P, row_bytes);
  return hipGetLastError();
}

}  // namespace vsa
