// Streaming HBM read: the bandwidth ceiling the weight-streaming expert kernels are
// measured against. Every 16-byte chunk of the buffer is read once with a non-temporal
// load (as the expert kernels read their weights) and folded into an XOR of all dwords,
// which does not depend on the order of the reads.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__global__ __launch_bounds__(64) void xor_clear_kernel(uint32_t* out) {
  if (threadIdx.x == 0) *out = 0u;
}

// Block b reads chunks [b * per, (b + 1) * per) front to back, eight 4 KB steps in flight,
// and the grid's last block also the remainder: each block is one sequential stream (on
// MI355X block-contiguous streams read ~15% faster than a grid-stride sweep).
__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4_t* __restrict__ p, size_t n16, size_t per,
                                                       uint32_t* __restrict__ out) {
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = blockIdx.x + 1 == gridDim.x ? n16 : lo + per;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  size_t i = lo + threadIdx.x;
  for (; i + 7 * 256 < hi; i += 8 * 256) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = load_nt_u32x4(p + i + u * 256);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < hi; i += 256) acc ^= load_nt_u32x4(p + i);
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  if ((threadIdx.x & 63) == 0 && x) atomicXor(out, x);
}

}  // namespace

hipError_t launch_hbm_read(const void* buf, size_t bytes, uint32_t* checksum, hipStream_t s) {
  hipLaunchKernelGGL(xor_clear_kernel, dim3(1), dim3(64), 0, s, checksum);
  const size_t n16 = bytes / 16;
  if (n16) {
    // 8192 blocks (32 per compute unit) of at least one 4 KB step each
    size_t blocks = n16 / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const u32x4_t*)buf, n16,
                       n16 / blocks, checksum);
  }
  return hipGetLastError();
}

}  // namespace moe
