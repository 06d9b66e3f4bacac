// read_ceiling.hip -- a read-only pass over device memory, for gfx950.
//
// The weight-streaming GEMV moves one byte per weight from HBM and almost
// nothing else, so the rate at which a kernel can do nothing but read HBM is
// the practical ceiling it is measured against, beside the published peak.
// Every 16-byte word of the buffer is read once with the same non-temporal
// loads the GEMV uses (eight in flight per thread, grid-stride over a grid
// sized to the chip) and folded by XOR so that no load can be dropped; each
// workgroup writes one 32-bit word.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"

namespace fp8w {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void k_read_xor(const uint8_t* __restrict__ buf, int64_t words,
                                                       uint32_t* __restrict__ out) {
  __shared__ uint32_t part[kThreads / kWave];
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < words; base += stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t w = base + (int64_t)u * kThreads;
      v[u] = w < words ? ld_stream_u4(buf, (size_t)w * 16) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) r ^= part[w];
    st_global<uint32_t>(out, (size_t)blockIdx.x * 4, r);
  }
}

}  // namespace

int64_t read_ceiling_blocks(int64_t bytes, int64_t max_blocks) {
  const int64_t words = bytes / 16;
  const int64_t per_block = (int64_t)kThreads * kUnroll;
  const int64_t need = (words + per_block - 1) / per_block;
  return need < max_blocks ? need : max_blocks;
}

hipError_t launch_read_ceiling(const void* buf, int64_t bytes, uint32_t* out, int64_t blocks,
                               hipStream_t stream) {
  hipLaunchKernelGGL(k_read_xor, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const uint8_t*>(buf), bytes / 16, out);
  return hipGetLastError();
}

}  // namespace fp8w
