// Plain read stream: the achievable HBM read rate on this GPU, measured the
// way the decode kernel reads its selected pages (16-byte loads, many in
// flight per lane).  It is a yardstick for the memory-bound calls, not a
// step of the method.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;   // 16-byte loads in flight per lane

// Each workgroup folds its share of the buffer (grid-stride over 16-byte
// chunks) into one XOR word, so nothing is written besides the sink and
// the loads cannot be dropped.
__global__ __launch_bounds__(kStreamThreads) void k_read_stream(const u32x4* __restrict__ src,
                                                                size_t n16, uint32_t* sink) {
  const size_t stride = size_t(gridDim.x) * kStreamThreads;
  size_t i = size_t(blockIdx.x) * kStreamThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    u32x4 w[kStreamUnroll];
#pragma unroll
    for (int j = 0; j < kStreamUnroll; ++j) w[j] = __builtin_nontemporal_load(src + i + j * stride);
#pragma unroll
    for (int j = 0; j < kStreamUnroll; ++j) acc ^= w[j][0] ^ w[j][1] ^ w[j][2] ^ w[j][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 w = src[i];
    acc ^= w[0] ^ w[1] ^ w[2] ^ w[3];
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  __shared__ uint32_t part[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int w = 0; w < kStreamThreads / 64; ++w) x ^= part[w];
    sink[blockIdx.x] = x;
  }
}

}  // namespace

hipError_t launch_read_stream(const void* src, size_t bytes, uint32_t* sink, int n_wg,
                              hipStream_t s) {
  k_read_stream<<<n_wg, kStreamThreads, 0, s>>>(static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace dsa
