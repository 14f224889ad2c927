// Plain read stream: the achievable HBM read rate on this GPU, measured the
// way the decode kernel reads its selected pages (16 KiB runs of 16-byte
// streaming loads, several in flight per lane).  It is a yardstick for the
// memory-bound calls, not a step of the method.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamLoads = 4;                                 // 16-byte loads in flight per lane
constexpr int kChunk16 = kStreamThreads * kStreamLoads;          // one chunk: 16 KiB

// Workgroup w reads the 16 KiB chunks w, w + grid, w + 2 grid, ... whole
// (each lane four 16-byte streaming loads per chunk, issued before any is
// used), then its share of the ragged tail; it folds everything it read
// into one XOR word, so nothing is written besides the sink and the loads
// cannot be dropped.  Contiguous chunks per workgroup measured faster on
// this GPU than a grid-wide stride over 16-byte units (7.2-7.3 against
// 6.3-6.8 TB/s on a 4 GiB buffer).
__global__ __launch_bounds__(kStreamThreads) void k_read_stream(const u32x4* __restrict__ src,
                                                                size_t n16, uint32_t* sink) {
  const size_t nchunk = n16 / kChunk16;
  uint32_t acc = 0;
  for (size_t c = blockIdx.x; c < nchunk; c += gridDim.x) {
    const u32x4* p = src + c * kChunk16 + threadIdx.x;
    u32x4 w[kStreamLoads];
#pragma unroll
    for (int j = 0; j < kStreamLoads; ++j) w[j] = __builtin_nontemporal_load(p + j * kStreamThreads);
#pragma unroll
    for (int j = 0; j < kStreamLoads; ++j) acc ^= w[j][0] ^ w[j][1] ^ w[j][2] ^ w[j][3];
  }
  for (size_t i = nchunk * kChunk16 + size_t(blockIdx.x) * kStreamThreads + threadIdx.x; i < n16;
       i += size_t(gridDim.x) * kStreamThreads) {
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
