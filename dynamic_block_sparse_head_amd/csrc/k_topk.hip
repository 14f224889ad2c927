// Top-k block selection plus the local window ([DMA] §五: after the causal
// mask keep the k highest-weight history positions, everything else -inf).
//
// One workgroup per score row.  Candidates become 64-bit keys
//   (order-preserving bits of the score) << 32 | (0xffffffff - index)
// so that "larger key" means "higher score, then lower index"; NaN maps to
// the lowest score bits and therefore ranks last.  The keys are sorted
// descending by a bitonic network in LDS; the first k are the selection.
// Selected and window blocks are flagged in LDS and compacted in index
// order, which writes each output row already ascending.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxN = 8192;

__device__ __forceinline__ uint32_t order_bits(float f) {
  if (__builtin_isnan(f)) return 0u;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kThreads) void k_topk(const float* __restrict__ scores, int n_q,
                                                   int n_k, int k, int n_local, int causal,
                                                   int32_t* __restrict__ idx,
                                                   int32_t* __restrict__ count) {
  __shared__ uint64_t keys[kMaxN];
  __shared__ uint8_t flag[kMaxN];
  __shared__ int part[kThreads + 1];

  const int row = blockIdx.x;            // over rows * n_q
  const int i = row % n_q;
  const float* srow = scores + size_t(row) * n_k;
  const int width = k + n_local;
  int last, w0, w1;                      // candidates 0..last, window w0..w1
  if (causal) {
    last = i - n_local;
    w0 = max(0, i - n_local + 1);
    w1 = i;
  } else {
    last = n_k - 1 - n_local;
    w0 = n_k - n_local;
    w1 = n_k - 1;
  }
  const int ncand = max(0, last + 1);
  const int span = max(w1 + 1, ncand);   // flags needed for blocks 0..span-1

  for (int j = threadIdx.x; j < span; j += kThreads)
    flag[j] = (j >= w0 && j <= w1) || (ncand <= k && j < ncand);

  if (ncand > k && k > 0) {
    int P = 1;
    while (P < ncand) P <<= 1;
    for (int j = threadIdx.x; j < P; j += kThreads)
      keys[j] = (j < ncand) ? ((uint64_t(order_bits(srow[j])) << 32) | (0xffffffffu - uint32_t(j)))
                            : 0ull;
    __syncthreads();
    // bitonic sort, descending
    for (int size = 2; size <= P; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = threadIdx.x; t < P / 2; t += kThreads) {
          const int lo = 2 * t - (t & (stride - 1));
          const int hi = lo + stride;
          const bool desc = ((lo & size) == 0);
          const uint64_t a = keys[lo], b = keys[hi];
          if ((a < b) == desc) {
            keys[lo] = b;
            keys[hi] = a;
          }
        }
        __syncthreads();
      }
    }
    for (int t = threadIdx.x; t < k; t += kThreads)
      flag[0xffffffffu - uint32_t(keys[t] & 0xffffffffu)] = 1;
  }
  __syncthreads();

  // ascending compaction of the flagged blocks
  const int chunk = (span + kThreads - 1) / kThreads;
  const int c0 = threadIdx.x * chunk;
  const int c1 = min(span, c0 + chunk);
  int c = 0;
  for (int j = c0; j < c1; ++j) c += flag[j];
  part[threadIdx.x + 1] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    part[0] = 0;
    for (int t = 1; t <= kThreads; ++t) part[t] += part[t - 1];
  }
  __syncthreads();
  int32_t* orow = idx + size_t(row) * width;
  int pos = part[threadIdx.x];
  for (int j = c0; j < c1; ++j)
    if (flag[j]) orow[pos++] = j;
  const int total = part[kThreads];
  for (int t = total + threadIdx.x; t < width; t += kThreads) orow[t] = -1;
  if (threadIdx.x == 0) count[row] = total;
}

}  // namespace

hipError_t launch_topk(const float* scores, int rows, int n_q, int n_k, int k, int n_local,
                       int causal, int32_t* idx, int32_t* count, hipStream_t s) {
  k_topk<<<rows * n_q, kThreads, 0, s>>>(scores, n_q, n_k, k, n_local, causal, idx, count);
  return hipGetLastError();
}

}  // namespace dsa
