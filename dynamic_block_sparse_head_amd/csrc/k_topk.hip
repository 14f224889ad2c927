// Top-k block selection plus the local window ([DMA] §五: after the causal
// mask keep the k highest-weight history positions, everything else -inf).
//
// Rows of up to 2048 candidates use one wave per row (bisection for the k-th
// largest key, see k_topk_wave); longer rows use one workgroup per row.
// Candidates become 64-bit keys
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

// Rows of up to 64*E candidates: one wave per row, no LDS and no barrier.
// Lane l holds candidates l, l+64, ... as the same 64-bit keys.  The k-th
// largest key T is found bit by bit from the top (T grows while at least k
// keys are >= T); keys are unique, so exactly k candidates satisfy key >= T.
// Chosen and window blocks are then compacted in index order with ballots.
template <int E>
__global__ __launch_bounds__(kThreads) void k_topk_wave(const float* __restrict__ scores, int n_rows,
                                                        int n_q, int n_k, int k, int n_local,
                                                        int causal, int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ count) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= n_rows) return;          // the whole wave leaves together
  const int i = row % n_q;
  const float* srow = scores + size_t(row) * n_k;
  const int width = k + n_local;
  int last, w0, w1;
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

  uint64_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = e * 64 + lane;
    key[e] = (j < ncand) ? ((uint64_t(order_bits(srow[j])) << 32) | (0xffffffffu - uint32_t(j))) : 0ull;
  }
  const bool take_all = ncand <= k;
  uint64_t T = 0;
  if (!take_all && k > 0) {
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t cand = T | (1ull << bit);
      int c = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) c += __popcll(__ballot(key[e] >= cand));
      if (c >= k) T = cand;
    }
  }

  int32_t* orow = idx + size_t(row) * width;
  int base = 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = e * 64 + lane;
    const bool sel = j < ncand && (take_all || (k > 0 && key[e] >= T));
    const bool f = sel || (j >= w0 && j <= w1);
    const uint64_t mask = __ballot(f);
    if (f) orow[base + __popcll(mask & below)] = j;
    base += __popcll(mask);
  }
  for (int t = base + lane; t < width; t += 64) orow[t] = -1;
  if (lane == 0) count[row] = base;
}

}  // namespace

hipError_t launch_topk(const float* scores, int rows, int n_q, int n_k, int k, int n_local,
                       int causal, int32_t* idx, int32_t* count, hipStream_t s) {
  const int n_rows = rows * n_q;
  const int grid = (n_rows + kThreads / 64 - 1) / (kThreads / 64);
#define DSA_TOPK_WAVE(E)                                                                    \
  k_topk_wave<E><<<grid, kThreads, 0, s>>>(scores, n_rows, n_q, n_k, k, n_local, causal, idx, \
                                           count)
  if (n_k <= 64) DSA_TOPK_WAVE(1);
  else if (n_k <= 128) DSA_TOPK_WAVE(2);
  else if (n_k <= 256) DSA_TOPK_WAVE(4);
  else if (n_k <= 512) DSA_TOPK_WAVE(8);
  else if (n_k <= 1024) DSA_TOPK_WAVE(16);
  else if (n_k <= 2048) DSA_TOPK_WAVE(32);
  else k_topk<<<n_rows, kThreads, 0, s>>>(scores, n_q, n_k, k, n_local, causal, idx, count);
#undef DSA_TOPK_WAVE
  return hipGetLastError();
}

}  // namespace dsa
