// Top-k block selection plus the local window ([DMA] §五: after the causal
// mask keep the k highest-weight history positions, everything else -inf).
//
// Order: higher score first, equal scores by lower index, NaN below every
// number.  Each score becomes its order-preserving 32-bit pattern (NaN -> 0).
// The k-th largest pattern T is found by bisection from the top bit down
// (T grows while at least k candidates are >= T); the selection is every
// candidate above T plus the lowest-indexed candidates equal to T, as many
// as are still missing.  Counts come from wave ballots, so a row needs no
// sort and no LDS traffic beyond a few counters.  The chosen and the window
// blocks are written in index order, i.e. each output row comes out
// ascending, padded with -1.
//
// Layout: W waves own one row (W = 1: four rows per 256-thread workgroup,
// no barriers), each lane E candidates; candidate j sits in chunk j / 64,
// chunk c = e * W + w held by wave w as element e, so loads are coalesced
// and chunk order is index order.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

__device__ __forceinline__ uint32_t order_bits(float f) {
  if (__builtin_isnan(f)) return 0u;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }

// Sum of a wave-uniform value over the W waves of the row.  `slot` alternates
// between calls so one barrier per call suffices.
template <int W>
__device__ __forceinline__ int row_total(int v, int (*red)[W], int& slot) {
  if constexpr (W == 1) {
    return v;
  } else {
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[slot][w] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) t += red[slot][i];
    slot ^= 1;
    return t;
  }
}

// Exclusive prefix over the row, in index order, of per-chunk counts (mine[e]
// is this wave's count for chunk e * W + w).  Returns the bases of this
// wave's chunks and the row total.
template <int E, int W>
__device__ __forceinline__ int chunk_prefix(const int (&mine)[E], int (&base)[E], int* pre) {
  if constexpr (W == 1) {
    int run = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      base[e] = run;
      run += mine[e];
    }
    return run;
  } else {
    constexpr int NC = E * W;
    constexpr int PER = (NC + 63) / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) {
#pragma unroll
      for (int e = 0; e < E; ++e) pre[e * W + w] = mine[e];
    }
    __syncthreads();
    if (w == 0) {
      int v[PER];
      int s = 0;
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int c = lane * PER + p;
        v[p] = (c < NC) ? pre[c] : 0;
        s += v[p];
      }
      int incl = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      int run = incl - s;
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int c = lane * PER + p;
        if (c < NC) pre[c] = run;
        run += v[p];
      }
      if (lane == 63) pre[NC] = incl;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) base[e] = pre[e * W + w];
    const int total = pre[NC];
    __syncthreads();  // the table is reused by the next call
    return total;
  }
}

template <int E, int W>
__global__ __launch_bounds__(W == 1 ? 256 : 64 * W) void k_topk(
    const float* __restrict__ scores, int n_rows, int n_q, int n_k, int k, int n_local, int causal,
    int row_block, int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  __shared__ int red[2][W];
  __shared__ int pre[E * W + 1];
  const int lane = threadIdx.x & 63;
  const int w = (W == 1) ? 0 : (threadIdx.x >> 6);
  const int row = (W == 1) ? blockIdx.x * 4 + (threadIdx.x >> 6) : blockIdx.x;
  if (row >= n_rows) return;  // W == 1: the whole wave; W > 1: the whole workgroup
  const int i = (row % n_q) / row_block;   // the row's query block
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
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  int jj[E];
  uint32_t bits[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    jj[e] = (e * W + w) * 64 + lane;
    bits[e] = (jj[e] < ncand) ? order_bits(srow[jj[e]]) : 0u;
  }

  int slot = 0;
  bool f[E];
  if (ncand <= k || k == 0) {
    const bool all = k > 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      f[e] = (all && jj[e] < ncand) || (jj[e] >= w0 && jj[e] <= w1);
  } else {
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = T | (1u << bit);
      int n = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) n += popc(__ballot(jj[e] < ncand && bits[e] >= c));
      if (row_total<W>(n, red, slot) >= k) T = c;
    }
    int gt = 0, tc[E], tb[E];
    uint64_t tm[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      gt += popc(__ballot(jj[e] < ncand && bits[e] > T));
      tm[e] = __ballot(jj[e] < ncand && bits[e] == T);
      tc[e] = popc(tm[e]);
    }
    const int need = k - row_total<W>(gt, red, slot);
    chunk_prefix<E, W>(tc, tb, pre);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool valid = jj[e] < ncand;
      const bool tie_in = bits[e] == T && tb[e] + popc(tm[e] & below) < need;
      f[e] = (valid && (bits[e] > T || tie_in)) || (jj[e] >= w0 && jj[e] <= w1);
    }
  }

  uint64_t fm[E];
  int fc[E], fb[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    fm[e] = __ballot(f[e]);
    fc[e] = popc(fm[e]);
  }
  const int total = chunk_prefix<E, W>(fc, fb, pre);
  int32_t* orow = idx + size_t(row) * width;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (f[e]) orow[fb[e] + popc(fm[e] & below)] = jj[e];
  for (int t = total + w * 64 + lane; t < width; t += 64 * W) orow[t] = -1;
  if (w == 0 && lane == 0) count[row] = total;
}

template <int W>
hipError_t launch_w(int E, const float* scores, int n_rows, int n_q, int n_k, int k, int n_local,
                    int causal, int row_block, int32_t* idx, int32_t* count, hipStream_t s) {
  const int threads = (W == 1) ? 256 : 64 * W;
  const int grid = (W == 1) ? (n_rows + 3) / 4 : n_rows;
#define DSA_TOPK(EE)                                                                          \
  k_topk<EE, W><<<grid, threads, 0, s>>>(scores, n_rows, n_q, n_k, k, n_local, causal, \
                                         row_block, idx, count)
  switch (E) {
    case 1: DSA_TOPK(1); break;
    case 2: DSA_TOPK(2); break;
    case 4: DSA_TOPK(4); break;
    case 8: DSA_TOPK(8); break;
    case 16: DSA_TOPK(16); break;
    case 32: DSA_TOPK(32); break;
    default: return hipErrorInvalidValue;
  }
#undef DSA_TOPK
  return hipGetLastError();
}

int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

}  // namespace

// One wave per row when there are enough rows to fill the chip (or the rows
// are short); otherwise eight waves share a row so that few long rows (decode:
// one per sequence and KV head) still spread over many CUs.
hipError_t launch_topk(const float* scores, int rows, int n_q, int n_k, int k, int n_local,
                       int causal, int row_block, int32_t* idx, int32_t* count, hipStream_t s) {
  const int n_rows = rows * n_q;
  if (n_rows == 0) return hipSuccess;
  if ((n_rows >= 512 && n_k <= 2048) || n_k <= 256)
    return launch_w<1>(pow2_at_least((n_k + 63) / 64), scores, n_rows, n_q, n_k, k, n_local,
                       causal, row_block, idx, count, s);
  return launch_w<8>(pow2_at_least((n_k + 511) / 512), scores, n_rows, n_q, n_k, k, n_local,
                     causal, row_block, idx, count, s);
}

}  // namespace dsa
