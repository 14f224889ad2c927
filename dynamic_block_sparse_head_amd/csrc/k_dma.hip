// Value-driven dynamic weights ([DMA] §四-§五): each history position gets a
// weight from its value row alone, delta = exp(A softplus(v . Delta)), per
// KV head; a key block weighs as much as its heaviest position, and the
// block weights are laid out as a causal score matrix so the ordinary top-k
// selection can keep the heaviest blocks of every query block.
//
// One workgroup per (sequence and KV head, key block): D/8 lanes per
// position (16 bytes of v each), a shuffle reduction per position, the
// block maximum through LDS.  float32 arithmetic.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void load8f(const uint16_t* p, float* f) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16lo(w[e]);
    f[2 * e + 1] = bf16hi(w[e]);
  }
}
__device__ __forceinline__ void load8f(const float* p, float* f) {
  const floatx4 a = *reinterpret_cast<const floatx4*>(p);
  const floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = a[e];
    f[4 + e] = b[e];
  }
}

// log(1 + e^x) without overflow
__device__ __forceinline__ float softplus(float x) { return x > 20.f ? x : log1pf(expf(x)); }

template <typename T>
__global__ __launch_bounds__(kThreads) void k_dma_weights(const T* __restrict__ v, int Hkv, int S,
                                                          int D, const float* __restrict__ proj,
                                                          const float* __restrict__ gain, int block,
                                                          int nb, float* __restrict__ weights,
                                                          float* __restrict__ scores) {
  __shared__ float red[kThreads];
  const int j = blockIdx.x, bg = blockIdx.y, g = bg % Hkv;
  const int lpp = D / 8;                       // lanes per position (a power of two <= 16)
  const int ppp = kThreads / lpp;              // positions per pass
  const int sub = threadIdx.x % lpp, slot = threadIdx.x / lpp;
  float pj[8];
  load8f(proj + size_t(g) * D + sub * 8, pj);
  const float A = gain[g];
  const int s0 = j * block, s1 = min(S, s0 + block);
  float mx = -__builtin_inff();
  for (int s = s0 + slot; s < s0 + ((s1 - s0 + ppp - 1) / ppp) * ppp; s += ppp) {
    float dot = 0.f;
    if (s < s1) {
      float x[8];
      load8f(v + (size_t(bg) * S + s) * D + sub * 8, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(x[e], pj[e], dot);
    }
    for (int o = lpp / 2; o > 0; o /= 2) dot += __shfl_xor(dot, o);
    if (s < s1) {
      const float w = expf(A * softplus(dot));
      if (sub == 0) weights[size_t(bg) * S + s] = w;
      mx = fmaxf(mx, w);
    }
  }
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o /= 2) {
    if (int(threadIdx.x) < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
    __syncthreads();
  }
  const float wj = red[0];
  if (scores == nullptr) return;
  float* col = scores + size_t(bg) * nb * nb + j;   // column j of the [nb, nb] matrix
  for (int i = threadIdx.x; i < nb; i += kThreads) col[size_t(i) * nb] = i >= j ? wj : -__builtin_inff();
}

}  // namespace

hipError_t launch_dma_weights(int dtype, const void* v, int B, int Hkv, int S, int D,
                              const float* proj, const float* gain, int block, float* weights,
                              float* block_scores, hipStream_t s) {
  const int nb = (S + block - 1) / block;
  dim3 grid(nb, B * Hkv);
  if (dtype == 1)
    k_dma_weights<uint16_t><<<grid, kThreads, 0, s>>>(static_cast<const uint16_t*>(v), Hkv, S, D,
                                                      proj, gain, block, nb, weights, block_scores);
  else
    k_dma_weights<float><<<grid, kThreads, 0, s>>>(static_cast<const float*>(v), Hkv, S, D, proj,
                                                   gain, block, nb, weights, block_scores);
  return hipGetLastError();
}

}  // namespace dsa
