// Single-query decode attention over selected KV-cache pages.
//
// [SF] §二-§四: a page-level decode method keeps the whole cache and reads
// only the pages it selects; [NSA] §01/§04: decoding re-reads the history
// for every new token and scattered reads are slow, so whole pages are
// streamed with coalesced 16-byte loads.
//
// Work split: every (sequence, KV group) row of selected pages is cut into
// chunks of 512 tokens' worth of pages; one workgroup per chunk computes, for the
// group's G query heads, the chunk's running max, exp-sum and unnormalised
// weighted value sum.  A merge kernel combines the chunks of each
// (sequence, head) in chunk order (deterministic, no atomics).
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxTok = 512;   // tokens per workgroup: 8 pages of 64, 4 of 128, ...

int pages_per_split(int page) { return page >= kMaxTok ? 1 : kMaxTok / page; }

__device__ __forceinline__ void unpack8(const u32x4& w, float* f) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16lo(w[e]);
    f[2 * e + 1] = bf16hi(w[e]);
  }
}

// Sum over the 16 lanes of a DPP row (every lane gets the total).
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // lane ^ 1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // lane ^ 2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)); // half-row mirror
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)); // row mirror
  return x;
}

constexpr int kUnroll = 8;   // token rows in flight per thread

// grid (nsplit, B*Hkv)
template <int D, int G>
__global__ __launch_bounds__(kThreads) void k_decode_split(DecodeArgs a, int nsplit, int ppsplit) {
  constexpr int CPR = D / 8;              // lanes per token row (8 dims each)
  constexpr int TPI = kThreads / CPR;     // tokens per pass
  static_assert(CPR == 16 || CPR == 8, "row reduction assumes 8 or 16 lanes per token");
  __shared__ float sc[G][kMaxTok];
  __shared__ float red[TPI][G][D];
  __shared__ float stat[G][2];

  const int split = blockIdx.x, bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int cnt = min(a.count[bg], a.idx_width);
  const int n_pages = a.L / a.page;
  const int p0 = split * ppsplit;
  const int np = max(0, min(cnt, p0 + ppsplit) - p0);
  const int ntok = np * a.page;
  const int dc = threadIdx.x % CPR, tg = threadIdx.x / CPR;
  const float c = a.scale * kLog2e;

  // K and V of this (sequence, KV head): out-of-range pages read as zeros
  const uint32_t kv_bytes = uint32_t(a.L) * D * 2;
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc(static_cast<const uint16_t*>(a.k) + size_t(bg) * a.L * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs =
      make_rsrc(static_cast<const uint16_t*>(a.v) + size_t(bg) * a.L * D, kv_bytes);
  const int32_t* pages = a.idx + size_t(bg) * a.idx_width + p0;

  float q[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) +
                                                    (size_t(b) * a.Hq + g * G + h) * D + dc * 8);
    unpack8(w, q[h]);
  }
  // byte offset of a token row inside the cache (page validity folded in)
  auto row_off = [&](int tok, bool& ok) -> uint32_t {
    const int pg = tok < ntok ? pages[tok / a.page] : -1;
    ok = pg >= 0 && pg < n_pages;
    return ok ? uint32_t((pg * a.page + tok % a.page) * D + dc * 8) * 2u : 0xffffffffu;
  };

  // scores of every token of the chunk, for every head
  for (int base = 0; base < ntok; base += TPI * kUnroll) {
    u32x4 kw[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t off = row_off(base + u * TPI + tg, ok[u]);
      kw[u] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float kf[8];
      unpack8(kw[u], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(q[h][e], kf[e], s);
        s = (CPR == 16) ? row16_sum(s) : s;
        if (CPR == 8) {
          s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0xB1, 0xF, 0xF, false));
          s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x4E, 0xF, 0xF, false));
          s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x141, 0xF, 0xF, false));
        }
        const int tok = base + u * TPI + tg;
        if (dc == 0 && tok < ntok) sc[h][tok] = ok[u] ? s * c : -__builtin_inff();
      }
    }
  }
  __syncthreads();

  // per-head max and exp-sum (one wave per head, fixed order)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int h = wave; h < G; h += kThreads / 64) {
    float mx = -__builtin_inff();
    for (int t = lane; t < ntok; t += 64) mx = fmaxf(mx, sc[h][t]);
#pragma unroll
    for (int o = 32; o > 0; o /= 2) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float mu = (mx == -__builtin_inff()) ? 0.f : mx;
    float ls = 0.f;
    for (int t = lane; t < ntok; t += 64) {
      const float p = fast_exp2(sc[h][t] - mu);
      sc[h][t] = p;
      ls += p;
    }
#pragma unroll
    for (int o = 32; o > 0; o /= 2) ls += __shfl_xor(ls, o);
    if (lane == 0) {
      stat[h][0] = mx;
      stat[h][1] = ls;
    }
  }
  __syncthreads();

  // weighted value sums
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  for (int base = 0; base < ntok; base += TPI * kUnroll) {
    u32x4 vw[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t off = row_off(base + u * TPI + tg, ok[u]);
      vw[u] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tok = base + u * TPI + tg;
      if (!ok[u]) continue;
      float vf[8];
      unpack8(vw[u], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = sc[h][tok];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tg][h][dc * 8 + e] = acc[h][e];
  __syncthreads();

  for (int e = threadIdx.x; e < G * D; e += kThreads) {
    const int h = e / D, d = e % D;
    float s = 0.f;
    for (int t = 0; t < TPI; ++t) s += red[t][h][d];
    float* part = a.partial + ((size_t(b) * a.Hq + g * G + h) * nsplit + split) * (D + 2);
    part[d] = s;
    if (d == 0) {
      part[D] = ntok > 0 ? stat[h][0] : -__builtin_inff();
      part[D + 1] = ntok > 0 ? stat[h][1] : 0.f;
    }
  }
}

// grid (B*Hq); combine the chunks of one (sequence, head)
template <int D>
__global__ __launch_bounds__(D) void k_decode_merge(const float* __restrict__ partial, int nsplit,
                                                    uint16_t* __restrict__ out) {
  const int bh = blockIdx.x, d = threadIdx.x;
  const float* p = partial + size_t(bh) * nsplit * (D + 2);
  float M = -__builtin_inff();
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, p[s * (D + 2) + D]);
  float L = 0.f, o = 0.f;
  if (M != -__builtin_inff()) {
    for (int s = 0; s < nsplit; ++s) {
      const float w = fast_exp2(p[s * (D + 2) + D] - M);
      L = fmaf(p[s * (D + 2) + D + 1], w, L);
      o = fmaf(p[s * (D + 2) + d], w, o);
    }
  }
  out[size_t(bh) * D + d] = f32_to_bf16(L > 0.f ? o / L : 0.f);
}

template <int D, int G>
hipError_t run(const DecodeArgs& a, hipStream_t s) {
  const int pps = pages_per_split(a.page);
  const int nsplit = (a.idx_width + pps - 1) / pps;
  k_decode_split<D, G><<<dim3(nsplit, a.B * a.Hkv), kThreads, 0, s>>>(a, nsplit, pps);
  k_decode_merge<D><<<a.B * a.Hq, D, 0, s>>>(a.partial, nsplit, static_cast<uint16_t*>(a.out));
  return hipGetLastError();
}

template <int D>
hipError_t run_d(const DecodeArgs& a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return run<D, 1>(a, s);
    case 2: return run<D, 2>(a, s);
    case 4: return run<D, 4>(a, s);
    default: return run<D, 8>(a, s);
  }
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int idx_width, int page, int D) {
  (void)Hkv;
  const int pps = pages_per_split(page);
  const size_t nsplit = (size_t(idx_width) + pps - 1) / pps;
  return size_t(B) * Hq * nsplit * (D + 2) * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  return a.D == 128 ? run_d<128>(a, s) : run_d<64>(a, s);
}

}  // namespace dsa
