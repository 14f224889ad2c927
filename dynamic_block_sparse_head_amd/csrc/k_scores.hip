// Block and page importance scores.
//
//  * Pooled prefill scores ([DMA] §四-§五: an importance score per history
//    position from its content, causal mask before selection; [SA] "策略":
//    blocks as the unit): score[b,g,i,j] = (sum over the group's query
//    heads of the mean query of block i) . (mean key of block j), j <= i.
//    Two kernels: a pooling pass that reads Q and K once (HBM bound) and a
//    small float64 dot-product pass over the pooled vectors.
//  * Page bounds for decode ([SF] §二-§四, page-level selection with the full
//    cache kept): sum over heads and dims of max(q*kmin, q*kmax).
//  * Page min/max metadata: element-wise extremes of each page's keys.
//
// All sums are float64 in a fixed order, so results are deterministic and
// agree with an exact float64 evaluation to ~1e-15 relative.
#include <type_traits>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
typedef float floatx8 __attribute__((ext_vector_type(8)));

// Load 8 consecutive elements as float.
__device__ __forceinline__ void load8(const uint16_t* p, float* f) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16lo(w[e]);
    f[2 * e + 1] = bf16hi(w[e]);
  }
}
__device__ __forceinline__ void load8(const float* p, float* f) {
  const floatx4 a = *reinterpret_cast<const floatx4*>(p);
  const floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = a[e];
    f[4 + e] = b[e];
  }
}

// out[bu, i, :] = sum over hpu heads of mean over the rows of block i.
// grid (nb, B*U, 2) with U = Hq / SH selection units: z = 0 pools the
// queries (the SH heads of each unit summed), z = 1 the keys (one KV head
// per bu < B*Hkv).  Each thread owns 8 columns and a strided set of rows.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_pool(const T* __restrict__ q, const T* __restrict__ k,
                                                   int Hq, int S, int D, int block, int SH, int Hkv,
                                                   double* __restrict__ out_q,
                                                   double* __restrict__ out_k) {
  __shared__ double red[kThreads * 8];
  const bool keys = blockIdx.z != 0;
  const int U = keys ? Hkv : Hq / SH;   // units (keys: KV heads) per sequence
  const int bg = blockIdx.y;
  if (keys && int(bg) >= int(gridDim.y) / (Hq / SH) * Hkv) return;   // whole workgroup
  const T* __restrict__ x = keys ? k : q;
  const int H = keys ? Hkv : Hq;
  const int hpg = keys ? 1 : SH;
  double* __restrict__ out = keys ? out_k : out_q;
  const int i = blockIdx.x;
  const int b = bg / U, g = bg % U;
  const int ncg = D / 8;
  const int nrg = kThreads / ncg;
  const int cg = threadIdx.x % ncg;
  const int rg = threadIdx.x / ncg;
  const int row0 = i * block;
  const int nrows = min(block, S - row0);
  const int R = hpg * nrows;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int r = rg; r < R; r += nrg) {
    const int hh = r / nrows, row = r % nrows;
    const size_t off = ((size_t(b) * H + size_t(g) * hpg + hh) * S + row0 + row) * D + cg * 8;
    float f[8];
    load8(x + off, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += double(f[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg * D + cg * 8 + e] = acc[e];
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += kThreads) {
    double s = 0.0;
    for (int r = 0; r < nrg; ++r) s += red[r * D + d];
    out[(size_t(bg) * gridDim.x + i) * D + d] = s / double(nrows);
  }
}

// scores[bu, i, j] = qs[bu, i, :] . kb[kv(bu), j, :] for j <= i, -inf above
// the diagonal, kv(bu) the KV head of selection unit bu (U units and Hkv KV
// heads per sequence).  32x32 output tile per workgroup; thread (ti, tj)
// owns rows ti, ti+16 and columns tj, tj+16, i.e. four independent float64
// dot products fed from LDS (two query and two key values per step).
template <int D>
__global__ __launch_bounds__(kThreads) void k_pooled_dot(const double* __restrict__ qs,
                                                         const double* __restrict__ kb, int nb,
                                                         int U, int Hkv,
                                                         float* __restrict__ scores) {
  extern __shared__ double lds[];  // [32][D+2] queries, then [32][D+2] keys
  const int bg = blockIdx.z;
  const int kvh = (bg / U) * Hkv + (bg % U) / (U / Hkv);   // its KV head (row of kb)
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  const int ti = threadIdx.x / 16, tj = threadIdx.x % 16;
  float* srow = scores + size_t(bg) * nb * nb;
  if (j0 > i0 + 31) {  // whole tile above the diagonal
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int i = i0 + ti + 16 * r, j = j0 + tj + 16 * c;
        if (i < nb && j < nb) srow[size_t(i) * nb + j] = -__builtin_inff();
      }
    return;
  }
  const int ld = D + 2;  // even: rows stay 16-byte aligned
  double* lq = lds;
  double* lk = lds + 32 * ld;
  // all loads of the two 32-row slabs are issued before any LDS store
  constexpr int hd = D / 2, NPT = 32 * hd / kThreads;
  double2 ra[NPT], rc[NPT];
#pragma unroll
  for (int x = 0; x < NPT; ++x) {
    const int e = threadIdx.x + x * kThreads;
    const int r = e / hd, d = (e % hd) * 2;
    ra[x] = double2{0.0, 0.0};
    rc[x] = double2{0.0, 0.0};
    if (i0 + r < nb) ra[x] = *reinterpret_cast<const double2*>(qs + (size_t(bg) * nb + i0 + r) * D + d);
    if (j0 + r < nb) rc[x] = *reinterpret_cast<const double2*>(kb + (size_t(kvh) * nb + j0 + r) * D + d);
  }
#pragma unroll
  for (int x = 0; x < NPT; ++x) {
    const int e = threadIdx.x + x * kThreads;
    const int r = e / hd, d = (e % hd) * 2;
    *reinterpret_cast<double2*>(lq + r * ld + d) = ra[x];
    *reinterpret_cast<double2*>(lk + r * ld + d) = rc[x];
  }
  __syncthreads();
  const double* q0 = lq + ti * ld;
  const double* q1 = lq + (ti + 16) * ld;
  const double* k0 = lk + tj * ld;
  const double* k1 = lk + (tj + 16) * ld;
  double a00 = 0.0, a01 = 0.0, a10 = 0.0, a11 = 0.0;
  for (int d = 0; d < D; d += 2) {
    const double2 x0 = *reinterpret_cast<const double2*>(q0 + d);
    const double2 x1 = *reinterpret_cast<const double2*>(q1 + d);
    const double2 y0 = *reinterpret_cast<const double2*>(k0 + d);
    const double2 y1 = *reinterpret_cast<const double2*>(k1 + d);
    a00 = __builtin_fma(x0.x, y0.x, a00);
    a01 = __builtin_fma(x0.x, y1.x, a01);
    a10 = __builtin_fma(x1.x, y0.x, a10);
    a11 = __builtin_fma(x1.x, y1.x, a11);
    a00 = __builtin_fma(x0.y, y0.y, a00);
    a01 = __builtin_fma(x0.y, y1.y, a01);
    a10 = __builtin_fma(x1.y, y0.y, a10);
    a11 = __builtin_fma(x1.y, y1.y, a11);
  }
  const double acc[2][2] = {{a00, a01}, {a10, a11}};
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int i = i0 + ti + 16 * r, j = j0 + tj + 16 * c;
      if (i < nb && j < nb) srow[size_t(i) * nb + j] = (j <= i) ? float(acc[r][c]) : -__builtin_inff();
    }
}

// Page bound scores.  Each page is handled by D/8 lanes (8 dims each) and
// each lane covers kPagesPerThread pages, whose bound loads are issued before
// the group's G query vectors are staged in LDS, so the two latencies overlap.
constexpr int kPagesPerThread = 4;

template <typename T>
__global__ __launch_bounds__(kThreads) void k_page_scores(const T* __restrict__ q,
                                                          const T* __restrict__ kmin,
                                                          const T* __restrict__ kmax, int Hq,
                                                          int Hkv, int nP, int D,
                                                          float* __restrict__ scores) {
  extern __shared__ float lq[];  // [G][D]
  const int bg = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv;
  const int lpp = D / 8;                 // lanes per page
  const int ppw = kThreads / lpp;        // pages per workgroup and slot
  const int sub = threadIdx.x % lpp;
  // Raw 16-byte (bf16) or 32-byte (float) chunks, converted when used.
  using Raw = typename std::conditional<sizeof(T) == 2, u32x4, floatx8>::type;
  int pg[kPagesPerThread];
  Raw rlo[kPagesPerThread], rhi[kPagesPerThread];
#pragma unroll
  for (int t = 0; t < kPagesPerThread; ++t) {
    pg[t] = (blockIdx.x * kPagesPerThread + t) * ppw + threadIdx.x / lpp;
    if (pg[t] < nP) {
      const size_t off = (size_t(bg) * nP + pg[t]) * D + sub * 8;
      rlo[t] = *reinterpret_cast<const Raw*>(kmin + off);
      rhi[t] = *reinterpret_cast<const Raw*>(kmax + off);
    }
  }
  for (int e = threadIdx.x; e < G * D; e += kThreads) {
    const size_t off = (size_t(b) * Hq + size_t(g) * G) * D + e;
    if constexpr (sizeof(T) == 2) lq[e] = bf16_to_f32(q[off]);
    else lq[e] = q[off];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < kPagesPerThread; ++t) {
    double acc = 0.0;
    if (pg[t] < nP) {
      float lo[8], hi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (sizeof(T) == 2) {
          lo[e] = (e & 1) ? bf16hi(rlo[t][e / 2]) : bf16lo(rlo[t][e / 2]);
          hi[e] = (e & 1) ? bf16hi(rhi[t][e / 2]) : bf16lo(rhi[t][e / 2]);
        } else {
          lo[e] = rlo[t][e];
          hi[e] = rhi[t][e];
        }
      }
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float qf = lq[h * D + sub * 8 + e];
          if constexpr (sizeof(T) == 2) {
            // bf16 x bf16 fits a float mantissa: products (in float's normal
            // range) and their max are exact in float; only the sum needs
            // float64.
            acc += double(fmaxf(qf * lo[e], qf * hi[e]));
          } else {
            const double qd = double(qf);
            acc += fmax(qd * double(lo[e]), qd * double(hi[e]));
          }
        }
      }
    }
    for (int o = lpp / 2; o > 0; o /= 2) acc += __shfl_xor(acc, o);
    if (pg[t] < nP && sub == 0) scores[size_t(bg) * nP + pg[t]] = float(acc);
  }
}

// bf16 page bound scores for a compile-time group size.  Since kmax >= kmin,
// max(q kmin, q kmax) is q kmax for q >= 0 and q kmin otherwise, so a page's
// score is sum over d of kmax_d P_d + kmin_d N_d with P_d (N_d) the sum of the
// group's non-negative (negative) query components in dimension d.  P and N
// are formed once per lane in float64 (exact for bf16 inputs); each page then
// costs two float64 FMAs per dimension instead of a float64 add per head and
// dimension.  Each workgroup walks kIters slots of pages with the next slot's
// bound loads in flight while the current one is reduced; no LDS, no barrier.
constexpr int kIters = 4;

//
// PAGED: the summaries live in a pool [n_pool, Hkv, D]; logical page p of
// sequence b reads pool page page_table[b][p], and pages at or past
// ceil(seq_len[b] / page) (or naming no pool page) score -inf.
// One float64 lane value moved by a DPP pattern (both halves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(u)), CTRL, 0xF, 0xF, false));
  const uint32_t hi = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(u >> 32)), CTRL, 0xF, 0xF, false));
  return __builtin_bit_cast(double, uint64_t(hi) << 32 | lo);
}

// Sum over the n (8 or 16) lanes of a page (a DPP row group, or half of
// one); every lane gets the total.
__device__ __forceinline__ double page_sum(double x, int n) {
  x += dpp_f64<0xB1>(x);    // lane ^ 1
  x += dpp_f64<0x4E>(x);    // lane ^ 2
  x += dpp_f64<0x141>(x);   // half-row mirror: the other quad of the 8
  if (n == 16) x += dpp_f64<0x140>(x);   // row mirror: the other 8 of the 16
  return x;
}

template <int G, bool PAGED>
__global__ __launch_bounds__(kThreads) void k_page_scores_bf16(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ kmin,
                                                               const uint16_t* __restrict__ kmax,
                                                               int Hq, int Hkv, int nP, int D,
                                                               float* __restrict__ scores,
                                                               PageScoreArgs pa) {
  const int bg = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int npg = PAGED ? min(nP, (pa.seq_len[b] + pa.page - 1) / pa.page) : nP;
  const int lpp = D / 8;
  const int ppw = kThreads / lpp;
  const int sub = threadIdx.x % lpp;
  double pos[8], neg[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) pos[e] = neg[e] = 0.0;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(q + (size_t(b) * Hq + size_t(g) * G + h) * D + sub * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (e & 1) ? bf16hi(w[e / 2]) : bf16lo(w[e / 2]);
      if (x >= 0.f) pos[e] += double(x);
      else neg[e] += double(x);
    }
  }
  u32x4 rlo[2][kPagesPerThread], rhi[2][kPagesPerThread];
  bool live[2][kPagesPerThread];   // the page exists (always, unless PAGED)
  auto page_of = [&](int it, int t) {
    return ((blockIdx.x * kIters + it) * kPagesPerThread + t) * ppw + int(threadIdx.x) / lpp;
  };
  auto load = [&](int it, int buf) {
#pragma unroll
    for (int t = 0; t < kPagesPerThread; ++t) {
      const int p = page_of(it, t);
      live[buf][t] = false;
      if (p < npg) {
        size_t off;
        if constexpr (PAGED) {
          const int phys = pa.page_table[size_t(b) * nP + p];
          if (phys < 0 || phys >= pa.n_pool) continue;
          off = (size_t(phys) * Hkv + g) * D + sub * 8;
        } else {
          off = (size_t(bg) * nP + p) * D + sub * 8;
        }
        live[buf][t] = true;
        // streaming loads: every bound is read once per call
        rlo[buf][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kmin + off));
        rhi[buf][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kmax + off));
      }
    }
  };
  load(0, 0);
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    if (it + 1 < kIters) load(it + 1, (it + 1) & 1);
#pragma unroll
    for (int t = 0; t < kPagesPerThread; ++t) {
      const int p = page_of(it, t);
      double acc = 0.0;
      if (live[it & 1][t]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float lo = (e & 1) ? bf16hi(rlo[it & 1][t][e / 2]) : bf16lo(rlo[it & 1][t][e / 2]);
          const float hi = (e & 1) ? bf16hi(rhi[it & 1][t][e / 2]) : bf16lo(rhi[it & 1][t][e / 2]);
          acc = __builtin_fma(double(hi), pos[e], acc);
          acc = __builtin_fma(double(lo), neg[e], acc);
        }
      }
      acc = page_sum(acc, lpp);
      if (p < nP && sub == 0)
        scores[size_t(bg) * nP + p] = live[it & 1][t] ? float(acc) : -__builtin_inff();
    }
  }
}

// Element-wise min and max over each page.  grid (nP, B*Hkv).
template <typename T>
__global__ __launch_bounds__(kThreads) void k_page_minmax(const T* __restrict__ k, int L, int D,
                                                          int page, T* __restrict__ kmin,
                                                          T* __restrict__ kmax) {
  __shared__ float rmin[kThreads * 8];
  __shared__ float rmax[kThreads * 8];
  const int p = blockIdx.x, bg = blockIdx.y;
  const int nP = L / page;
  const int ncg = D / 8, nrg = kThreads / ncg;
  const int cg = threadIdx.x % ncg, rg = threadIdx.x / ncg;
  float mn[8], mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mn[e] = __builtin_inff();
    mx[e] = -__builtin_inff();
  }
  for (int r = rg; r < page; r += nrg) {
    float f[8];
    load8(k + (size_t(bg) * L + size_t(p) * page + r) * D + cg * 8, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mn[e] = fminf(mn[e], f[e]);
      mx[e] = fmaxf(mx[e], f[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    rmin[rg * D + cg * 8 + e] = mn[e];
    rmax[rg * D + cg * 8 + e] = mx[e];
  }
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float a = __builtin_inff(), c = -__builtin_inff();
    for (int r = 0; r < nrg && r < page; ++r) {
      a = fminf(a, rmin[r * D + d]);
      c = fmaxf(c, rmax[r * D + d]);
    }
    const size_t off = (size_t(bg) * nP + p) * D + d;
    if constexpr (sizeof(T) == 2) {
      kmin[off] = f32_to_bf16(a);   // exact: a is a bf16 value
      kmax[off] = f32_to_bf16(c);
    } else {
      kmin[off] = a;
      kmax[off] = c;
    }
  }
}

}  // namespace

hipError_t launch_pooled_scores(const PoolScoreArgs& a, hipStream_t s) {
  const int nb = (a.S + a.block - 1) / a.block;
  const int U = a.Hq / a.sel_heads;
  dim3 grid(nb, a.B * U, 2);
  if (a.dtype == 1)
    k_pool<uint16_t><<<grid, kThreads, 0, s>>>(static_cast<const uint16_t*>(a.q),
                                               static_cast<const uint16_t*>(a.k), a.Hq, a.S, a.D,
                                               a.block, a.sel_heads, a.Hkv, a.ws_q, a.ws_k);
  else
    k_pool<float><<<grid, kThreads, 0, s>>>(static_cast<const float*>(a.q),
                                            static_cast<const float*>(a.k), a.Hq, a.S, a.D,
                                            a.block, a.sel_heads, a.Hkv, a.ws_q, a.ws_k);
  const int nt = (nb + 31) / 32;
  const size_t lds = size_t(2) * 32 * (a.D + 2) * sizeof(double);
  if (a.D == 128)
    k_pooled_dot<128><<<dim3(nt, nt, a.B * U), kThreads, lds, s>>>(a.ws_q, a.ws_k, nb, U, a.Hkv,
                                                                   a.scores);
  else
    k_pooled_dot<64><<<dim3(nt, nt, a.B * U), kThreads, lds, s>>>(a.ws_q, a.ws_k, nb, U, a.Hkv,
                                                                  a.scores);
  return hipGetLastError();
}

hipError_t launch_page_scores(const PageScoreArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  if (a.dtype == 1 && (G == 1 || G == 2 || G == 4 || G == 8)) {
    const int ppb = kThreads / (a.D / 8) * kPagesPerThread * kIters;
    dim3 grid((a.nP + ppb - 1) / ppb, a.B * a.Hkv);
    const auto* q = static_cast<const uint16_t*>(a.q);
    const auto* lo = static_cast<const uint16_t*>(a.kmin);
    const auto* hi = static_cast<const uint16_t*>(a.kmax);
#define DSA_PS(GG)                                                                          \
  (a.page_table ? k_page_scores_bf16<GG, true><<<grid, kThreads, 0, s>>>(q, lo, hi, a.Hq, a.Hkv, \
                                                                         a.nP, a.D, a.scores, a) \
                : k_page_scores_bf16<GG, false><<<grid, kThreads, 0, s>>>(q, lo, hi, a.Hq, a.Hkv, \
                                                                          a.nP, a.D, a.scores, a))
    switch (G) {
      case 1: DSA_PS(1); break;
      case 2: DSA_PS(2); break;
      case 4: DSA_PS(4); break;
      default: DSA_PS(8); break;
    }
#undef DSA_PS
    return hipGetLastError();
  }
  const int ppb = kThreads / (a.D / 8) * kPagesPerThread;
  dim3 grid((a.nP + ppb - 1) / ppb, a.B * a.Hkv);
  const size_t lds = size_t(a.Hq / a.Hkv) * a.D * sizeof(float);
  if (a.dtype == 1)
    k_page_scores<uint16_t><<<grid, kThreads, lds, s>>>(
        static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.kmin),
        static_cast<const uint16_t*>(a.kmax), a.Hq, a.Hkv, a.nP, a.D, a.scores);
  else
    k_page_scores<float><<<grid, kThreads, lds, s>>>(
        static_cast<const float*>(a.q), static_cast<const float*>(a.kmin),
        static_cast<const float*>(a.kmax), a.Hq, a.Hkv, a.nP, a.D, a.scores);
  return hipGetLastError();
}

hipError_t launch_page_minmax(int dtype, const void* k, int B, int Hkv, int L, int D, int page,
                              void* kmin, void* kmax, hipStream_t s) {
  dim3 grid(L / page, B * Hkv);
  if (dtype == 1)
    k_page_minmax<uint16_t><<<grid, kThreads, 0, s>>>(static_cast<const uint16_t*>(k), L, D, page,
                                                      static_cast<uint16_t*>(kmin),
                                                      static_cast<uint16_t*>(kmax));
  else
    k_page_minmax<float><<<grid, kThreads, 0, s>>>(static_cast<const float*>(k), L, D, page,
                                                   static_cast<float*>(kmin),
                                                   static_cast<float*>(kmax));
  return hipGetLastError();
}

}  // namespace dsa
