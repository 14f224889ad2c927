// Single-query decode attention over selected KV-cache pages.
//
// [SF] §二-§四: a page-level decode method keeps the whole cache and reads
// only the pages it selects; [NSA] §01/§04: decoding re-reads the history
// for every new token and scattered reads are slow, so whole pages are
// streamed with coalesced 16-byte loads.
//
// Work split: every (sequence, KV group) row of selected pages is cut into
// chunks of about 512 tokens' worth of pages; one workgroup per chunk
// computes, for the group's G query heads, the chunk's running max, exp-sum
// and unnormalised weighted value sum.  A merge kernel combines the chunks
// of each (sequence, head) in chunk order (deterministic, no atomics).
#include <mutex>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

// Partial results of dsa_sparse_attn_decode_noalloc: one copy per GPU, held
// until the process ends.  Host code never names it directly (on the host
// the name is only a stand-in for the symbol): decode_scratch() looks up
// each device's address once and kernels receive that address.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

constexpr int kThreads = 256;
constexpr int kMaxTok = 512;   // tokens per workgroup: 8 pages of 64, 4 of 128, ...
constexpr int kBatch = 4;      // token rows per thread per pipeline stage

int pages_per_split(int page) { return page >= kMaxTok ? 1 : kMaxTok / page; }

// Chunks per (sequence, KV head) row of selected pages.  When the rows are
// few enough, just enough chunks (at most one per page) that the grid is
// one round of the chip's concurrent workgroups (256 CUs x 3 at this
// kernel's register use): every workgroup then streams for the whole call
// and starts only once (128K decode: 86 us against 95 us with chunks of
// 512 tokens).  Otherwise chunks of about kMaxTok tokens, with the count
// nudged so the grid fills whole rounds: a partly filled last round would
// leave most CUs idle while its few chunks stream.  The row's pages are
// then spread evenly over its chunks.
constexpr int kSlots = 256 * 3;
int split_count(int rows, int idx_width, int page) {
  if (rows * 2 <= kSlots) return max(1, min(idx_width, (kSlots + rows - 1) / rows));
  const int pps = pages_per_split(page);
  const int base = (idx_width + pps - 1) / pps;
  int best = base;
  long long best_cost = -1;
  for (int n = max(1, base - base / 4); n <= base + base / 4 + 1; ++n) {
    const long long rounds = (static_cast<long long>(rows) * n + kSlots - 1) / kSlots;
    const long long cost = rounds * ((idx_width + n - 1) / n);   // rounds x pages per chunk
    if (best_cost < 0 || cost < best_cost) {
      best = n;
      best_cost = cost;
    }
  }
  return best;
}

__device__ __forceinline__ void unpack8(const u32x4& w, float* f) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16lo(w[e]);
    f[2 * e + 1] = bf16hi(w[e]);
  }
}

// Sum over the N (8 or 16) lanes of a DPP row group; every lane gets the total.
template <int N>
__device__ __forceinline__ float row_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // lane ^ 1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // lane ^ 2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)); // half-row mirror
  if (N == 16)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)); // row mirror
  return x;
}

// DPP within a row of 16 lanes: lane r reads lane r ^ 8, the lane mirrored
// in its half row (bits 0-2 flipped), in its quad (bits 0-1 flipped), r ^ 1,
// r - 4 and r - 8 (rotations), or lane n (broadcast)
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppRor8 = 0x128, kDppRor4 = 0x124, kDppRor12 = 0x12C, kDppHalfMirror = 0x141,
              kDppQuadRev = 0x1B, kDppQuadSwap = 0xB1, kDppBcast0 = 0x150;
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(x), CTRL, 0xF, 0xF, false));
}

// One stage of a reduce-scatter over the lanes of a row: the lane keeps the
// N values whose index bit matches `bit` (its own lane bit) and adds the
// partner's copies of them; it sends the other N.  x[0..2N) -> y[0..N).
template <int N, int CTRL>
__device__ __forceinline__ void scatter_stage(const float* x, float* y, bool bit) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const float send = bit ? x[j] : x[j + N];
    const float keep = bit ? x[j + N] : x[j];
    y[j] = keep + dpp<CTRL>(send);
  }
}

// grid (nsplit, B*Hkv).  PAGED: the cache is a pool [P, Hkv, PAGE, D]
// shared by the batch, logical page p of sequence b lives in pool page
// page_table[b][p], and only tokens below seq_len[b] exist (rows past it,
// pages past it and pool ids out of range score -inf with zero values).
// The chunk's tokens are walked in slabs of
// kBatch * NG consecutive tokens; group tg of D/8 lanes takes rows
// tg, tg + NG, ... of each slab, with an online softmax.  Page numbers are
// uniform per row of a slab (pages are whole multiples of NG tokens), so
// every load is a buffer load with a per-thread constant offset plus a
// scalar row offset; the next slab's K and V are in flight while the
// current one is used.  The NG group partials are merged in LDS in order.
template <int D, int G, int PAGE, bool PAGED>
__global__ __launch_bounds__(kThreads) void k_decode_split(DecodeArgs a, int nsplit) {
  constexpr int CPR = D / 8;              // lanes per token row (8 dims each)
  constexpr int NG = kThreads / CPR;      // token groups
  constexpr int SLAB = kBatch * NG;       // tokens per pipeline stage
  static_assert(CPR == 16 || CPR == 8, "row reduction assumes 8 or 16 lanes per token");
  static_assert(PAGE % NG == 0, "a page holds whole rows of token groups");
  __shared__ float g_m[NG][G], g_l[NG][G];
  __shared__ float g_acc[NG][G][D];

  const int split = blockIdx.x, bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int cnt = min(a.count[bg], a.idx_width);
  const int len = PAGED ? a.seq_len[b] : a.L;        // tokens in this sequence's cache
  const int n_pages = (len + PAGE - 1) / PAGE;
  const int p0 = int((static_cast<long long>(split) * max(cnt, 0)) / nsplit);
  const int np = int((static_cast<long long>(split + 1) * max(cnt, 0)) / nsplit) - p0;
  const int ntok = np * PAGE;
  const int dc = threadIdx.x % CPR, tg = threadIdx.x / CPR;
  const float c = a.scale * kLog2e;
  const int32_t* pages = a.idx + size_t(bg) * a.idx_width + p0;

  // K and V of this (sequence, KV head); a missing token reads zeros
  const uint32_t kv_bytes = PAGED ? 0u : uint32_t(a.L) * D * 2;
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc(static_cast<const uint16_t*>(a.k) + size_t(bg) * a.L * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs =
      make_rsrc(static_cast<const uint16_t*>(a.v) + size_t(bg) * a.L * D, kv_bytes);
  const uint32_t lane_off = uint32_t(tg * D + dc * 8) * 2u;

  // this lane's 8 dimensions of the query rows, as bf16 pairs: a score is
  // four bf16 pair products (v_dot2, exact products, float32 sums) per lane,
  // summed over the row's lanes, times scale*log2(e) (scores in log2 units)
  u32x4 q[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    q[h] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) +
                                           (size_t(b) * a.Hq + g * G + h) * D + dc * 8);

  // scalar byte offset of row block u of slab sl (0xffffffff: absent, reads zeros)
  auto row_base = [&](int sl, int u) -> uint32_t {
    const int t = sl * SLAB + u * NG;               // first token of this row block
    if (t >= ntok) return 0xffffffffu;
    const int pg = pages[t / PAGE];
    if (pg < 0 || pg >= n_pages) return 0xffffffffu;
    return uint32_t(pg * PAGE + t % PAGE) * uint32_t(D * 2);
  };
  // PAGED: first element of row block u of slab sl in the pool (null: absent)
  // and the logical position of its first row
  const uint16_t* kpool = static_cast<const uint16_t*>(a.k);
  const uint16_t* vpool = static_cast<const uint16_t*>(a.v);
  auto pool_row = [&](int sl, int u, int& tok0) -> size_t {
    const int t = sl * SLAB + u * NG;
    tok0 = 0x7fffffff;
    if (t >= ntok) return ~size_t(0);
    const int pg = pages[t / PAGE];
    if (pg < 0 || pg >= n_pages) return ~size_t(0);
    const int phys = a.page_table[size_t(b) * a.max_pages + pg];
    if (phys < 0 || phys >= a.n_pool) return ~size_t(0);
    tok0 = pg * PAGE + t % PAGE;
    return ((size_t(phys) * a.Hkv + g) * PAGE + t % PAGE) * D;
  };

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -__builtin_inff();
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  struct Batch {
    u32x4 k[kBatch], v[kBatch];
    uint32_t base[kBatch];   // contiguous: row offset; PAGED: 1 if this lane's row exists
  };
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  auto fetch = [&](int sl, Batch& bt) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if constexpr (PAGED) {
        int tok0;
        const size_t e = pool_row(sl, u, tok0);
        const bool ok = e != ~size_t(0) && tok0 + tg < len;   // the row exists and is written
        const size_t off = ok ? e + tg * D + dc * 8 : 0;
        bt.base[u] = ok ? 1u : 0xffffffffu;
        // streaming loads, as below (a buffer descriptor cannot span a pool
        // of 4 GiB or more, so these are global loads)
        bt.k[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kpool + off));
        bt.v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vpool + off));
      } else {
        bt.base[u] = row_base(sl, u);
        // streaming loads (nt): the pages are read once per call; measured
        // 87 -> 78 us on the 128K decode against cached loads
        bt.k[u] = __builtin_amdgcn_raw_buffer_load_b128(krs, lane_off, bt.base[u], 2);
        bt.v[u] = __builtin_amdgcn_raw_buffer_load_b128(vrs, lane_off, bt.base[u], 2);
      }
    }
  };
  // D = 128 with 4 heads per group: a row of 16 lanes holds kBatch = 4
  // tokens x 4 heads = 16 (token, head) pairs, pair j = 4 u + h.  Each lane's
  // 16 partial dot products are reduce-scattered over the row (four DPP
  // stages, 15 adds in all instead of 64 for a reduction to every lane), so
  // lane r owns pair r: one score, one exponential and one row-sum term per
  // lane; the heads' maxima and the 16 probabilities reach every lane of the
  // row by DPP broadcasts.  lp: this lane's share of its head's row sum.
  constexpr bool kPairs = (CPR == 16 && G == 4 && kBatch == 4);
  const int hr = dc & 3;   // (kPairs) the head of this lane's pair
  float lp = 0.f;
  auto consume_pairs = [&](const Batch& bt) {
    if constexpr (kPairs) {
      float part[16];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const bf16x8 kv = __builtin_bit_cast(bf16x8, bt.k[u]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const bf16x8 qv = __builtin_bit_cast(bf16x8, q[h]);
          float s = 0.f;
          s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(qv, qv, 0, 1), __builtin_shufflevector(kv, kv, 0, 1), s, false);
          s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(qv, qv, 2, 3), __builtin_shufflevector(kv, kv, 2, 3), s, false);
          s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(qv, qv, 4, 5), __builtin_shufflevector(kv, kv, 4, 5), s, false);
          s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(qv, qv, 6, 7), __builtin_shufflevector(kv, kv, 6, 7), s, false);
          part[u * 4 + h] = s;
        }
      }
      float w8[8], w4[4], w2[2], w1[1];
      scatter_stage<8, kDppRor8>(part, w8, dc & 8);
      scatter_stage<4, kDppHalfMirror>(w8, w4, dc & 4);
      scatter_stage<2, kDppQuadRev>(w4, w2, dc & 2);
      scatter_stage<1, kDppQuadSwap>(w2, w1, dc & 1);
      bool ok = false;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) ok = (dc >> 2) == u ? bt.base[u] != 0xffffffffu : ok;
      const float sc = ok ? w1[0] * c : -__builtin_inff();
      // the head's maximum over the 4 tokens, then every head's on every lane
      float mx = fmaxf(sc, dpp<kDppRor8>(sc));
      mx = fmaxf(mx, dpp<kDppRor4>(mx));
      float mt[G];
      mt[0] = dpp<kDppBcast0 + 0>(mx);
      mt[1] = dpp<kDppBcast0 + 1>(mx);
      mt[2] = dpp<kDppBcast0 + 2>(mx);
      mt[3] = dpp<kDppBcast0 + 3>(mx);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (mt[h] > m[h]) {   // uniform across the lanes of a token group
          const float alpha = fast_exp2(m[h] - mt[h]);
          lp = hr == h ? lp * alpha : lp;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
          m[h] = mt[h];
        }
      }
      float mh = m[0];
#pragma unroll
      for (int h = 1; h < G; ++h) mh = hr == h ? m[h] : mh;
      const float p = fast_exp2(sc - (mh == -__builtin_inff() ? 0.f : mh));
      lp += p;
      // P.V over token pairs (0, 1) and (2, 3): the probabilities rounded to
      // bf16 (as the prefill kernels feed P to the matrix core), one v_dot2 per
      // (token pair, head, dimension) on the bf16 pairs of the two tokens'
      // values (exact products, float32 sums).  Lane 8 up + h packs its
      // probability with lane 8 up + 4 + h's (token 2 up + 1, same head), and
      // the 8 pairs reach every lane of the row.
      const uint32_t pk = pack_bf16x2(p, dpp<kDppRor12>(p));
      uint32_t pkj[8];
#define DSA_BCAST(UP, H) pkj[4 * UP + H] = dpp_u<kDppBcast0 + 8 * UP + H>(pk);
      DSA_BCAST(0, 0) DSA_BCAST(0, 1) DSA_BCAST(0, 2) DSA_BCAST(0, 3)
      DSA_BCAST(1, 0) DSA_BCAST(1, 1) DSA_BCAST(1, 2) DSA_BCAST(1, 3)
#undef DSA_BCAST
#pragma unroll
      for (int up = 0; up < 2; ++up) {
        const u32x4 va = PAGED && bt.base[2 * up] == 0xffffffffu ? zero4 : bt.v[2 * up];
        const u32x4 vb = PAGED && bt.base[2 * up + 1] == 0xffffffffu ? zero4 : bt.v[2 * up + 1];
        uint32_t vv[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          vv[2 * w] = __builtin_amdgcn_perm(vb[w], va[w], 0x05040100u);       // low halves
          vv[2 * w + 1] = __builtin_amdgcn_perm(vb[w], va[w], 0x07060302u);   // high halves
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const bf16x2 pp = __builtin_bit_cast(bf16x2, pkj[4 * up + h]);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc[h][e] = __builtin_amdgcn_fdot2_f32_bf16(pp, __builtin_bit_cast(bf16x2, vv[e]), acc[h][e], false);
        }
      }
    }
  };
  auto consume = [&](const Batch& bt) {
    if constexpr (kPairs) {
      consume_pairs(bt);
      return;
    }
    float sc[kBatch][G];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bool ok = bt.base[u] != 0xffffffffu;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        // (pairs taken with shufflevector: a bit_cast of a vector element
        // subscript here compiled to element 0 for every e)
        const bf16x8 qv = __builtin_bit_cast(bf16x8, q[h]), kv = __builtin_bit_cast(bf16x8, bt.k[u]);
        float s = 0.f;
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(qv, qv, 0, 1), __builtin_shufflevector(kv, kv, 0, 1), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(qv, qv, 2, 3), __builtin_shufflevector(kv, kv, 2, 3), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(qv, qv, 4, 5), __builtin_shufflevector(kv, kv, 4, 5), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(qv, qv, 6, 7), __builtin_shufflevector(kv, kv, 6, 7), s, false);
        s = row_sum<CPR>(s) * c;
        sc[u][h] = ok ? s : -__builtin_inff();
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mt = sc[0][h];
#pragma unroll
      for (int u = 1; u < kBatch; ++u) mt = fmaxf(mt, sc[u][h]);
      if (mt > m[h]) {   // uniform across the lanes of a token group
        const float alpha = fast_exp2(m[h] - mt);
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
        m[h] = mt;
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      float vf[8];
      // a missing row contributes nothing: its (pool) values may be anything
      unpack8(PAGED && bt.base[u] == 0xffffffffu ? zero4 : bt.v[u], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = fast_exp2(sc[u][h] - (m[h] == -__builtin_inff() ? 0.f : m[h]));
        l[h] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
      }
    }
  };

  const int nslab = (ntok + SLAB - 1) / SLAB;
  Batch A, B;
  if (nslab > 0) fetch(0, A);
  for (int sl = 0; sl < nslab; sl += 2) {
    if (sl + 1 < nslab) fetch(sl + 1, B);
    consume(A);
    if (sl + 1 >= nslab) break;
    if (sl + 2 < nslab) fetch(sl + 2, A);
    consume(B);
  }

  if constexpr (kPairs) {
    // each head's row sum: the shares of the 4 lanes holding its pairs
    float x = lp + dpp<kDppRor8>(lp);
    x += dpp<kDppRor4>(x);
    l[0] = dpp<kDppBcast0 + 0>(x);
    l[1] = dpp<kDppBcast0 + 1>(x);
    l[2] = dpp<kDppBcast0 + 2>(x);
    l[3] = dpp<kDppBcast0 + 3>(x);
  }
  if (dc == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      g_m[tg][h] = m[h];
      g_l[tg][h] = l[h];
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) g_acc[tg][h][dc * 8 + e] = acc[h][e];
  __syncthreads();

  for (int e = threadIdx.x; e < G * D; e += kThreads) {
    const int h = e / D, d = e % D;
    float M = -__builtin_inff();
    for (int t = 0; t < NG; ++t) M = fmaxf(M, g_m[t][h]);
    float Ls = 0.f, O = 0.f;
    if (M != -__builtin_inff()) {
      for (int t = 0; t < NG; ++t) {
        const float w = fast_exp2(g_m[t][h] - M);
        Ls = fmaf(g_l[t][h], w, Ls);
        O = fmaf(g_acc[t][h][d], w, O);
      }
    }
    float* part = a.partial + ((size_t(b) * a.Hq + g * G + h) * nsplit + split) * (D + 2);
    part[d] = O;
    if (d == 0) {
      part[D] = M;
      part[D + 1] = Ls;
    }
  }
}

// grid (B*Hq); combine the chunks of one (sequence, head) in chunk order
template <int D>
__global__ __launch_bounds__(D) void k_decode_merge(const float* __restrict__ partial, int nsplit,
                                                    uint16_t* __restrict__ out) {
  const int bh = blockIdx.x, d = threadIdx.x;
  const float* p = partial + size_t(bh) * nsplit * (D + 2);
  float M = -__builtin_inff(), L = 0.f, O = 0.f;
  // Splits are read eight at a time so their loads overlap; the combine
  // still runs in split order.
  constexpr int kChunk = 8;
  for (int s0 = 0; s0 < nsplit; s0 += kChunk) {
    float ms[kChunk], ls[kChunk], os[kChunk];
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int s = s0 + c;
      ms[c] = -__builtin_inff();
      ls[c] = os[c] = 0.f;
      if (s < nsplit) {
        ms[c] = p[s * (D + 2) + D];
        ls[c] = p[s * (D + 2) + D + 1];
        os[c] = p[s * (D + 2) + d];
      }
    }
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      if (ms[c] == -__builtin_inff()) continue;        // empty chunk or past the end
      const float mn = fmaxf(M, ms[c]);
      const float wo = fast_exp2(M - mn), ws = fast_exp2(ms[c] - mn);   // M = -inf gives wo = 0
      L = L * wo + ls[c] * ws;
      O = O * wo + os[c] * ws;
      M = mn;
    }
  }
  out[size_t(bh) * D + d] = f32_to_bf16(L > 0.f ? O / L : 0.f);
}

template <int D, int G, int PAGE>
hipError_t run(const DecodeArgs& a, hipStream_t s) {
  const int nsplit = split_count(a.B * a.Hkv, a.idx_width, PAGE);
  if (a.page_table)
    k_decode_split<D, G, PAGE, true><<<dim3(nsplit, a.B * a.Hkv), kThreads, 0, s>>>(a, nsplit);
  else
    k_decode_split<D, G, PAGE, false><<<dim3(nsplit, a.B * a.Hkv), kThreads, 0, s>>>(a, nsplit);
  k_decode_merge<D><<<a.B * a.Hq, D, 0, s>>>(a.partial, nsplit, static_cast<uint16_t*>(a.out));
  return hipGetLastError();
}

template <int D, int G>
hipError_t run_p(const DecodeArgs& a, hipStream_t s) {
  switch (a.page) {
    case 32: return run<D, G, 32>(a, s);
    case 64: return run<D, G, 64>(a, s);
    case 128: return run<D, G, 128>(a, s);
    case 256: return run<D, G, 256>(a, s);
    default: return run<D, G, 512>(a, s);
  }
}

template <int D>
hipError_t run_d(const DecodeArgs& a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return run_p<D, 1>(a, s);
    case 2: return run_p<D, 2>(a, s);
    case 4: return run_p<D, 4>(a, s);
    default: return run_p<D, 8>(a, s);
  }
}

// Append one token per sequence to a paged cache: grid B.  Token
// t = seq_len[b] goes to row t % page of pool page page_table[b][t / page];
// its key is folded into that page's element-wise min/max (the page's first
// token sets them); then seq_len[b] = t + 1.  A sequence whose page slot or
// pool id is out of range is left unchanged.
__global__ __launch_bounds__(kThreads) void k_paged_append(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, int Hkv, int D,
    int page, int max_pages, const int32_t* __restrict__ page_table, int32_t* seq_len, int n_pool,
    uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool, uint16_t* __restrict__ kmin,
    uint16_t* __restrict__ kmax) {
  const int b = blockIdx.x;
  const int t = seq_len[b];
  const int p = t / page, r = t % page;
  const bool ok = t >= 0 && p < max_pages;
  const int phys = ok ? page_table[size_t(b) * max_pages + p] : -1;
  if (phys < 0 || phys >= n_pool) return;   // whole workgroup
  for (int e = threadIdx.x; e < Hkv * D; e += kThreads) {
    const int g = e / D, d = e % D;
    const uint16_t kb = k_new[(size_t(b) * Hkv + g) * D + d];
    const size_t row = ((size_t(phys) * Hkv + g) * page + r) * D + d;
    k_pool[row] = kb;
    v_pool[row] = v_new[(size_t(b) * Hkv + g) * D + d];
    const size_t m = (size_t(phys) * Hkv + g) * D + d;
    if (r == 0) {
      kmin[m] = kb;
      kmax[m] = kb;
    } else {
      const float x = bf16_to_f32(kb);
      if (x < bf16_to_f32(kmin[m])) kmin[m] = kb;
      if (x > bf16_to_f32(kmax[m])) kmax[m] = kb;
    }
  }
  __syncthreads();   // every thread has read seq_len[b]
  if (threadIdx.x == 0) seq_len[b] = t + 1;
}

}  // namespace

hipError_t launch_paged_append(const void* k_new, const void* v_new, int B, int Hkv, int D,
                               int page, int max_pages, const int32_t* page_table,
                               int32_t* seq_len, int n_pool, void* k_pool, void* v_pool,
                               void* kmin, void* kmax, hipStream_t s) {
  k_paged_append<<<B, kThreads, 0, s>>>(
      static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), Hkv, D, page,
      max_pages, page_table, seq_len, n_pool, static_cast<uint16_t*>(k_pool),
      static_cast<uint16_t*>(v_pool), static_cast<uint16_t*>(kmin), static_cast<uint16_t*>(kmax));
  return hipGetLastError();
}

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int idx_width, int page, int D) {
  const size_t nsplit = split_count(B * Hkv, idx_width, page);
  return size_t(B) * Hq * nsplit * (D + 2) * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  return a.D == 128 ? run_d<128>(a, s) : run_d<64>(a, s);
}

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace dsa
