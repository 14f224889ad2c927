// Three-branch attention support kernels ([NSA] §03: a compressed branch
// that scans summaries of the history, a selected branch over important
// blocks, a sliding branch, fused per token by gates).
//
//  * k_compress: summaries = plain means of `len` keys (values) every
//    `stride` tokens, rounded once to bf16.
//  * k_cmp_block_scores: second pass of the compressed branch.  With the
//    branch's log-sum-exp known, it recomputes each row's probabilities over
//    the summaries (bf16 MFMA), sums them over the rows and heads of a query
//    block, and spreads each summary's mass over the key blocks it overlaps
//    in proportion to the overlap: the importance that ranks blocks for the
//    selected branch.  One workgroup per (group, query block), so the
//    reduction order is fixed.
//  * k_cmp_token_scores: the same probabilities kept per query token (summed
//    over the group's heads only): per-token selection scores.
//  * k_combine: out = sum over branches of sigmoid(gate logit) * branch output.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

// grid (ceil(n_cmp*D/8 / 256), B*Hkv, 2).  Sums in float64 (exact for
// bf16 inputs of any realistic spread), one division, one rounding to bf16.
__global__ __launch_bounds__(256) void k_compress(const uint16_t* __restrict__ k,
                                                  const uint16_t* __restrict__ v, int S, int D,
                                                  int len, int stride, int n_cmp,
                                                  uint16_t* __restrict__ ck,
                                                  uint16_t* __restrict__ cv) {
  const int cpr = D / 8;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= n_cmp * cpr) return;
  const int cidx = e / cpr, dc = e % cpr;
  const int bg = blockIdx.y;
  const uint16_t* src = (blockIdx.z == 0 ? k : v) + (size_t(bg) * S + size_t(cidx) * stride) * D + dc * 8;
  double acc[8] = {0., 0., 0., 0., 0., 0., 0., 0.};
  for (int r = 0; r < len; ++r) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(src + size_t(r) * D);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      acc[2 * x] += double(bf16lo(w[x]));
      acc[2 * x + 1] += double(bf16hi(w[x]));
    }
  }
  const double n = double(len);
  u32x4 o;
#pragma unroll
  for (int x = 0; x < 4; ++x)
    o[x] = uint32_t(f64_to_bf16(acc[2 * x] / n)) | (uint32_t(f64_to_bf16(acc[2 * x + 1] / n)) << 16);
  uint16_t* dst = (blockIdx.z == 0 ? ck : cv) + (size_t(bg) * n_cmp + cidx) * D + dc * 8;
  *reinterpret_cast<u32x4*>(dst) = o;
}

// x of lane l % 32 plus x of lane 32 + l % 32, on every lane
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr int kNW = 4;      // waves per workgroup of the per-token kernel

// Block-score kernel shape: NW waves of QT 32-row tiles each (the query
// rows a workgroup holds at once: one chunk of its group's rows).
constexpr int kBsNW = 8;
constexpr int kBsQT = 1;

// grid (B*Hkv*nqb), NW*64 threads; dynamic LDS: colsum[n_cmp] floats.
// Every summary tile's per-wave column sums meet in a small exchange buffer;
// one wave (rotating with the tile) adds them, in wave order, into colsum, so
// the reduction order is fixed.
template <int D, int NW, int QT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4 / QT, 4 / QT)))
void k_cmp_block_scores(CmpScoreArgs a, int nqb) {
  constexpr int ROWS = NW * 32 * QT;                         // rows per chunk
  constexpr int CSTR = D + 8;
  constexpr int CPR = D / 8;                                  // 16-byte chunks per summary
  constexpr int CPT = (32 * CPR + NW * 64 - 1) / (NW * 64);   // chunks per thread per tile
  constexpr int NP = QT * D / 16;                             // products per wave per tile
  constexpr int NE = QT * 16;                                 // scores per lane per tile
  constexpr int EPS = (NE + NP - 1) / NP;                     // exponentials per product
  __shared__ __attribute__((aligned(16))) uint16_t c_lds[2][32 * CSTR];
  __shared__ float xsum[2][NW][32];
  extern __shared__ float colsum[];

  // later query blocks see more summaries: start them first
  const int bg = blockIdx.x / nqb, i = nqb - 1 - int(blockIdx.x % nqb);
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int sb = a.sel_block;
  const int t0 = i * sb, t1 = min(a.S, t0 + sb) - 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const float c = a.scale * kLog2e;

  for (int x = threadIdx.x; x < a.n_cmp; x += NW * 64) colsum[x] = 0.f;

  int c_hi = -1;
  if (t1 >= a.len - 1) c_hi = min(a.n_cmp - 1, (t1 - (a.len - 1)) / a.stride);
  const int nkt = c_hi < 0 ? 0 : c_hi / 32 + 1;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(static_cast<const uint16_t*>(a.ck) + size_t(bg) * a.n_cmp * D,
                                               uint32_t(a.n_cmp) * D * 2);
  const uint16_t* qp = static_cast<const uint16_t*>(a.q);

  // summary tile staging: global -> registers two tiles ahead -> LDS
  u32x4 st[CPT];
  auto load = [&](int kt) {
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      const int e = threadIdx.x + cc * NW * 64;
      if (e < 32 * CPR)   // past n_cmp the buffer range check returns zeros
        st[cc] = __builtin_amdgcn_raw_buffer_load_b128(crs, uint32_t(((kt * 32 + e / CPR) * D + (e % CPR) * 8) * 2), 0, 0);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      const int e = threadIdx.x + cc * NW * 64;
      if (e < 32 * CPR) *reinterpret_cast<u32x4*>(&c_lds[buf][(e / CPR) * CSTR + (e % CPR) * 8]) = st[cc];
    }
  };
  // the column sums of tile kt (parked by every wave before the last
  // barrier) into colsum, by wave kt % NW
  auto flush = [&](int kt) __attribute__((always_inline)) {
    const int cs = kt * 32 + col;
    if (wave == kt % NW && half == 0 && cs < a.n_cmp) {
      float t = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) t += xsum[kt & 1][w2][col];
      colsum[cs] += t;
    }
  };

  const int total_rows = G * sb;
  const int nchunks = (total_rows + ROWS - 1) / ROWS;
  for (int chunk = 0; chunk < nchunks; ++chunk) {
    // this wave's query rows, their Q operands and base-2 log-sum-exp.  A
    // 32-row tile lies in one head (sel_block is a multiple of 32), so the
    // token of accumulator row (rr/4)*8 + half*4 + rr%4 is tbase + (rr/4)*8
    // + rr%4: the visibility test needs no per-row table
    bf16x8 qf[QT][D / 16];
    float lse2[QT][16];
    int tbase[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int r = chunk * ROWS + wave * 32 * QT + qt * 32 + col;
      const int hh = r / sb;
      const int t = t0 + r % sb;
      const bool ok = hh < G && t <= t1;
      const uint16_t* src = qp + ((size_t(b) * a.Hq + g * G + (ok ? hh : 0)) * a.S + (ok ? t : t0)) * D + half * 8;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(src + ks * 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[qt][ks][e] = ok ? v[e] : static_cast<__bf16>(0.0f);
      }
      // rows of the accumulator tile held by this lane: (rr/4)*8 + half*4 + rr%4
      const int rbase = chunk * ROWS + wave * 32 * QT + qt * 32;
      tbase[qt] = t0 + rbase % sb + half * 4;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int r2 = rbase + (rr >> 2) * 8 + half * 4 + (rr & 3);
        const int h2 = r2 / sb, tt = t0 + r2 % sb;
        const bool ok2 = h2 < G && tt <= t1;
        const float l2 = ok2 ? a.lse[(size_t(b) * a.Hq + g * G + h2) * a.S + tt] * kLog2e : 0.f;
        // rows outside the block get +inf (probability 0 everywhere); rows
        // that see no summary have lse -inf and are cut by the visibility test
        lse2[qt][rr] = !ok2 ? __builtin_inff() : (l2 == -__builtin_inff() ? 0.f : l2);
      }
    }

    // Tiles whose summaries all end at or before the block's first token
    // (every row sees them) form a prefix, tiles [0, nfull); they run as a
    // software pipeline: while the exponentials of tile kt run, the products
    // of tile kt + 1 are issued (in an order fixed by scheduling barriers)
    // and tile kt + 2 is on its way from memory.  The remaining (diagonal)
    // tiles, one or two per row chunk, run one at a time with the
    // visibility test as the first product's accumulator (-inf where a row
    // cannot see the summary, so the exponential of a hidden pair is 0 with
    // no per-score select).
    int nfull = 0;
    if (t0 - a.len + 1 >= 0) {
      const int m = (t0 - a.len + 1) / a.stride;   // summaries 0..m end at or before t0
      nfull = m >= 31 ? min(nkt, (m - 31) / 32 + 1) : 0;
    }
    float pp[4];
    auto park = [&](int kt) __attribute__((always_inline)) {
      // lane holds summary kt*32+col for 16 rows of each row tile
      const float part = sum_halves((pp[0] + pp[1]) + (pp[2] + pp[3]));
      if (half == 0) xsum[kt & 1][wave][col] = part;
    };
    // exponentials of cur into pp; with NXT, the products of the tile in LDS
    // buffer buf into nxt (zero accumulator) between them
    auto step = [&](auto NXT, int buf, floatx16 (&cur)[QT], floatx16 (&nxt)[QT])
        __attribute__((always_inline)) {
      constexpr bool kNxt = decltype(NXT)::value;
      const uint16_t* cl = &c_lds[buf][col * CSTR + half * 8];
      bf16x8 cb[2];
      if constexpr (kNxt) cb[0] = *reinterpret_cast<const bf16x8*>(cl);
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        if constexpr (kNxt) {
          const int ks = j / QT, qt = j % QT;
          if (qt == 0 && ks + 1 < D / 16) cb[(ks + 1) & 1] = *reinterpret_cast<const bf16x8*>(cl + (ks + 1) * 16);
          nxt[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[qt][ks], cb[ks & 1], ks == 0 ? floatx16{} : nxt[qt],
                                                             0, 0, 0);
        }
#pragma unroll
        for (int e = EPS * j; e < EPS * j + EPS; ++e) {
          if (e < NE) {
            const int qt = e >> 4, rr = e & 15;
            const float p = fast_exp2(fmaf(cur[qt][rr], c, -lse2[qt][rr]));
            pp[rr & 3] = e < 4 ? p : pp[rr & 3] + p;   // four independent chains
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto products = [&](int buf, floatx16 (&acc)[QT], bool zero_init) __attribute__((always_inline)) {
      const uint16_t* cl = &c_lds[buf][col * CSTR + half * 8];
      if (zero_init) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) acc[qt] = floatx16{};
      }
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 cb = *reinterpret_cast<const bf16x8*>(cl + ks * 16);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          acc[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[qt][ks], cb, acc[qt], 0, 0, 0);
      }
    };
    // one pipelined full tile: NXT when tile kt + 1 is full too.  Buffer
    // kt & 1 held tile kt, whose products every wave issued before the
    // previous barrier, so tile kt + 2 goes there.
    auto iter_full = [&](auto NXT, int kt, floatx16 (&cur)[QT], floatx16 (&nxt)[QT])
        __attribute__((always_inline)) {
      if (kt + 2 < nkt) load(kt + 2);
      if (kt > 0) flush(kt - 1);
      step(NXT, (kt + 1) & 1, cur, nxt);
      park(kt);
      if (kt + 2 < nkt) store(kt & 1);
      __syncthreads();
    };

    floatx16 sa[QT], sb2[QT];
    if (nkt > 0) {
      load(0);
      store(0);
      __syncthreads();
      if (nfull > 0) products(0, sa, true);
      if (nkt > 1) {
        load(1);
        store(1);
      }
      __syncthreads();   // tile 1 in LDS; every wave is done with tile 0's buffer
    }
    int kt = 0;
    for (; kt + 2 < nfull; kt += 2) {
      iter_full(std::true_type{}, kt, sa, sb2);
      iter_full(std::true_type{}, kt + 1, sb2, sa);
    }
    if (kt + 1 < nfull) {
      iter_full(std::true_type{}, kt, sa, sb2);
      iter_full(std::false_type{}, kt + 1, sb2, sa);
    } else if (kt < nfull) {
      iter_full(std::false_type{}, kt, sa, sb2);
    }
    for (kt = nfull; kt < nkt; ++kt) {
      if (kt + 2 < nkt) load(kt + 2);
      if (kt > 0) flush(kt - 1);
      const int cend = (kt * 32 + col) * a.stride + a.len - 1;   // last token of this lane's summary
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int lim = tbase[qt] - cend;   // row visible iff its offset >= -lim
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          sa[qt][rr] = ((rr >> 2) * 8 + (rr & 3) + lim >= 0) ? 0.f : -__builtin_inff();
      }
      products(kt & 1, sa, false);
      step(std::false_type{}, 0, sa, sb2);
      park(kt);
      if (kt + 2 < nkt) {
        __syncthreads();   // every wave is done with tile kt's buffer
        store(kt & 1);
      }
      __syncthreads();
    }
    // the last tile's sums (every wave parked them before the last barrier;
    // the next chunk's first park comes after two more barriers)
    if (nkt > 0) flush(nkt - 1);
  }
  __syncthreads();

  // spread each summary's mass over the key blocks it overlaps
  const int nb = (a.S + sb - 1) / sb;
  const float norm = 1.f / (float(t1 - t0 + 1) * float(G));
  float* out = a.scores + (size_t(bg) * nqb + i) * nb;
  for (int j = threadIdx.x; j < nb; j += NW * 64) {
    const int j0 = j * sb, j1 = j * sb + sb - 1;
    int c0 = (j0 - a.len + 1 + a.stride - 1);
    c0 = c0 <= 0 ? 0 : c0 / a.stride;
    const int c1 = min(c_hi, j1 / a.stride);
    float acc = 0.f;
    for (int cc = c0; cc <= c1; ++cc) {
      const int a0 = cc * a.stride, a1 = a0 + a.len - 1;
      const int ov = min(a1, j1) - max(a0, j0) + 1;
      if (ov > 0) acc += colsum[cc] * (float(ov) / float(a.len));
    }
    out[j] = acc * norm;
  }
}

// Per-token selection scores (the method's own granularity: each query token
// ranks the key blocks for its KV group).  One workgroup per (group, 32
// consecutive tokens); wave w holds the Q operands of heads w, w + 4, ...
// (HPW heads, G <= 4 HPW), so the summary tile staged in LDS is shared by
// all heads of the group.  Per summary tile each wave adds its heads'
// probabilities into one 32 x 32 partial (token x summary) and parks it in
// LDS; the workgroup then forms the block scores of the blocks whose last
// overlapping summary lies in this tile, reading this tile's and the
// previous tile's partials (a block spans fewer than 32 summaries, checked
// by the caller).  Blocks past the last tile any of the 32 tokens can see
// are written at the last tile (their remaining summaries are invisible, 0).
// Output [B,Hkv,S,nb]; the head mean makes a row that sees a summary sum to 1.
constexpr int kTokRows = 32;
constexpr int kPStride = 33;   // padded partial row (floats)

template <int D, int HPW>
__global__ __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_cmp_token_scores(CmpScoreArgs a, int ntt) {
  constexpr int CSTR = D + 8;
  constexpr int CPR = D / 8;
  constexpr int CPT = (32 * CPR + kNW * 64 - 1) / (kNW * 64);
  __shared__ __attribute__((aligned(16))) uint16_t c_lds[2][32 * CSTR];
  __shared__ float part[2][kNW][kTokRows * kPStride];
  __shared__ __attribute__((aligned(16))) float lse_lds[kNW * HPW][kTokRows];

  const int bg = blockIdx.x / ntt, tt = ntt - 1 - int(blockIdx.x % ntt);   // longest first
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int t0 = tt * kTokRows, t1 = min(a.S, t0 + kTokRows) - 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const float c = a.scale * kLog2e;
  const int nb = (a.S + a.sel_block - 1) / a.sel_block;
  float* out = a.scores + (size_t(bg) * a.S + t0) * nb;
  const float inv_g = 1.f / float(G);

  int c_hi = -1;
  if (t1 >= a.len - 1) c_hi = min(a.n_cmp - 1, (t1 - (a.len - 1)) / a.stride);
  const int nkt = c_hi < 0 ? 0 : c_hi / 32 + 1;
  if (nkt == 0) {   // no token of the tile sees a summary: all scores 0
    for (int e = threadIdx.x; e < (t1 - t0 + 1) * nb; e += kNW * 64) out[e] = 0.f;
    return;
  }

  // Q operands of this wave's heads (rows = the 32 tokens), base-2 lse in LDS
  bf16x8 qf[HPW][D / 16];
  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
#pragma unroll
  for (int hi = 0; hi < HPW; ++hi) {
    const int h = hi * kNW + wave;
    const int t = t0 + col;
    const bool ok = h < G && t <= t1;
    const uint16_t* src = qp + ((size_t(b) * a.Hq + g * G + (ok ? h : 0)) * a.S + (ok ? t : t0)) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(src + ks * 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[hi][ks][e] = ok ? v[e] : static_cast<__bf16>(0.0f);
    }
    if (half == 0) {
      float l2 = __builtin_inff();   // no such head / token: probability 0
      if (ok) {
        const float l = a.lse[(size_t(b) * a.Hq + g * G + h) * a.S + t] * kLog2e;
        l2 = (l == -__builtin_inff()) ? 0.f : l;   // sees no summary: cut by the mask
      }
      lse_lds[hi * kNW + wave][col] = l2;
    }
  }

  const __amdgpu_buffer_rsrc_t crs = make_rsrc(static_cast<const uint16_t*>(a.ck) + size_t(bg) * a.n_cmp * D,
                                               uint32_t(a.n_cmp) * D * 2);
  u32x4 st[CPT];
  auto load = [&](int kt) {
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      const int e = threadIdx.x + cc * kNW * 64;
      if (e < 32 * CPR)
        st[cc] = __builtin_amdgcn_raw_buffer_load_b128(crs, uint32_t(((kt * 32 + e / CPR) * D + (e % CPR) * 8) * 2), 0, 0);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      const int e = threadIdx.x + cc * kNW * 64;
      if (e < 32 * CPR) *reinterpret_cast<u32x4*>(&c_lds[buf][(e / CPR) * CSTR + (e % CPR) * 8]) = st[cc];
    }
  };

  // last token of each accumulator row held by this lane (-1 past the sequence)
  int tlim[16];
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int tt2 = t0 + (rr >> 2) * 8 + half * 4 + (rr & 3);
    tlim[rr] = tt2 <= t1 ? tt2 : -1;
  }

  // blocks emitted after tile m: those whose last overlapping summary
  // floor((j*sb + sb - 1) / stride) lies at or before tile m's last summary
  auto last_block = [&](int m) {
    const int v = (32 * m + 32) * a.stride - a.sel_block;
    return v < 0 ? -1 : v / a.sel_block;
  };

  load(0);
  store(0);
  __syncthreads();
  int jlo = 0;
  for (int m = 0; m < nkt; ++m) {
    const int buf = m & 1;
    if (m + 1 < nkt) load(m + 1);
    float acc[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) acc[rr] = 0.f;
    const int cs = m * 32 + col;                    // this lane's summary
    const int cend = cs * a.stride + a.len - 1;     // its last token
    const bool all_vis = (m * 32 + 31) * a.stride + a.len - 1 <= t0;
    bf16x8 cb[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      cb[ks] = *reinterpret_cast<const bf16x8*>(&c_lds[buf][col * CSTR + ks * 16 + half * 8]);
#pragma unroll
    for (int hi = 0; hi < HPW; ++hi) {
      if (hi * kNW + wave >= G) break;   // wave-uniform
      floatx16 sacc = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[hi][ks], cb[ks], sacc, 0, 0, 0);
      const float* lrow = lse_lds[hi * kNW + wave];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const floatx4 l4 = *reinterpret_cast<const floatx4*>(lrow + q4 * 8 + half * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = q4 * 4 + r;
          const float p = fast_exp2(fmaf(sacc[rr], c, -l4[r]));
          acc[rr] += (all_vis || cend <= tlim[rr]) ? p : 0.f;
        }
      }
    }
    float* pw = part[buf][wave];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) pw[((rr >> 2) * 8 + half * 4 + (rr & 3)) * kPStride + col] = acc[rr];
    if (m + 1 < nkt) store(buf ^ 1);
    __syncthreads();

    // block scores of blocks jlo .. jhi for the 32 tokens
    const int jhi = (m == nkt - 1) ? nb - 1 : min(nb - 1, last_block(m));
    const int nbt = jhi - jlo + 1;
    const int cmax = min(32 * m + 31, a.n_cmp - 1);
    for (int e = threadIdx.x; e < kTokRows * nbt; e += kNW * 64) {
      const int r = e / nbt, j = jlo + e % nbt;
      if (t0 + r > t1) continue;
      const int j0 = j * a.sel_block, j1 = j0 + a.sel_block - 1;
      int c0 = j0 - a.len + 1;
      c0 = c0 <= 0 ? 0 : (c0 + a.stride - 1) / a.stride;
      const int c1 = min(cmax, j1 / a.stride);
      float v = 0.f;
      for (int cc = c0; cc <= c1; ++cc) {
        const int a0 = cc * a.stride, a1 = a0 + a.len - 1;
        const int ov = min(a1, j1) - max(a0, j0) + 1;
        const float* pc = &part[(cc >> 5) & 1][0][r * kPStride + (cc & 31)];
        float ps = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kNW; ++w2) ps += pc[w2 * kTokRows * kPStride];
        if (ov > 0) v += ps * (float(ov) / float(a.len));
      }
      out[size_t(r) * nb + j] = v * inv_g;
    }
    jlo = jhi + 1;
    __syncthreads();   // the partials of tile m - 1 are overwritten next
  }
}

// grid-stride over 8-element chunks of the outputs
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ o1,
                                                 const uint16_t* __restrict__ o2,
                                                 const uint16_t* __restrict__ o3,
                                                 const float* __restrict__ z, int Hq, int S, int D,
                                                 size_t nchunks, uint16_t* __restrict__ out) {
  const int cpr = D / 8;
  for (size_t e = size_t(blockIdx.x) * 256 + threadIdx.x; e < nchunks; e += size_t(gridDim.x) * 256) {
    const size_t row = e / cpr;            // (b*Hq + h)*S + t
    const int t = int(row % S);
    const size_t bh = row / S;
    const int h = int(bh % Hq);
    const size_t b = bh / Hq;
    const float* zz = z + ((b * S + t) * Hq + h) * 3;
    const float g1 = 1.f / (1.f + __expf(-zz[0]));
    const float g2 = 1.f / (1.f + __expf(-zz[1]));
    const float g3 = 1.f / (1.f + __expf(-zz[2]));
    const u32x4 a = *reinterpret_cast<const u32x4*>(o1 + e * 8);
    const u32x4 bb = *reinterpret_cast<const u32x4*>(o2 + e * 8);
    const u32x4 cc = *reinterpret_cast<const u32x4*>(o3 + e * 8);
    u32x4 r;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float lo = g1 * bf16lo(a[x]) + g2 * bf16lo(bb[x]) + g3 * bf16lo(cc[x]);
      const float hi = g1 * bf16hi(a[x]) + g2 * bf16hi(bb[x]) + g3 * bf16hi(cc[x]);
      r[x] = pack_bf16x2(lo, hi);
    }
    *reinterpret_cast<u32x4*>(out + e * 8) = r;
  }
}

}  // namespace

hipError_t launch_nsa_compress(const void* k, const void* v, int B, int Hkv, int S, int D,
                               int len, int stride, void* ck, void* cv, hipStream_t s) {
  const int n_cmp = (S - len) / stride + 1;
  const int work = n_cmp * (D / 8);
  k_compress<<<dim3((work + 255) / 256, B * Hkv, 2), 256, 0, s>>>(
      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), S, D, len, stride, n_cmp,
      static_cast<uint16_t*>(ck), static_cast<uint16_t*>(cv));
  return hipGetLastError();
}

hipError_t launch_cmp_block_scores(const CmpScoreArgs& a, hipStream_t s) {
  const int nqb = (a.S + a.sel_block - 1) / a.sel_block;
  const size_t lds = size_t(a.n_cmp) * sizeof(float);
  if (a.D == 128)
    k_cmp_block_scores<128, kBsNW, kBsQT><<<a.B * a.Hkv * nqb, kBsNW * 64, lds, s>>>(a, nqb);
  else
    k_cmp_block_scores<64, kBsNW, kBsQT><<<a.B * a.Hkv * nqb, kBsNW * 64, lds, s>>>(a, nqb);
  return hipGetLastError();
}

hipError_t launch_cmp_token_scores(const CmpScoreArgs& a, hipStream_t s) {
  const int ntt = (a.S + kTokRows - 1) / kTokRows;
  const int G = a.Hq / a.Hkv;
  const int grid = a.B * a.Hkv * ntt;
#define DSA_TS(DD, HH) k_cmp_token_scores<DD, HH><<<grid, kNW * 64, 0, s>>>(a, ntt)
  if (a.D == 128) {
    if (G <= 4) DSA_TS(128, 1);
    else if (G <= 8) DSA_TS(128, 2);
    else DSA_TS(128, 4);
  } else {
    if (G <= 4) DSA_TS(64, 1);
    else if (G <= 8) DSA_TS(64, 2);
    else DSA_TS(64, 4);
  }
#undef DSA_TS
  return hipGetLastError();
}

hipError_t launch_nsa_combine(const void* o1, const void* o2, const void* o3, const float* z,
                              int B, int Hq, int S, int D, void* out, hipStream_t s) {
  const size_t nchunks = size_t(B) * Hq * S * (D / 8);
  const size_t blocks = (nchunks + 255) / 256;
  const unsigned grid = unsigned(blocks < 65536 ? blocks : 65536);
  k_combine<<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(o1), static_cast<const uint16_t*>(o2),
                                 static_cast<const uint16_t*>(o3), z, Hq, S, D, nchunks,
                                 static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace dsa
