// Exact softmax attention restricted to a set of key tiles per query block.
//
// [DMA] §四-§五: positions outside the selection get weight exactly zero and
// their query.key products are never computed; skipping them gives the same
// result as the masked dense computation.  [NSA] §03: the same kernel runs
// the sliding branch (token window) and the compressed branch (keys are
// summaries, visible once their last token is in the past).
//
// bf16 kernel (gfx950 MFMA):
//   * A workgroup owns one query block of one KV group and packs the group's
//     query heads into its rows (GQA packing), so every K/V tile staged in
//     LDS feeds G heads.  Each wave owns 32*QT query rows.
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16: the key axis lands in each
//     lane's 16 accumulator registers and the query axis across lanes, so
//     row max / row sum need only in-lane work plus one exchange between the
//     two 32-lane halves.
//   * O^T += V^T . P^T, again 32x32x16: P is converted in registers straight
//     into the B operand; V is written to LDS transposed, with the key order
//     permuted inside every 16-key group so each lane's 8 keys are contiguous.
//   * Online softmax in base 2 (v_exp_f32), float32 statistics; the causal /
//     window / summary mask is only evaluated on tiles that cut the visible
//     region.  K/V tiles are double-buffered in LDS with register prefetch.
//   * Workgroup ids are remapped so each XCD works on one contiguous range of
//     (group, query block) pairs and its L2 holds that group's K/V.
//
// float32 kernel: one thread per query row, K/V tiles in LDS, VALU math.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

struct TileSpec {
  int mode, block, Skv, window, len, stride;
  const int32_t* idx_row;  // index mode
  int tpb;                 // key tiles per selected block
  int kt;                  // keys per tile
  int first_tile;          // window mode
};

// Keys of tile n start here.
__device__ __forceinline__ int tile_key0(const TileSpec& ts, int n) {
  if (ts.mode == MODE_INDEX) return ts.idx_row[n / ts.tpb] * ts.block + (n % ts.tpb) * ts.kt;
  if (ts.mode == MODE_WINDOW) return (ts.first_tile + n) * ts.kt;
  return n * ts.kt;
}

__device__ __forceinline__ bool visible(const TileSpec& ts, int t, int s) {
  if (s >= ts.Skv || s < 0) return false;
  if (ts.mode == MODE_INDEX) return s <= t;
  if (ts.mode == MODE_WINDOW) return s <= t && s > t - ts.window;
  return s * ts.stride + ts.len - 1 <= t;
}

// True when every key of the tile is visible to every row in [t0, t1].
__device__ __forceinline__ bool tile_full(const TileSpec& ts, int key0, int t0, int t1) {
  const int k1 = key0 + ts.kt - 1;
  if (k1 >= ts.Skv) return false;
  if (ts.mode == MODE_INDEX) return k1 <= t0;
  if (ts.mode == MODE_WINDOW) return k1 <= t0 && key0 > t1 - ts.window;
  return k1 * ts.stride + ts.len - 1 <= t0;
}

// Number of key tiles for query rows [t0, t1] and the spec to walk them.
__device__ __forceinline__ int make_tiles(const AttnArgs& a, int bg, int i, int t0, int t1, int kt,
                                          TileSpec& ts) {
  ts.mode = a.mode;
  ts.block = a.block;
  ts.Skv = a.Skv;
  ts.window = a.window;
  ts.len = a.cmp_len;
  ts.stride = a.cmp_stride;
  ts.kt = kt;
  ts.idx_row = nullptr;
  ts.tpb = 1;
  ts.first_tile = 0;
  if (a.mode == MODE_INDEX) {
    const int nqb = (a.S + a.block - 1) / a.block;
    ts.tpb = a.block / kt;
    ts.idx_row = a.idx + (size_t(bg) * nqb + i) * a.idx_width;
    const int cnt = a.count[size_t(bg) * nqb + i];
    return max(0, min(cnt, a.idx_width)) * ts.tpb;
  }
  if (a.mode == MODE_WINDOW) {
    const int lo = max(0, t0 - a.window + 1);
    ts.first_tile = lo / kt;
    return t1 / kt - ts.first_tile + 1;
  }
  if (t1 < a.cmp_len - 1) return 0;
  const int c_hi = min(a.Skv - 1, (t1 - (a.cmp_len - 1)) / a.cmp_stride);
  return c_hi / kt + 1;
}

// ------------------------------------------------------------------ bf16
template <int D, int KT, int QT, int NW>
__global__ __launch_bounds__(NW * 64) void k_attn_bf16(AttnArgs a, int wg_per_qb, int nqb,
                                                       int per_xcd, int total) {
  constexpr int NT = NW * 64;
  constexpr int ROWS = NW * 32 * QT;
  constexpr int KSTR = D + 8;   // bf16 elements per K row in LDS (16 B pad)
  constexpr int VSTR = KT + 8;  // bf16 elements per V^T row in LDS (16 B pad)
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int NCHUNK = KT * CPR;
  constexpr int CH = (NCHUNK + NT - 1) / NT;  // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][KT * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][D * VSTR];

  const int w = xcd_work_id(per_xcd);
  if (w >= total) return;
  const int sub = w % wg_per_qb;
  const int rest = w / wg_per_qb;
  const int i = nqb - 1 - rest % nqb;   // later query blocks see more keys: start them first
  const int bg = rest / nqb;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int t0 = i * a.block;
  const int t1 = min(a.S, t0 + a.block) - 1;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;

  const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kp = static_cast<const uint16_t*>(a.k) + size_t(bg) * a.Skv * D;
  const uint16_t* __restrict__ vp = static_cast<const uint16_t*>(a.v) + size_t(bg) * a.Skv * D;

  int row_t[QT], row_h[QT];
  bool row_ok[QT];
  bf16x8 qf[QT][D / 16];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = sub * ROWS + wave * 32 * QT + qt * 32 + col;
    const int hh = r / a.block;
    row_t[qt] = t0 + r % a.block;
    row_h[qt] = g * G + hh;
    row_ok[qt] = hh < G && row_t[qt] < a.S;
    const uint16_t* src = qp + ((size_t(b) * a.Hq + row_h[qt]) * a.S + row_t[qt]) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      if (row_ok[qt]) {
        qf[qt][ks] = *reinterpret_cast<const bf16x8*>(src + ks * 16);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[qt][ks][e] = static_cast<__bf16>(0.0f);
      }
    }
  }

  floatx16 o[QT][D / 32];
  float m[QT], l[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = -__builtin_inff();
    l[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qt][dt][r] = 0.f;
  }

  TileSpec ts;
  const int ntiles = make_tiles(a, bg, i, t0, t1, KT, ts);
  const float c = a.scale * kLog2e;

  u32x4 kreg[CH], vreg[CH];
  auto gload = [&](int n) {
    const int key0 = tile_key0(ts, n);
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
      const int e = threadIdx.x + ch * NT;
      const int key = key0 + e / CPR, dc = e % CPR;
      if ((NCHUNK % NT == 0 || e < NCHUNK) && key >= 0 && key < a.Skv) {
        kreg[ch] = *reinterpret_cast<const u32x4*>(kp + size_t(key) * D + dc * 8);
        vreg[ch] = *reinterpret_cast<const u32x4*>(vp + size_t(key) * D + dc * 8);
      } else {
        kreg[ch] = u32x4{0u, 0u, 0u, 0u};
        vreg[ch] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
      const int e = threadIdx.x + ch * NT;
      if (NCHUNK % NT != 0 && e >= NCHUNK) break;
      const int key = e / CPR, dc = e % CPR;
      *reinterpret_cast<u32x4*>(&k_lds[buf][key * KSTR + dc * 8]) = kreg[ch];
      // V^T with bits 2 and 3 of the key offset swapped (see header comment)
      const int pos = (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
      uint16_t* vt = &v_lds[buf][dc * 8 * VSTR + pos];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        vt[(2 * e2) * VSTR] = uint16_t(vreg[ch][e2] & 0xffffu);
        vt[(2 * e2 + 1) * VSTR] = uint16_t(vreg[ch][e2] >> 16);
      }
    }
  };

  if (ntiles > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();

  for (int n = 0; n < ntiles; ++n) {
    const int buf = n & 1;
    if (n + 1 < ntiles) gload(n + 1);

    floatx16 s[KT / 32][QT];
#pragma unroll
    for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][qt][r] = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT / 32; ++kt) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 ka =
            *reinterpret_cast<const bf16x8*>(&k_lds[buf][(kt * 32 + col) * KSTR + ks * 16 + half * 8]);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          s[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[qt][ks], s[kt][qt], 0, 0, 0);
      }
    }

    const int key0 = tile_key0(ts, n);
    if (!tile_full(ts, key0, t0, t1)) {
#pragma unroll
      for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kt * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
            if (!visible(ts, row_t[qt], key)) s[kt][qt][r] = -__builtin_inff();
          }
    }

#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][qt][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m[qt], mx * c);
      const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
      const float alpha = fast_exp2(m[qt] - m_use);
      m[qt] = m_new;
      float ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[kt][qt][r], c, -m_use));
          s[kt][qt][r] = p;
          ls += p;
        }
      l[qt] = l[qt] * alpha + ls;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[qt][dt][r] *= alpha;
    }

#pragma unroll
    for (int ks = 0; ks < KT / 16; ++ks) {
      bf16x8 pb[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[qt][e] = static_cast<__bf16>(s[ks >> 1][qt][(ks & 1) * 8 + e]);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const bf16x8 va =
            *reinterpret_cast<const bf16x8*>(&v_lds[buf][(dt * 32 + col) * VSTR + ks * 16 + half * 8]);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          o[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[qt], o[qt][dt], 0, 0, 0);
      }
    }

    if (n + 1 < ntiles) swrite(buf ^ 1);
    __syncthreads();
  }

  uint16_t* __restrict__ op = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float lt = l[qt] + __shfl_xor(l[qt], 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (!row_ok[qt]) continue;
    uint16_t* dst = op + ((size_t(b) * a.Hq + row_h[qt]) * a.S + row_t[qt]) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        u32x2 pk;
        pk[0] = pack_bf16x2(o[qt][dt][rr * 4 + 0] * inv, o[qt][dt][rr * 4 + 1] * inv);
        pk[1] = pack_bf16x2(o[qt][dt][rr * 4 + 2] * inv, o[qt][dt][rr * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(dst + dt * 32 + rr * 8 + half * 4) = pk;
      }
    if (a.lse && half == 0)
      a.lse[(size_t(b) * a.Hq + row_h[qt]) * a.S + row_t[qt]] =
          lt > 0.f ? (m[qt] + __builtin_log2f(lt)) * kLn2 : -__builtin_inff();
  }
}

// ----------------------------------------------------------------- float32
template <int D>
__global__ __launch_bounds__(256) void k_attn_f32(AttnArgs a, int nqb) {
  constexpr int KT = 32;
  __shared__ float k_lds[KT][D];
  __shared__ float v_lds[KT][D];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.Hkv, g = h / G, bg = b * a.Hkv + g;
  const int t0 = i * a.block;
  const int t1 = min(a.S, t0 + a.block) - 1;
  const int t = t0 + threadIdx.x;
  const bool ok = threadIdx.x < a.block && t < a.S;
  const float* kp = static_cast<const float*>(a.k) + size_t(bg) * a.Skv * D;
  const float* vp = static_cast<const float*>(a.v) + size_t(bg) * a.Skv * D;

  float qv[D], ov[D];
  const float* qrow = static_cast<const float*>(a.q) + ((size_t(b) * a.Hq + h) * a.S + (ok ? t : t0)) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = qrow[d];
    ov[d] = 0.f;
  }
  float m = -__builtin_inff(), l = 0.f;

  TileSpec ts;
  const int ntiles = make_tiles(a, bg, i, t0, t1, KT, ts);
  for (int n = 0; n < ntiles; ++n) {
    const int key0 = tile_key0(ts, n);
    __syncthreads();
    for (int e = threadIdx.x; e < KT * D; e += blockDim.x) {
      const int key = key0 + e / D;
      const bool in = key >= 0 && key < a.Skv;
      k_lds[e / D][e % D] = in ? kp[size_t(key) * D + e % D] : 0.f;
      v_lds[e / D][e % D] = in ? vp[size_t(key) * D + e % D] : 0.f;
    }
    __syncthreads();
#pragma unroll 1
    for (int kk = 0; kk < KT; ++kk) {
      if (!visible(ts, t, key0 + kk)) continue;
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(qv[d], k_lds[kk][d], dot);
      const float sc = dot * a.scale;
      if (sc > m) {  // new running maximum: rescale what was accumulated
        const float alpha = expf(m - sc);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) ov[d] *= alpha;
        m = sc;
      }
      const float p = expf(sc - m);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) ov[d] = fmaf(p, v_lds[kk][d], ov[d]);
    }
  }
  if (!ok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* orow = static_cast<float*>(a.out) + ((size_t(b) * a.Hq + h) * a.S + t) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) orow[d] = ov[d] * inv;
  if (a.lse) a.lse[(size_t(b) * a.Hq + h) * a.S + t] = l > 0.f ? m + logf(l) : -__builtin_inff();
}

template <int D, int KT, int QT, int NW>
hipError_t run_bf16(const AttnArgs& a, hipStream_t s) {
  constexpr int ROWS = NW * 32 * QT;
  const int nqb = (a.S + a.block - 1) / a.block;
  const int G = a.Hq / a.Hkv;
  const int wg_per_qb = (G * a.block + ROWS - 1) / ROWS;
  const int total = a.B * a.Hkv * nqb * wg_per_qb;
  const int per_xcd = (total + kNumXcd - 1) / kNumXcd;
  k_attn_bf16<D, KT, QT, NW><<<per_xcd * kNumXcd, NW * 64, 0, s>>>(a, wg_per_qb, nqb, per_xcd, total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const int nqb = (a.S + a.block - 1) / a.block;
  if (a.dtype == 0) {
    dim3 grid(nqb, a.Hq, a.B);
    const int threads = ((a.block + 63) / 64) * 64;
    if (a.D == 64) k_attn_f32<64><<<grid, threads, 0, s>>>(a, nqb);
    else k_attn_f32<128><<<grid, threads, 0, s>>>(a, nqb);
    return hipGetLastError();
  }
  // key tile = 64 keys unless index-mode blocks are 32 tokens long
  const bool kt32 = (a.mode == MODE_INDEX && a.block % 64 != 0);
  if (a.D == 128) return kt32 ? run_bf16<128, 32, 1, 8>(a, s) : run_bf16<128, 64, 1, 8>(a, s);
  return kt32 ? run_bf16<64, 32, 1, 8>(a, s) : run_bf16<64, 64, 1, 8>(a, s);
}

}  // namespace dsa
