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
#include <type_traits>

#include "dsa_device.h"
#include "dsa_internal.h"

// Generic bf16 kernel: query rows per workgroup = kAttnWaves waves x 32.
constexpr int kAttnWaves = 8;
// Wave priority while issuing matrix instructions: a wave in its MFMA phase
// wins issue over a wave doing softmax on the same SIMD.
constexpr int kMfmaPrio = 1;
// Minimum waves per SIMD the register allocation of the 8-wave kernels
// must allow.
#define DSA_ATTN_WAVES_PER_EU 2

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

// Keys visible to row t form one interval [lo, hi] in every mode (within a
// selected block in index mode); an empty interval has hi < lo.
__device__ __forceinline__ void row_range(const AttnArgs& a, int t, int& lo, int& hi) {
  if (a.mode == MODE_INDEX) {
    lo = 0;
    hi = min(t, a.Skv - 1);
  } else if (a.mode == MODE_WINDOW) {
    lo = max(0, t - a.window + 1);
    hi = min(t, a.Skv - 1);
  } else {
    lo = 0;
    hi = t >= a.cmp_len - 1 ? min(a.Skv - 1, (t - (a.cmp_len - 1)) / a.cmp_stride) : -1;
  }
}

// ------------------------------------------------------------------ bf16
// The two 32-lane halves of a wave hold the same 32 query columns; this
// returns (value of lane l%32, value of lane 32 + l%32) on every lane.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A row's running maximum is only moved (and its accumulators rescaled)
// when a new logit exceeds it by more than this many powers of two; until
// then probabilities are exp2 of at most this value.  The result is the
// same softmax: numerator and denominator share the reference maximum.
constexpr float kLazyRescale = 8.0f;

// (two-wave instances stage a tile in more registers per lane and run one
// wave per SIMD)
template <int D, int KT, int QT, int NW>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(NW >= 4 ? DSA_ATTN_WAVES_PER_EU : 1)))
void k_attn_bf16(AttnArgs a, int wg_per_qb, int nqb,
                                                       int per_xcd, int total) {
  constexpr int NT = NW * 64;
  constexpr int ROWS = NW * 32 * QT;
  constexpr int KSTR = D + 8;   // bf16 elements per K row in LDS (16 B pad: conflict-free reads)
  constexpr int VSTR = KT + 8;  // bf16 elements per V^T row in LDS
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int KCH = KT * CPR; // K chunks per tile
  constexpr int KCT = (KCH + NT - 1) / NT;
  constexpr int NKG = KT / 4;   // 4-key groups per tile
  constexpr int VGR = NKG * CPR;  // V groups (4 keys x 8 dims) per tile
  constexpr int VGT = (VGR + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][KT * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][D * VSTR];

  // Contiguous work per XCD keeps a group's K/V in that XCD's L2.  The
  // compressed branch is the exception: its work grows with the query block
  // (a contiguous range would give some XCDs only the longest blocks) and its
  // summaries are small, so its workgroups stay in dispatch order, dealt
  // round-robin over the XCDs.
  const int w = a.mode == MODE_CMP ? int(blockIdx.x) : xcd_work_id(per_xcd);
  if (w >= total) return;
  const int sub = w % wg_per_qb;
  const int rest = w / wg_per_qb;
  const int i = nqb - 1 - rest % nqb;   // later query blocks see more keys: start them first
  // (sequence, selection unit): SH query heads sharing one index list and
  // their KV head (SH = G unless the caller selects per query head)
  const int SH = a.sel_heads, U = a.Hq / SH;
  const int bu = rest / nqb;
  const int b = bu / U, u = bu % U;
  const int bg = b * a.Hkv + (u * SH) / (a.Hq / a.Hkv);
  const int t0 = i * a.block;
  const int t1 = min(a.S, t0 + a.block) - 1;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;

  const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(a.q);
  // K/V of this KV head through buffer descriptors: loads outside the
  // group's rows (ragged tails, padding) return zeros without a branch
  const uint32_t kv_bytes = uint32_t(a.Skv) * D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(static_cast<const uint16_t*>(a.k) + size_t(bg) * a.Skv * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(static_cast<const uint16_t*>(a.v) + size_t(bg) * a.Skv * D, kv_bytes);

  int row_t[QT], row_h[QT];
  bool row_ok[QT];
  bf16x8 qf[QT][D / 16];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = sub * ROWS + wave * 32 * QT + qt * 32 + col;
    const int hh = r / a.block;
    row_t[qt] = t0 + r % a.block;
    row_h[qt] = u * SH + hh;
    row_ok[qt] = hh < SH && row_t[qt] < a.S;
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
  int row_lo[QT], row_hi[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = -__builtin_inff();
    l[qt] = 0.f;
    row_range(a, row_t[qt], row_lo[qt], row_hi[qt]);
    // relative to this lane's key offset inside a 32-key accumulator tile
    row_lo[qt] -= half * 4;
    row_hi[qt] -= half * 4;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qt][dt][r] = 0.f;
  }
  // a tile needs no mask when every key is visible to every row of the block
  int blk_lo, blk_hi, dummy;
  row_range(a, t1, blk_lo, dummy);
  row_range(a, t0, dummy, blk_hi);

  TileSpec ts;
  const int ntiles = make_tiles(a, bu, i, t0, t1, KT, ts);
  const float c = a.scale * kLog2e;

  // K: one 16-byte chunk per (key, 8 dims).  V: four keys x 8 dims per
  // thread, so the transposed store writes 4 consecutive keys (8 bytes) of
  // one V^T row; the 16 lanes of a row group write 16 different key groups
  // (conflict-free).
  struct Stage {
    u32x4 k[KCT];
    u32x4 v[VGT][4];
  };
  // per-thread byte offsets inside a tile; the tile's start is a scalar offset
  uint32_t koff[KCT], voff[VGT];
#pragma unroll
  for (int ch = 0; ch < KCT; ++ch) {
    const int e = threadIdx.x + ch * NT;
    koff[ch] = uint32_t((e / CPR) * D + (e % CPR) * 8) * 2u;
  }
#pragma unroll
  for (int ch = 0; ch < VGT; ++ch) {
    const int e = threadIdx.x + ch * NT;
    voff[ch] = uint32_t(((e % NKG) * 4) * D + (e / NKG) * 8) * 2u;
  }
  auto gload = [&](int n, Stage& st) {
    const uint32_t base = uint32_t(tile_key0(ts, n)) * uint32_t(D * 2);  // wraps for key < 0: reads 0
#pragma unroll
    for (int ch = 0; ch < KCT; ++ch) {
      if (KCH % NT != 0 && int(threadIdx.x) + ch * NT >= KCH) break;
      st.k[ch] = __builtin_amdgcn_raw_buffer_load_b128(krs, koff[ch], base, 0);
    }
#pragma unroll
    for (int ch = 0; ch < VGT; ++ch) {
      if (VGR % NT != 0 && int(threadIdx.x) + ch * NT >= VGR) break;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        st.v[ch][j] = __builtin_amdgcn_raw_buffer_load_b128(vrs, voff[ch] + j * D * 2, base, 0);
    }
  };
  auto swrite = [&](const Stage& st, int buf) {
#pragma unroll
    for (int ch = 0; ch < KCT; ++ch) {
      const int e = threadIdx.x + ch * NT;
      if (KCH % NT != 0 && e >= KCH) break;
      *reinterpret_cast<u32x4*>(&k_lds[buf][(e / CPR) * KSTR + (e % CPR) * 8]) = st.k[ch];
    }
#pragma unroll
    for (int ch = 0; ch < VGT; ++ch) {
      const int e = threadIdx.x + ch * NT;
      if (VGR % NT != 0 && e >= VGR) break;
      const int kg = e % NKG, dc = e / NKG;
      // key offset -> position with bits 2 and 3 swapped, so the 8 keys one
      // lane feeds to the P.V product are adjacent in its V^T row
      const int k4 = kg * 4;
      const int pos = (k4 & ~12) | ((k4 & 4) << 1) | ((k4 & 8) >> 1);
      uint16_t* vt = &v_lds[buf][dc * 8 * VSTR + pos];
#pragma unroll
      for (int x = 0; x < 4; ++x) {   // dims dc*8 + 2x (low halves) and 2x+1 (high halves)
        u32x2 lo2, hi2;
        lo2[0] = __builtin_amdgcn_perm(st.v[ch][1][x], st.v[ch][0][x], 0x05040100u);
        lo2[1] = __builtin_amdgcn_perm(st.v[ch][3][x], st.v[ch][2][x], 0x05040100u);
        hi2[0] = __builtin_amdgcn_perm(st.v[ch][1][x], st.v[ch][0][x], 0x07060302u);
        hi2[1] = __builtin_amdgcn_perm(st.v[ch][3][x], st.v[ch][2][x], 0x07060302u);
        *reinterpret_cast<u32x2*>(vt + (2 * x) * VSTR) = lo2;
        *reinterpret_cast<u32x2*>(vt + (2 * x + 1) * VSTR) = hi2;
      }
    }
  };

  // one tile: S^T = K Q^T, mask, online softmax, O^T += V^T P^T
  auto tile = [&](int n, int buf) {
    floatx16 s[KT / 32][QT];
#pragma unroll
    for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][qt][r] = 0.f;
    __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
      for (int kt = 0; kt < KT / 32; ++kt) {
        const bf16x8 ka =
            *reinterpret_cast<const bf16x8*>(&k_lds[buf][(kt * 32 + col) * KSTR + ks * 16 + half * 8]);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          s[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[qt][ks], s[kt][qt], 0, 0, 0);
      }
    }

    __builtin_amdgcn_s_setprio(0);
    const int key0 = tile_key0(ts, n);
    if (key0 < blk_lo || key0 + KT - 1 > blk_hi) {   // wave-uniform
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int lo = row_lo[qt] - key0, hi = row_hi[qt] - key0;
#pragma unroll
        for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = kt * 32 + (r >> 2) * 8 + (r & 3);
            s[kt][qt][r] = (off < lo || off > hi) ? -__builtin_inff() : s[kt][qt][r];
          }
      }
    }

    bf16x8 pb[KT / 16][QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][qt][r]);
      const float mt = half_max(mx) * c;
      const bool grow = mt > m[qt] + kLazyRescale;
      if (__any(grow)) {
        // lanes that do not grow keep alpha = 1 (their m may still be -inf)
        const float alpha = grow ? fast_exp2(m[qt] - mt) : 1.f;   // 0 when m was -inf
        const float m_new = grow ? mt : m[qt];
        m[qt] = m_new;
        l[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[qt][dt][r] *= alpha;
      }
      const float mu = (m[qt] == -__builtin_inff()) ? 0.f : m[qt];
      float ls = 0.f;
#pragma unroll
      for (int ks = 0; ks < KT / 16; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(fmaf(s[ks >> 1][qt][(ks & 1) * 8 + e], c, -mu));
          ls += p;
          pb[ks][qt][e] = static_cast<__bf16>(p);
        }
      }
      l[qt] += ls;
    }

    __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
    for (int ks = 0; ks < KT / 16; ++ks) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const bf16x8 va =
            *reinterpret_cast<const bf16x8*>(&v_lds[buf][(dt * 32 + col) * VSTR + ks * 16 + half * 8]);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          o[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks][qt], o[qt][dt], 0, 0, 0);
      }
    }

    __builtin_amdgcn_s_setprio(0);
  };

  // Global loads run two tiles ahead of the math through two register
  // stages (A holds even tiles, B odd ones); LDS is double-buffered.
  Stage A, B;
  if (ntiles > 0) {
    gload(0, A);
    if (ntiles > 1) gload(1, B);
    swrite(A, 0);
  }
  __syncthreads();
  for (int n = 0; n < ntiles; n += 2) {
    if (n + 2 < ntiles) gload(n + 2, A);
    tile(n, 0);
    if (n + 1 < ntiles) swrite(B, 1);
    __syncthreads();
    if (n + 1 >= ntiles) break;
    if (n + 3 < ntiles) gload(n + 3, B);
    tile(n + 1, 1);
    if (n + 2 < ntiles) swrite(A, 0);
    __syncthreads();
  }

  uint16_t* __restrict__ op = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float lt = half_sum(l[qt]);
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

// ---------------------------------------------- bf16, D = 128, 64-key tiles
// Same math as k_attn_bf16, different data layout and staging:
//  * Per tile every wave runs Q.K, the softmax and P.V of its 32 rows; one
//    barrier per tile.  K and V of tile n+1 are loaded into registers at the
//    start of tile n (16 bytes x 4 per thread) and stored to the other LDS
//    buffer at its end.
//  * LDS holds K and V row-major in 1 KB chunks of four 256-byte key rows;
//    the rows a chunk holds make the operand reads free of bank conflicts
//    without padded rows: K chunk j (0..15) holds keys j, j+16, j+32, j+48
//    and starts at byte j * 1040 (the 16 keys of one ds_read_b128 phase lie
//    in chunks whose starts differ by 16 bytes modulo 256); V chunk j holds
//    keys 16 (j / 4) + 4 q + j % 4 (q = 0..3) and starts at byte j * 1088
//    (the four keys of one transposed read lie 64 bytes apart modulo 256).
//  * The P.V operand V^T comes from transposed LDS reads (ds_read_b64_tr_b16:
//    four keys of one dimension per lane), so V needs no register shuffle.
//  * Query rows load through one buffer descriptor per group, and the first
//    key of every tile is kept in a lane and read with v_readlane, so the
//    tile loop touches memory only for the K/V stream.
// persistent workgroups per XCD: 32 CUs, one resident workgroup each
constexpr int kAttnSlotsPerXcd = 32;
namespace d128 {
constexpr int D = 128, KT = 64, NW = 8, NT = NW * 64;
constexpr int KCH = 1040, VCH = 1088;  // chunk pitch in bytes
constexpr int KBYTES = 16 * KCH, VBYTES = 16 * VCH;
constexpr int kMaxTiles = 128;         // key tiles per query block (lane table)
}  // namespace d128

#define DSA_LDS_BF16X4(p) ((__attribute__((address_space(3))) bf16x4*)(p))

// BIAS: every key carries an additive logit term (key_bias, per KV head and
// position), staged per tile next to K.
// UNION: per-query-head lists (one selection unit per head).  A workgroup
// still packs the group's heads into its rows; it walks the union of its
// heads' lists (each tile staged once) and every wave runs the products
// only for the tiles its own head selected.
template <bool BIAS, bool UNION = false>
__global__ __launch_bounds__(d128::NT) __attribute__((amdgpu_waves_per_eu(DSA_ATTN_WAVES_PER_EU)))
void k_attn_bf16_d128(AttnArgs a, int wg_per_qb, int nqb, int per_xcd, int total) {
  using namespace d128;
  constexpr int ROWS = NW * 32;
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][KBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vbuf[2][VBYTES];
  __shared__ __attribute__((aligned(16))) float kbias[2][BIAS ? KT : 4];   // key_bias / scale
  __shared__ uint32_t ubits[UNION ? 256 : 1];        // union bitmap over key blocks
  __shared__ int ulist[UNION ? kMaxTiles : 1];       // union, ascending
  __shared__ int ucount;
  // epilogue: each wave's 32 output rows, 16-byte chunks XOR-swizzled by
  // row, and their log-sum-exp values
  __shared__ __attribute__((aligned(16))) uint8_t ostage[NW][32 * D * 2];
  __shared__ float lstage[NW][32];

  // Contiguous work per XCD keeps a group's K/V in that XCD's L2.  The
  // compressed branch is the exception: its work grows with the query block
  // (a contiguous range would give some XCDs only the longest blocks) and its
  // summaries are small, so its workgroups stay in dispatch order, dealt
  // round-robin over the XCDs.
  // Persistent workgroups: one per slot of the chip; workgroup j of XCD x
  // takes items x * per_xcd + j, + nwg, ... of that XCD's range.  The
  // compressed branch is launched with one workgroup per item (w_step =
  // grid = total: a single pass).
  const int nwg = int(gridDim.x) / kNumXcd;
  const int xcd = int(blockIdx.x) % kNumXcd, slot = int(blockIdx.x) / kNumXcd;
  const int w_first = a.mode == MODE_CMP ? int(blockIdx.x) : xcd * per_xcd + slot;
  const int w_end = a.mode == MODE_CMP ? total : min(total, (xcd + 1) * per_xcd);
  const int w_step = a.mode == MODE_CMP ? int(gridDim.x) : nwg;
  if (w_first >= w_end) return;

  // (sequence, selection unit): SH query heads sharing one index list and
  // their KV head (SH = G unless the caller selects per query head; the
  // union variant maps rows as per group and reads each head's own list)
  const int SH = UNION ? a.Hq / a.Hkv : a.sel_heads, U = a.Hq / SH;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  const uint32_t kv_bytes = uint32_t(a.Skv) * D * 2;
  const float c = a.scale * kLog2e;
  const float inv_scale = 1.f / a.scale;
  // The lane index as an opaque value: per-item address arithmetic derived
  // from it is redone per item instead of being hoisted out of the item
  // loop, where it would hold registers across the tile loop.
  auto item_lane = [&]() __attribute__((always_inline)) -> int {
    int x = lane;
    asm volatile("" : "+v"(x));
    return x;
  };

  // Staging: wave w moves K chunks and V chunks 2w and 2w + 1 of a tile;
  // lane l carries bytes [16 l, 16 l + 16) of each.
  uint32_t kvo[2], vvo[2];
  {
    const int q = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {
      const int j = 2 * wave + j2;
      kvo[j2] = uint32_t((16 * q + j) * 256 + c16 * 16);
      vvo[j2] = uint32_t((16 * (j / 4) + 4 * q + (j % 4)) * 256 + c16 * 16);
    }
  }
  // per-lane byte offsets of the operand reads (the rest are immediates)
  const uint32_t k_rd = (col & 15) * KCH + (col >> 4) * 256 + half * 16;
  const uint32_t v_rd = ((lane & 15) >> 2) * VCH + half * 256 + ((lane >> 4) & 1) * 32 + (lane & 3) * 8;

  // ---- the running item: set by begin() while the previous item finishes
  int sub = 0, b = 0, u = 0, t0 = 0;       // unit coordinates (uniform)
  int row_t = 0, row_h = 0;                // this lane's query row
  bool row_ok = false;
  int row_lo = 0, row_hi = -1, blk_lo = 0, blk_hi = -1;
  int ntiles = 0;
  uint64_t sel_lo = ~0ull, sel_hi = ~0ull;   // UNION: the tiles this wave's head selected
  // First key of every tile, held across lanes (tile n in lane n % 64 of
  // word n / 64) and read back with v_readlane: no memory access and no wait
  // inside the tile loop.  The launcher sends query blocks with more than
  // kMaxTiles tiles to k_attn_bf16.
  int key0_w0 = 0, key0_w1 = 0;
  __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k, 0u), vrs = make_rsrc(a.v, 0u), brs = make_rsrc(a.q, 0u);
  bf16x8 qf[D / 16];
  u32x4 stk[2], stv[2];
  u32x4 stb = {0u, 0u, 0u, 0u};   // BIAS: four key terms (wave 0, lanes 0..15)

  auto key0_of = [&](int n) __attribute__((always_inline)) -> int {
    const int lo = __builtin_amdgcn_readlane(key0_w0, n & 63);
    const int hi = __builtin_amdgcn_readlane(key0_w1, n & 63);
    return n < 64 ? lo : hi;
  };
  auto load_k = [&](int n) __attribute__((always_inline)) {
    const uint32_t base = uint32_t(key0_of(n)) * uint32_t(D * 2);
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) stk[j2] = __builtin_amdgcn_raw_buffer_load_b128(krs, kvo[j2], base, 0);
    if constexpr (BIAS)
      if (wave == 0 && lane < KT / 4)
        stb = __builtin_amdgcn_raw_buffer_load_b128(brs, uint32_t(lane * 16), uint32_t(key0_of(n)) * 4u, 0);
  };
  auto load_v = [&](int n) __attribute__((always_inline)) {
    const uint32_t base = uint32_t(key0_of(n)) * uint32_t(D * 2);
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) stv[j2] = __builtin_amdgcn_raw_buffer_load_b128(vrs, vvo[j2], base, 0);
  };
  auto store_k = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2)
      *reinterpret_cast<u32x4*>(&kbuf[buf][(2 * wave + j2) * KCH + lane * 16]) = stk[j2];
    if constexpr (BIAS)
      if (wave == 0 && lane < KT / 4) {
        floatx4 bv = __builtin_bit_cast(floatx4, stb);
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[e] *= inv_scale;
        *reinterpret_cast<floatx4*>(&kbias[buf][lane * 4]) = bv;
      }
  };
  auto store_v = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2)
      *reinterpret_cast<u32x4*>(&vbuf[buf][(2 * wave + j2) * VCH + lane * 16]) = stv[j2];
  };

  // list row of item w in index mode (per selection unit and query block)
  auto item_lrow = [&](int w) __attribute__((always_inline)) -> size_t {
    const int rest = w / wg_per_qb;
    return size_t(rest / nqb) * nqb + (nqb - 1 - rest % nqb);
  };
  const bool prefetch_list = !UNION && a.mode == MODE_INDEX;
  // index mode: the next item's count and list entries lane, lane + 64,
  // requested while the running item computes
  int nx_cnt = 0, nx_e0 = 0, nx_e1 = 0;
  auto fetch_list = [&](int w) __attribute__((always_inline)) {
    if constexpr (!UNION) {
      const size_t lrow = item_lrow(w);
      const int32_t* lst = a.idx + lrow * a.idx_width;
      const int ln = item_lane();
      nx_cnt = a.count[lrow];
      nx_e0 = ln < a.idx_width ? lst[ln] : 0;
      nx_e1 = ln + 64 < a.idx_width ? lst[ln + 64] : 0;
    }
  };

  // begin(w): coordinates of item w, its query rows (registers), its key
  // tiles and the loads of its first tile.  In index mode the list comes
  // from fetch_list(w), issued earlier.
  auto begin = [&](int w) __attribute__((always_inline)) {
    sub = w % wg_per_qb;
    const int rest = w / wg_per_qb;
    const int i = nqb - 1 - rest % nqb;   // later query blocks see more keys: start them first
    const int bu = rest / nqb;
    b = bu / U;
    u = bu % U;
    const int bg = b * a.Hkv + (u * SH) / (a.Hq / a.Hkv);
    t0 = i * a.block;
    const int t1 = min(a.S, t0 + a.block) - 1;
    krs = make_rsrc(static_cast<const uint16_t*>(a.k) + size_t(bg) * a.Skv * D, kv_bytes);
    vrs = make_rsrc(static_cast<const uint16_t*>(a.v) + size_t(bg) * a.Skv * D, kv_bytes);
    // (BIAS only; without it the descriptor covers nothing and is never used)
    brs = make_rsrc(BIAS ? a.key_bias + size_t(bg) * a.Skv : a.q, BIAS ? uint32_t(a.Skv) * 4 : 0u);

    // this lane's query row; rows past the group or the sequence read zeros
    const int ln = item_lane();
    const int r = sub * ROWS + wave * 32 + (ln & 31);
    const int hh = r / a.block;
    row_t = t0 + r % a.block;
    row_ok = hh < SH && row_t < a.S;
    row_h = u * SH + (row_ok ? hh : 0);
    row_range(a, row_t, row_lo, row_hi);
    row_lo -= half * 4;
    row_hi -= half * 4;
    int dummy;
    row_range(a, t1, blk_lo, dummy);
    row_range(a, t0, dummy, blk_hi);

    if constexpr (UNION) {
      // union of the lists of the heads in this workgroup (64-token blocks:
      // one tile per block), via a bitmap over the key blocks
      const int nbk = (a.Skv + KT - 1) / KT, nwords = (nbk + 31) >> 5;
      for (int e = threadIdx.x; e < nwords; e += NT) ubits[e] = 0u;
      __syncthreads();
      const int hw = (sub * ROWS + wave * 32) / a.block;   // this wave's head in the group
      const bool hw_ok = hw < SH;
      const size_t lrow = (size_t(b) * a.Hq + u * SH + (hw_ok ? hw : 0)) * nqb + i;
      const int cnt = hw_ok ? max(0, min(a.count[lrow], a.idx_width)) : 0;
      const int32_t* lst = a.idx + lrow * a.idx_width;
      for (int e = lane; e < cnt; e += 64) {
        const int j = lst[e];
        if (j >= 0 && j < nbk) atomicOr(&ubits[j >> 5], 1u << (j & 31));
      }
      __syncthreads();
      if (wave == 0) {   // bitmap -> ascending list (lane l scans words 4l .. 4l + 3)
        uint32_t wv[4];
        int c4 = 0;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int wi = lane * 4 + x;
          wv[x] = wi < nwords ? ubits[wi] : 0u;
          c4 += __popc(wv[x]);
        }
        int incl = c4;
#pragma unroll
        for (int o2 = 1; o2 < 64; o2 <<= 1) {
          const int y = __shfl_up(incl, o2);
          if (lane >= o2) incl += y;
        }
        int pos = incl - c4;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          uint32_t bits = wv[x];
          while (bits) {
            if (pos < kMaxTiles) ulist[pos] = (lane * 4 + x) * 32 + __builtin_ctz(bits);
            ++pos;
            bits &= bits - 1;
          }
        }
        if (lane == 63) ucount = min(incl, kMaxTiles);
      }
      __syncthreads();
      ntiles = ucount;
      // membership of union tile n in this wave's list: binary search (the
      // list is ascending)
      auto member = [&](int n) -> bool {
        if (n >= ntiles) return false;
        const int j = ulist[n];
        int lo = 0, hi = cnt - 1;
        while (lo <= hi) {
          const int mid = (lo + hi) >> 1;
          const int v = lst[mid];
          if (v == j) return true;
          if (v < j) lo = mid + 1; else hi = mid - 1;
        }
        return false;
      };
      sel_lo = __ballot(member(lane));
      sel_hi = __ballot(member(lane + 64));
      key0_w0 = lane < ntiles ? ulist[lane] * KT : 0;
      key0_w1 = lane + 64 < ntiles ? ulist[lane + 64] * KT : 0;
    } else if (a.mode == MODE_INDEX) {
      // tile n is part n % tpb of listed block n / tpb (list entries past
      // the count are never used)
      const int tpb = a.block / KT;
      ntiles = max(0, min(nx_cnt, a.idx_width)) * tpb;
      auto key0 = [&](int n) -> int {
        const int e = n / tpb;
        const int v0 = __shfl(nx_e0, e & 63), v1 = __shfl(nx_e1, e & 63);
        return (e < 64 ? v0 : v1) * a.block + (n % tpb) * KT;
      };
      const int k0 = key0(ln), k1 = key0(ln + 64);
      key0_w0 = ln < ntiles ? k0 : 0;
      key0_w1 = ln + 64 < ntiles ? k1 : 0;
    } else {
      TileSpec ts;
      ntiles = make_tiles(a, bu, i, t0, t1, KT, ts);
      key0_w0 = lane < ntiles ? tile_key0(ts, lane) : 0;
      key0_w1 = lane + 64 < ntiles ? tile_key0(ts, lane + 64) : 0;
    }
    {
      // one descriptor over the unit's query heads; rows that are not ours
      // get an offset past its end and read zeros
      const __amdgpu_buffer_rsrc_t qrs = make_rsrc(
          static_cast<const uint16_t*>(a.q) + (size_t(b) * a.Hq + size_t(u) * SH) * a.S * D,
          uint32_t(SH) * a.S * D * 2);
      const uint32_t qoff = row_ok ? uint32_t((hh * a.S + row_t) * D + (ln >> 5) * 8) * 2u : 0x80000000u;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff, ks * 32, 0));
    }
    if (ntiles > 0) {
      load_k(0);
      load_v(0);
    }
  };

  float alpha = 1.f;     // pending rescale of o (lazy softmax)
  bool rescale = false;
  floatx16 o[D / 32];
  float m, l;
  floatx16 s[KT / 32];   // S^T of the tile between its Q.K and its softmax
  bf16x8 pb[KT / 16];    // P^T of the tile between its softmax and its P.V

  // Operand reads run one k-step ahead of the MFMAs that use them; the
  // scheduling barriers keep the compiler from hoisting every read of the
  // phase to its top (which would need ~128 more registers).
  auto qk = [&](int buf) __attribute__((always_inline)) {
    const uint8_t* kb = &kbuf[buf][0] + k_rd;
    constexpr int KS2 = D / 32;   // steps of two k-slices: 4 MFMAs each
    bf16x8 ka[2][2][KT / 32];
    auto rd = [&](int st, bf16x8 (&dst)[2][KT / 32]) __attribute__((always_inline)) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kt = 0; kt < KT / 32; ++kt)
          dst[h][kt] = *reinterpret_cast<const bf16x8*>(kb + kt * 512 + (2 * st + h) * 32);
    };
    rd(0, ka[0]);
#pragma unroll
    for (int st = 0; st < KS2; ++st) {
      if (st + 1 < KS2) rd(st + 1, ka[(st + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kt = 0; kt < KT / 32; ++kt)
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[st & 1][h][kt], qf[2 * st + h],
                                                          st == 0 && h == 0 ? floatx16{} : s[kt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto pv = [&](int buf) __attribute__((always_inline)) {
    if (rescale) {   // wave-uniform
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
      alpha = 1.f;
      rescale = false;
    }
    const uint8_t* vb = &vbuf[buf][0] + v_rd;
    bf16x8 va[2][D / 32];
    auto rd = [&](int ks, bf16x8 (&dst)[D / 32]) __attribute__((always_inline)) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(DSA_LDS_BF16X4(vb + ks * 4352 + dt * 64));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(DSA_LDS_BF16X4(vb + ks * 4352 + 512 + dt * 64));
        dst[dt] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    rd(0, va[0]);
#pragma unroll
    for (int ks = 0; ks < KT / 16; ++ks) {
      if (ks + 1 < KT / 16) rd(ks + 1, va[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks & 1][dt], pb[ks], o[dt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto softmax = [&](int n) __attribute__((always_inline)) {
    const int key0 = key0_of(n);
    if constexpr (BIAS) {   // logit += key_bias: in units of s, key_bias / scale
#pragma unroll
      for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const floatx4 b4 = *reinterpret_cast<const floatx4*>(&kbias[n & 1][kt * 32 + e4 * 8 + half * 4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[kt][e4 * 4 + e] += b4[e];
        }
    }
    if (key0 < blk_lo || key0 + KT - 1 > blk_hi) {   // wave-uniform
      asm volatile("");   // a real branch: if-converting it would copy s
      const int lo = row_lo - key0, hi = row_hi - key0;
#pragma unroll
      for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int off = kt * 32 + (e >> 2) * 8 + (e & 3);
          s[kt][e] = (off < lo || off > hi) ? -__builtin_inff() : s[kt][e];
        }
    }
    // four independent chains: with one softmax wave per SIMD, latency and
    // not issue rate would bound a single chain
    float mx4[4] = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
#pragma unroll
    for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx4[e & 3] = fmaxf(mx4[e & 3], s[kt][e]);
    const float mt = half_max(fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]))) * c;
    const bool grow = mt > m + kLazyRescale;
    if (__any(grow)) {
      // o is rescaled at the start of the P.V of this tile, before the
      // tile adds to it
      const float a_ = grow ? fast_exp2(m - mt) : 1.f;   // 0 when m was -inf
      m = grow ? mt : m;
      l *= a_;
      alpha *= a_;
      rescale = true;
    }
    const float mu = (m == -__builtin_inff()) ? 0.f : m;
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KT / 16; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = fast_exp2(fmaf(s[ks >> 1][(ks & 1) * 8 + e], c, -mu));
        ls[e & 3] += p;
        pb[ks][e] = static_cast<__bf16>(p);
      }
    l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };

  // Per item: the first tile goes to LDS (its loads were issued while the
  // previous item finished), then the previous item's staged output leaves,
  // then the tile loop; the epilogue requests the next item's query rows and
  // first tile before it stages this item's output, so no wait for those
  // loads ever covers output stores.
  bool pend = false;   // staged output of the previous item still in LDS (uniform)
  int p_b = 0, p_u = 0, p_sub = 0, p_t0 = 0;
  uint16_t* __restrict__ op = static_cast<uint16_t*>(a.out);
  auto flush = [&]() __attribute__((always_inline)) {
    // the wave's 32 rows: consecutive positions of one head (the launcher
    // sends blocks that are not a multiple of 32 rows elsewhere); four whole
    // 256-byte rows per store, marked streaming (nothing here reads them
    // back, and they should not displace K/V lines from the caches)
    const uint8_t* stg = &ostage[wave][0];
    const int rw = p_sub * ROWS + wave * 32;
    const int hr = rw / a.block;
    const int tr0 = p_t0 + rw % a.block;
    if (hr < SH) {
      uint16_t* wb = op + ((size_t(p_b) * a.Hq + p_u * SH + hr) * a.S + tr0) * D;
      const int ln = item_lane();
      const int c16 = ln & 15;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int R = 4 * j + (ln >> 4);
        const u32x4 v4 = *reinterpret_cast<const u32x4*>(stg + R * 256 + ((c16 ^ (R & 15)) << 4));
        if (tr0 + R < a.S) __builtin_nontemporal_store(v4, reinterpret_cast<u32x4*>(wb + R * D + c16 * 8));
      }
      if (a.lse && ln < 32 && tr0 + ln < a.S)
        a.lse[(size_t(p_b) * a.Hq + p_u * SH + hr) * a.S + tr0 + ln] = lstage[wave][ln];
    }
  };

  if (prefetch_list) fetch_list(w_first);
  begin(w_first);
  for (int w = w_first; w < w_end; w += w_step) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
    m = -__builtin_inff();
    l = 0.f;
    alpha = 1.f;
    rescale = false;
    // the next item, or this one again after the last: begin() and
    // fetch_list() then run unconditionally (their registers need no merge
    // of two versions; the repeated loads are never used)
    const int w_next = w + w_step < w_end ? w + w_step : w;   // uniform

    if (ntiles > 0) {
      store_k(0);
      store_v(0);
    }
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): query rows and first tile landed on every path
    if (pend) {
      flush();
      pend = false;
    }
    if (prefetch_list) fetch_list(w_next);
    for (int n = 0; n < ntiles; ++n) {
      const bool more = n + 1 < ntiles;
      if (more) {
        load_k(n + 1);
        load_v(n + 1);
      }
      const bool mine = !UNION || (((n < 64 ? sel_lo : sel_hi) >> (n & 63)) & 1);   // wave-uniform
      if (mine) {
        __builtin_amdgcn_s_setprio(kMfmaPrio);
        qk(n & 1);
        __builtin_amdgcn_s_setprio(0);
        softmax(n);
        __builtin_amdgcn_s_setprio(kMfmaPrio);
        pv(n & 1);
        __builtin_amdgcn_s_setprio(0);
      }
      if (more) {
        store_k((n + 1) & 1);
        store_v((n + 1) & 1);
      }
      __syncthreads();
    }

    const int e_sub = sub, e_b = b, e_u = u, e_t0 = t0;
    const int e_row_t = row_t, e_row_h = row_h;
    const bool e_row_ok = row_ok;
    const float lt = half_sum(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse_v = lt > 0.f ? (m + __builtin_log2f(lt)) * kLn2 : -__builtin_inff();
    const size_t orow = ((size_t(e_b) * a.Hq + e_row_h) * a.S + e_row_t) * D;
    uint16_t* dst = op + orow;
    if (a.gate_z != nullptr) {
      if (e_row_ok) {
        // gated combine with the other two branches' outputs (this branch
        // in float32, the others as stored), rounded once
        const float* z = a.gate_z + ((size_t(e_b) * a.S + e_row_t) * a.Hq + e_row_h) * 3;
        const float g1 = 1.f / (1.f + __expf(-z[0]));
        const float g2 = 1.f / (1.f + __expf(-z[1]));
        const float g3 = inv / (1.f + __expf(-z[2]));
        const uint16_t* p1 = static_cast<const uint16_t*>(a.gate_o1) + orow;
        const uint16_t* p2 = static_cast<const uint16_t*>(a.gate_o2) + orow;
        // a half row's loads before its stores: the stores may alias them
        // as far as the compiler knows, so interleaving would serialise
        // every load
#pragma unroll
        for (int d2 = 0; d2 < D / 64; ++d2) {
          u32x2 w1[2][4], w2[2][4];
#pragma unroll
          for (int dh = 0; dh < 2; ++dh)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int off = (2 * d2 + dh) * 32 + rr * 8 + half * 4;
              w1[dh][rr] = *reinterpret_cast<const u32x2*>(p1 + off);
              w2[dh][rr] = *reinterpret_cast<const u32x2*>(p2 + off);
            }
#pragma unroll
          for (int dh = 0; dh < 2; ++dh)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int dt = 2 * d2 + dh;
              u32x2 pk;
#pragma unroll
              for (int x = 0; x < 2; ++x) {
                const float lo = g1 * bf16lo(w1[dh][rr][x]) + g2 * bf16lo(w2[dh][rr][x]) + g3 * o[dt][rr * 4 + 2 * x];
                const float hi = g1 * bf16hi(w1[dh][rr][x]) + g2 * bf16hi(w2[dh][rr][x]) + g3 * o[dt][rr * 4 + 2 * x + 1];
                pk[x] = pack_bf16x2(lo, hi);
              }
              *reinterpret_cast<u32x2*>(dst + dt * 32 + rr * 8 + half * 4) = pk;
            }
        }
      }
      if (a.lse && half == 0 && e_row_ok) a.lse[(size_t(e_b) * a.Hq + e_row_h) * a.S + e_row_t] = lse_v;
    }
    begin(w_next);
    if (a.gate_z == nullptr) {
      // A lane holds 8-byte pieces of its own row, so direct stores would
      // touch 32 rows per instruction.  The wave's 32 rows go to LDS (16-byte
      // chunks XOR-swizzled by row) and leave as whole rows in flush().
      uint8_t* stg = &ostage[wave][0];
      const int ln = item_lane();
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          u32x2 pk;
          pk[0] = pack_bf16x2(o[dt][rr * 4 + 0] * inv, o[dt][rr * 4 + 1] * inv);
          pk[1] = pack_bf16x2(o[dt][rr * 4 + 2] * inv, o[dt][rr * 4 + 3] * inv);
          *reinterpret_cast<u32x2*>(stg + (ln & 31) * 256 + (((dt * 4 + rr) ^ (ln & 15)) << 4) + (ln >> 5) * 8) = pk;
        }
      if (ln < 32) lstage[wave][ln] = lse_v;
      pend = true;
      p_b = e_b;
      p_u = e_u;
      p_sub = e_sub;
      p_t0 = e_t0;
    }
  }
  if (pend) {   // this wave's own LDS writes, read back in program order
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    flush();
  }
}

// -------------------------- bf16, D = 128, software-pipelined within each wave
// The tiles, LDS layouts and MFMA shapes of k_attn_bf16_d128 (eight waves of
// 32 query rows, two waves per SIMD), with each wave's softmax moved into
// the shadow of its own matrix products.  Measured on gfx950: a wave that
// issues its own products keeps the matrix core busy while it runs a few
// independent vector instructions between them, and two such waves per SIMD
// do better still; a wave whose vector work waits for its own products (the
// plain order Q.K, softmax, P.V) leaves the other wave to fill the gaps,
// which it does poorly.  So:
//  * keys advance in steps of 32 (the two halves of a 64-key LDS tile);
//  * step g issues P.V of step g-2 and Q.K of step g on the matrix core and,
//    between those products, the softmax of step g-1 (scores and
//    probabilities are double-buffered by step parity);
//  * P.V trails Q.K by two steps, i.e. one 64-key tile: tile n's keys and
//    tile n-1's values are read while tile n+1's keys and tile n's values
//    stream into the other buffers by direct-to-LDS loads; one barrier per
//    tile;
//  * the softmax's common path takes no maximum: probabilities are taken
//    against the row's current reference and summed in float32; a step in
//    which some lane's 16-key partial sum exceeds 2^8 (or whose row has no
//    reference yet) takes the slow path, which moves the reference as the
//    other kernels do and redoes that step's probabilities.
namespace w2 {
constexpr int D = 128, KT = 64, NW = 8, NT = NW * 64, ROWS = NW * 32;
constexpr int KCH = d128::KCH, VCH = d128::VCH, KBYTES = d128::KBYTES, VBYTES = d128::VBYTES;
constexpr int kMaxTiles = 128;
// a lane's partial sum of one step above this (or not a number) sends the
// step through the slow path
constexpr float kSumLimit = 256.0f;
}  // namespace w2

// 16 bytes per lane from global memory straight into LDS: from a wave-uniform
// base plus a per-lane 32-bit byte offset (no vector address arithmetic), and
// lane l's bytes land at dst + 16 l (dst uniform across the wave).  Issued
// from inline assembly so the compiler does not wait for these loads before
// unrelated LDS reads; the kernel waits for them itself (vmcnt) before the
// barrier that publishes a tile.  The instruction writes no register.
__device__ __forceinline__ void lds_load16_base(const void* base, uint32_t off, void* dst) {
  const uint64_t b = uint64_t(uintptr_t(base));
  // (the builtin returns a signed int: widen each half as unsigned)
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(b)));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(b >> 32)));
  const uint64_t sb = uint64_t(hi) << 32 | uint64_t(lo);
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t(dst)));
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sb), "s"(m0) : "memory", "m0");
}

// BIAS: every key carries an additive logit term (key_bias, per KV head and
// key; the value-driven mask): a tile's terms, divided by the softmax scale,
// sit in LDS beside its keys and enter each step's first Q.K product as its
// accumulator, so the scores come out with the term added.
template <bool BIAS>
__global__ __launch_bounds__(w2::NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_attn_bf16_d128_pipe(AttnArgs a, int wg_per_qb, int nqb, int per_xcd, int total) {
  using namespace w2;
  // K and V double-buffered; each wave stages its output rows (32 x 256 B)
  // in a region of its own, so the next item's first tile can load while
  // this item's output is still being written out
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * KBYTES + 2 * VBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t ostage[NW][32 * D * 2];
  __shared__ float lstage[NW][32];
  __shared__ __attribute__((aligned(16))) float kbias[2][BIAS ? KT : 4];   // key_bias / scale, by K buffer
  uint8_t* const kbase = smem;
  uint8_t* const vbase = smem + 2 * KBYTES;

  // persistent workgroups (one per CU): a contiguous range of items per XCD,
  // or for the compressed branch (items differ in length) every grid-th item.
  // An XCD's range runs longest items first and is dealt out round by round,
  // forward in even rounds and backward in odd ones, so that the workgroup
  // that took a round's longest item takes the next round's shortest (the
  // short items of the earliest query blocks then even out instead of
  // piling onto the same workgroups).
  const int nwg = int(gridDim.x) / kNumXcd;
  const int xcd = int(blockIdx.x) % kNumXcd, slot = int(blockIdx.x) / kNumXcd;
  const int w_end = a.mode == MODE_CMP ? total : min(total, (xcd + 1) * per_xcd);
  auto item_of = [&](int r) __attribute__((always_inline)) -> int {
    if (a.mode == MODE_CMP) return int(blockIdx.x) + r * int(gridDim.x);
    return xcd * per_xcd + r * nwg + ((r & 1) ? nwg - 1 - slot : slot);
  };

  const int SH = a.sel_heads, U = a.Hq / SH;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  const float c = a.scale * kLog2e;
  const uint32_t k_rd = (col & 15) * KCH + (col >> 4) * 256 + half * 16;
  const uint32_t v_rd = ((lane & 15) >> 2) * VCH + half * 256 + ((lane >> 4) & 1) * 32 + (lane & 3) * 8;
  // direct-to-LDS staging: wave w moves K chunks 2w, 2w+1 (chunk j holds keys
  // j, j+16, j+32, j+48) and V chunks 2w, 2w+1 (chunk j holds keys
  // 16 (j/4) + 4 q + j%4, q = 0..3); lane l carries row l/16 of a chunk,
  // bytes 16 (l%16) .. 16 (l%16) + 15 of its key
  const int lq = lane >> 4, lc = lane & 15;
  // byte offsets of this lane's 16 bytes within a whole tile, per chunk
  const uint32_t k_off0 = uint32_t((16 * lq + 2 * wave) * D * 2 + lc * 16);
  const uint32_t k_off1 = k_off0 + D * 2;
  const uint32_t v_off0 = uint32_t((16 * ((2 * wave) >> 2) + 4 * lq + ((2 * wave) & 3)) * D * 2 + lc * 16);
  const uint32_t v_off1 = v_off0 + D * 2;   // chunk 2w+1: the next key of the same quad

  // per item (n_sel: tiles of the listed blocks when a window pass follows
  // them, else -1)
  int ntiles = 0, n_sel = -1, key0_w0 = 0, key0_w1 = 0;
  int row_lo = 0, row_hi = -1, blk_lo = 0, blk_hi = -1;
  bf16x8 qf[D / 16];
  floatx16 o[D / 32];
  floatx16 s[2];       // S^T of a 32-key step, by step parity
  u32x4 pb[2][2];      // its probabilities (bf16 pairs) as the P.V operand, by step parity
  float m = 0.f, l = 0.f, lsum = 0.f, alpha = 1.f;
  bool rescale = false;
  const uint16_t* kg = nullptr;
  const uint16_t* vg = nullptr;

  auto key0_of = [&](int n) __attribute__((always_inline)) -> int {
    const int lo = __builtin_amdgcn_readlane(key0_w0, n & 63);
    const int hi = __builtin_amdgcn_readlane(key0_w1, n & 63);
    return n < 64 ? lo : hi;
  };
  // BIAS: the item's key terms (a descriptor over the group's keys; reads
  // past the sequence return zeros) and the next tile's four terms per lane
  // of wave 0, lanes 0..15, on their way to LDS
  __amdgpu_buffer_rsrc_t brs = make_rsrc(a.q, 0u);
  u32x4 stb = {0u, 0u, 0u, 0u};
  const float inv_scale = 1.f / a.scale;
  auto bias_load = [&](int n) __attribute__((always_inline)) {
    if constexpr (BIAS)
      if (wave == 0 && lane < KT / 4)
        stb = __builtin_amdgcn_raw_buffer_load_b128(brs, uint32_t(lane * 16), uint32_t(key0_of(n)) * 4u, 0);
  };
  auto bias_store = [&](int n) __attribute__((always_inline)) {
    if constexpr (BIAS)
      if (wave == 0 && lane < KT / 4) {
        floatx4 bv = __builtin_bit_cast(floatx4, stb);
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[e] *= inv_scale;
        *reinterpret_cast<floatx4*>(&kbias[n & 1][lane * 4]) = bv;
      }
  };
  auto kbuf = [&](int n) __attribute__((always_inline)) -> uint8_t* { return kbase + (n & 1) * KBYTES; };
  auto vbuf = [&](int n) __attribute__((always_inline)) -> uint8_t* { return vbase + (n & 1) * VBYTES; };
  // One tile's loads for this wave: K chunks 2w, 2w+1 of tile nk and V
  // chunks 2w, 2w+1 of tile nv (nk or nv < 0: none), each from a
  // wave-uniform base plus a per-lane byte offset.  A tile that starts before
  // the sequence or reaches past its end reads clamped rows instead (through
  // offsets from the group's first row): keys past the end are masked for
  // every row, and a list entry outside the sequence cannot send a load
  // outside the buffer.
  struct TileLoads {
    const uint16_t* kb;
    const uint16_t* vb;
    uint32_t ko0, ko1, vo0, vo1;
    uint8_t* kd;
    uint8_t* vd;
    bool k, v;
  };
  auto plan = [&](int nk, int nv) __attribute__((always_inline)) -> TileLoads {
    TileLoads r;
    r.k = nk >= 0;
    r.v = nv >= 0;
    r.kd = kbuf(nk) + (2 * wave) * KCH;
    r.vd = vbuf(nv) + (2 * wave) * VCH;
    r.kb = kg;
    r.vb = vg;
    r.ko0 = k_off0;
    r.ko1 = k_off1;
    r.vo0 = v_off0;
    r.vo1 = v_off1;
    if (r.k) {
      const int key0 = key0_of(nk);
      if (key0 >= 0 && key0 + KT <= a.Skv) {   // uniform: the whole tile inside
        r.kb = kg + size_t(key0) * D;
      } else {
        r.ko0 = uint32_t(min(max(key0 + 16 * lq + 2 * wave, 0), a.Skv - 1) * D * 2 + lc * 16);
        r.ko1 = uint32_t(min(max(key0 + 16 * lq + 2 * wave + 1, 0), a.Skv - 1) * D * 2 + lc * 16);
      }
    }
    if (r.v) {
      const int key0 = key0_of(nv);
      if (key0 >= 0 && key0 + KT <= a.Skv) {
        r.vb = vg + size_t(key0) * D;
      } else {
        const int k0 = key0 + 16 * ((2 * wave) >> 2) + 4 * lq + ((2 * wave) & 3);
        r.vo0 = uint32_t(min(max(k0, 0), a.Skv - 1) * D * 2 + lc * 16);
        r.vo1 = uint32_t(min(max(k0 + 1, 0), a.Skv - 1) * D * 2 + lc * 16);
      }
    }
    return r;
  };
  // load q (0..3: K chunk 2w, 2w+1, V chunk 2w, 2w+1) of a planned tile
  auto issue = [&](const TileLoads& r, int q) __attribute__((always_inline)) {
    if (q < 2) {
      if (r.k) lds_load16_base(r.kb, q ? r.ko1 : r.ko0, r.kd + q * KCH);
    } else {
      if (r.v) lds_load16_base(r.vb, q == 3 ? r.vo1 : r.vo0, r.vd + (q - 2) * VCH);
    }
  };
  auto wait_loads = [&]() __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  // probabilities of the step in s[P] against reference mu into pb[P];
  // lsum = this lane's float32 sum of them (the slow path's recomputation)
  auto probs = [&](auto P, float mu) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float pe[8];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = fast_exp2(fmaf(s[p][kk * 8 + e], c, -mu));
        acc[e & 3] += x;
        pe[e] = x;
        if (e & 1) pb[p][kk][e >> 1] = pack_bf16x2(pe[e - 1], x);
      }
    lsum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  };

  // One step, in explicit issue order: NPV products of P.V (step gpv, operand
  // pb[parity of gpv]) and NQK of Q.K (step gqk, into s[parity of gqk]) on
  // the matrix core, each product's operand read from LDS two products
  // ahead, and after each product one sixteenth of the common-path softmax
  // of the step in s[PS] against the current reference (when SM): score e's
  // probability, score e-1's contribution to the row sum and, every second
  // score, the bf16 pair of scores e-2 and e-1 (one score behind, so that no
  // instruction waits for the exponential just issued).  The scheduling
  // barriers keep this order.
  auto body = [&](auto NPV, auto NQK, auto SM, auto PS, int gpv, int gqk, auto&& after) __attribute__((always_inline)) {
    constexpr int npv = decltype(NPV)::value, nqk = decltype(NQK)::value;
    constexpr bool sm = decltype(SM)::value;
    constexpr int ps = decltype(PS)::value;   // parity of the softmax step
    constexpr int pp = ps ^ 1;                // parity of the P.V and Q.K steps
    constexpr int N = npv + nqk;
    constexpr int NI = N > 16 ? N : 16;
    const uint8_t* vp = vbuf(gpv >> 1) + (gpv & 1) * 2 * 4352 + v_rd;
    const uint8_t* kp = kbuf(gqk >> 1) + (gqk & 1) * 512 + k_rd;
    (void)vp;
    (void)kp;
    auto read_op = [&](auto I) __attribute__((always_inline)) -> bf16x8 {
      constexpr int i = decltype(I)::value;
      if constexpr (i < npv) {
        constexpr int kk = i / 4, dt = i % 4;
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(DSA_LDS_BF16X4(vp + kk * 4352 + dt * 64));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(DSA_LDS_BF16X4(vp + kk * 4352 + 512 + dt * 64));
        return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      } else {
        constexpr int ks = i - npv;
        return *reinterpret_cast<const bf16x8*>(kp + ks * 32);
      }
    };
    const float nmu = -m;
    float pe[16];
    float acc[4];
    bf16x8 op[3];
    // BIAS: the step's key terms, the first Q.K product's accumulator (read
    // with that product's operand); keys of accumulator element e are
    // 8 (e / 4) + 4 half + e % 4 of the step's 32
    floatx16 binit = {};
    auto read_bias = [&]() __attribute__((always_inline)) {
      if constexpr (BIAS) {
        const float* kb = &kbias[(gqk >> 1) & 1][(gqk & 1) * 32 + half * 4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const floatx4 b4 = *reinterpret_cast<const floatx4*>(kb + 8 * j);
#pragma unroll
          for (int e = 0; e < 4; ++e) binit[4 * j + e] = b4[e];
        }
      }
    };
    if constexpr (N > 0) op[0] = read_op(std::integral_constant<int, 0>{});
    if constexpr (N > 1) op[1] = read_op(std::integral_constant<int, 1>{});
    if constexpr (nqk > 0 && npv < 2) read_bias();
    __builtin_amdgcn_sched_barrier(0);
    // score j into the row sum; after an odd j, the bf16 pair (j-1, j)
    auto sum_pair = [&](auto J) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
      if constexpr (j < 4) acc[j] = pe[j];
      else acc[j % 4] += pe[j];
      if constexpr (j % 2 == 1) {
        uint32_t w = pack_bf16x2(pe[j - 1], pe[j]);
        asm volatile("" : "+v"(w));   // converted here, in the products' shadow
        pb[ps][j / 8][(j % 8) / 2] = w;
      }
    };
    auto one = [&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      if constexpr (i + 2 < N) op[(i + 2) % 3] = read_op(std::integral_constant<int, i + 2>{});
      if constexpr (nqk > 0 && npv >= 2 && i + 2 == npv) read_bias();
      if constexpr (i < npv) {
        constexpr int kk = i / 4, dt = i % 4;
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % 3], __builtin_bit_cast(bf16x8, pb[pp][kk]), o[dt], 0, 0, 0);
      } else if constexpr (i < N) {
        constexpr int ks = i - npv;
        s[pp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % 3], qf[ks], ks == 0 ? binit : s[pp], 0, 0, 0);
      }
      after(I);
      if constexpr (sm && i < 16) {
        pe[i] = fast_exp2(fmaf(s[ps][i], c, nmu));
        if constexpr (i >= 1) sum_pair(std::integral_constant<int, i - 1>{});
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    [&]<int... Is>(std::integer_sequence<int, Is...>) __attribute__((always_inline)) {
      (one(std::integral_constant<int, Is>{}), ...);
    }(std::make_integer_sequence<int, NI>{});
    if constexpr (sm) {
      sum_pair(std::integral_constant<int, 15>{});
      lsum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
  };
  // after the common-path softmax of the step in s[PS]: the slow path where
  // needed, then the row sum
  auto finish = [&](auto PS) __attribute__((always_inline)) {
    if (__any(!(lsum <= kSumLimit))) {   // wave-uniform, rare
      asm volatile("");
      constexpr int p = decltype(PS)::value;
      float mx = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[p][e]);
      const float mt = half_max(mx) * c;
      const bool grow = mt > m + kLazyRescale;
      if (__any(grow)) {
        const float a_ = grow ? fast_exp2(m - mt) : 1.f;   // 0 when there was no reference
        m = grow ? mt : m;
        l *= a_;
        alpha *= a_;
        rescale = true;
      }
      probs(PS, m == -__builtin_inff() ? 0.f : m);
    }
    l += lsum;
  };
  // keys of step g (in s[P]) outside the row's visible interval -> -inf
  // (steps that cut the block's visible region only)
  auto mask = [&](auto P, int g) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    const int key0 = key0_of(g >> 1) + (g & 1) * 32;
    if (key0 < blk_lo || key0 + 31 > blk_hi) {   // wave-uniform
      asm volatile("");
      const int lo = row_lo - key0, hi = row_hi - key0;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int off = (e >> 2) * 8 + (e & 3);
        s[p][e] = (off < lo || off > hi) ? -__builtin_inff() : s[p][e];
      }
    }
  };
  auto apply_rescale = [&]() __attribute__((always_inline)) {
    if (rescale) {   // wave-uniform
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
      alpha = 1.f;
      rescale = false;
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using T = std::true_type;
  using F = std::false_type;

  // step g: P.V of step g-2 (when PV), Q.K of step g (when QK), softmax of
  // step g-1 (when SM); G is g's parity.  Even steps start a tile: they issue
  // the loads of the next tile's keys and this tile's values; odd steps that
  // computed Q.K end it with the barrier that publishes those loads.
  auto step = [&](auto PV, auto QK, auto SM, auto G, int g) __attribute__((always_inline)) {
    constexpr bool pv = decltype(PV)::value, qk = decltype(QK)::value, sm = decltype(SM)::value;
    constexpr int gp = decltype(G)::value;
    using PS = std::integral_constant<int, gp ^ 1>;   // parity of step g-1
    using NP = std::integral_constant<int, pv ? 8 : 0>;
    using NQ = std::integral_constant<int, qk ? 8 : 0>;
    // even steps start the loads of the next tile's keys and this tile's
    // values (issued together: spreading them over the products measured
    // slower)
    if constexpr (qk && gp == 0) {
      const int n = g >> 1;
      const TileLoads tl = plan(n + 1 < ntiles ? n + 1 : -1, n);
      issue(tl, 0);
      issue(tl, 1);
      issue(tl, 2);
      issue(tl, 3);
      if (n + 1 < ntiles) bias_load(n + 1);
    }
    auto after = [&](auto) __attribute__((always_inline)) {};
    if constexpr (sm) mask(PS{}, g - 1);
    if constexpr (pv) apply_rescale();
    body(NP{}, NQ{}, std::integral_constant<bool, sm>{}, PS{}, g - 2, g, after);
    if constexpr (sm) finish(PS{});
    if constexpr (qk && gp == 1) {
      if (BIAS && (g >> 1) + 1 < ntiles) bias_store((g >> 1) + 1);
      wait_loads();
      __syncthreads();
    }
  };

  // item coordinates
  int sub = 0, b = 0, u = 0, t0 = 0;
  auto item_lane = [&]() __attribute__((always_inline)) -> int {
    int x = lane;
    asm volatile("" : "+v"(x));   // keeps list loads on the vector path
    return x;
  };
  // index mode: the next item's count and list entries lane, lane + 64,
  // requested while the running item computes
  int nx_cnt = 0, nx_e0 = 0, nx_e1 = 0;
  auto fetch_list = [&](int w) __attribute__((always_inline)) {
    if (a.mode == MODE_INDEX) {
      const int rest = w / wg_per_qb;
      const size_t lrow = size_t(rest / nqb) * nqb + (nqb - 1 - rest % nqb);
      const int32_t* lst = a.idx + lrow * a.idx_width;
      const int ln = item_lane();
      nx_cnt = a.count[lrow + (ln & 0x40000000)];   // (ln < 2^30: the entry itself)
      nx_e0 = ln < a.idx_width ? lst[ln] : 0;
      nx_e1 = ln + 64 < a.idx_width ? lst[ln + 64] : 0;
    }
  };
  // begin(w): coordinates of item w, its query rows (registers), its key
  // tiles and the loads of its first tile's keys; in index mode the list
  // comes from fetch_list(w), issued earlier
  auto begin = [&](int w) __attribute__((always_inline)) {
    w = __builtin_amdgcn_readfirstlane(w);
    sub = w % wg_per_qb;
    const int rest = w / wg_per_qb;
    const int i = nqb - 1 - rest % nqb;   // later query blocks see more keys: start them first
    const int bu = rest / nqb;
    b = bu / U;
    u = bu % U;
    const int bg = __builtin_amdgcn_readfirstlane(b * a.Hkv + (u * SH) / (a.Hq / a.Hkv));
    t0 = i * a.block;
    const int t1 = min(a.S, t0 + a.block) - 1;
    kg = static_cast<const uint16_t*>(a.k) + size_t(bg) * a.Skv * D;
    vg = static_cast<const uint16_t*>(a.v) + size_t(bg) * a.Skv * D;
    if constexpr (BIAS) brs = make_rsrc(a.key_bias + size_t(bg) * a.Skv, uint32_t(a.Skv) * 4u);

    // this lane's query row; rows past the unit or the sequence compute on
    // zeros and are not stored
    {
      const __amdgpu_buffer_rsrc_t qrs = make_rsrc(
          static_cast<const uint16_t*>(a.q) + (size_t(b) * a.Hq + size_t(u) * SH) * a.S * D,
          uint32_t(SH) * a.S * D * 2);
      const int r = sub * ROWS + wave * 32 + col;
      const int hh = r / a.block;
      const int row_t = t0 + r % a.block;
      const bool row_ok = hh < SH && row_t < a.S;
      row_range(a, row_t, row_lo, row_hi);
      row_lo -= half * 4;
      row_hi -= half * 4;
      const uint32_t qoff = row_ok ? uint32_t((hh * a.S + row_t) * D + half * 8) * 2u : 0x80000000u;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff, ks * 32, 0));
      int dummy;
      row_range(a, t1, blk_lo, dummy);
      row_range(a, t0, dummy, blk_hi);
    }
    if (a.mode == MODE_INDEX) {
      // tile n is part n % tpb of listed block n / tpb (entries past the
      // count are never used)
      const int tpb = a.block / KT;
      // (every lane loaded the same count)
      const int nsel = max(0, min(__builtin_amdgcn_readfirstlane(nx_cnt), a.idx_width)) * tpb;
      // a window pass: the window's tiles follow the listed ones
      const int wfirst = max(0, t0 - a.then_window + 1) / KT;
      ntiles = a.then_window > 0 ? nsel + t1 / KT - wfirst + 1 : nsel;
      n_sel = a.then_window > 0 ? nsel : -1;
      auto key0 = [&](int n) -> int {
        const int e = n / tpb;
        const int v0 = __shfl(nx_e0, e & 63), v1 = __shfl(nx_e1, e & 63);
        return n < nsel ? (e < 64 ? v0 : v1) * a.block + (n % tpb) * KT : (wfirst + n - nsel) * KT;
      };
      const int ln = item_lane();
      const int k0 = key0(ln), k1 = key0(ln + 64);
      key0_w0 = ln < ntiles ? k0 : 0;
      key0_w1 = ln + 64 < ntiles ? k1 : 0;
    } else {
      TileSpec ts;
      ntiles = make_tiles(a, bu, i, t0, t1, KT, ts);
      key0_w0 = lane < ntiles ? tile_key0(ts, lane) : 0;
      key0_w1 = lane + 64 < ntiles ? tile_key0(ts, lane + 64) : 0;
    }
    if (ntiles > 0) {
      const TileLoads t0l = plan(0, -1);
      issue(t0l, 0);
      issue(t0l, 1);
      bias_load(0);
    }
  };

  // Window pass after the listed blocks.  switch_a runs once the listed
  // blocks' last softmax step is done (their row sum is final): it parks the
  // row sum, restarts the softmax statistics and moves the visible intervals
  // to the window; the listed blocks' last P.V product (and any rescale it
  // still owes) runs in the next step.  switch_b runs after it: the listed
  // blocks' output, normalised and rounded to bf16 as a separate call would
  // store it, goes into this wave's staging region (free until the
  // epilogue), and the accumulators restart.
  auto switch_a = [&]() __attribute__((always_inline)) {
    const float lt = half_sum(l);
    if (half == 0) lstage[wave][col] = lt;
    m = -__builtin_inff();
    l = 0.f;
    const int r = sub * ROWS + wave * 32 + col;
    const int row_t = t0 + r % a.block;
    const int t1 = min(a.S, t0 + a.block) - 1;
    const int W = a.then_window;
    row_lo = max(0, row_t - W + 1) - half * 4;
    row_hi = min(row_t, a.Skv - 1) - half * 4;
    blk_lo = max(0, t1 - W + 1);
    blk_hi = min(t0, a.Skv - 1);
  };
  auto switch_b = [&]() __attribute__((always_inline)) {
    const float lt = lstage[wave][col];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint8_t* stg = &ostage[wave][0];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        u32x2 pk;
        pk[0] = pack_bf16x2(o[dt][rr * 4 + 0] * inv, o[dt][rr * 4 + 1] * inv);
        pk[1] = pack_bf16x2(o[dt][rr * 4 + 2] * inv, o[dt][rr * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(stg + col * 256 + (((dt * 4 + rr) ^ (col & 15)) << 4) + half * 8) = pk;
      }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] = floatx16{};
  };

  // the staged output of the previous item leaves: the wave's 32 rows are
  // consecutive positions of one head (blocks are a multiple of 32 rows),
  // whole 256-byte rows per store, streaming (nothing here reads them back)
  bool pend = false;   // uniform
  int p_b = 0, p_u = 0, p_sub = 0, p_t0 = 0;
  auto flush = [&]() __attribute__((always_inline)) {
    const uint8_t* stg = &ostage[wave][0];
    const int rw = p_sub * ROWS + wave * 32;
    const int hr = rw / a.block;
    const int tr0 = p_t0 + rw % a.block;
    if (hr < SH) {
      uint16_t* wb = static_cast<uint16_t*>(a.out) + ((size_t(p_b) * a.Hq + p_u * SH + hr) * a.S + tr0) * D;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int R = 4 * j + lq;
        const u32x4 v4 = *reinterpret_cast<const u32x4*>(stg + R * 256 + ((lc ^ (R & 15)) << 4));
        if (tr0 + R < a.S) __builtin_nontemporal_store(v4, reinterpret_cast<u32x4*>(wb + R * D + lc * 8));
      }
      if (a.lse && lane < 32 && tr0 + lane < a.S)
        a.lse[(size_t(p_b) * a.Hq + p_u * SH + hr) * a.S + tr0 + lane] = lstage[wave][lane];
    }
  };

  // Per item: wait for its query rows and first keys, write out the
  // previous item's staged output, request the next item's list, run the
  // tile loop; then request the next item's query rows and first keys
  // before staging this item's output, so that those loads run under the
  // staging and the stores.
  // (item numbers grow with the round, so the first one past the range ends
  // the loop)
  int w = item_of(0);
  if (w < w_end) {
    fetch_list(w);
    begin(w);
  }
  for (int r = 1; w < w_end; ++r) {
    // the next item, or this one again after the last (those loads are
    // never used; running begin() unconditionally keeps one version of its
    // registers)
    const int w_after = item_of(r);
    const int w_next = w_after < w_end ? w_after : w;   // uniform
    m = -__builtin_inff();
    l = 0.f;
    alpha = 1.f;
    rescale = false;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] = floatx16{};

    wait_loads();
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the query rows too
    if (ntiles > 0) bias_store(0);
    __syncthreads();
    if (pend) {
      flush();
      pend = false;
    }
    fetch_list(w_next);

    if (ntiles > 0) {
      if (n_sel == 0) {   // nothing listed: the window pass from the start
        switch_a();
        switch_b();
      }
      step(F{}, T{}, F{}, I0{}, 0);
      step(F{}, T{}, T{}, I1{}, 1);
      for (int n = 1; n < ntiles; ++n) {
        step(T{}, T{}, T{}, I0{}, 2 * n);
        if (n == n_sel) switch_a();   // uniform
        step(T{}, T{}, T{}, I1{}, 2 * n + 1);
        if (n == n_sel) switch_b();
      }
      step(T{}, F{}, T{}, I0{}, 2 * ntiles);
      step(T{}, F{}, F{}, I1{}, 2 * ntiles + 1);
    }
    __syncthreads();   // every wave is done with the tile buffers

    const float lt = half_sum(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float mu = m == -__builtin_inff() ? 0.f : m;
    const float lse_v = lt > 0.f ? (mu + __builtin_log2f(lt)) * kLn2 : -__builtin_inff();
    p_b = b;
    p_u = u;
    p_sub = sub;
    p_t0 = t0;
    begin(w_next);

    // the wave's 32 rows into its staging region, 16-byte chunks
    // XOR-swizzled by row
    uint8_t* stg = &ostage[wave][0];
    if (a.gate_z == nullptr) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          u32x2 pk;
          pk[0] = pack_bf16x2(o[dt][rr * 4 + 0] * inv, o[dt][rr * 4 + 1] * inv);
          pk[1] = pack_bf16x2(o[dt][rr * 4 + 2] * inv, o[dt][rr * 4 + 3] * inv);
          *reinterpret_cast<u32x2*>(stg + col * 256 + (((dt * 4 + rr) ^ (col & 15)) << 4) + half * 8) = pk;
        }
    } else {
      // gated combine with the other two branches' outputs: sigmoid(z0) o1 +
      // sigmoid(z1) o2 + sigmoid(z2) (this branch, float32), rounded once.
      // The lane's pieces of both rows are all loaded before any is used.
      // After a window pass o2 is the listed blocks' output, staged in this
      // lane's own places of the staging region (overwritten below).
      const int r = p_sub * ROWS + wave * 32 + col;
      const int hh = r / a.block;
      const int row_t = p_t0 + r % a.block;
      const bool ok = hh < SH && row_t < a.S;
      const int h = p_u * SH + (ok ? hh : 0);
      const size_t orow = ((size_t(p_b) * a.Hq + h) * a.S + (ok ? row_t : 0)) * D;
      float g1 = 0.f, g2 = 0.f, g3 = 0.f;
      u32x2 w1[D / 32][4], w2[D / 32][4];
      const uint16_t* p1 = static_cast<const uint16_t*>(a.gate_o1) + orow;
      const uint16_t* p2 = static_cast<const uint16_t*>(a.gate_o2) + orow;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          w1[dt][rr] = ok ? *reinterpret_cast<const u32x2*>(p1 + dt * 32 + rr * 8 + half * 4) : u32x2{0u, 0u};
          if (a.then_window > 0)
            w2[dt][rr] = *reinterpret_cast<const u32x2*>(stg + col * 256 + (((dt * 4 + rr) ^ (col & 15)) << 4) + half * 8);
          else
            w2[dt][rr] = ok ? *reinterpret_cast<const u32x2*>(p2 + dt * 32 + rr * 8 + half * 4) : u32x2{0u, 0u};
        }
      if (ok) {
        const float* z = a.gate_z + ((size_t(p_b) * a.S + row_t) * a.Hq + h) * 3;
        g1 = 1.f / (1.f + __expf(-z[0]));
        g2 = 1.f / (1.f + __expf(-z[1]));
        g3 = inv / (1.f + __expf(-z[2]));
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          u32x2 pk;
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const float lo = g1 * bf16lo(w1[dt][rr][x]) + g2 * bf16lo(w2[dt][rr][x]) + g3 * o[dt][rr * 4 + 2 * x];
            const float hi = g1 * bf16hi(w1[dt][rr][x]) + g2 * bf16hi(w2[dt][rr][x]) + g3 * o[dt][rr * 4 + 2 * x + 1];
            pk[x] = pack_bf16x2(lo, hi);
          }
          *reinterpret_cast<u32x2*>(stg + col * 256 + (((dt * 4 + rr) ^ (col & 15)) << 4) + half * 8) = pk;
        }
    }
    if (half == 0) lstage[wave][col] = lse_v;
    pend = true;
    w = w_after;
  }
  if (pend) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    flush();
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
  const int bu = b * (a.Hq / a.sel_heads) + h / a.sel_heads;   // index rows of h's selection unit
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
  const int ntiles = make_tiles(a, bu, i, t0, t1, KT, ts);
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
      const float sc = dot * a.scale + (a.key_bias ? a.key_bias[size_t(bg) * a.Skv + key0 + kk] : 0.f);
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

// Upper bound on the key tiles of one query block (as make_tiles counts them).
int attn_max_tiles(const AttnArgs& a, int kt) {
  if (a.mode == MODE_INDEX)
    return a.idx_width * (a.block / kt) + (a.then_window > 0 ? (a.then_window + a.block) / kt + 2 : 0);
  if (a.mode == MODE_WINDOW) return (a.window + a.block) / kt + 2;
  return (a.Skv + kt - 1) / kt;
}

template <int D, int KT, int QT, int NW>
hipError_t run_bf16(const AttnArgs& a, hipStream_t s) {
  constexpr int ROWS = NW * 32 * QT;
  const int nqb = (a.S + a.block - 1) / a.block;
  const int wg_per_qb = (a.sel_heads * a.block + ROWS - 1) / ROWS;
  const int total = a.B * (a.Hq / a.sel_heads) * nqb * wg_per_qb;
  const int per_xcd = (total + kNumXcd - 1) / kNumXcd;
  k_attn_bf16<D, KT, QT, NW><<<per_xcd * kNumXcd, NW * 64, 0, s>>>(a, wg_per_qb, nqb, per_xcd, total);
  return hipGetLastError();
}

}  // namespace

namespace {
// per-query-head lists through the union kernel: 64-token blocks, the
// group's heads filling whole workgroups, every union within the lane table
bool uses_d128_union(const AttnArgs& a) {
  constexpr int ROWS = d128::NW * 32;
  const int G = a.Hq / a.Hkv;
  const int heads_per_wg = ROWS / 64;
  return a.dtype == 1 && a.D == 128 && a.mode == MODE_INDEX && a.block == 64 && a.sel_heads == 1 &&
         G > 1 && (G * 64) % ROWS == 0 && a.key_bias == nullptr && a.gate_z == nullptr &&
         heads_per_wg * a.idx_width <= d128::kMaxTiles && (a.S + 63) / 64 <= 256 * 32;
}

// the software-pipelined kernel: 64-token blocks (key tiles of whole blocks,
// each wave's 32 rows inside one head), whole workgroups of rows
bool uses_pipe(const AttnArgs& a) {
  return a.dtype == 1 && a.D == 128 && a.block % 64 == 0 && a.sel_heads * a.block >= 256 &&
         (a.gate_z == nullptr || a.mode == MODE_WINDOW || a.then_window > 0) &&
         attn_max_tiles(a, 64) <= w2::kMaxTiles;
}

bool uses_d128(const AttnArgs& a) {
  const bool kt32 = (a.mode == MODE_INDEX && a.block % 64 != 0);
  return a.dtype == 1 && a.D == 128 && !kt32 && a.block % 32 == 0 && a.sel_heads * a.block >= 256 &&
         attn_max_tiles(a, 64) <= d128::kMaxTiles;
}
}  // namespace

bool attention_supported(const AttnArgs& a) {
  // the additive key term exists in the float32 kernel and the D = 128 one;
  // the gated-combine epilogue in the D = 128 one
  if (a.gate_z != nullptr && !uses_d128(a)) return false;
  // the window pass after the listed blocks exists in the pipelined kernel only
  if (a.then_window > 0 && (a.mode != MODE_INDEX || !uses_pipe(a))) return false;
  return a.key_bias == nullptr || a.dtype == 0 || uses_d128(a);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (!attention_supported(a)) return hipErrorInvalidValue;
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
  // a selection unit with fewer rows than an eight-wave workgroup (per-head
  // selection) runs the generic kernel with as many waves as it has rows
  const int unit_rows = a.sel_heads * a.block;
  if (uses_d128_union(a)) {
    constexpr int ROWS = d128::NW * 32;
    const int wg_per_qb = ((a.Hq / a.Hkv) * a.block + ROWS - 1) / ROWS;
    const int total = a.B * a.Hkv * nqb * wg_per_qb;
    const int per_xcd = (total + kNumXcd - 1) / kNumXcd;
    const int grid = kNumXcd * min(per_xcd, kAttnSlotsPerXcd);
    k_attn_bf16_d128<false, true><<<grid, d128::NT, 0, s>>>(a, wg_per_qb, nqb, per_xcd, total);
    return hipGetLastError();
  }
  if (unit_rows < 256) {
    const int nw = unit_rows <= 64 ? 2 : 4;
    if (a.D == 128)
      return kt32 ? (nw == 2 ? run_bf16<128, 32, 1, 2>(a, s) : run_bf16<128, 32, 1, 4>(a, s))
                  : (nw == 2 ? run_bf16<128, 64, 1, 2>(a, s) : run_bf16<128, 64, 1, 4>(a, s));
    return kt32 ? (nw == 2 ? run_bf16<64, 32, 1, 2>(a, s) : run_bf16<64, 32, 1, 4>(a, s))
                : (nw == 2 ? run_bf16<64, 64, 1, 2>(a, s) : run_bf16<64, 64, 1, 4>(a, s));
  }
  if (uses_pipe(a)) {
    constexpr int ROWS = w2::ROWS;
    const int wg_per_qb = (a.sel_heads * a.block + ROWS - 1) / ROWS;
    const int total = a.B * (a.Hq / a.sel_heads) * nqb * wg_per_qb;
    const int per_xcd = (total + kNumXcd - 1) / kNumXcd;
    // persistent workgroups, one per CU: contiguous item ranges per XCD, or
    // for the compressed branch (items differ in length, longest first)
    // every 256th item of the whole list (a workgroup per item instead
    // measured 3% slower: no item pipelining)
    const int grid = a.mode == MODE_CMP ? min(total, kNumXcd * kAttnSlotsPerXcd)
                                        : kNumXcd * min(per_xcd, kAttnSlotsPerXcd);
    if (a.key_bias)
      k_attn_bf16_d128_pipe<true><<<grid, w2::NT, 0, s>>>(a, wg_per_qb, nqb, per_xcd, total);
    else
      k_attn_bf16_d128_pipe<false><<<grid, w2::NT, 0, s>>>(a, wg_per_qb, nqb, per_xcd, total);
    return hipGetLastError();
  }
  if (uses_d128(a)) {
    constexpr int ROWS = d128::NW * 32;
    const int wg_per_qb = (a.sel_heads * a.block + ROWS - 1) / ROWS;
    const int total = a.B * (a.Hq / a.sel_heads) * nqb * wg_per_qb;
    const int per_xcd = (total + kNumXcd - 1) / kNumXcd;
    // one resident workgroup per CU (registers allow two waves per SIMD); the
    // compressed branch, whose items differ in length, keeps one workgroup
    // per item so that the dispatcher balances them
    const int grid = a.mode == MODE_CMP ? total : kNumXcd * min(per_xcd, kAttnSlotsPerXcd);
    if (a.key_bias)
      k_attn_bf16_d128<true><<<grid, d128::NT, 0, s>>>(a, wg_per_qb, nqb, per_xcd, total);
    else
      k_attn_bf16_d128<false><<<grid, d128::NT, 0, s>>>(a, wg_per_qb, nqb, per_xcd, total);
    return hipGetLastError();
  }
  if (a.D == 128)
    return kt32 ? run_bf16<128, 32, 1, kAttnWaves>(a, s) : run_bf16<128, 64, 1, kAttnWaves>(a, s);
  return kt32 ? run_bf16<64, 32, 1, kAttnWaves>(a, s) : run_bf16<64, 64, 1, kAttnWaves>(a, s);
}

}  // namespace dsa
