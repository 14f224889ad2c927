// Backward of block-sparse causal attention in index mode ([DMA] §四-§五: the
// sparse computation stays differentiable; positions the mask removes get
// exactly zero gradient, kept positions the ordinary softmax gradient).
//
// For a row t with visible keys, P = softmax(scale q_t.k_s) is recomputed
// from the forward's log-sum-exp, and with dP_s = do_t.v_s and
// D_t = do_t.o_t (k_bwd_rowterm):
//     dS_s = P_s (dP_s - D_t),   dq_t = scale sum_s dS_s k_s,
//     dk_s = scale sum_t dS_s q_t,   dv_s = sum_t P_s do_t.
// k_bwd_dq walks, per (group, query block), the key tiles of the selected
// blocks (the forward's index lists).  k_bwd_dkdv walks, per (group, key
// block), the query blocks that selected it; k_bwd_invert builds those
// lists from the forward's, ascending, so every gradient is a sum in a fixed
// order (no atomics) and runs are bit-reproducible.
//
// All products run on v_mfma_f32_32x32x16_bf16 over 32x32 tiles with float32
// accumulation; P and dS enter the second products rounded to bf16.  Tiles in
// LDS are row-major with rows padded to D + 8 elements; the transposed
// operands (K^T, Q^T, dO^T) come from ds_read_b64_tr_b16.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kT = 32;         // rows and keys per MFMA tile

#define DSA_LDS_BF16X4(p) ((__attribute__((address_space(3))) bf16x4*)(p))

__device__ __forceinline__ bf16x8 lds_b128(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// A operand of a transposed tile: lane l gets 8 entries of column
// (dim) c0 + l % 32 from rows k-group ks2: rows ks2*16 + {h*4 .. h*4+3} and
// ks2*16 + 8 + {h*4 .. h*4+3} with h = l / 32 (the key order the
// accumulator layout gives the matching B operand).  `base` points at the
// tile's row 0, `pitch` is the row pitch in elements.
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* base, int pitch, int ks2, int c0, int lane) {
  const int h = lane >> 5, g2 = (lane >> 4) & 1, r4 = (lane & 15) >> 2, c4 = lane & 3;
  const int col = c0 + g2 * 16 + c4 * 4;
  const uint16_t* p0 = base + (ks2 * 16 + h * 4 + r4) * pitch + col;
  const uint16_t* p1 = p0 + 8 * pitch;
  const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(DSA_LDS_BF16X4(p0));
  const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(DSA_LDS_BF16X4(p1));
  return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Accumulator row of register r for lane half h (32x32 tile).
__device__ __forceinline__ int acc_row(int r, int h) { return (r >> 2) * 8 + h * 4 + (r & 3); }

// Per row (rows = B*Hq*S; D/8 lanes per row): D_t = sum_d dO[t,d] O[t,d]
// and the forward's log-sum-exp in base 2, lse2_t = lse_t log2(e).
__global__ __launch_bounds__(256) void k_bwd_rowterm(const uint16_t* __restrict__ out,
                                                     const uint16_t* __restrict__ dout,
                                                     const float* __restrict__ lse, int rows,
                                                     int D, float* __restrict__ dt,
                                                     float* __restrict__ lse2) {
  const int lpr = D / 8;
  const int r = int((size_t(blockIdx.x) * 256 + threadIdx.x) / lpr);
  const int sub = threadIdx.x % lpr;
  float acc = 0.f;
  if (r < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(out + size_t(r) * D + sub * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dout + size_t(r) * D + sub * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += bf16lo(a[e]) * bf16lo(b[e]) + bf16hi(a[e]) * bf16hi(b[e]);
  }
  for (int o = lpr / 2; o > 0; o /= 2) acc += __shfl_xor(acc, o);
  if (r < rows && sub == 0) {
    dt[r] = acc;
    lse2[r] = lse[r] * kLog2e;
  }
}

// inv[bg, j, :inv_cnt] = ascending query blocks i whose index row lists key
// block j.  One wave per (group, key block); membership by binary search in
// the ascending row, compaction by ballots (index order).
__global__ __launch_bounds__(256) void k_bwd_invert(const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ count, int nbg,
                                                    int nb, int width, int32_t* __restrict__ inv,
                                                    int32_t* __restrict__ inv_cnt) {
  const int w = blockIdx.x * 4 + int(threadIdx.x >> 6);
  if (w >= nbg * nb) return;   // whole wave
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int bg = w / nb, j = w % nb;
  int total = 0;
  for (int i0 = j; i0 < nb; i0 += 64) {   // causal selection: only i >= j lists j
    const int i = i0 + lane;
    bool has = false;
    if (i < nb) {
      const int32_t* row = idx + (size_t(bg) * nb + i) * width;
      int lo = 0, hi = min(count[size_t(bg) * nb + i], width) - 1;
      while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        const int x = row[mid];
        if (x == j) {
          has = true;
          break;
        }
        if (x < j) lo = mid + 1;
        else hi = mid - 1;
      }
    }
    const uint64_t m = __ballot(has);
    if (has) inv[(size_t(bg) * nb + j) * nb + total + __popcll(m & below)] = i;
    total += __popcll(m);
  }
  if (lane == 0) inv_cnt[size_t(bg) * nb + j] = total;
}

// The backward's kernel arguments: the public call's tensors plus the
// workspace pieces (row terms and inverted lists).
struct BwdK {
  const uint16_t *q, *k, *v, *dout;
  const float* lse2;     // [B,Hq,S] forward log-sum-exp, base 2
  const float* dt;       // [B,Hq,S]
  const int32_t *idx, *count, *inv, *inv_cnt;
  int B, Hq, Hkv, S, block, idx_width, nqb;
  float scale;
  uint16_t *dq, *dk, *dv;
};

__device__ __forceinline__ bf16x8 ld_row8(const uint16_t* p, bool ok) {
  const u32x4 x = ok ? *reinterpret_cast<const u32x4*>(p) : u32x4{0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, x);
}

// dq for one (group, query block, slice of nw*32 rows): nw waves of 32 rows
// (rows enumerate head-major: row r -> head r / block, position r % block).
// Key tiles of 32 from the selected blocks; per tile S^T = K Q^T and
// dP^T = V dO^T (keys on accumulator rows, the lane's row on its column),
// dS^T = P^T (dP^T - D), dq^T += K^T dS^T.
template <int D>
__global__ __launch_bounds__(512) void k_bwd_dq(BwdK a, int wg_per_qb, int per_xcd, int total) {
  constexpr int PITCH = D + 8;
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint16_t kl[kT * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t vl[kT * PITCH];

  const int w = xcd_work_id(per_xcd);
  if (w >= total) return;               // whole workgroup, before any barrier
  const int nt = blockDim.x;
  const int sub = w % wg_per_qb;
  const int i = (w / wg_per_qb) % a.nqb, bg = (w / wg_per_qb) / a.nqb;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const float c = a.scale * kLog2e;

  const int r = (sub * (nt >> 6) + wave) * 32 + col;
  const int hh = r / a.block;
  const int t = i * a.block + r % a.block;
  const bool row_ok = hh < G && t < a.S;
  const size_t row = (size_t(b) * a.Hq + g * G + (row_ok ? hh : 0)) * a.S + (row_ok ? t : 0);
  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    qf[ks] = ld_row8(a.q + row * D + ks * 16 + half * 8, row_ok);
    df[ks] = ld_row8(a.dout + row * D + ks * 16 + half * 8, row_ok);
  }
  const float lse2 = row_ok ? a.lse2[row] : 0.f;
  const float dterm = row_ok ? a.dt[row] : 0.f;

  floatx16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.f;

  const int tpb = a.block / kT;
  const int32_t* irow = a.idx + (size_t(bg) * a.nqb + i) * a.idx_width;
  const int ntiles = min(a.count[size_t(bg) * a.nqb + i], a.idx_width) * tpb;
  const uint16_t* kg = a.k + size_t(bg) * a.S * D;
  const uint16_t* vg = a.v + size_t(bg) * a.S * D;

  for (int n = 0; n < ntiles; ++n) {
    const int key0 = irow[n / tpb] * a.block + (n % tpb) * kT;
    __syncthreads();   // the previous tile is consumed
    for (int e = threadIdx.x; e < kT * CPR; e += nt) {
      const int kr = e / CPR, cc = e % CPR;
      const bool ok = unsigned(key0 + kr) < unsigned(a.S);   // a bad list entry reads nothing
      const size_t off = size_t(ok ? key0 + kr : 0) * D + cc * 8;
      const u32x4 z = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&kl[kr * PITCH + cc * 8]) = ok ? *reinterpret_cast<const u32x4*>(kg + off) : z;
      *reinterpret_cast<u32x4*>(&vl[kr * PITCH + cc * 8]) = ok ? *reinterpret_cast<const u32x4*>(vg + off) : z;
    }
    __syncthreads();
    floatx16 s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(&kl[col * PITCH + ks * 16 + half * 8]), qf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(&vl[col * PITCH + ks * 16 + half * 8]), df[ks], dp, 0, 0, 0);
    }
    bf16x8 dsb[2];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int key = key0 + acc_row(rr, half);
      const bool vis = row_ok && key <= t && unsigned(key) < unsigned(a.S);
      const float p = vis ? fast_exp2(fmaf(s[rr], c, -lse2)) : 0.f;
      dsb[rr >> 3][rr & 7] = static_cast<__bf16>(p * (dp[rr] - dterm));
    }
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(kl, PITCH, ks2, dt * 32, lane), dsb[ks2], acc[dt], 0, 0, 0);
  }

  if (!row_ok) return;
  uint16_t* dst = a.dq + row * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      u32x2 pk;
      pk[0] = pack_bf16x2(acc[dt][r4 * 4 + 0] * a.scale, acc[dt][r4 * 4 + 1] * a.scale);
      pk[1] = pack_bf16x2(acc[dt][r4 * 4 + 2] * a.scale, acc[dt][r4 * 4 + 3] * a.scale);
      *reinterpret_cast<u32x2*>(dst + dt * 32 + r4 * 8 + half * 4) = pk;
    }
}

// dk, dv for one (group, key block): block / 32 waves, wave w owning keys
// 32w .. 32w + 31 of the block (K and V rows stay in LDS).  Walks every
// (query block that selected it, head of the group, 32-row tile) in that
// order; per tile S = Q K^T and dP = dO V^T (the tile's rows on accumulator
// rows, the lane's key on its column), P, dS = P (dP - D), then
// dv^T += dO^T P and dk^T += Q^T dS.
template <int D>
__global__ __launch_bounds__(512) void k_bwd_dkdv(BwdK a, int per_xcd, int total) {
  constexpr int PITCH = D + 8;
  constexpr int CPR = D / 8;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int w = xcd_work_id(per_xcd);
  if (w >= total) return;
  const int nt = blockDim.x;
  uint16_t* kl = smem;                           // [block][PITCH]
  uint16_t* vl = kl + a.block * PITCH;           // [block][PITCH]
  uint16_t* ql = vl + a.block * PITCH;           // [32][PITCH]
  uint16_t* dl = ql + kT * PITCH;                // [32][PITCH]
  float* lsel = reinterpret_cast<float*>(dl + kT * PITCH);   // [32] base-2 lse, +inf past S
  float* dtl = lsel + kT;                                      // [32]

  const int j = w % a.nqb, bg = w / a.nqb;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int lane = threadIdx.x & 63, kw = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const float c = a.scale * kLog2e;
  const uint16_t* kg = a.k + size_t(bg) * a.S * D;
  const uint16_t* vg = a.v + size_t(bg) * a.S * D;
  const int kb0 = j * a.block;
  const u32x4 z = u32x4{0u, 0u, 0u, 0u};

  for (int e = threadIdx.x; e < a.block * CPR; e += nt) {
    const int kr = e / CPR, cc = e % CPR;
    const bool ok = kb0 + kr < a.S;
    const size_t off = size_t(ok ? kb0 + kr : 0) * D + cc * 8;
    *reinterpret_cast<u32x4*>(&kl[kr * PITCH + cc * 8]) = ok ? *reinterpret_cast<const u32x4*>(kg + off) : z;
    *reinterpret_cast<u32x4*>(&vl[kr * PITCH + cc * 8]) = ok ? *reinterpret_cast<const u32x4*>(vg + off) : z;
  }

  floatx16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dka[dt][e] = 0.f;
      dva[dt][e] = 0.f;
    }

  const int key = kb0 + kw * kT + col;          // this lane's key
  const uint16_t* kme = &kl[(kw * kT + col) * PITCH];
  const uint16_t* vme = &vl[(kw * kT + col) * PITCH];
  const int32_t* inv = a.inv + (size_t(bg) * a.nqb + j) * a.nqb;
  const int rtp = a.block / kT;                 // 32-row tiles per query block
  const int ntiles = a.inv_cnt[size_t(bg) * a.nqb + j] * G * rtp;

  for (int n = 0; n < ntiles; ++n) {
    const int i = inv[n / (G * rtp)];
    const int h = (n / rtp) % G, rt = n % rtp;
    const int t0 = i * a.block + rt * kT;
    const size_t row0 = (size_t(b) * a.Hq + g * G + h) * a.S;
    __syncthreads();   // K/V staged (first tile) or the previous tile consumed
    for (int e = threadIdx.x; e < kT * CPR; e += nt) {
      const int rr = e / CPR, cc = e % CPR;
      const bool ok = t0 + rr < a.S;
      const size_t off = (row0 + (ok ? t0 + rr : 0)) * D + cc * 8;
      *reinterpret_cast<u32x4*>(&ql[rr * PITCH + cc * 8]) = ok ? *reinterpret_cast<const u32x4*>(a.q + off) : z;
      *reinterpret_cast<u32x4*>(&dl[rr * PITCH + cc * 8]) = ok ? *reinterpret_cast<const u32x4*>(a.dout + off) : z;
    }
    for (int rr = threadIdx.x; rr < kT; rr += nt) {
      const bool ok = t0 + rr < a.S;
      lsel[rr] = ok ? a.lse2[row0 + t0 + rr] : __builtin_inff();
      dtl[rr] = ok ? a.dt[row0 + t0 + rr] : 0.f;
    }
    __syncthreads();
    floatx16 s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(&ql[col * PITCH + ks * 16 + half * 8]),
                                                  lds_b128(kme + ks * 16 + half * 8), s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(&dl[col * PITCH + ks * 16 + half * 8]),
                                                   lds_b128(vme + ks * 16 + half * 8), dp, 0, 0, 0);
    }
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int qr = acc_row(rr, half);
      const int tt = t0 + qr;
      const bool vis = key <= tt && key < a.S && tt < a.S;
      const float p = vis ? fast_exp2(fmaf(s[rr], c, -lsel[qr])) : 0.f;
      pb[rr >> 3][rr & 7] = static_cast<__bf16>(p);
      dsb[rr >> 3][rr & 7] = static_cast<__bf16>(p * (dp[rr] - dtl[qr]));
    }
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        dva[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(dl, PITCH, ks2, dt * 32, lane), pb[ks2], dva[dt], 0, 0, 0);
        dka[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(ql, PITCH, ks2, dt * 32, lane), dsb[ks2], dka[dt], 0, 0, 0);
      }
  }

  if (key >= a.S) return;
  uint16_t* dko = a.dk + (size_t(bg) * a.S + key) * D;
  uint16_t* dvo = a.dv + (size_t(bg) * a.S + key) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      u32x2 pk, pv;
      pk[0] = pack_bf16x2(dka[dt][r4 * 4 + 0] * a.scale, dka[dt][r4 * 4 + 1] * a.scale);
      pk[1] = pack_bf16x2(dka[dt][r4 * 4 + 2] * a.scale, dka[dt][r4 * 4 + 3] * a.scale);
      pv[0] = pack_bf16x2(dva[dt][r4 * 4 + 0], dva[dt][r4 * 4 + 1]);
      pv[1] = pack_bf16x2(dva[dt][r4 * 4 + 2], dva[dt][r4 * 4 + 3]);
      *reinterpret_cast<u32x2*>(dko + dt * 32 + r4 * 8 + half * 4) = pk;
      *reinterpret_cast<u32x2*>(dvo + dt * 32 + r4 * 8 + half * 4) = pv;
    }
}

// ------------------------------------------------ D = 128, blocks of 64 / 128
// Tiles of 256-byte rows (128 bf16) are staged with direct-to-LDS loads
// (global_load_lds_dwordx4: lane l of a wave fills bytes 16 l .. 16 l + 15 of
// a 1 KB run, so one instruction moves four rows) into double buffers: the
// next tile streams in while the current one is used, one barrier per tile.
// Chunk c (16 bytes) of row r sits at byte r * 256 + ((c ^ swz(r)) << 4).
// With swz(r) = 4 (r mod 4) + (r / 4 mod 4):
//  * 16 lanes reading the same chunk of 16 consecutive rows (an MFMA operand
//    row per lane) hit 16 different 16-byte bank groups;
//  * a transposed read (ds_read_b64_tr_b16: 4 consecutive rows x 64 bytes
//    per 32 lanes) puts the four rows in four different 64-byte groups;
// so both ways of reading a tile are free of bank conflicts, and as the
// swizzle is an XOR, each read costs one v_xor on a per-lane base.
namespace f128 {
constexpr int D = 128, ROWB = 256;
constexpr int kDqList = 256;     // index-list entries a dq workgroup keeps in LDS
constexpr int kDkdvList = 1024;  // inverted-list entries a dk/dv workgroup keeps in LDS

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

typedef __attribute__((address_space(3))) void* lds_ptr;

// Direct-to-LDS loads (16 or 4 bytes per lane; lane l writes at dst + l *
// size, dst wave-uniform), written as inline assembly: issued through the
// builtin, the compiler waits for every one of them in flight before the
// next LDS read of any buffer, which would drain the prefetch of the next
// tile before the current one is used.  The kernels wait for them
// explicitly (wait_vm) instead.  They write no register, so nothing the
// compiler tracks is left in flight.
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t(dst)));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
}
// As dma16, from a wave-uniform base plus a per-lane 32-bit byte offset
// (the address lives in scalar registers; one vector register per lane).
__device__ __forceinline__ void dma16_base(const void* base, uint32_t off, void* dst) {
  const uint64_t b = uint64_t(uintptr_t(base));
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(b)));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(b >> 32)));
  const uint64_t sb = uint64_t(hi) << 32 | uint64_t(lo);
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t(dst)));
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sb), "s"(m0) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* src, void* dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t(dst)));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
}

// Rows 0..63 of a tile (src = row 0; rows >= nvalid read row nvalid - 1,
// which may lie before the tile when nvalid <= 0 but is always a real row)
// into dst[0 .. 16 KB); wave `wave` of `nw` issues runs wave, wave + nw, ...
__device__ __forceinline__ void dma_rows64(const uint16_t* src, int nvalid, uint8_t* dst, int wave,
                                           int nw, int lane) {
  const int cl = (lane & 15) ^ ((lane >> 4) << 2);
  for (int k = wave; k < 16; k += nw) {
    const int r = min(4 * k + (lane >> 4), nvalid - 1);
    const int c = cl ^ (k & 3);
    dma16(src + ptrdiff_t(r) * D + c * 8, dst + k * 1024);
  }
}

// Rows 0..63 of a tile that lies wholly inside the sequence.  Wave w of nw
// issues runs w + nw j; with nw a multiple of 4 the swizzle of every run is
// the same per lane, so one per-lane offset (dma_lane_off) serves them all.
__device__ __forceinline__ uint32_t dma_lane_off(int wave, int lane) {
  const int cl = (lane & 15) ^ ((lane >> 4) << 2);
  return uint32_t((4 * wave + (lane >> 4)) * ROWB + ((cl ^ (wave & 3)) << 4));
}
__device__ __forceinline__ void dma_rows64_full(const uint16_t* src, uint8_t* dst, int wave, int nw,
                                                uint32_t lane_off) {
  const uint8_t* s8 = reinterpret_cast<const uint8_t*>(src) + lane_off;
  for (int k = wave, j = 0; k < 16; k += nw, ++j)
    dma16(s8 + j * nw * 4 * ROWB, dst + k * 1024);
}

// MFMA operand (8 bf16 of one row) at per-lane base `base` (row * 256 with
// the row's swizzle and the lane half folded in) for k-step ks.
__device__ __forceinline__ bf16x8 rd_row(const uint8_t* buf, uint32_t base, int ks) {
  return *reinterpret_cast<const bf16x8*>(buf + (base ^ uint32_t(ks << 5)));
}

// Per-lane base of rd_row for tile row `row`.
__device__ __forceinline__ uint32_t row_base(int row, int half) {
  return uint32_t(row * ROWB) | uint32_t((swz(row) ^ half) << 4);
}

// Transposed operand (see tr_operand) from a swizzled tile: rows
// r0 + ks2 * 16 + {h*4 .. h*4+3, 8 + h*4 ..}, dims dt * 32 + lane % 32.
// lt0 / lt8 are the per-lane bases of the two row groups (tr_bases).
__device__ __forceinline__ bf16x8 rd_tr(const uint8_t* buf, uint32_t lt0, uint32_t lt8, int ks2, int dt) {
  const uint32_t x = uint32_t(dt << 6);
  const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      DSA_LDS_BF16X4(buf + ks2 * 16 * ROWB + (lt0 ^ x)));
  const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      DSA_LDS_BF16X4(buf + ks2 * 16 * ROWB + (lt8 ^ x)));
  return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void tr_bases(int r0, int lane, uint32_t& lt0, uint32_t& lt8) {
  const int h = lane >> 5, g2 = (lane >> 4) & 1, r4 = (lane & 15) >> 2, c4 = lane & 3;
  const int low = g2 * 2 + (c4 >> 1);
  const int ra = r0 + h * 4 + r4, rb = ra + 8;
  lt0 = uint32_t(ra * ROWB) | uint32_t((low ^ swz(ra)) << 4) | uint32_t((c4 & 1) << 3);
  lt8 = uint32_t(rb * ROWB) | uint32_t((low ^ swz(rb)) << 4) | uint32_t((c4 & 1) << 3);
}

// Workgroup barrier for the staged loops: waits for this wave's LDS
// operations only.  The direct-to-LDS loads are waited for explicitly
// (wait_vm) before it, so a load still streaming into another buffer does
// not hold the barrier, as a full fence would.  The memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N) (N < 16): all but this wave's last N vector-memory
// operations have completed (they complete in issue order)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

}  // namespace f128

// dq, D = 128: as k_bwd_dq, with 64-key steps (two 32-key halves per wave)
// and K/V tiles staged by direct-to-LDS loads into two buffers.
template <int BLK>
__global__ __launch_bounds__(512) void k_bwd_dq_d128(BwdK a, int wg_per_qb, int per_xcd, int total) {
  using namespace f128;
  constexpr int NW = 8, SPB = BLK / 64;   // 64-key steps per selected block
  __shared__ __attribute__((aligned(1024))) uint8_t kv0[2 * 64 * ROWB];   // K rows, then V rows
  __shared__ __attribute__((aligned(1024))) uint8_t kv1[2 * 64 * ROWB];
  __shared__ int lst[kDqList];            // the selected blocks (the launcher checks they fit)

  const int w = xcd_work_id(per_xcd);
  if (w >= total) return;
  const int sub = w % wg_per_qb;
  const int i = (w / wg_per_qb) % a.nqb, bg = (w / wg_per_qb) / a.nqb;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int col = lane & 31, half = lane >> 5;
  const float c = a.scale * kLog2e;

  const int r = (sub * NW + wave) * 32 + col;
  const int hh = r / BLK;
  const int t = i * BLK + r % BLK;
  const bool row_ok = hh < G && t < a.S;
  const size_t row = (size_t(b) * a.Hq + g * G + (row_ok ? hh : 0)) * a.S + (row_ok ? t : 0);
  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    qf[ks] = ld_row8(a.q + row * D + ks * 16 + half * 8, row_ok);
    df[ks] = ld_row8(a.dout + row * D + ks * 16 + half * 8, row_ok);
  }
  const float lse2 = row_ok ? a.lse2[row] : 0.f;
  const float dterm = row_ok ? a.dt[row] : 0.f;
  const int tlim = row_ok ? min(t, a.S - 1) : -1;   // last visible key of this row

  floatx16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.f;

  const int32_t* irow = a.idx + (size_t(bg) * a.nqb + i) * a.idx_width;
  const int cnt = min(a.count[size_t(bg) * a.nqb + i], a.idx_width);
  const int nsteps = cnt * SPB;
  const uint16_t* kg = a.k + size_t(bg) * a.S * D;
  const uint16_t* vg = a.v + size_t(bg) * a.S * D;
  auto key0_of = [&](int entry, int n) __attribute__((always_inline)) {
    return entry * BLK + (n % SPB) * 64;
  };
  const uint32_t dma_off = dma_lane_off(wave, lane);
  auto stage = [&](int key0, uint8_t* dst) __attribute__((always_inline)) {
    if (key0 >= 0 && key0 + 64 <= a.S) {
      dma_rows64_full(kg + size_t(key0) * D, dst, wave, NW, dma_off);
      dma_rows64_full(vg + size_t(key0) * D, dst + 64 * ROWB, wave, NW, dma_off);
    } else {
      const int k0 = min(max(key0, 0), a.S - 1);   // a bad list entry reads in bounds
      dma_rows64(kg + size_t(k0) * D, a.S - k0, dst, wave, NW, lane);
      dma_rows64(vg + size_t(k0) * D, a.S - k0, dst + 64 * ROWB, wave, NW, lane);
    }
  };

  auto step = [&](int key0, const uint8_t* cur) __attribute__((always_inline)) {
#pragma unroll 1
    for (int kh = 0; kh < 2; ++kh) {
      const uint32_t la = row_base(kh * 32 + col, half);
      uint32_t lt0, lt8;
      tr_bases(kh * 32, lane, lt0, lt8);
      floatx16 s = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_row(cur, la, ks), qf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_row(cur + 64 * ROWB, la, ks), df[ks], dp, 0, 0, 0);
      }
      bf16x8 dsb[2];
      // key key0 + 32 kh + acc_row(rr, half) is visible iff it is <= tlim
      const int lim = tlim - key0 - kh * 32 - half * 4;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const bool vis = (rr >> 2) * 8 + (rr & 3) <= lim;
        const float p = vis ? fast_exp2(fmaf(s[rr], c, -lse2)) : 0.f;
        dsb[rr >> 3][rr & 7] = static_cast<__bf16>(p * (dp[rr] - dterm));
      }
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_tr(cur, lt0, lt8, ks2, dt), dsb[ks2], acc[dt], 0, 0, 0);
    }
  };

  // Two buffers: tile n + 1 streams in while tile n is used.  The list
  // sits in LDS, so finding a tile's keys costs no memory round trip.
  if (nsteps > 0) {
    for (int e = threadIdx.x; e < cnt; e += NW * 64) lst[e] = irow[e];
    __syncthreads();
    auto entry = [&](int n) __attribute__((always_inline)) { return lst[n / SPB]; };
    int k0 = key0_of(entry(0), 0), k1 = 0;
    stage(k0, kv0);
    wait_vm<0>();
    __syncthreads();
    auto phase = [&](int n, int& kc, const uint8_t* cb, int& kp, uint8_t* pb) __attribute__((always_inline)) {
      const bool pf = n + 1 < nsteps;
      if (pf) {
        kp = key0_of(entry(n + 1), n + 1);
        stage(kp, pb);
      }
      step(kc, cb);
      wait_vm<0>();   // tile n + 1 has landed (each wave waits for its own loads)
      lds_barrier();
    };
    for (int n = 0; n < nsteps; n += 2) {
      phase(n, k0, kv0, k1, kv1);
      if (n + 1 >= nsteps) break;
      phase(n + 1, k1, kv1, k0, kv0);
    }
  }

  if (!row_ok) return;
  uint16_t* dst = a.dq + row * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      u32x2 pk;
      pk[0] = pack_bf16x2(acc[dt][r4 * 4 + 0] * a.scale, acc[dt][r4 * 4 + 1] * a.scale);
      pk[1] = pack_bf16x2(acc[dt][r4 * 4 + 2] * a.scale, acc[dt][r4 * 4 + 3] * a.scale);
      *reinterpret_cast<u32x2*>(dst + dt * 32 + r4 * 8 + half * 4) = pk;
    }
}

// dk, dv, D = 128: as k_bwd_dkdv, with 64-row steps shared by four waves
// (wave w: keys 32 (w mod BLK/32) .. and the rows 32 r .. of each step with
// r = w div (BLK/32) for BLK 64, both halves in turn for BLK 128); K and V
// stay in LDS, Q and dO tiles stream through direct-to-LDS buffers (three
// for BLK 64, two for BLK 128), the row terms through registers of wave 0.
template <int BLK>
__global__ __launch_bounds__(256) void k_bwd_dkdv_d128(BwdK a, int per_xcd, int total) {
  using namespace f128;
  // four waves: BLK 64 -> 2 key tiles x 2 row halves; BLK 128 -> 4 key tiles,
  // each wave taking both row halves of a step in turn
  constexpr int NKT = BLK / 32, NW = 4, RH = NW / NKT, RTP = BLK / 64;
  constexpr int NB = BLK == 64 ? 3 : 2;   // Q/dO buffers (LDS: 2 BLK + 64 NB rows of 512 B)
  __shared__ __attribute__((aligned(1024))) uint8_t kv[2 * BLK * ROWB];   // K rows, then V rows
  // a tile buffer: Q rows, dO rows, then the row terms (lse, D) of its rows
  constexpr int QDB = 2 * 64 * ROWB + 2 * 64 * 4;
  __shared__ __attribute__((aligned(1024))) uint8_t qd0[QDB];
  __shared__ __attribute__((aligned(1024))) uint8_t qd1[QDB];
  __shared__ __attribute__((aligned(1024))) uint8_t qd2[NB == 3 ? QDB : 1024];
  float* const rt0 = reinterpret_cast<float*>(qd0 + 2 * 64 * ROWB);
  float* const rt1 = reinterpret_cast<float*>(qd1 + 2 * 64 * ROWB);
  float* const rt2 = reinterpret_cast<float*>(qd2 + (NB == 3 ? 2 * 64 * ROWB : 0));
  __shared__ int lst[kDkdvList];          // the inverted list (the launcher checks it fits)

  const int w = xcd_work_id(per_xcd);
  if (w >= total) return;
  const int j = w % a.nqb, bg = w / a.nqb;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int kt = wave % NKT, rh0 = wave / NKT;
  const int col = lane & 31, half = lane >> 5;
  const float c = a.scale * kLog2e;
  const int kb0 = j * BLK;

  floatx16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dka[dt][e] = 0.f;
      dva[dt][e] = 0.f;
    }

  const int key = kb0 + kt * 32 + col;          // this lane's key
  const int32_t* inv = a.inv + (size_t(bg) * a.nqb + j) * a.nqb;
  const int nsteps = a.inv_cnt[size_t(bg) * a.nqb + j] * G * RTP;

  // tile n: query block inv[n / (G RTP)], head (n / RTP) mod G, rows 64 (n mod RTP) ..
  struct Tile { int t0; size_t row0; };
  auto tile_of = [&](int i, int n) __attribute__((always_inline)) -> Tile {
    const int h = (n / RTP) % G;
    return Tile{i * BLK + (n % RTP) * 64, (size_t(b) * a.Hq + g * G + h) * a.S};
  };
  const uint32_t dma_off = dma_lane_off(wave, lane);
  auto stage = [&](const Tile& tl, uint8_t* dst) __attribute__((always_inline)) {
    const int nv = a.S - tl.t0;
    if (nv >= 64) {
      dma_rows64_full(a.q + (tl.row0 + tl.t0) * D, dst, wave, NW, dma_off);
      dma_rows64_full(a.dout + (tl.row0 + tl.t0) * D, dst + 64 * ROWB, wave, NW, dma_off);
    } else {
      dma_rows64(a.q + (tl.row0 + tl.t0) * D, nv, dst, wave, NW, lane);
      dma_rows64(a.dout + (tl.row0 + tl.t0) * D, nv, dst + 64 * ROWB, wave, NW, lane);
    }
  };
  // row terms of a tile (base-2 lse, then D), streamed by wave 0: one row
  // per lane, rows past S read row S - 1 (their weights are masked)
  auto stage_rt = [&](const Tile& tl, float* dst) __attribute__((always_inline)) {
    if (wave == 0) {
      const size_t rr = tl.row0 + min(tl.t0 + lane, a.S - 1);
      dma4(a.lse2 + rr, dst);
      dma4(a.dt + rr, dst + 64);
    }
  };

  const uint32_t lb = row_base(kt * 32 + col, half);       // K / V rows (B operand)

  // this wave's K and V rows (the B operands of every step), loaded once
  bf16x8 kf[D / 16], vf[D / 16];

  // One step: every LDS operand of a product is requested before the
  // product starts, so a single wave per SIMD is not left waiting on LDS
  // latency between the MFMAs.
  auto step = [&](int t0, const uint8_t* cur, const float* rtc) __attribute__((always_inline)) {
#pragma unroll 1
   for (int rh = rh0; rh < 2; rh += RH) {
    const uint32_t la = row_base(rh * 32 + col, half);     // Q / dO rows (A operand)
    uint32_t lt0, lt8;
    tr_bases(rh * 32, lane, lt0, lt8);                     // Q^T / dO^T (transposed A)
    bf16x8 qa[D / 16], da[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qa[ks] = rd_row(cur, la, ks);
      da[ks] = rd_row(cur + 64 * ROWB, la, ks);
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the requests ahead of the products
    floatx16 s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ks], kf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[ks], vf[ks], dp, 0, 0, 0);
    }
    bf16x8 tq[2][D / 32], td[2][D / 32];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        td[ks2][dt] = rd_tr(cur + 64 * ROWB, lt0, lt8, ks2, dt);
        tq[ks2][dt] = rd_tr(cur, lt0, lt8, ks2, dt);
      }
    __builtin_amdgcn_sched_barrier(0);   // ... and ahead of the softmax arithmetic
    bf16x8 pb[2], dsb[2];
    // every row of this wave's half at or after every key of its tile, all
    // inside the sequence: no masking
    const int r_lo = t0 + rh * 32, k_hi = kb0 + kt * 32 + 31;
    const bool full = k_hi <= r_lo && r_lo + 31 < a.S && k_hi < a.S;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int qr0 = rh * 32 + q4 * 8 + half * 4;
      const floatx4 l4 = *reinterpret_cast<const floatx4*>(rtc + qr0);
      const floatx4 d4 = *reinterpret_cast<const floatx4*>(rtc + 64 + qr0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = q4 * 4 + e;
        if (full) {
          const float p = fast_exp2(fmaf(s[rr], c, -l4[e]));
          pb[rr >> 3][rr & 7] = static_cast<__bf16>(p);
          dsb[rr >> 3][rr & 7] = static_cast<__bf16>(p * (dp[rr] - d4[e]));
        } else {
          const int tt = t0 + qr0 + e;
          const bool vis = key <= tt && key < a.S && tt < a.S;
          const float p = vis ? fast_exp2(fmaf(s[rr], c, -l4[e])) : 0.f;
          pb[rr >> 3][rr & 7] = static_cast<__bf16>(p);
          dsb[rr >> 3][rr & 7] = static_cast<__bf16>(vis ? p * (dp[rr] - d4[e]) : 0.f);
        }
      }
    }
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        dva[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(td[ks2][dt], pb[ks2], dva[dt], 0, 0, 0);
        dka[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[ks2][dt], dsb[ks2], dka[dt], 0, 0, 0);
      }
   }
  };

  if (nsteps > 0) {
    const int nv = a.S - kb0;
    const uint16_t* kg = a.k + (size_t(bg) * a.S + kb0) * D;
    const uint16_t* vg = a.v + (size_t(bg) * a.S + kb0) * D;
#pragma unroll
    for (int part = 0; part < RTP; ++part) {
      dma_rows64(kg + size_t(part) * 64 * D, nv - part * 64, kv + part * 64 * ROWB, wave, NW, lane);
      dma_rows64(vg + size_t(part) * 64 * D, nv - part * 64, kv + (BLK + part * 64) * ROWB, wave, NW, lane);
    }
    // NB buffers: tile n + NB - 1 streams in while tile n is used.  The
    // list sits in LDS, so finding a tile's rows costs no memory round trip;
    // the row terms stream like the rows (direct-to-LDS, one float a lane).
    const int ninv = nsteps / (G * RTP);
    for (int e = threadIdx.x; e < ninv; e += NW * 64) lst[e] = inv[e];
    __syncthreads();
    auto entry = [&](int n) __attribute__((always_inline)) { return lst[n / (G * RTP)]; };
    constexpr int kOps = 8;   // direct-to-LDS loads per wave and tile (16 runs each of Q, dO over 4 waves)
    Tile T0 = tile_of(entry(0), 0), T1 = T0, T2 = T0;
    stage_rt(T0, rt0);
    stage(T0, qd0);
    if (NB == 3 && nsteps > 1) {
      T1 = tile_of(entry(1), 1);
      stage_rt(T1, rt1);
      stage(T1, qd1);
    }
    wait_vm<0>();
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      kf[ks] = rd_row(kv, lb, ks);
      vf[ks] = rd_row(kv + BLK * ROWB, lb, ks);
    }
    auto phase = [&](int n, const Tile& tc, const uint8_t* cb, const float* cr, Tile& tp, uint8_t* pb,
                     float* pr) __attribute__((always_inline)) {
      const int m = n + NB - 1;
      const bool pf = m < nsteps;
      if (pf) {
        tp = tile_of(entry(m), m);
        stage_rt(tp, pr);
        stage(tp, pb);
      }
      step(tc.t0, cb, cr);
      // tile n + 1 has landed (each wave waits for its own loads); with three
      // buffers the eight row loads of tile n + 2, issued last, may still be
      // in flight
      if (NB == 3 && pf) wait_vm<kOps>();
      else wait_vm<0>();
      lds_barrier();
    };
    for (int n = 0; n < nsteps; n += NB) {
      if constexpr (NB == 3) {
        phase(n, T0, qd0, rt0, T2, qd2, rt2);
        if (n + 1 >= nsteps) break;
        phase(n + 1, T1, qd1, rt1, T0, qd0, rt0);
        if (n + 2 >= nsteps) break;
        phase(n + 2, T2, qd2, rt2, T1, qd1, rt1);
      } else {
        phase(n, T0, qd0, rt0, T1, qd1, rt1);
        if (n + 1 >= nsteps) break;
        phase(n + 1, T1, qd1, rt1, T0, qd0, rt0);
      }
    }
  }

  if constexpr (RH == 2) {
    // the second row half's waves hand their sums to the first half's
    // (the Q/dO buffers are free: the last step ended with a barrier)
    float* xk = reinterpret_cast<float*>(qd0) + kt * 64 * 64 + lane;
    float* xv = reinterpret_cast<float*>(qd1) + kt * 64 * 64 + lane;
    if (rh0 == 1) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          xk[(dt * 16 + e) * 64] = dka[dt][e];
          xv[(dt * 16 + e) * 64] = dva[dt][e];
        }
    }
    __syncthreads();
    if (rh0 == 1) return;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        dka[dt][e] += xk[(dt * 16 + e) * 64];
        dva[dt][e] += xv[(dt * 16 + e) * 64];
      }
  }

  if (key >= a.S) return;
  uint16_t* dko = a.dk + (size_t(bg) * a.S + key) * D;
  uint16_t* dvo = a.dv + (size_t(bg) * a.S + key) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      u32x2 pk, pv;
      pk[0] = pack_bf16x2(dka[dt][r4 * 4 + 0] * a.scale, dka[dt][r4 * 4 + 1] * a.scale);
      pk[1] = pack_bf16x2(dka[dt][r4 * 4 + 2] * a.scale, dka[dt][r4 * 4 + 3] * a.scale);
      pv[0] = pack_bf16x2(dva[dt][r4 * 4 + 0], dva[dt][r4 * 4 + 1]);
      pv[1] = pack_bf16x2(dva[dt][r4 * 4 + 2], dva[dt][r4 * 4 + 3]);
      *reinterpret_cast<u32x2*>(dko + dt * 32 + r4 * 8 + half * 4) = pk;
      *reinterpret_cast<u32x2*>(dvo + dt * 32 + r4 * 8 + half * 4) = pv;
    }
}

// dk, dv, D = 128, blocks of 64: eight waves in pairs.  For key tile kt and
// row half rh, wave A (waves 0..3) computes S = Q K^T, P and dv^T += dO^T P;
// wave B (waves 4..7) computes dP = dO V^T, dS = P (dP - D) with A's P
// (the bf16 values A's own product takes, through LDS) and dk^T += Q^T dS.
// Each wave holds one accumulator set and one fixed operand (K or V rows),
// so two waves fit a SIMD and one's softmax and operand reads run beside the
// other's products (a single wave holding both sets keeps the matrix core
// about a quarter busy).  Tiles and summation order are those of
// k_bwd_dkdv_d128; dS differs from it only by the bf16 rounding of P.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_bwd_dkdv_pair(BwdK a, int per_xcd, int total) {
  using namespace f128;
  constexpr int BLK = 64, NKT = BLK / 32, NW = 8, NB = 3;
  __shared__ __attribute__((aligned(1024))) uint8_t kv[2 * BLK * ROWB];   // K rows, then V rows
  // a tile buffer: Q rows, dO rows, then the row terms (lse, D) of its rows
  constexpr int QDB = 2 * 64 * ROWB + 2 * 64 * 4 + 512;   // (padded to a multiple of 1 KB)
  __shared__ __attribute__((aligned(1024))) uint8_t qd[NB][QDB];
  auto rt_of = [&](int buf) __attribute__((always_inline)) {
    return reinterpret_cast<float*>(&qd[buf][2 * 64 * ROWB]);
  };
  // a pair's P in bf16 (the operand A multiplies with), by step parity:
  // group h of lane l's 16 values at [h][l] (consecutive lanes in
  // consecutive 16-byte slots: no bank conflicts)
  __shared__ __attribute__((aligned(16))) bf16x8 xp[2][NW / 2][2][64];
  __shared__ int lst[kDkdvList];          // the inverted list (the launcher checks it fits)

  const int w = xcd_work_id(per_xcd);
  if (w >= total) return;
  const int j = w % a.nqb, bg = w / a.nqb;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const bool role_b = wave >= NW / 2;     // uniform
  const int pr = wave % (NW / 2);         // the pair: waves pr and pr + 4 share a SIMD
  const int kt = pr % NKT, rh = pr / NKT;
  const int col = lane & 31, half = lane >> 5;
  const float c = a.scale * kLog2e;
  const int kb0 = j * BLK;

  floatx16 acc[D / 32];   // dv^T (A) or dk^T (B)
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.f;

  const int key = kb0 + kt * 32 + col;          // this lane's key
  const int32_t* inv = a.inv + (size_t(bg) * a.nqb + j) * a.nqb;
  const int nsteps = a.inv_cnt[size_t(bg) * a.nqb + j] * G;

  // tile n: query block inv[n / G], head n mod G, its 64 rows
  struct Tile { int t0; size_t row0; };
  auto tile_of = [&](int i, int n) __attribute__((always_inline)) -> Tile {
    return Tile{i * BLK, (size_t(b) * a.Hq + g * G + n % G) * a.S};
  };
  const uint32_t dma_off = dma_lane_off(wave, lane);
  auto stage = [&](const Tile& tl, uint8_t* dst) __attribute__((always_inline)) {
    const int nv = a.S - tl.t0;
    if (nv >= 64) {   // runs wave and wave + 8 of each array (see dma_rows64_full)
      const uint8_t* qs = reinterpret_cast<const uint8_t*>(a.q + (tl.row0 + tl.t0) * D);
      const uint8_t* ds = reinterpret_cast<const uint8_t*>(a.dout + (tl.row0 + tl.t0) * D);
#pragma unroll
      for (int jr = 0; jr < 16 / NW; ++jr) {
        dma16_base(qs + jr * NW * 4 * ROWB, dma_off, dst + (wave + jr * NW) * 1024);
        dma16_base(ds + jr * NW * 4 * ROWB, dma_off, dst + 64 * ROWB + (wave + jr * NW) * 1024);
      }
    } else {
      dma_rows64(a.q + (tl.row0 + tl.t0) * D, nv, dst, wave, NW, lane);
      dma_rows64(a.dout + (tl.row0 + tl.t0) * D, nv, dst + 64 * ROWB, wave, NW, lane);
    }
  };
  // row terms of a tile (base-2 lse, then D), streamed by wave 0: one row
  // per lane, rows past S read row S - 1 (their weights are masked)
  auto stage_rt = [&](const Tile& tl, float* dst) __attribute__((always_inline)) {
    if (wave == 0) {
      const size_t rr = tl.row0 + min(tl.t0 + lane, a.S - 1);
      dma4(a.lse2 + rr, dst);
      dma4(a.dt + rr, dst + 64);
    }
  };

  const uint32_t lb = row_base(kt * 32 + col, half);       // K / V rows (B operand)
  const uint32_t la = row_base(rh * 32 + col, half);       // Q / dO rows (A operand)
  uint32_t lt0, lt8;
  tr_bases(rh * 32, lane, lt0, lt8);                       // Q^T / dO^T (transposed A operand)
  bf16x8 kvf[D / 16];   // A: this wave's K rows; B: its V rows

  // The second products trail the first by one step: the P that A parks in
  // step n is published by the barrier that ends the step, and B forms dS
  // from it in step n + 1, from its dP - D of step n; each wave holds its
  // transposed operands (and A its P) of step n in registers until then.
  // One barrier per step.
  bf16x8 trp[2][D / 32];     // the previous step's transposed operands
  bf16x8 opp[2];             // A: the previous step's P in bf16
  floatx16 xprev;            // B: the previous step's dP - D
  auto second_prev = [&](int ppar) __attribute__((always_inline)) {
    bf16x8 op[2];
    if (role_b) {
      const bf16x8 pb[2] = {xp[ppar][pr][0][lane], xp[ppar][pr][1][lane]};
#pragma unroll
      for (int rr = 0; rr < 16; ++rr)   // a hidden pair has P = 0, so its dS is 0 as well
        op[rr >> 3][rr & 7] = static_cast<__bf16>(static_cast<float>(pb[rr >> 3][rr & 7]) * xprev[rr]);
    } else {
      op[0] = opp[0];
      op[1] = opp[1];
    }
    // dO^T P (A) or Q^T dS (B)
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(trp[ks2][dt], op[ks2], acc[dt], 0, 0, 0);
  };

  // One step: A requests its Q operands, B its dO operands; the previous
  // step's second product; the first product (S or dP) and, under it, this
  // step's transposed operands (dO^T for A, Q^T for B); A forms P and parks
  // it, B keeps dP - D.
  auto step = [&](int t0, const uint8_t* cur, const float* rtc, int par, bool prev)
      __attribute__((always_inline)) {
    const uint8_t* rows = cur + (role_b ? 64 * ROWB : 0);
    const uint8_t* trs = cur + (role_b ? 0 : 64 * ROWB);
    // the per-lane operand addresses are formed here, each step, rather than
    // kept live for every buffer across the loop
    uint32_t la_ = la, lt0_ = lt0, lt8_ = lt8;
    asm volatile("" : "+v"(la_), "+v"(lt0_), "+v"(lt8_));
    bf16x8 ra[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) ra[ks] = rd_row(rows, la_, ks);
    __builtin_amdgcn_sched_barrier(0);   // keep the requests ahead of the products
    if (prev) second_prev(par ^ 1);
    floatx16 x = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[ks], kvf[ks], x, 0, 0, 0);
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) trp[ks2][dt] = rd_tr(trs, lt0_, lt8_, ks2, dt);
    __builtin_amdgcn_sched_barrier(0);   // ... and ahead of the softmax arithmetic
    if (!role_b) {
      // every row of this half at or after every key of its tile, all inside
      // the sequence: no masking
      const int r_lo = t0 + rh * 32, k_hi = kb0 + kt * 32 + 31;
      const bool full = k_hi <= r_lo && r_lo + 31 < a.S && k_hi < a.S;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int qr0 = rh * 32 + q4 * 8 + half * 4;
        const floatx4 l4 = *reinterpret_cast<const floatx4*>(rtc + qr0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = q4 * 4 + e;
          float p;
          if (full) {
            p = fast_exp2(fmaf(x[rr], c, -l4[e]));
          } else {
            const int tt = t0 + qr0 + e;
            const bool vis = key <= tt && key < a.S && tt < a.S;
            p = vis ? fast_exp2(fmaf(x[rr], c, -l4[e])) : 0.f;
          }
          opp[rr >> 3][rr & 7] = static_cast<__bf16>(p);
        }
      }
      xp[par][pr][0][lane] = opp[0];
      xp[par][pr][1][lane] = opp[1];
    } else {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int qr0 = rh * 32 + q4 * 8 + half * 4;
        const floatx4 d4 = *reinterpret_cast<const floatx4*>(rtc + 64 + qr0);
#pragma unroll
        for (int e = 0; e < 4; ++e) xprev[q4 * 4 + e] = x[q4 * 4 + e] - d4[e];
      }
    }
  };

  if (nsteps > 0) {
    const int nv = a.S - kb0;
    dma_rows64(a.k + (size_t(bg) * a.S + kb0) * D, nv, kv, wave, NW, lane);
    dma_rows64(a.v + (size_t(bg) * a.S + kb0) * D, nv, kv + BLK * ROWB, wave, NW, lane);
    // NB buffers: tile n + 2 streams in while tile n is used.  The list sits
    // in LDS, so finding a tile's rows costs no memory round trip; the row
    // terms stream like the rows (direct-to-LDS, one float a lane).
    const int ninv = nsteps / G;
    for (int e = threadIdx.x; e < ninv; e += NW * 64) lst[e] = inv[e];
    __syncthreads();
    auto entry = [&](int n) __attribute__((always_inline)) { return lst[n / G]; };
    constexpr int kOps = 4;   // direct-to-LDS row loads per wave and tile (16 runs each of Q, dO over 8 waves)
    {
      const Tile t = tile_of(entry(0), 0);
      stage_rt(t, rt_of(0));
      stage(t, qd[0]);
    }
    if (nsteps > 1) {
      const Tile t = tile_of(entry(1), 1);
      stage_rt(t, rt_of(1));
      stage(t, qd[1]);
    }
    wait_vm<0>();
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) kvf[ks] = rd_row(kv + (role_b ? BLK * ROWB : 0), lb, ks);
    // one loop body (the buffer of tile n is n mod NB, kept as a rotating
    // index), so the accumulators stay in one set of registers
    int cb = 0;
    for (int n = 0; n < nsteps; ++n) {
      const int pbuf = cb == 0 ? NB - 1 : cb - 1;   // (n + NB - 1) mod NB
      const bool pf = n + NB - 1 < nsteps;
      if (pf) {
        const Tile tp = tile_of(entry(n + NB - 1), n + NB - 1);
        stage_rt(tp, rt_of(pbuf));
        stage(tp, qd[pbuf]);
      }
      step(entry(n) * BLK, qd[cb], rt_of(cb), n & 1, n > 0);
      // tile n + 1 has landed (each wave waits for its own loads); the row
      // loads of tile n + 2, issued last, may still be in flight
      if (pf) wait_vm<kOps>();
      else wait_vm<0>();
      lds_barrier();
      cb = cb == NB - 1 ? 0 : cb + 1;
    }
    // the last step's second products (B's P was published by the last
    // barrier)
    second_prev((nsteps - 1) & 1);
  }

  // the second row half's waves hand their sums to the first half's (the
  // tile buffers are free: the last step ended with a barrier)
  float* xs = reinterpret_cast<float*>(qd[role_b ? 1 : 0]) + kt * 64 * 64 + lane;
  if (rh == 1) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) xs[(dt * 16 + e) * 64] = acc[dt][e];
  }
  __syncthreads();
  if (rh == 1) return;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] += xs[(dt * 16 + e) * 64];

  if (key >= a.S) return;
  const float sc = role_b ? a.scale : 1.f;
  uint16_t* dst = (role_b ? a.dk : a.dv) + (size_t(bg) * a.S + key) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      u32x2 pk;
      pk[0] = pack_bf16x2(acc[dt][r4 * 4 + 0] * sc, acc[dt][r4 * 4 + 1] * sc);
      pk[1] = pack_bf16x2(acc[dt][r4 * 4 + 2] * sc, acc[dt][r4 * 4 + 3] * sc);
      *reinterpret_cast<u32x2*>(dst + dt * 32 + r4 * 8 + half * 4) = pk;
    }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

template <int BLK>
hipError_t launch_d128(const BwdK& k, hipStream_t s) {
  const int nbg = k.B * k.Hkv;
  const int rows = (k.Hq / k.Hkv) * BLK;
  const int wg_per_qb = (rows + 255) / 256;
  const int total_q = nbg * k.nqb * wg_per_qb;
  const int per_xcd_q = (total_q + kNumXcd - 1) / kNumXcd;
  k_bwd_dq_d128<BLK><<<per_xcd_q * kNumXcd, 512, 0, s>>>(k, wg_per_qb, per_xcd_q, total_q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int total_k = nbg * k.nqb;
  const int per_xcd_k = (total_k + kNumXcd - 1) / kNumXcd;
  if constexpr (BLK == 64)
    k_bwd_dkdv_pair<<<per_xcd_k * kNumXcd, 512, 0, s>>>(k, per_xcd_k, total_k);
  else
    k_bwd_dkdv_d128<BLK><<<per_xcd_k * kNumXcd, 256, 0, s>>>(k, per_xcd_k, total_k);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BwdK& k, hipStream_t s) {
  const int G = k.Hq / k.Hkv;
  const int nbg = k.B * k.Hkv;
  // dq: waves of 32 rows, at most 8 per workgroup
  const int rows = G * k.block;
  const int nw = min(8, (rows + 31) / 32);
  const int wg_per_qb = (rows + nw * 32 - 1) / (nw * 32);
  const int total_q = nbg * k.nqb * wg_per_qb;
  const int per_xcd_q = (total_q + kNumXcd - 1) / kNumXcd;
  k_bwd_dq<D><<<per_xcd_q * kNumXcd, nw * 64, 0, s>>>(k, wg_per_qb, per_xcd_q, total_q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int total_k = nbg * k.nqb;
  const int per_xcd_k = (total_k + kNumXcd - 1) / kNumXcd;
  const size_t lds = size_t(2 * k.block + 2 * kT) * (D + 8) * 2 + 2 * kT * sizeof(float);
  k_bwd_dkdv<D><<<per_xcd_k * kNumXcd, (k.block / kT) * 64, lds, s>>>(k, per_xcd_k, total_k);
  return hipGetLastError();
}

}  // namespace

size_t attn_backward_workspace_bytes(int B, int Hq, int Hkv, int S, int block) {
  const size_t nb = (size_t(S) + block - 1) / block;
  return 2 * align256(size_t(B) * Hq * S * sizeof(float)) +
         align256(size_t(B) * Hkv * nb * nb * sizeof(int32_t)) +
         align256(size_t(B) * Hkv * nb * sizeof(int32_t));
}

hipError_t launch_attn_backward(const AttnBwdArgs& a, hipStream_t s) {
  const int nqb = (a.S + a.block - 1) / a.block;
  char* ws = static_cast<char*>(a.workspace);
  float* dt = reinterpret_cast<float*>(ws);
  ws += align256(size_t(a.B) * a.Hq * a.S * sizeof(float));
  float* lse2 = reinterpret_cast<float*>(ws);
  ws += align256(size_t(a.B) * a.Hq * a.S * sizeof(float));
  int32_t* inv = reinterpret_cast<int32_t*>(ws);
  ws += align256(size_t(a.B) * a.Hkv * nqb * nqb * sizeof(int32_t));
  int32_t* inv_cnt = reinterpret_cast<int32_t*>(ws);

  const int rows = a.B * a.Hq * a.S;
  const int lpr = a.D / 8;
  k_bwd_rowterm<<<int((size_t(rows) * lpr + 255) / 256), 256, 0, s>>>(
      static_cast<const uint16_t*>(a.out), static_cast<const uint16_t*>(a.dout), a.lse, rows, a.D, dt,
      lse2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nbg = a.B * a.Hkv;
  k_bwd_invert<<<(nbg * nqb + 3) / 4, 256, 0, s>>>(a.idx, a.count, nbg, nqb, a.idx_width, inv,
                                                    inv_cnt);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  BwdK k{static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
         static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.dout),
         lse2, dt, a.idx, a.count, inv, inv_cnt,
         a.B, a.Hq, a.Hkv, a.S, a.block, a.idx_width, nqb, a.scale,
         static_cast<uint16_t*>(a.dq), static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv)};
  // the staged kernels keep the index lists in LDS and read row terms of a
  // 64-row tile by clamping to row S - 1
  const bool staged = a.D == 128 && a.idx_width <= f128::kDqList && nqb <= f128::kDkdvList &&
                      a.S >= 64;
  if (staged && a.block == 64) return launch_d128<64>(k, s);
  if (staged && a.block == 128) return launch_d128<128>(k, s);
  return a.D == 128 ? launch_d<128>(k, s) : launch_d<64>(k, s);
}

}  // namespace dsa
