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

// D_t = sum_d dO[t,d] O[t,d] over rows = B*Hq*S; D/8 lanes per row.
__global__ __launch_bounds__(256) void k_bwd_rowterm(const uint16_t* __restrict__ out,
                                                     const uint16_t* __restrict__ dout, int rows,
                                                     int D, float* __restrict__ dt) {
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
  if (r < rows && sub == 0) dt[r] = acc;
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
  const float* lse;      // [B,Hq,S] natural log
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
  const float lse2 = row_ok ? a.lse[row] * kLog2e : 0.f;
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
      lsel[rr] = ok ? a.lse[row0 + t0 + rr] * kLog2e : __builtin_inff();
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

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

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
  return align256(size_t(B) * Hq * S * sizeof(float)) +
         align256(size_t(B) * Hkv * nb * nb * sizeof(int32_t)) +
         align256(size_t(B) * Hkv * nb * sizeof(int32_t));
}

hipError_t launch_attn_backward(const AttnBwdArgs& a, hipStream_t s) {
  const int nqb = (a.S + a.block - 1) / a.block;
  char* ws = static_cast<char*>(a.workspace);
  float* dt = reinterpret_cast<float*>(ws);
  ws += align256(size_t(a.B) * a.Hq * a.S * sizeof(float));
  int32_t* inv = reinterpret_cast<int32_t*>(ws);
  ws += align256(size_t(a.B) * a.Hkv * nqb * nqb * sizeof(int32_t));
  int32_t* inv_cnt = reinterpret_cast<int32_t*>(ws);

  const int rows = a.B * a.Hq * a.S;
  const int lpr = a.D / 8;
  k_bwd_rowterm<<<int((size_t(rows) * lpr + 255) / 256), 256, 0, s>>>(
      static_cast<const uint16_t*>(a.out), static_cast<const uint16_t*>(a.dout), rows, a.D, dt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nbg = a.B * a.Hkv;
  k_bwd_invert<<<(nbg * nqb + 3) / 4, 256, 0, s>>>(a.idx, a.count, nbg, nqb, a.idx_width, inv,
                                                    inv_cnt);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  BwdK k{static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
         static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.dout),
         a.lse, dt, a.idx, a.count, inv, inv_cnt,
         a.B, a.Hq, a.Hkv, a.S, a.block, a.idx_width, nqb, a.scale,
         static_cast<uint16_t*>(a.dq), static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv)};
  return a.D == 128 ? launch_d<128>(k, s) : launch_d<64>(k, s);
}

}  // namespace dsa
