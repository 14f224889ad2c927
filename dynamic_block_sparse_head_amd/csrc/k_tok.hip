// Selected branch with per-token block lists ([NSA] §03 at the method's own
// granularity: every query token picks the key blocks for its KV group, and
// all query heads of the group attend to that token's blocks).
//
// The G heads of one token form the MFMA tile (16 x 16 x 32 bf16, heads
// padded to 16).  Scores are computed transposed, S^T = K Q^T (rows = keys,
// columns = heads), so each lane owns one head column: the row maximum needs
// only two cross-lane steps, the running rescale is a per-lane scalar, and
// the probabilities already sit in the B-operand layout of O^T = V^T P^T.
//
// Neighbouring tokens pick mostly the same blocks, so a workgroup takes 8
// consecutive tokens of one (sequence, KV group), one wave each, builds the
// union of their lists (LDS bitmap -> ascending list) and streams every
// union block through LDS once (direct-to-LDS loads, double buffered, one
// barrier per block); each wave runs the MFMAs only for the blocks of its
// own list.  K/V rows are 256 bytes (D = 128); chunk c (16 bytes) of row r
// sits at byte r * 256 + ((c ^ (r mod 16)) << 4), which keeps both the
// K-operand reads (16 rows, one chunk each) and the transposed V reads
// (ds_read_b64_tr_b16: 4 rows x 32 bytes per 16 lanes) spread over the banks.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr;
#define DSA_LDS_BF16X4(p) ((__attribute__((address_space(3))) bf16x4*)(p))

constexpr int kD = 128;
constexpr int kRowB = 256;     // bytes per K / V row
constexpr int kTW = 8;         // tokens (waves) per workgroup
constexpr int kMaxList = 64;   // blocks per token list
constexpr int kMaxWords = 256; // bitmap words: up to 8192 key blocks

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int BLK>
__global__ __launch_bounds__(kTW * 64) void k_attn_tok(AttnArgs a, int ntile, int per_xcd) {
  constexpr int NKT = BLK / 16;        // 16-key tiles per block
  constexpr int NKK = BLK / 32;        // 32-key contraction steps per block
  constexpr int RUNS = BLK * 2 / 4;    // 1 KB runs (4 rows) per block, K then V
  constexpr int VOFF = BLK * kRowB;
  __shared__ __attribute__((aligned(1024))) uint8_t kv0[2 * BLK * kRowB];
  __shared__ __attribute__((aligned(1024))) uint8_t kv1[2 * BLK * kRowB];
  __shared__ uint32_t bitmap[kMaxWords];
  __shared__ int32_t ulist[kMaxWords * 32 < kTW * kMaxList ? kMaxWords * 32 : kTW * kMaxList];
  __shared__ int n_union;

  const int id = xcd_work_id(per_xcd);
  if (id >= a.B * a.Hkv * ntile) return;   // whole workgroup
  const int bg = id / ntile, tile = id % ntile;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, q4 = lane >> 4;
  const int t = tile * kTW + wave;
  const bool live = t < a.S;
  const int nb = (a.S + BLK - 1) / BLK;
  const int nwords = (nb + 31) >> 5;

  // this token's list: lane l holds entry l
  int cnt = 0, myent = 0x7fffffff;
  if (live) {
    const size_t row = size_t(bg) * a.S + t;
    cnt = min(a.count[row], a.idx_width);
    if (lane < cnt) myent = a.idx[row * a.idx_width + lane];
  }
  for (int e = threadIdx.x; e < nwords; e += kTW * 64) bitmap[e] = 0u;
  __syncthreads();
  if (lane < cnt && myent >= 0 && myent < nb) atomicOr(&bitmap[myent >> 5], 1u << (myent & 31));
  __syncthreads();
  if (wave == 0) {   // bitmap -> ascending union list
    constexpr int WPL = kMaxWords / 64;
    uint32_t w[WPL];
    int c = 0;
#pragma unroll
    for (int x = 0; x < WPL; ++x) {
      const int wi = lane * WPL + x;
      w[x] = wi < nwords ? bitmap[wi] : 0u;
      c += __popc(w[x]);
    }
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    int pos = incl - c;
#pragma unroll
    for (int x = 0; x < WPL; ++x) {
      uint32_t bits = w[x];
      while (bits) {
        ulist[pos++] = (lane * WPL + x) * 32 + __builtin_ctz(bits);
        bits &= bits - 1;
      }
    }
    if (lane == 63) n_union = incl;
  }
  __syncthreads();
  const int U = n_union;

  // Q^T operand: lane -> head i16, dims q4 * 32 + ks * 8 .. + 8 (the K
  // operand uses the same dims per k-slot, so the sum over D is exact)
  bf16x8 qb[4];
  {
    const bool ok = live && i16 < G;
    const uint16_t* src = static_cast<const uint16_t*>(a.q) +
                          ((size_t(b) * a.Hq + g * G + (ok ? i16 : 0)) * a.S + (live ? t : 0)) * kD + q4 * 32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(src + ks * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) qb[ks][e] = ok ? v[e] : static_cast<__bf16>(0.0f);
    }
  }

  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + size_t(bg) * a.S * kD;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + size_t(bg) * a.S * kD;
  // runs wave, wave + 8, ... of block j into `dst` (rows past the sequence
  // repeat its last row: those keys are masked, their values finite)
  auto stage = [&](int j, uint8_t* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int k = wave; k < RUNS; k += kTW) {
      const bool isv = k >= RUNS / 2;
      const int r = (isv ? k - RUNS / 2 : k) * 4 + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      const int row = min(j * BLK + r, a.S - 1);
      const uint16_t* src = (isv ? vbase : kbase) + size_t(row) * kD + c * 8;
      __builtin_amdgcn_global_load_lds(src, (lds_ptr)(dst + k * 1024), 16, 0, 0);
    }
  };

  const float c2 = a.scale * kLog2e;
  floatx4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff(), l = 0.f;
  int p = 0;   // next entry of this token's list

  auto compute = [&](int j, const uint8_t* buf) __attribute__((always_inline)) {
    const int key0 = j * BLK;
    floatx4 s[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      s[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
            buf + (kt * 16 + i16) * kRowB + (((q4 * 4 + ks) ^ i16) << 4));
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[ks], s[kt], 0, 0, 0);
      }
    }
    // lane holds keys key0 + kt*16 + q4*4 + r of head i16
    const bool edge = key0 + BLK - 1 > t;
    float bm = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = s[kt][r] * c2;
        if (edge && key0 + kt * 16 + q4 * 4 + r > t) x = -__builtin_inff();
        s[kt][r] = x;
        bm = fmaxf(bm, x);
      }
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mn = fmaxf(m, bm);
    const float mu = mn == -__builtin_inff() ? 0.f : mn;
    const float alpha = fast_exp2(m - mu);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    bf16x8 pb[NKK];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = fast_exp2(s[kt][r] - mu);
        l += e;
        pb[kt >> 1][(kt & 1) * 4 + r] = static_cast<__bf16>(e);
      }
    // V^T operand: lane -> dim dt*16 + i16, keys 32kk + 4q4 + 0..3 and
    // 32kk + 16 + 4q4 + 0..3 (the key order of pb)
    const uint8_t* vb = buf + VOFF;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int r1 = kk * 32 + q4 * 4 + (i16 >> 2);
      const uint32_t rowoff = uint32_t(r1 * kRowB) | uint32_t((i16 & 1) << 3);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int cc = dt * 2 + ((i16 & 3) >> 1);
        const uint32_t off = rowoff | uint32_t((cc ^ (r1 & 15)) << 4);
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(DSA_LDS_BF16X4(vb + off));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(DSA_LDS_BF16X4(vb + off + 16 * kRowB));
        const bf16x8 va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[kk], o[dt], 0, 0, 0);
      }
    }
  };

  auto phase = [&](int u, const uint8_t* cur, uint8_t* nxt) __attribute__((always_inline)) {
    wait_vm0();       // this wave's part of block u has landed
    lds_barrier();    // ... and everyone's; block u - 1 (in nxt) is done
    if (u + 1 < U) stage(ulist[u + 1], nxt);
    const int j = ulist[u];
    if (p < cnt && __builtin_amdgcn_readlane(myent, p) == j) {   // wave-uniform
      ++p;
      compute(j, cur);
    }
  };
  if (U > 0) stage(ulist[0], kv0);
  for (int u = 0; u < U; u += 2) {
    phase(u, kv0, kv1);
    if (u + 1 >= U) break;
    phase(u + 1, kv1, kv0);
  }

  if (!live || i16 >= G) return;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int h = g * G + i16;
  const size_t orow = (size_t(b) * a.Hq + h) * a.S + t;
  uint16_t* op = static_cast<uint16_t*>(a.out) + orow * kD + q4 * 4;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    u32x2 w;
    w[0] = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
    w[1] = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
    *reinterpret_cast<u32x2*>(op + dt * 16) = w;
  }
  if (a.lse != nullptr && q4 == 0)
    a.lse[orow] = l > 0.f ? (m + __log2f(l)) * kLn2 : -__builtin_inff();
}

}  // namespace

bool token_attention_supported(const AttnArgs& a) {
  const int nb = (a.S + a.block - 1) / a.block;
  return a.dtype == 1 && a.D == kD && a.Hq / a.Hkv <= 16 && a.idx_width <= kMaxList &&
         nb <= kMaxWords * 32 && (a.block == 32 || a.block == 64 || a.block == 128);
}

hipError_t launch_token_attention(const AttnArgs& a, hipStream_t s) {
  const int ntile = (a.S + kTW - 1) / kTW;
  const int total = a.B * a.Hkv * ntile;
  const int per_xcd = (total + kNumXcd - 1) / kNumXcd;
  const int grid = per_xcd * kNumXcd;
  switch (a.block) {
    case 32: k_attn_tok<32><<<grid, kTW * 64, 0, s>>>(a, ntile, per_xcd); break;
    case 64: k_attn_tok<64><<<grid, kTW * 64, 0, s>>>(a, ntile, per_xcd); break;
    case 128: k_attn_tok<128><<<grid, kTW * 64, 0, s>>>(a, ntile, per_xcd); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dsa
