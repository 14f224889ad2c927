// Selected branch with per-token block lists ([NSA] §03 at the method's own
// granularity: every query token picks the key blocks for its KV group, and
// all query heads of the group attend to that token's blocks).
//
// The G heads of one token form the MFMA tile (16 x 16 x 32 bf16, heads
// padded to 16).  Scores are computed transposed, S^T = K Q^T (rows = keys,
// columns = heads), so each lane owns one head column: the row maximum needs
// two cross-lane steps, the running rescale is a per-lane scalar, and the
// probabilities already sit in the B-operand layout of O^T = V^T P^T.  The
// A-operand row r of 16-key sub-tile h in a 32-key half block is key
// 8 (r / 4) + 4 h + r % 4, so lane quarter q ends up holding keys 8q .. 8q+7:
// one contiguous 8-key run, the k-slots of the V^T operand.
//
// One wave per (sequence, KV group, token), no barriers.  Different tokens'
// lists overlap little, so each wave streams its own blocks in 32-key
// halves, the next half in flight while the current one is used: K and V
// rows go to the wave's own LDS slot (direct-to-LDS loads, two slots), K
// read back as the A operand, V through transposed reads (ds_read_b64_tr_b16)
// as V^T.  A row r of a half is 256 bytes; chunk c sits at byte
// r * 256 + ((c ^ swz(r)) << 4) with swz(r) = (r mod 16) ^ 4 (r / 16 mod 2),
// so the 16 rows that one transposed read touches, and the 16 rows whose
// same chunk 16 lanes read for the A operand, land on 16 different 16-byte
// bank groups.  The loads are issued from inline assembly: through the
// builtin, the compiler would wait for all of them before any LDS read
// (it cannot tell the slots apart), draining the next half's loads; the
// loop waits for them itself (wait_vm).
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

#define DSA_LDS_BF16X4(p) ((__attribute__((address_space(3))) bf16x4*)(p))

// direct-to-LDS load of 16 bytes per lane: lane l writes dst + 16 l (dst
// wave-uniform); writes no register
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t(dst)));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
}

constexpr int kD = 128;
constexpr int kRowB = 256;     // bytes per K / V row
constexpr int kTW = 4;         // tokens (waves) per workgroup
constexpr int kMaxList = 64;   // blocks per token list
constexpr int kHalfB = 32 * kRowB;   // K (or V) bytes of one 32-key half block
constexpr float kLazy = 8.f;         // log2 headroom before the running maximum moves

__device__ __forceinline__ int vswz(int r) { return (r & 15) ^ (((r >> 4) & 1) << 2); }

// s_waitcnt vmcnt(N): all but this wave's last N vector-memory operations
// have completed (they complete in issue order); lgkm / exp counts untouched
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__global__ __launch_bounds__(kTW * 64) void k_attn_tok(AttnArgs a, int ntile, int per_xcd) {
  constexpr int BLK = 64;
  // per wave, two slots of one half each: K rows, then V rows
  __shared__ __attribute__((aligned(1024))) uint8_t vs0[kTW][2 * kHalfB];
  __shared__ __attribute__((aligned(1024))) uint8_t vs1[kTW][2 * kHalfB];

  const int id = xcd_work_id(per_xcd);
  if (id >= a.B * a.Hkv * ntile) return;
  const int bg = id / ntile, tile = id % ntile;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = tile * kTW + wave;
  if (t >= a.S) return;   // no barriers below: a wave may leave alone
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int i16 = lane & 15, q4 = lane >> 4;

  // this token's list: lane l holds entry l
  const size_t lrow = size_t(bg) * a.S + t;
  const int cnt = __builtin_amdgcn_readfirstlane(max(0, min(a.count[lrow], a.idx_width)));
  const int myent = lane < cnt ? a.idx[lrow * a.idx_width + lane] : 0;

  // Q^T operand: lane -> head i16, dims ks*32 + q4*8 .. + 8 (the K operand
  // uses the same dims per k-slot, so the sum over D is exact)
  bf16x8 qb[4];
  {
    const bool ok = i16 < G;
    const uint16_t* src = static_cast<const uint16_t*>(a.q) +
                          ((size_t(b) * a.Hq + g * G + (ok ? i16 : 0)) * a.S + t) * kD + q4 * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(src + ks * 32);
#pragma unroll
      for (int e = 0; e < 8; ++e) qb[ks][e] = ok ? v[e] : static_cast<__bf16>(0.0f);
    }
  }

  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + size_t(bg) * a.S * kD;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + size_t(bg) * a.S * kD;
  // K A-operand rows of this lane in a half: sub-tile h -> key 8 (i16/4) + 4 h + i16 % 4;
  // k-step ks reads chunk q4 + 4 ks of that row
  uint32_t koff[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = (i16 >> 2) * 8 + 4 * h + (i16 & 3);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) koff[h][ks] = uint32_t(r * kRowB + (((q4 + 4 * ks) ^ vswz(r)) << 4));
  }
  // direct-to-LDS: run k (4 rows) -> rows 4k + lane/16, position lane % 16
  const int vr = lane >> 4;

  // half n of the list: block entry n / 2, keys 32 (n % 2) ..
  auto key0_of = [&](int n) { return __builtin_amdgcn_readlane(myent, n >> 1) * BLK + (n & 1) * 32; };
  // 16 loads per half: K runs into dst, V runs into dst + kHalfB
  auto issue = [&](int key0, uint8_t* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = k * 4 + vr;
      const int row = max(0, min(key0 + r, a.S - 1));   // outside: masked keys, finite values
      const int c = (lane & 15) ^ vswz(r);
      dma16(kbase + size_t(row) * kD + c * 8, dst + k * 1024);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = k * 4 + vr;
      const int row = max(0, min(key0 + r, a.S - 1));
      const int c = (lane & 15) ^ vswz(r);
      dma16(vbase + size_t(row) * kD + c * 8, dst + kHalfB + k * 1024);
    }
  };

  const float c2 = a.scale * kLog2e;
  floatx4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff(), l = 0.f;

  // transposed-read offsets: rows 8 q4 + i16/4 (+4), chunk 2 dt + (i16 % 4) / 2
  const int r1 = q4 * 8 + (i16 >> 2), r2 = r1 + 4;
  const uint32_t ro1 = uint32_t(r1 * kRowB + ((i16 & 1) << 3)), ro2 = uint32_t(r2 * kRowB + ((i16 & 1) << 3));
  const int s1 = vswz(r1), s2 = vswz(r2), cl = (i16 & 3) >> 1;

  auto compute = [&](int key0, const uint8_t* slot) __attribute__((always_inline)) {
    const uint8_t* vsrc = slot + kHalfB;
    bf16x8 kr[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kr[h][ks] = *reinterpret_cast<const bf16x8*>(slot + koff[h][ks]);
    floatx4 s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        s[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[h][ks], qb[ks], s[h], 0, 0, 0);
    }
    // lane holds keys key0 + 8 q4 + 4 h + i of head i16
    const bool edge = key0 < 0 || key0 + 31 > t;   // keys past t (or before 0) masked
    float bm = -__builtin_inff();
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = s[h][i] * c2;
        if (edge && unsigned(key0 + q4 * 8 + h * 4 + i) > unsigned(t)) x = -__builtin_inff();
        s[h][i] = x;
        bm = fmaxf(bm, x);
      }
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    // lazy rescale: the reference maximum moves only when the block's maximum
    // exceeds it by more than 2^kLazy (probabilities stay <= 2^kLazy), so the
    // accumulators are rescaled rarely once the first blocks are in
    if (__builtin_amdgcn_ballot_w64(bm > m + kLazy) != 0) {   // wave-uniform
      const float mn = bm > m + kLazy ? bm : m;
      const float alpha = fast_exp2(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    }
    const float mu = m == -__builtin_inff() ? 0.f : m;
    bf16x8 pb;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = fast_exp2(s[h][i] - mu);
        l += e;
        pb[h * 4 + i] = static_cast<__bf16>(e);
      }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int cc = dt * 2 + cl;
      const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          DSA_LDS_BF16X4(vsrc + (ro1 | uint32_t((cc ^ s1) << 4))));
      const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          DSA_LDS_BF16X4(vsrc + (ro2 | uint32_t((cc ^ s2) << 4))));
      const bf16x8 va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[dt], 0, 0, 0);
    }
  };

  const int total = 2 * cnt;
  uint8_t* sa = vs0[wave];
  uint8_t* sb = vs1[wave];
  // the half after the last one re-reads the last half into the idle slot,
  // so every phase issues the same 16 loads and waits the same way
  auto phase = [&](int n, const uint8_t* sc, uint8_t* sn) __attribute__((always_inline)) {
    issue(key0_of(min(n + 1, total - 1)), sn);
    wait_vm<16>();   // half n's runs landed (the 16 just issued may not have)
    compute(key0_of(n), sc);
  };
  if (total > 0) {
    issue(key0_of(0), sa);
    for (int n = 0; n < total; n += 2) {
      phase(n, sa, sb);
      if (n + 1 >= total) break;
      phase(n + 1, sb, sa);
    }
    wait_vm<0>();   // the spare re-read has landed before the wave ends
  }

  if (i16 >= G) return;
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
  return a.dtype == 1 && a.D == kD && a.Hq / a.Hkv <= 16 && a.idx_width <= kMaxList &&
         a.block == 64;
}

hipError_t launch_token_attention(const AttnArgs& a, hipStream_t s) {
  const int ntile = (a.S + kTW - 1) / kTW;
  const int total = a.B * a.Hkv * ntile;
  const int per_xcd = (total + kNumXcd - 1) / kNumXcd;
  k_attn_tok<<<per_xcd * kNumXcd, kTW * 64, 0, s>>>(a, ntile, per_xcd);
  return hipGetLastError();
}

}  // namespace dsa
