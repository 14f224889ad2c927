// Internal declarations shared by the C-ABI layer and the HIP kernels of
// libdsa.so.  Nothing here is part of the public interface (include/dsa.h).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dsa {

// ---------------------------------------------------------------- launches
// Every launcher enqueues on `stream` and returns the launch status.  The
// arguments were validated by the C-ABI layer before any launcher runs.

struct PoolScoreArgs {
  int dtype;
  const void* q;     // [B,Hq,S,D]
  const void* k;     // [B,Hkv,S,D]
  int B, Hq, Hkv, S, D, block;
  int sel_heads;     // query heads per selection unit (Hq/Hkv: per KV group; 1: per query head)
  double* ws_q;      // [B*Hq/sel_heads, nb, D]  unit-summed pooled queries
  double* ws_k;      // [B*Hkv, nb, D]  pooled keys
  float* scores;     // [B,Hq/sel_heads,nb,nb]
};
hipError_t launch_pooled_scores(const PoolScoreArgs& a, hipStream_t s);

struct PageScoreArgs {
  int dtype;
  const void* q;     // [B,Hq,D]
  const void* kmin;  // [B,Hkv,nP,D]; paged: [n_pool,Hkv,D]
  const void* kmax;
  int B, Hq, Hkv, nP, D;
  float* scores;     // [B,Hkv,nP]  (paged: nP = max_pages)
  // paged (page_table != null): page p of sequence b is pool page
  // page_table[b][p]; pages at or past ceil(seq_len[b]/page) score -inf
  const int32_t* page_table;
  const int32_t* seq_len;
  int page, n_pool;
};
hipError_t launch_page_scores(const PageScoreArgs& a, hipStream_t s);

hipError_t launch_page_minmax(int dtype, const void* k, int B, int Hkv, int L, int D, int page,
                              void* kmin, void* kmax, hipStream_t s);

// Row r of each n_q-row matrix belongs to query block (r % n_q) / row_block
// (row_block = 1: the rows are the query blocks; > 1: per-token rows).
hipError_t launch_topk(const float* scores, int rows, int n_q, int n_k, int k, int n_local,
                       int causal, int row_block, int32_t* idx, int32_t* count, hipStream_t s);

enum AttnMode { MODE_INDEX = 0, MODE_WINDOW = 1, MODE_CMP = 2 };

struct AttnArgs {
  int dtype;
  const void* q;        // [B,Hq,S,D]
  const void* k;        // [B,Hkv,Skv,D]
  const void* v;        // [B,Hkv,Skv,D]
  void* out;            // [B,Hq,S,D]
  float* lse;           // [B,Hq,S] or null
  const int32_t* idx;   // index mode: [B,Hkv,nqb,idx_width]
  const int32_t* count; // index mode: [B,Hkv,nqb]
  int B, Hq, Hkv, S, Skv, D;
  int block;            // query rows per query block (and key block size in index mode)
  int idx_width;
  int mode;
  int window;           // window mode: tokens
  int cmp_len, cmp_stride;  // compressed mode: summary c ends at c*stride+len-1
  int sel_heads;        // query heads sharing one index row (Hq/Hkv unless per-head lists)
  const float* key_bias;  // [B,Hkv,Skv] additive logit term per key, or null
  // gated combine in the epilogue (gate_z != null): out = sigmoid(z0) gate_o1
  // + sigmoid(z1) gate_o2 + sigmoid(z2) (this attention's output), z =
  // gate_z[b][t][h][0..2]; gate_o1 / gate_o2 [B,Hq,S,D] in the output dtype
  const void* gate_o1;
  const void* gate_o2;
  const float* gate_z;
  float scale;
  // index mode (pipelined D = 128 kernel): after its listed blocks, every
  // row also attends to the token window of this many keys ending at the row
  // (a second softmax); with gate_z the epilogue combines the two, the
  // listed blocks' output taking gate_o2's place.  0: no window pass.
  int then_window;
};
// Whether some kernel serves this configuration (host-side check).
bool attention_supported(const AttnArgs& a);
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
// Per-token lists (idx [B,Hkv,S,idx_width], count [B,Hkv,S]; key blocks of
// a.block tokens): every head of group g at row t attends to keys <= t of
// the blocks listed for (b, g, t).
bool token_attention_supported(const AttnArgs& a);
hipError_t launch_token_attention(const AttnArgs& a, hipStream_t s);

hipError_t launch_dma_weights(int dtype, const void* v, int B, int Hkv, int S, int D,
                              const float* proj, const float* gain, int block, float* weights,
                              float* block_scores, hipStream_t s);

struct AttnBwdArgs {
  const void* q;        // [B,Hq,S,D] bf16
  const void* k;        // [B,Hkv,S,D]
  const void* v;
  const void* out;      // forward output [B,Hq,S,D]
  const float* lse;     // forward log-sum-exp [B,Hq,S]
  const void* dout;     // [B,Hq,S,D]
  const int32_t* idx;   // [B,Hkv,nqb,idx_width]
  const int32_t* count; // [B,Hkv,nqb]
  int B, Hq, Hkv, S, D, block, idx_width;
  float scale;
  void* workspace;      // attn_backward_workspace_bytes()
  void *dq, *dk, *dv;   // [B,Hq,S,D], [B,Hkv,S,D], [B,Hkv,S,D]
};
size_t attn_backward_workspace_bytes(int B, int Hq, int Hkv, int S, int block);
hipError_t launch_attn_backward(const AttnBwdArgs& a, hipStream_t s);

struct DecodeArgs {
  const void* q;        // [B,Hq,D] bf16
  const void* k;        // [B,Hkv,L,D]
  const void* v;
  const int32_t* idx;   // [B,Hkv,idx_width]
  const int32_t* count; // [B,Hkv]
  int B, Hq, Hkv, L, D, idx_width, page;
  float scale;
  float* partial;       // workspace
  void* out;            // [B,Hq,D] bf16
  // paged cache (page_table != null): k, v are pools [n_pool, Hkv, page, D]
  const int32_t* page_table;  // [B, max_pages] pool page of each logical page
  const int32_t* seq_len;     // [B] tokens per sequence (L unused)
  int max_pages, n_pool;
};
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int idx_width, int page, int D);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// Size of the per-device scratch array of the non-allocating decode, and
// its address on the current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
hipError_t decode_scratch(void** ptr);
hipError_t launch_paged_append(const void* k_new, const void* v_new, int B, int Hkv, int D,
                               int page, int max_pages, const int32_t* page_table,
                               int32_t* seq_len, int n_pool, void* k_pool, void* v_pool,
                               void* kmin, void* kmax, hipStream_t s);

hipError_t launch_nsa_compress(const void* k, const void* v, int B, int Hkv, int S, int D,
                               int len, int stride, void* ck, void* cv, hipStream_t s);

struct CmpScoreArgs {
  const void* q;        // [B,Hq,S,D] bf16
  const void* ck;       // [B,Hkv,n_cmp,D] bf16
  const float* lse;     // [B,Hq,S] from the compressed-branch attention
  int B, Hq, Hkv, S, n_cmp, D, len, stride, sel_block;
  float scale;
  float* scores;        // [B,Hkv,nb,nb]
};
hipError_t launch_cmp_block_scores(const CmpScoreArgs& a, hipStream_t s);
// scores [B,Hkv,S,nb]: per query token (sum over the group's heads / G);
// needs Hq/Hkv <= 16 and (sel_block + len - 2) / stride <= 31
hipError_t launch_cmp_token_scores(const CmpScoreArgs& a, hipStream_t s);

// XOR of every 32-bit word of src [bytes / 4] folded into sink [n_wg], one
// word per workgroup (bytes a multiple of 16).
hipError_t launch_read_stream(const void* src, size_t bytes, uint32_t* sink, int n_wg,
                              hipStream_t s);

hipError_t launch_nsa_combine(const void* o1, const void* o2, const void* o3, const float* z,
                              int B, int Hq, int S, int D, void* out, hipStream_t s);

}  // namespace dsa
