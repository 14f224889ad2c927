// C-ABI entry points of libdsa.so: argument validation, workspace carving
// and kernel dispatch.  Validation runs entirely on the host and makes no
// HIP call, so a rejected call enqueues nothing and touches no output.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/dsa.h"
#include "dsa_internal.h"

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

#define REQUIRE_PTR(p)                                                        \
  do {                                                                        \
    if ((p) == nullptr) return fail(DSA_E_ARG, "%s must not be NULL", #p);    \
    if (!aligned16(p)) return fail(DSA_E_ARG, "%s must be 16-byte aligned", #p); \
  } while (0)

int check_dtype(int dtype, bool f32_ok) {
  if (dtype == DSA_BF16) return DSA_OK;
  if (dtype == DSA_F32 && f32_ok) return DSA_OK;
  if (dtype == DSA_F32) return fail(DSA_E_UNSUPPORTED, "dtype DSA_F32 is not supported by this call");
  return fail(DSA_E_ARG, "unknown dtype %d", dtype);
}

int check_heads(int B, int Hq, int Hkv) {
  REQUIRE(B >= 1, DSA_E_ARG, "B must be >= 1 (got %d)", B);
  REQUIRE(Hq >= 1 && Hkv >= 1, DSA_E_ARG, "head counts must be >= 1 (Hq=%d, Hkv=%d)", Hq, Hkv);
  REQUIRE(Hq % Hkv == 0, DSA_E_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  // launch grids put B, B*Hkv or Hq in a 16-bit grid dimension
  REQUIRE(B <= 65535 && Hq <= 65535 && (long long)B * Hkv <= 65535, DSA_E_UNSUPPORTED,
          "B (%d), Hq (%d) and B*Hkv must be at most 65535", B, Hq);
  return DSA_OK;
}

int check_dim(int D) {
  REQUIRE(D == 64 || D == 128, DSA_E_UNSUPPORTED, "head dim %d not supported (64 or 128)", D);
  return DSA_OK;
}

int check_block(int block, const char* what) {
  REQUIRE(block > 0, DSA_E_ARG, "%s must be > 0 (got %d)", what, block);
  REQUIRE(block % 32 == 0 && block <= 256, DSA_E_UNSUPPORTED,
          "%s %d not supported (a multiple of 32, at most 256)", what, block);
  return DSA_OK;
}

// largest element count a kernel may address with 64-bit offsets but 32-bit
// row indices: keep every row count below 2^31
bool rows_fit(long long a, long long b, long long c) { return a * b * c < (1ll << 31); }

// The attention kernels address one KV group's query rows [G, S, D] and its
// keys [S, D] through buffer descriptors with 32-bit byte ranges and 32-bit
// element offsets: a group's G*S*D elements must stay below 2^31.
int check_group_extent(long long G, long long S, long long D, const char* dim) {
  REQUIRE(G * S * D < (1ll << 31), DSA_E_UNSUPPORTED,
          "one KV group's rows (%lld * %s * D = %lld elements) must stay below 2^31, the range of "
          "the kernels' 32-bit buffer offsets",
          G, dim, G * S * D);
  return DSA_OK;
}

#define TRY(x)                     \
  do {                             \
    const int _st = (x);           \
    if (_st != DSA_OK) return _st; \
  } while (0)

}  // namespace

extern "C" {

int dsa_version(void) { return DSA_VERSION; }

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_E_ARG: return "DSA_E_ARG: invalid argument";
    case DSA_E_UNSUPPORTED: return "DSA_E_UNSUPPORTED: no kernel for this configuration";
    case DSA_E_WORKSPACE: return "DSA_E_WORKSPACE: workspace missing or too small";
    case DSA_E_HIP: return "DSA_E_HIP: HIP launch failure";
    default: return "unknown dsa status";
  }
}

const char* dsa_last_error(void) { return g_err.c_str(); }

size_t dsa_block_scores_workspace_size(int kind, int B, int Hq, int Hkv, int n, int D, int block) {
  if ((kind != DSA_SCORE_POOLED && kind != DSA_SCORE_POOLED_HEAD) || B <= 0 || Hq <= 0 || Hkv <= 0 ||
      n <= 0 || D <= 0 || block <= 0)
    return 0;
  const size_t nb = (size_t(n) + block - 1) / block;
  const size_t units = kind == DSA_SCORE_POOLED ? size_t(Hkv) : size_t(Hq);
  return (units + Hkv) * B * nb * D * sizeof(double);
}

int dsa_block_scores(int kind, int dtype, const void* q, const void* k_or_kmin, const void* kmax,
                     int B, int Hq, int Hkv, int n, int D, int block, void* workspace,
                     size_t workspace_bytes, float* scores, void* stream) {
  g_err.clear();
  TRY(check_dtype(dtype, true));
  TRY(check_heads(B, Hq, Hkv));
  TRY(check_dim(D));
  REQUIRE(n >= 1, DSA_E_ARG, "n must be >= 1 (got %d)", n);
  REQUIRE_PTR(q);
  REQUIRE_PTR(k_or_kmin);
  REQUIRE_PTR(scores);
  auto s = static_cast<hipStream_t>(stream);
  if (kind == DSA_SCORE_POOLED || kind == DSA_SCORE_POOLED_HEAD) {
    TRY(check_block(block, "block"));
    REQUIRE(kmax == nullptr, DSA_E_ARG, "kmax must be NULL for pooled scores");
    REQUIRE(rows_fit(B, Hq, n), DSA_E_ARG, "B*Hq*n too large");
    const size_t need = dsa_block_scores_workspace_size(kind, B, Hq, Hkv, n, D, block);
    REQUIRE(workspace != nullptr && workspace_bytes >= need, DSA_E_WORKSPACE,
            "pooled scores need a workspace of %zu bytes (got %zu)", need, workspace_bytes);
    REQUIRE_PTR(workspace);
    const int nb = (n + block - 1) / block;
    const int sel_heads = kind == DSA_SCORE_POOLED ? Hq / Hkv : 1;
    dsa::PoolScoreArgs a{dtype, q, k_or_kmin, B, Hq, Hkv, n, D, block, sel_heads,
                         static_cast<double*>(workspace),
                         static_cast<double*>(workspace) + size_t(B) * (Hq / sel_heads) * nb * D,
                         scores};
    return hip_status(dsa::launch_pooled_scores(a, s), "dsa_block_scores");
  }
  if (kind == DSA_SCORE_PAGE_BOUND) {
    REQUIRE_PTR(kmax);
    REQUIRE(Hq / Hkv <= 64, DSA_E_UNSUPPORTED, "at most 64 query heads per KV head");
    dsa::PageScoreArgs a{dtype, q, k_or_kmin, kmax, B, Hq, Hkv, n, D, scores};
    return hip_status(dsa::launch_page_scores(a, s), "dsa_block_scores");
  }
  return fail(DSA_E_ARG, "unknown score kind %d", kind);
}

int dsa_topk_select(const float* scores, int rows, int n_q, int n_k, int k, int n_local,
                    int causal, int32_t* idx, int32_t* count, void* stream) {
  g_err.clear();
  REQUIRE(rows >= 1 && n_q >= 1 && n_k >= 1, DSA_E_ARG,
          "rows, n_q, n_k must be >= 1 (got %d, %d, %d)", rows, n_q, n_k);
  REQUIRE(k >= 0, DSA_E_ARG, "k must be >= 0 (got %d)", k);
  REQUIRE(n_local >= 0, DSA_E_ARG, "n_local must be >= 0 (got %d)", n_local);
  REQUIRE(k + n_local >= 1, DSA_E_ARG, "k + n_local must be >= 1");
  REQUIRE(n_k <= 8192, DSA_E_UNSUPPORTED, "n_k %d exceeds 8192", n_k);
  REQUIRE(!causal || n_q <= n_k, DSA_E_ARG, "causal selection needs n_q <= n_k (%d > %d)", n_q, n_k);
  REQUIRE(causal || n_local <= n_k, DSA_E_ARG, "n_local (%d) exceeds n_k (%d)", n_local, n_k);
  REQUIRE(rows_fit(rows, n_q, 1), DSA_E_ARG, "rows*n_q too large");
  REQUIRE_PTR(scores);
  REQUIRE(idx != nullptr && count != nullptr, DSA_E_ARG, "idx and count must not be NULL");
  return hip_status(dsa::launch_topk(scores, rows, n_q, n_k, k, n_local, causal, 1, idx, count,
                                     static_cast<hipStream_t>(stream)),
                    "dsa_topk_select");
}

int dsa_topk_select_tokens(const float* scores, int rows, int S, int n_k, int k, int n_local,
                           int block, int32_t* idx, int32_t* count, void* stream) {
  g_err.clear();
  REQUIRE(rows >= 1 && S >= 1 && n_k >= 1, DSA_E_ARG,
          "rows, S, n_k must be >= 1 (got %d, %d, %d)", rows, S, n_k);
  REQUIRE(block >= 1, DSA_E_ARG, "block must be >= 1 (got %d)", block);
  REQUIRE(k >= 0, DSA_E_ARG, "k must be >= 0 (got %d)", k);
  REQUIRE(n_local >= 0, DSA_E_ARG, "n_local must be >= 0 (got %d)", n_local);
  REQUIRE(k + n_local >= 1, DSA_E_ARG, "k + n_local must be >= 1");
  REQUIRE(n_k <= 8192, DSA_E_UNSUPPORTED, "n_k %d exceeds 8192", n_k);
  REQUIRE((S + block - 1) / block <= n_k, DSA_E_ARG,
          "the last token's block (%d) is past n_k (%d)", (S + block - 1) / block - 1, n_k);
  REQUIRE(rows_fit(rows, S, 1), DSA_E_ARG, "rows*S too large");
  REQUIRE_PTR(scores);
  REQUIRE(idx != nullptr && count != nullptr, DSA_E_ARG, "idx and count must not be NULL");
  return hip_status(dsa::launch_topk(scores, rows, S, n_k, k, n_local, 1, block, idx, count,
                                     static_cast<hipStream_t>(stream)),
                    "dsa_topk_select_tokens");
}

static int prefill_impl(int dtype, const void* q, const void* k, const void* v, int B, int Hq,
                        int Hkv, int S, int D, const int32_t* idx, const int32_t* count,
                        int idx_width, int block, int window, int sel_heads,
                        const float* key_bias, float scale, void* out, float* lse,
                        void* stream) {
  TRY(check_dtype(dtype, true));
  TRY(check_heads(B, Hq, Hkv));
  TRY(check_dim(D));
  TRY(check_block(block, "block"));
  REQUIRE(S >= 1, DSA_E_ARG, "S must be >= 1 (got %d)", S);
  REQUIRE(rows_fit(B, Hq, S), DSA_E_ARG, "B*Hq*S too large");
  TRY(check_group_extent(Hq / Hkv, S, D, "S"));
  REQUIRE(scale > 0.f, DSA_E_ARG, "scale must be > 0");
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(out);
  const bool index_mode = idx != nullptr || count != nullptr;
  if (index_mode) {
    REQUIRE(idx != nullptr && count != nullptr, DSA_E_ARG, "idx and count must both be given");
    REQUIRE(window == 0, DSA_E_ARG, "window must be 0 in index mode (got %d)", window);
    REQUIRE(idx_width >= 1, DSA_E_ARG, "idx_width must be >= 1 (got %d)", idx_width);
  } else {
    REQUIRE(window >= 1, DSA_E_ARG, "window mode needs window >= 1 (got %d)", window);
  }
  dsa::AttnArgs a{};
  a.dtype = dtype;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.idx = idx;
  a.count = count;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.S = S;
  a.Skv = S;
  a.D = D;
  a.block = block;
  a.idx_width = idx_width;
  a.mode = index_mode ? dsa::MODE_INDEX : dsa::MODE_WINDOW;
  a.window = window;
  a.cmp_len = 1;
  a.cmp_stride = 1;
  a.sel_heads = sel_heads;
  a.key_bias = key_bias;
  a.scale = scale;
  REQUIRE(dsa::attention_supported(a), DSA_E_UNSUPPORTED,
          "key_bias needs D = 128, blocks of 64k tokens and at least 256 rows per selection unit "
          "(bf16), or DSA_F32");
  return hip_status(dsa::launch_attention(a, static_cast<hipStream_t>(stream)),
                    "dsa_sparse_attn_prefill");
}

int dsa_sparse_attn_prefill(int dtype, const void* q, const void* k, const void* v, int B, int Hq,
                            int Hkv, int S, int D, const int32_t* idx, const int32_t* count,
                            int idx_width, int block, int window, float scale, void* out,
                            float* lse, void* stream) {
  g_err.clear();
  TRY(check_heads(B, Hq, Hkv));
  return prefill_impl(dtype, q, k, v, B, Hq, Hkv, S, D, idx, count, idx_width, block, window,
                      Hq / Hkv, nullptr, scale, out, lse, stream);
}

int dsa_sparse_attn_prefill_ex(int dtype, const void* q, const void* k, const void* v, int B,
                               int Hq, int Hkv, int S, int D, const int32_t* idx,
                               const int32_t* count, int idx_width, int block, int sel_heads,
                               const float* key_bias, float scale, void* out, float* lse,
                               void* stream) {
  g_err.clear();
  TRY(check_heads(B, Hq, Hkv));
  REQUIRE(sel_heads >= 1 && (Hq / Hkv) % sel_heads == 0, DSA_E_ARG,
          "sel_heads (%d) must divide Hq/Hkv (%d)", sel_heads, Hq / Hkv);
  REQUIRE(idx != nullptr && count != nullptr, DSA_E_ARG, "idx and count must not be NULL");
  if (key_bias != nullptr) REQUIRE_PTR(key_bias);
  return prefill_impl(dtype, q, k, v, B, Hq, Hkv, S, D, idx, count, idx_width, block, 0, sel_heads,
                      key_bias, scale, out, lse, stream);
}

int dsa_dma_weights(int dtype, const void* v, int B, int Hkv, int S, int D, const float* proj,
                    const float* gain, int block, float* weights, float* block_scores,
                    void* stream) {
  g_err.clear();
  TRY(check_dtype(dtype, true));
  TRY(check_heads(B, Hkv, Hkv));
  TRY(check_dim(D));
  TRY(check_block(block, "block"));
  REQUIRE(S >= 1, DSA_E_ARG, "S must be >= 1 (got %d)", S);
  REQUIRE(rows_fit(B, Hkv, S), DSA_E_ARG, "B*Hkv*S too large");
  const long long nb = (S + block - 1) / block;
  REQUIRE(nb <= 65535, DSA_E_UNSUPPORTED, "at most 65535 blocks");
  REQUIRE((long long)B * Hkv * nb * nb < (1ll << 31), DSA_E_ARG, "B*Hkv*nb*nb too large");
  REQUIRE_PTR(v);
  REQUIRE_PTR(proj);
  REQUIRE(gain != nullptr, DSA_E_ARG, "gain must not be NULL");
  REQUIRE(weights != nullptr, DSA_E_ARG, "weights must not be NULL");
  return hip_status(dsa::launch_dma_weights(dtype, v, B, Hkv, S, D, proj, gain, block, weights,
                                            block_scores, static_cast<hipStream_t>(stream)),
                    "dsa_dma_weights");
}

size_t dsa_sparse_attn_prefill_backward_workspace_size(int B, int Hq, int Hkv, int S, int D,
                                                       int block) {
  (void)D;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || block <= 0) return 0;
  return dsa::attn_backward_workspace_bytes(B, Hq, Hkv, S, block);
}

int dsa_sparse_attn_prefill_backward(int dtype, const void* q, const void* k, const void* v,
                                     const void* out, const float* lse, const void* dout, int B,
                                     int Hq, int Hkv, int S, int D, const int32_t* idx,
                                     const int32_t* count, int idx_width, int block, float scale,
                                     void* workspace, size_t workspace_bytes, void* dq, void* dk,
                                     void* dv, void* stream) {
  g_err.clear();
  TRY(check_dtype(dtype, false));
  TRY(check_heads(B, Hq, Hkv));
  TRY(check_dim(D));
  TRY(check_block(block, "block"));
  REQUIRE(S >= 1, DSA_E_ARG, "S must be >= 1 (got %d)", S);
  REQUIRE(rows_fit(B, Hq, S), DSA_E_ARG, "B*Hq*S too large");
  TRY(check_group_extent(Hq / Hkv, S, D, "S"));
  REQUIRE(scale > 0.f, DSA_E_ARG, "scale must be > 0");
  REQUIRE(idx_width >= 1, DSA_E_ARG, "idx_width must be >= 1 (got %d)", idx_width);
  const long long nb = (S + block - 1) / block;
  REQUIRE((long long)B * Hkv * nb * nb < (1ll << 31), DSA_E_UNSUPPORTED,
          "B*Hkv*nb*nb too large for the inverted block lists");
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(out);
  REQUIRE_PTR(dout);
  REQUIRE_PTR(dq);
  REQUIRE_PTR(dk);
  REQUIRE_PTR(dv);
  REQUIRE(lse != nullptr, DSA_E_ARG, "lse must not be NULL");
  REQUIRE(idx != nullptr && count != nullptr, DSA_E_ARG, "idx and count must not be NULL");
  const size_t need = dsa::attn_backward_workspace_bytes(B, Hq, Hkv, S, block);
  REQUIRE(workspace != nullptr && workspace_bytes >= need, DSA_E_WORKSPACE,
          "the backward needs a workspace of %zu bytes (got %zu)", need, workspace_bytes);
  REQUIRE_PTR(workspace);
  dsa::AttnBwdArgs a{q,     k,   v,     out,   lse, dout, idx,       count,   B,  Hq, Hkv,
                     S,     D,   block, idx_width, scale, workspace, dq, dk, dv};
  return hip_status(dsa::launch_attn_backward(a, static_cast<hipStream_t>(stream)),
                    "dsa_sparse_attn_prefill_backward");
}

int dsa_page_minmax(int dtype, const void* k, int B, int Hkv, int L, int D, int page, void* kmin,
                    void* kmax, void* stream) {
  g_err.clear();
  TRY(check_dtype(dtype, true));
  TRY(check_heads(B, Hkv, Hkv));
  TRY(check_dim(D));
  REQUIRE(page >= 1, DSA_E_ARG, "page must be >= 1 (got %d)", page);
  REQUIRE(L >= page && L % page == 0, DSA_E_ARG, "L (%d) must be a positive multiple of page (%d)",
          L, page);
  REQUIRE_PTR(k);
  REQUIRE_PTR(kmin);
  REQUIRE_PTR(kmax);
  return hip_status(dsa::launch_page_minmax(dtype, k, B, Hkv, L, D, page, kmin, kmax,
                                            static_cast<hipStream_t>(stream)),
                    "dsa_page_minmax");
}

size_t dsa_sparse_attn_decode_workspace_size(int B, int Hq, int Hkv, int idx_width, int page, int D) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || idx_width <= 0 || page <= 0 || D <= 0) return 0;
  return dsa::decode_workspace_bytes(B, Hq, Hkv, idx_width, page, D);
}

static_assert(dsa::kDecodeScratchBytes == DSA_DECODE_NOALLOC_SCRATCH_BYTES,
              "the header and the kernels must agree on the decode scratch size");

// Validation shared by the two decode calls; workspace == nullptr selects
// the library's per-device scratch (dsa_sparse_attn_decode_noalloc).
static int decode_impl(int dtype, const void* q, const void* k_cache, const void* v_cache, int B,
                       int Hq, int Hkv, int L, int D, const int32_t* idx, const int32_t* count,
                       int idx_width, int page, float scale, void* workspace,
                       size_t workspace_bytes, bool noalloc, void* out, void* stream) {
  TRY(check_dtype(dtype, false));
  TRY(check_heads(B, Hq, Hkv));
  TRY(check_dim(D));
  const int G = Hq / Hkv;
  REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, DSA_E_UNSUPPORTED,
          "decode supports 1, 2, 4 or 8 query heads per KV head (got %d)", G);
  REQUIRE(page == 32 || page == 64 || page == 128 || page == 256 || page == 512, DSA_E_UNSUPPORTED,
          "page %d not supported (32, 64, 128, 256 or 512)", page);
  REQUIRE(L >= page && L % page == 0, DSA_E_ARG, "L (%d) must be a positive multiple of page (%d)",
          L, page);
  REQUIRE(idx_width >= 1 && idx_width <= L / page, DSA_E_ARG,
          "idx_width must be in [1, L/page] (got %d)", idx_width);
  TRY(check_group_extent(1, L, D, "L"));
  REQUIRE(B * Hkv <= 65535, DSA_E_UNSUPPORTED, "B*Hkv must be at most 65535");
  REQUIRE(scale > 0.f, DSA_E_ARG, "scale must be > 0");
  REQUIRE_PTR(q);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  REQUIRE_PTR(out);
  REQUIRE(idx != nullptr && count != nullptr, DSA_E_ARG, "idx and count must not be NULL");
  const size_t need = dsa::decode_workspace_bytes(B, Hq, Hkv, idx_width, page, D);
  if (noalloc) {
    REQUIRE(need <= DSA_DECODE_NOALLOC_SCRATCH_BYTES, DSA_E_WORKSPACE,
            "this decode needs %zu bytes of partial results, more than the %zu-byte scratch of "
            "dsa_sparse_attn_decode_noalloc (use dsa_sparse_attn_decode with a workspace)",
            need, size_t(DSA_DECODE_NOALLOC_SCRATCH_BYTES));
    const hipError_t e = dsa::decode_scratch(&workspace);
    if (e != hipSuccess) return hip_status(e, "dsa_sparse_attn_decode_noalloc: scratch lookup");
  } else {
    REQUIRE(workspace != nullptr && workspace_bytes >= need, DSA_E_WORKSPACE,
            "decode needs a workspace of %zu bytes (got %zu)", need, workspace_bytes);
    REQUIRE_PTR(workspace);
  }
  dsa::DecodeArgs a{q,  k_cache, v_cache, idx,   count, B, Hq, Hkv, L, D, idx_width, page,
                    scale, static_cast<float*>(workspace), out};
  return hip_status(dsa::launch_decode(a, static_cast<hipStream_t>(stream)),
                    noalloc ? "dsa_sparse_attn_decode_noalloc" : "dsa_sparse_attn_decode");
}

int dsa_sparse_attn_decode(int dtype, const void* q, const void* k_cache, const void* v_cache,
                           int B, int Hq, int Hkv, int L, int D, const int32_t* idx,
                           const int32_t* count, int idx_width, int page, float scale,
                           void* workspace, size_t workspace_bytes, void* out, void* stream) {
  g_err.clear();
  return decode_impl(dtype, q, k_cache, v_cache, B, Hq, Hkv, L, D, idx, count, idx_width, page,
                     scale, workspace, workspace_bytes, false, out, stream);
}

int dsa_sparse_attn_decode_noalloc(int dtype, const void* q, const void* k_cache,
                                   const void* v_cache, int B, int Hq, int Hkv, int L, int D,
                                   const int32_t* idx, const int32_t* count, int idx_width,
                                   int page, float scale, void* out, void* stream) {
  g_err.clear();
  return decode_impl(dtype, q, k_cache, v_cache, B, Hq, Hkv, L, D, idx, count, idx_width, page,
                     scale, nullptr, 0, true, out, stream);
}

// shared checks of the paged-cache calls
static int check_paged(int dtype, int B, int Hq, int Hkv, int D, int page, int max_pages,
                       const int32_t* page_table, const int32_t* seq_len, int n_pool) {
  TRY(check_dtype(dtype, false));
  TRY(check_heads(B, Hq, Hkv));
  TRY(check_dim(D));
  REQUIRE(page == 32 || page == 64 || page == 128 || page == 256 || page == 512, DSA_E_UNSUPPORTED,
          "page %d not supported (32, 64, 128, 256 or 512)", page);
  REQUIRE(max_pages >= 1, DSA_E_ARG, "max_pages must be >= 1 (got %d)", max_pages);
  REQUIRE(n_pool >= 1, DSA_E_ARG, "n_pool must be >= 1 (got %d)", n_pool);
  REQUIRE((long long)n_pool * Hkv * page * D < (1ll << 40), DSA_E_ARG, "pool too large");
  REQUIRE((long long)B * max_pages < (1ll << 31), DSA_E_ARG, "B*max_pages too large");
  REQUIRE(page_table != nullptr && seq_len != nullptr, DSA_E_ARG,
          "page_table and seq_len must not be NULL");
  return DSA_OK;
}

int dsa_paged_append(int dtype, const void* k_new, const void* v_new, int B, int Hkv, int D,
                     int page, int max_pages, const int32_t* page_table, int32_t* seq_len,
                     int n_pool, void* k_pool, void* v_pool, void* kmin, void* kmax,
                     void* stream) {
  g_err.clear();
  TRY(check_paged(dtype, B, Hkv, Hkv, D, page, max_pages, page_table, seq_len, n_pool));
  REQUIRE_PTR(k_new);
  REQUIRE_PTR(v_new);
  REQUIRE_PTR(k_pool);
  REQUIRE_PTR(v_pool);
  REQUIRE_PTR(kmin);
  REQUIRE_PTR(kmax);
  return hip_status(dsa::launch_paged_append(k_new, v_new, B, Hkv, D, page, max_pages, page_table,
                                             seq_len, n_pool, k_pool, v_pool, kmin, kmax,
                                             static_cast<hipStream_t>(stream)),
                    "dsa_paged_append");
}

int dsa_paged_page_scores(int dtype, const void* q, const void* kmin, const void* kmax, int B,
                          int Hq, int Hkv, int D, int page, int max_pages,
                          const int32_t* page_table, const int32_t* seq_len, int n_pool,
                          float* scores, void* stream) {
  g_err.clear();
  TRY(check_paged(dtype, B, Hq, Hkv, D, page, max_pages, page_table, seq_len, n_pool));
  const int G = Hq / Hkv;
  REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, DSA_E_UNSUPPORTED,
          "paged scores support 1, 2, 4 or 8 query heads per KV head (got %d)", G);
  REQUIRE(max_pages <= 65535 * 256, DSA_E_UNSUPPORTED, "max_pages too large");
  REQUIRE_PTR(q);
  REQUIRE_PTR(kmin);
  REQUIRE_PTR(kmax);
  REQUIRE(scores != nullptr, DSA_E_ARG, "scores must not be NULL");
  dsa::PageScoreArgs a{dtype, q, kmin, kmax, B, Hq, Hkv, max_pages, D, scores,
                       page_table, seq_len, page, n_pool};
  return hip_status(dsa::launch_page_scores(a, static_cast<hipStream_t>(stream)),
                    "dsa_paged_page_scores");
}

int dsa_paged_decode(int dtype, const void* q, const void* k_pool, const void* v_pool, int B,
                     int Hq, int Hkv, int D, int page, int max_pages, const int32_t* page_table,
                     const int32_t* seq_len, int n_pool, const int32_t* idx, const int32_t* count,
                     int idx_width, float scale, void* workspace, size_t workspace_bytes,
                     void* out, void* stream) {
  g_err.clear();
  TRY(check_paged(dtype, B, Hq, Hkv, D, page, max_pages, page_table, seq_len, n_pool));
  const int G = Hq / Hkv;
  REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, DSA_E_UNSUPPORTED,
          "decode supports 1, 2, 4 or 8 query heads per KV head (got %d)", G);
  REQUIRE(idx_width >= 1, DSA_E_ARG, "idx_width must be >= 1 (got %d)", idx_width);
  REQUIRE(B * Hkv <= 65535, DSA_E_UNSUPPORTED, "B*Hkv must be at most 65535");
  REQUIRE(scale > 0.f, DSA_E_ARG, "scale must be > 0");
  REQUIRE_PTR(q);
  REQUIRE_PTR(k_pool);
  REQUIRE_PTR(v_pool);
  REQUIRE_PTR(out);
  REQUIRE(idx != nullptr && count != nullptr, DSA_E_ARG, "idx and count must not be NULL");
  const size_t need = dsa::decode_workspace_bytes(B, Hq, Hkv, idx_width, page, D);
  REQUIRE(workspace != nullptr && workspace_bytes >= need, DSA_E_WORKSPACE,
          "decode needs a workspace of %zu bytes (got %zu)", need, workspace_bytes);
  REQUIRE_PTR(workspace);
  dsa::DecodeArgs a{q,     k_pool, v_pool, idx, count, B, Hq, Hkv, 0, D, idx_width, page,
                    scale, static_cast<float*>(workspace), out, page_table, seq_len, max_pages,
                    n_pool};
  return hip_status(dsa::launch_decode(a, static_cast<hipStream_t>(stream)), "dsa_paged_decode");
}

int dsa_nsa_compress(int dtype, const void* k, const void* v, int B, int Hkv, int S, int D, int len,
                     int stride, void* ck, void* cv, void* stream) {
  g_err.clear();
  TRY(check_dtype(dtype, false));
  TRY(check_heads(B, Hkv, Hkv));
  TRY(check_dim(D));
  REQUIRE(len >= 1 && stride >= 1, DSA_E_ARG, "len and stride must be >= 1 (got %d, %d)", len,
          stride);
  REQUIRE(S >= len, DSA_E_ARG, "S (%d) must be >= len (%d)", S, len);
  REQUIRE(B * Hkv <= 65535, DSA_E_UNSUPPORTED, "B*Hkv must be at most 65535");
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(ck);
  REQUIRE_PTR(cv);
  return hip_status(dsa::launch_nsa_compress(k, v, B, Hkv, S, D, len, stride, ck, cv,
                                             static_cast<hipStream_t>(stream)),
                    "dsa_nsa_compress");
}

int dsa_nsa_cmp_token_scores(int dtype, const void* q, const void* ck, const float* lse, int B,
                             int Hq, int Hkv, int S, int D, int len, int stride, int sel_block,
                             float scale, float* scores, void* stream) {
  g_err.clear();
  TRY(check_dtype(dtype, false));
  TRY(check_heads(B, Hq, Hkv));
  TRY(check_dim(D));
  TRY(check_block(sel_block, "sel_block"));
  REQUIRE(len >= 1 && stride >= 1, DSA_E_ARG, "len and stride must be >= 1 (got %d, %d)", len,
          stride);
  REQUIRE(S >= len, DSA_E_ARG, "S (%d) must be >= len (%d)", S, len);
  REQUIRE(rows_fit(B, Hq, S), DSA_E_ARG, "B*Hq*S too large");
  TRY(check_group_extent(Hq / Hkv, S, D, "S"));
  REQUIRE(scale > 0.f, DSA_E_ARG, "scale must be > 0");
  REQUIRE(Hq / Hkv <= 16, DSA_E_UNSUPPORTED, "at most 16 query heads per KV head (got %d)",
          Hq / Hkv);
  REQUIRE((sel_block + len - 2) / stride <= 31, DSA_E_UNSUPPORTED,
          "a selection block may overlap at most 32 summaries (sel_block %d, len %d, stride %d)",
          sel_block, len, stride);
  const int nb = (S + sel_block - 1) / sel_block;
  REQUIRE(rows_fit(B * Hkv, S, nb), DSA_E_ARG, "B*Hkv*S*nb too large");
  REQUIRE_PTR(q);
  REQUIRE_PTR(ck);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(scores);
  const int n_cmp = (S - len) / stride + 1;
  dsa::CmpScoreArgs c{q, ck, lse, B, Hq, Hkv, S, n_cmp, D, len, stride, sel_block, scale, scores};
  return hip_status(dsa::launch_cmp_token_scores(c, static_cast<hipStream_t>(stream)),
                    "dsa_nsa_cmp_token_scores");
}

int dsa_sparse_attn_tokens(int dtype, const void* q, const void* k, const void* v, int B, int Hq,
                           int Hkv, int S, int D, const int32_t* idx, const int32_t* count,
                           int idx_width, int block, float scale, void* out, float* lse,
                           void* stream) {
  g_err.clear();
  TRY(check_dtype(dtype, false));
  TRY(check_heads(B, Hq, Hkv));
  TRY(check_block(block, "block"));
  REQUIRE(D == 128, DSA_E_UNSUPPORTED, "per-token lists need D = 128 (got %d)", D);
  REQUIRE(Hq / Hkv <= 16, DSA_E_UNSUPPORTED, "at most 16 query heads per KV head (got %d)",
          Hq / Hkv);
  REQUIRE(S >= 1, DSA_E_ARG, "S must be >= 1 (got %d)", S);
  REQUIRE(idx_width >= 1 && idx_width <= 64, DSA_E_UNSUPPORTED,
          "idx_width must be in [1, 64] (got %d)", idx_width);
  REQUIRE(rows_fit(B, Hq, S), DSA_E_ARG, "B*Hq*S too large");
  TRY(check_group_extent(Hq / Hkv, S, D, "S"));
  REQUIRE(rows_fit(B * Hkv, S, idx_width), DSA_E_ARG, "B*Hkv*S*idx_width too large");
  REQUIRE(scale > 0.f, DSA_E_ARG, "scale must be > 0");
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(out);
  REQUIRE(idx != nullptr && count != nullptr, DSA_E_ARG, "idx and count must not be NULL");
  dsa::AttnArgs a{};
  a.dtype = dtype;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.idx = idx;
  a.count = count;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.S = S;
  a.Skv = S;
  a.D = D;
  a.block = block;
  a.idx_width = idx_width;
  a.mode = dsa::MODE_INDEX;
  a.sel_heads = Hq / Hkv;
  a.scale = scale;
  REQUIRE(dsa::token_attention_supported(a), DSA_E_UNSUPPORTED,
          "no per-token attention kernel for this configuration");
  return hip_status(dsa::launch_token_attention(a, static_cast<hipStream_t>(stream)),
                    "dsa_sparse_attn_tokens");
}

int dsa_nsa_cmp_attn(int dtype, const void* q, const void* ck, const void* cv, int B, int Hq,
                     int Hkv, int S, int D, int len, int stride, int sel_block, float scale,
                     void* out, float* lse, float* block_scores, void* stream) {
  g_err.clear();
  TRY(check_dtype(dtype, false));
  TRY(check_heads(B, Hq, Hkv));
  TRY(check_dim(D));
  TRY(check_block(sel_block, "sel_block"));
  REQUIRE(len >= 1 && stride >= 1, DSA_E_ARG, "len and stride must be >= 1 (got %d, %d)", len,
          stride);
  REQUIRE(S >= len, DSA_E_ARG, "S (%d) must be >= len (%d)", S, len);
  REQUIRE(rows_fit(B, Hq, S), DSA_E_ARG, "B*Hq*S too large");
  REQUIRE(scale > 0.f, DSA_E_ARG, "scale must be > 0");
  TRY(check_group_extent(Hq / Hkv, S, D, "S"));
  const int n_cmp = (S - len) / stride + 1;
  REQUIRE(n_cmp <= 8192, DSA_E_UNSUPPORTED, "at most 8192 summaries (got %d)", n_cmp);
  REQUIRE_PTR(q);
  REQUIRE_PTR(ck);
  REQUIRE_PTR(cv);
  REQUIRE_PTR(out);
  REQUIRE(lse != nullptr, DSA_E_ARG, "lse must not be NULL");
  auto s = static_cast<hipStream_t>(stream);
  dsa::AttnArgs a{};
  a.dtype = dtype;
  a.q = q;
  a.k = ck;
  a.v = cv;
  a.out = out;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.S = S;
  a.Skv = n_cmp;
  a.D = D;
  a.block = sel_block;
  a.mode = dsa::MODE_CMP;
  a.cmp_len = len;
  a.cmp_stride = stride;
  a.sel_heads = Hq / Hkv;
  a.key_bias = nullptr;
  a.scale = scale;
  int st = hip_status(dsa::launch_attention(a, s), "dsa_nsa_cmp_attn");
  if (st != DSA_OK || block_scores == nullptr) return st;
  dsa::CmpScoreArgs c{q, ck, lse, B, Hq, Hkv, S, n_cmp, D, len, stride, sel_block, scale,
                      block_scores};
  return hip_status(dsa::launch_cmp_block_scores(c, s), "dsa_nsa_cmp_attn");
}

int dsa_nsa_window_combine(int dtype, const void* q, const void* k, const void* v, int B, int Hq,
                           int Hkv, int S, int D, int window, float scale, const void* o_cmp,
                           const void* o_sel, const float* gate_logits, void* out,
                           void* stream) {
  g_err.clear();
  TRY(check_dtype(dtype, false));
  TRY(check_heads(B, Hq, Hkv));
  REQUIRE(D == 128, DSA_E_UNSUPPORTED, "the fused combine needs D = 128 (got %d)", D);
  REQUIRE(S >= 1, DSA_E_ARG, "S must be >= 1 (got %d)", S);
  REQUIRE(window >= 1, DSA_E_ARG, "window must be >= 1 (got %d)", window);
  REQUIRE(rows_fit(B, Hq, S), DSA_E_ARG, "B*Hq*S too large");
  TRY(check_group_extent(Hq / Hkv, S, D, "S"));
  REQUIRE(scale > 0.f, DSA_E_ARG, "scale must be > 0");
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(o_cmp);
  REQUIRE_PTR(o_sel);
  REQUIRE_PTR(gate_logits);
  REQUIRE_PTR(out);
  dsa::AttnArgs a{};
  a.dtype = dtype;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.S = S;
  a.Skv = S;
  a.D = D;
  a.block = 64;
  a.mode = dsa::MODE_WINDOW;
  a.window = window;
  a.cmp_len = 1;
  a.cmp_stride = 1;
  a.sel_heads = Hq / Hkv;
  a.gate_o1 = o_cmp;
  a.gate_o2 = o_sel;
  a.gate_z = gate_logits;
  a.scale = scale;
  REQUIRE(dsa::attention_supported(a), DSA_E_UNSUPPORTED,
          "the fused combine needs at least 4 query heads per KV head and a window of at most "
          "8000 tokens");
  return hip_status(dsa::launch_attention(a, static_cast<hipStream_t>(stream)),
                    "dsa_nsa_window_combine");
}

int dsa_nsa_select_window_combine(int dtype, const void* q, const void* k, const void* v, int B,
                                  int Hq, int Hkv, int S, int D, const int32_t* idx,
                                  const int32_t* count, int idx_width, int sel_block, int window,
                                  float scale, const void* o_cmp, const float* gate_logits,
                                  void* out, void* stream) {
  g_err.clear();
  TRY(check_dtype(dtype, false));
  TRY(check_heads(B, Hq, Hkv));
  REQUIRE(D == 128, DSA_E_UNSUPPORTED, "the fused branches need D = 128 (got %d)", D);
  TRY(check_block(sel_block, "sel_block"));
  REQUIRE(S >= 1, DSA_E_ARG, "S must be >= 1 (got %d)", S);
  REQUIRE(window >= 1, DSA_E_ARG, "window must be >= 1 (got %d)", window);
  REQUIRE(idx_width >= 1, DSA_E_ARG, "idx_width must be >= 1 (got %d)", idx_width);
  REQUIRE(rows_fit(B, Hq, S), DSA_E_ARG, "B*Hq*S too large");
  TRY(check_group_extent(Hq / Hkv, S, D, "S"));
  REQUIRE(scale > 0.f, DSA_E_ARG, "scale must be > 0");
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE(idx != nullptr && count != nullptr, DSA_E_ARG, "idx and count must not be NULL");
  REQUIRE_PTR(o_cmp);
  REQUIRE_PTR(gate_logits);
  REQUIRE_PTR(out);
  dsa::AttnArgs a{};
  a.dtype = dtype;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.idx = idx;
  a.count = count;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.S = S;
  a.Skv = S;
  a.D = D;
  a.block = sel_block;
  a.idx_width = idx_width;
  a.mode = dsa::MODE_INDEX;
  a.cmp_len = 1;
  a.cmp_stride = 1;
  a.sel_heads = Hq / Hkv;
  a.gate_o1 = o_cmp;
  a.gate_z = gate_logits;
  a.scale = scale;
  a.then_window = window;
  REQUIRE(dsa::attention_supported(a), DSA_E_UNSUPPORTED,
          "the fused branches need blocks of 64k tokens, at least 256 rows per query block and "
          "group, and idx_width * sel_block/64 + (window + sel_block)/64 + 2 <= 128");
  return hip_status(dsa::launch_attention(a, static_cast<hipStream_t>(stream)),
                    "dsa_nsa_select_window_combine");
}

int dsa_nsa_combine(int dtype, const void* o_cmp, const void* o_sel, const void* o_win,
                    const float* gate_logits, int B, int Hq, int S, int D, void* out,
                    void* stream) {
  g_err.clear();
  TRY(check_dtype(dtype, false));
  TRY(check_heads(B, Hq, Hq));
  TRY(check_dim(D));
  REQUIRE(S >= 1, DSA_E_ARG, "S must be >= 1 (got %d)", S);
  REQUIRE_PTR(o_cmp);
  REQUIRE_PTR(o_sel);
  REQUIRE_PTR(o_win);
  REQUIRE_PTR(gate_logits);
  REQUIRE_PTR(out);
  return hip_status(dsa::launch_nsa_combine(o_cmp, o_sel, o_win, gate_logits, B, Hq, S, D, out,
                                            static_cast<hipStream_t>(stream)),
                    "dsa_nsa_combine");
}

size_t dsa_read_stream_sink_words(void) { return 512; }   // two workgroups per CU

int dsa_read_stream(const void* src, size_t bytes, uint32_t* sink, size_t sink_words,
                    void* stream) {
  g_err.clear();
  REQUIRE_PTR(src);
  REQUIRE(sink != nullptr, DSA_E_ARG, "sink must not be NULL");
  REQUIRE(bytes >= 16 && bytes % 16 == 0, DSA_E_ARG,
          "bytes must be a positive multiple of 16 (got %zu)", bytes);
  REQUIRE(sink_words >= dsa_read_stream_sink_words(), DSA_E_WORKSPACE,
          "sink needs %zu words (got %zu)", dsa_read_stream_sink_words(), sink_words);
  return hip_status(dsa::launch_read_stream(src, bytes, sink, int(dsa_read_stream_sink_words()),
                                            static_cast<hipStream_t>(stream)),
                    "dsa_read_stream");
}

}  // extern "C"
