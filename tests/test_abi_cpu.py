"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments before enqueuing anything (the
validation layer makes no HIP call, so these run on a CPU-only host)."""
import ctypes
import os
import re

import pytest

from dynamic_block_sparse_head_amd import binding as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libdsa.so not built")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(L.LIB_PATH)
    names = _declared()
    assert len(names) == 28
    for n in names:
        assert hasattr(lib, n), f"{n} declared in dsa.h but not exported"
    assert set(names) == set(L.SIGNATURES), "binding prototypes out of sync with dsa.h"


def test_version_and_status_strings():
    lib = L.load()
    assert lib.dsa_version() == 101
    for st in (0, -1, -2, -3, -4):
        assert lib.dsa_status_string(st)
    assert lib.dsa_status_string(12345) == b"unknown dsa status"


FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10004)


def _err():
    return L.load().dsa_last_error().decode()


def test_topk_validation():
    lib = L.load()
    assert lib.dsa_topk_select(None, 1, 1, 8, 2, 1, 1, FAKE, FAKE, None) == L.DSA_E_ARG
    assert "scores" in _err()
    assert lib.dsa_topk_select(FAKE, 1, 1, 8, -1, 1, 1, FAKE, FAKE, None) == L.DSA_E_ARG
    assert lib.dsa_topk_select(FAKE, 1, 1, 8, 0, 0, 1, FAKE, FAKE, None) == L.DSA_E_ARG
    assert lib.dsa_topk_select(FAKE, 1, 1, 9000, 2, 1, 1, FAKE, FAKE, None) == L.DSA_E_UNSUPPORTED
    assert lib.dsa_topk_select(FAKE, 1, 9, 8, 2, 1, 1, FAKE, FAKE, None) == L.DSA_E_ARG  # n_q > n_k
    assert lib.dsa_topk_select(MISALIGNED, 1, 1, 8, 2, 1, 1, FAKE, FAKE, None) == L.DSA_E_ARG
    assert "aligned" in _err()


def test_prefill_validation():
    lib = L.load()
    f = lib.dsa_sparse_attn_prefill
    ok = dict(dtype=1, q=FAKE, k=FAKE, v=FAKE, B=1, Hq=4, Hkv=2, S=256, D=128, idx=FAKE, count=FAKE,
              width=3, block=64, window=0, scale=0.1, out=FAKE, lse=None, stream=None)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["dtype"], a["q"], a["k"], a["v"], a["B"], a["Hq"], a["Hkv"], a["S"], a["D"],
                 a["idx"], a["count"], a["width"], a["block"], a["window"], a["scale"], a["out"],
                 a["lse"], a["stream"])

    assert call(dtype=7) == L.DSA_E_ARG
    assert call(D=96) == L.DSA_E_UNSUPPORTED
    assert call(Hq=3) == L.DSA_E_ARG                      # Hq % Hkv
    assert call(block=48) == L.DSA_E_UNSUPPORTED
    assert call(block=0) == L.DSA_E_ARG
    assert call(q=None) == L.DSA_E_ARG
    assert call(count=None) == L.DSA_E_ARG                # idx without count
    assert call(window=64) == L.DSA_E_ARG                 # window in index mode
    assert call(idx=None, count=None, window=0) == L.DSA_E_ARG
    assert call(scale=0.0) == L.DSA_E_ARG
    assert call(S=0) == L.DSA_E_ARG
    assert call(B=70000) == L.DSA_E_UNSUPPORTED


def test_scores_and_decode_validation():
    lib = L.load()
    need = lib.dsa_block_scores_workspace_size(0, 1, 32, 8, 16384, 128, 64)
    assert need == 2 * 8 * 256 * 128 * 8
    st = lib.dsa_block_scores(0, 1, FAKE, FAKE, None, 1, 32, 8, 16384, 128, 64, FAKE, need - 8,
                              FAKE, None)
    assert st == L.DSA_E_WORKSPACE
    assert lib.dsa_block_scores(0, 1, FAKE, FAKE, FAKE, 1, 32, 8, 16384, 128, 64, FAKE, need,
                                FAKE, None) == L.DSA_E_ARG       # kmax with POOLED
    assert lib.dsa_block_scores(5, 1, FAKE, FAKE, None, 1, 32, 8, 16384, 128, 64, FAKE, need,
                                FAKE, None) == L.DSA_E_ARG       # unknown kind
    ws = lib.dsa_sparse_attn_decode_workspace_size(16, 32, 8, 102, 64, 128)
    assert ws == 16 * 32 * 6 * 130 * 4       # 6 chunks of 17 pages: one round of 768 workgroups
    dec = lib.dsa_sparse_attn_decode
    args = [1, FAKE, FAKE, FAKE, 16, 32, 8, 131072, 128, FAKE, FAKE, 102, 64, 0.1, FAKE, ws, FAKE,
            None]
    a = list(args); a[0] = 0
    assert dec(*a) == L.DSA_E_UNSUPPORTED                          # float32 decode
    a = list(args); a[12] = 96
    assert dec(*a) == L.DSA_E_UNSUPPORTED                          # page 96
    a = list(args); a[15] = ws - 1
    assert dec(*a) == L.DSA_E_WORKSPACE
    a = list(args); a[5] = 48
    assert dec(*a) == L.DSA_E_UNSUPPORTED                          # G = 6
    a = list(args); a[11] = 5000
    assert dec(*a) == L.DSA_E_ARG                                  # more pages than the cache


def test_selection_unit_validation():
    lib = L.load()
    g = lib.dsa_block_scores_workspace_size(0, 1, 32, 8, 16384, 128, 64)
    h = lib.dsa_block_scores_workspace_size(2, 1, 32, 8, 16384, 128, 64)
    assert h == (32 + 8) * 256 * 128 * 8 and g == 2 * 8 * 256 * 128 * 8
    f = lib.dsa_sparse_attn_prefill_ex
    args = [1, FAKE, FAKE, FAKE, 1, 32, 8, 2048, 128, FAKE, FAKE, 24, 64, 1, None, 0.1, FAKE, None,
            None]
    a = list(args); a[13] = 3
    assert f(*a) == L.DSA_E_ARG                                    # 3 does not divide G = 4
    assert "sel_heads" in _err()
    a = list(args); a[13] = 0
    assert f(*a) == L.DSA_E_ARG
    a = list(args); a[9] = None
    assert f(*a) == L.DSA_E_ARG                                    # index lists required
    a = list(args); a[12] = 48
    assert f(*a) == L.DSA_E_UNSUPPORTED                            # block 48
    a = list(args); a[14] = FAKE
    assert f(*a) == L.DSA_E_UNSUPPORTED                            # key bias with per-head units


def test_dma_weights_validation():
    lib = L.load()
    f = lib.dsa_dma_weights
    args = [1, FAKE, 1, 8, 2048, 128, FAKE, FAKE, 64, FAKE, FAKE, None]
    a = list(args); a[5] = 96
    assert f(*a) == L.DSA_E_UNSUPPORTED
    a = list(args); a[7] = None
    assert f(*a) == L.DSA_E_ARG and "gain" in _err()
    a = list(args); a[6] = MISALIGNED
    assert f(*a) == L.DSA_E_ARG
    a = list(args); a[8] = 33
    assert f(*a) == L.DSA_E_UNSUPPORTED


def test_paged_validation():
    lib = L.load()
    app = lib.dsa_paged_append
    args = [1, FAKE, FAKE, 4, 8, 128, 64, 100, FAKE, FAKE, 500, FAKE, FAKE, FAKE, FAKE, None]
    a = list(args); a[0] = 0
    assert app(*a) == L.DSA_E_UNSUPPORTED                          # float32
    a = list(args); a[6] = 48
    assert app(*a) == L.DSA_E_UNSUPPORTED                          # page 48
    a = list(args); a[9] = None
    assert app(*a) == L.DSA_E_ARG and "seq_len" in _err()
    a = list(args); a[10] = 0
    assert app(*a) == L.DSA_E_ARG                                  # empty pool
    dec = lib.dsa_paged_decode
    ws = lib.dsa_sparse_attn_decode_workspace_size(4, 32, 8, 10, 64, 128)
    args = [1, FAKE, FAKE, FAKE, 4, 32, 8, 128, 64, 100, FAKE, FAKE, 500, FAKE, FAKE, 10, 0.1, FAKE,
            ws, FAKE, None]
    a = list(args); a[18] = ws - 4
    assert dec(*a) == L.DSA_E_WORKSPACE
    a = list(args); a[5] = 48
    assert dec(*a) == L.DSA_E_UNSUPPORTED                          # G = 6
    a = list(args); a[13] = None
    assert dec(*a) == L.DSA_E_ARG
    sc = lib.dsa_paged_page_scores
    assert sc(1, FAKE, FAKE, FAKE, 4, 32, 8, 128, 64, 100, None, FAKE, 500, FAKE, None) == L.DSA_E_ARG


def test_backward_validation():
    lib = L.load()
    ws = lib.dsa_sparse_attn_prefill_backward_workspace_size(1, 32, 8, 16384, 128, 64)
    nb = 256
    assert ws == 2 * 32 * 16384 * 4 + 8 * nb * nb * 4 + 8 * nb * 4
    f = lib.dsa_sparse_attn_prefill_backward
    ok = dict(dtype=1, q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, dout=FAKE, B=1, Hq=32, Hkv=8,
              S=16384, D=128, idx=FAKE, count=FAKE, width=24, block=64, scale=0.1, ws=FAKE,
              ws_bytes=ws, dq=FAKE, dk=FAKE, dv=FAKE, stream=None)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["dtype"], a["q"], a["k"], a["v"], a["out"], a["lse"], a["dout"], a["B"],
                 a["Hq"], a["Hkv"], a["S"], a["D"], a["idx"], a["count"], a["width"], a["block"],
                 a["scale"], a["ws"], a["ws_bytes"], a["dq"], a["dk"], a["dv"], a["stream"])

    assert call(dtype=0) == L.DSA_E_UNSUPPORTED           # float32 backward
    assert call(D=96) == L.DSA_E_UNSUPPORTED
    assert call(block=40) == L.DSA_E_UNSUPPORTED
    assert call(ws_bytes=ws - 1) == L.DSA_E_WORKSPACE
    assert call(ws=None) == L.DSA_E_WORKSPACE
    assert call(lse=None) == L.DSA_E_ARG
    assert call(count=None) == L.DSA_E_ARG
    assert call(dk=MISALIGNED) == L.DSA_E_ARG
    assert "dk" in _err()
    assert call(width=0) == L.DSA_E_ARG
    assert call(scale=-1.0) == L.DSA_E_ARG
    assert call(Hq=12) == L.DSA_E_ARG                     # Hq % Hkv


def test_nsa_validation():
    lib = L.load()
    assert lib.dsa_nsa_compress(1, FAKE, FAKE, 1, 4, 16, 128, 32, 16, FAKE, FAKE, None) == L.DSA_E_ARG
    assert lib.dsa_nsa_cmp_attn(1, FAKE, FAKE, FAKE, 1, 64, 4, 32768, 128, 32, 16, 64, 0.1, FAKE,
                                None, None, None) == L.DSA_E_ARG         # lse required
    assert lib.dsa_nsa_combine(0, FAKE, FAKE, FAKE, FAKE, 1, 4, 8, 128, FAKE, None) == L.DSA_E_UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    import torch
    s = torch.zeros(1, 4, 4)
    idx = torch.zeros(1, 4, 2, dtype=torch.int32)
    cnt = torch.zeros(1, 4, dtype=torch.int32)
    with pytest.raises(ValueError):
        L.dsa_topk_select(s, 1, 1, True, idx, cnt)


def test_per_token_selection_validation():
    """Every call below fails validation (one bad argument each), so nothing
    is launched with the fake pointers."""
    lib = L.load()
    ts = lib.dsa_nsa_cmp_token_scores
    args = [1, FAKE, FAKE, FAKE, 1, 64, 4, 32768, 128, 32, 16, 64, 0.1, FAKE, None]
    a = list(args); a[5] = 68
    assert ts(*a) == L.DSA_E_UNSUPPORTED                           # G = 17
    a = list(args); a[10] = 2
    assert ts(*a) == L.DSA_E_UNSUPPORTED                           # block spans 47 summaries
    a = list(args); a[3] = None
    assert ts(*a) == L.DSA_E_ARG and "lse" in _err()
    a = list(args); a[0] = 0
    assert ts(*a) == L.DSA_E_UNSUPPORTED                           # float32
    tk = lib.dsa_topk_select_tokens
    assert tk(FAKE, 4, 32768, 511, 16, 0, 64, FAKE, FAKE, None) == L.DSA_E_ARG   # n_k < blocks
    assert tk(FAKE, 4, 32768, 512, 16, 0, 0, FAKE, FAKE, None) == L.DSA_E_ARG    # block 0
    assert tk(None, 4, 32768, 512, 16, 0, 64, FAKE, FAKE, None) == L.DSA_E_ARG
    at = lib.dsa_sparse_attn_tokens
    args = [1, FAKE, FAKE, FAKE, 1, 64, 4, 32768, 128, FAKE, FAKE, 16, 64, 0.1, FAKE, None, None]
    a = list(args); a[8] = 64
    assert at(*a) == L.DSA_E_UNSUPPORTED                           # D = 64
    a = list(args); a[11] = 65
    assert at(*a) == L.DSA_E_UNSUPPORTED                           # list too wide
    a = list(args); a[12] = 96
    assert at(*a) == L.DSA_E_UNSUPPORTED                           # block 96
    a = list(args); a[12] = 128
    assert at(*a) == L.DSA_E_UNSUPPORTED                           # block 128
    a = list(args); a[10] = None
    assert at(*a) == L.DSA_E_ARG
    a = list(args); a[5] = 128
    assert at(*a) == L.DSA_E_UNSUPPORTED                           # G = 32


def test_window_combine_validation():
    lib = L.load()
    f = lib.dsa_nsa_window_combine
    args = [1, FAKE, FAKE, FAKE, 1, 64, 4, 32768, 128, 512, 0.1, FAKE, FAKE, FAKE, FAKE, None]
    a = list(args); a[8] = 64
    assert f(*a) == L.DSA_E_UNSUPPORTED                            # D = 64
    a = list(args); a[9] = 0
    assert f(*a) == L.DSA_E_ARG                                    # no window
    a = list(args); a[13] = None
    assert f(*a) == L.DSA_E_ARG and "gate_logits" in _err()
    a = list(args); a[5] = 8
    assert f(*a) == L.DSA_E_UNSUPPORTED                            # G = 2: fewer than 256 rows
    a = list(args); a[9] = 9000
    assert f(*a) == L.DSA_E_UNSUPPORTED                            # window too long


def test_select_window_combine_validation():
    lib = L.load()
    f = lib.dsa_nsa_select_window_combine
    # q k v B Hq Hkv S D idx count width sel_block window scale o_cmp z out stream
    args = [1, FAKE, FAKE, FAKE, 1, 64, 4, 32768, 128, FAKE, FAKE, 16, 64, 512, 0.1, FAKE, FAKE,
            FAKE, None]
    a = list(args); a[8] = 64
    assert f(*a) == L.DSA_E_UNSUPPORTED                            # D = 64
    a = list(args); a[13] = 0
    assert f(*a) == L.DSA_E_ARG                                    # no window
    a = list(args); a[11] = 0
    assert f(*a) == L.DSA_E_ARG                                    # empty lists
    a = list(args); a[10] = None
    assert f(*a) == L.DSA_E_ARG and "count" in _err()
    a = list(args); a[16] = None
    assert f(*a) == L.DSA_E_ARG and "gate_logits" in _err()
    a = list(args); a[0] = 0
    assert f(*a) == L.DSA_E_UNSUPPORTED                            # float32
    a = list(args); a[12] = 32
    assert f(*a) == L.DSA_E_UNSUPPORTED                            # 32-token blocks
    a = list(args); a[5] = 8
    assert f(*a) == L.DSA_E_UNSUPPORTED                            # G = 2: fewer than 256 rows
    a = list(args); a[11] = 120
    assert f(*a) == L.DSA_E_UNSUPPORTED                            # 120 + 10 tiles > 128
    a = list(args); a[7] = 1 << 20; a[5] = 32; a[6] = 2
    assert f(*a) == L.DSA_E_UNSUPPORTED and "2^31" in _err()       # group beyond 32-bit offsets


def test_offsets_beyond_32_bits_are_rejected():
    """Kernels address one KV group's rows with 32-bit buffer offsets: a
    group of G * S * D >= 2^31 elements is refused before any launch, in
    every attention call and in decode (L * D).  (Every call here fails
    validation, so the fake pointers never reach a kernel.)"""
    lib = L.load()
    S = 1 << 20                                   # 16 heads per group * 2^20 * 128 = 2^31
    f = lib.dsa_sparse_attn_prefill
    assert f(1, FAKE, FAKE, FAKE, 1, 32, 2, S, 128, FAKE, FAKE, 24, 64, 0, 0.1, FAKE, None,
             None) == L.DSA_E_UNSUPPORTED
    assert "2^31" in _err()
    assert lib.dsa_nsa_window_combine(1, FAKE, FAKE, FAKE, 1, 32, 2, S, 128, 512, 0.1, FAKE, FAKE,
                                      FAKE, FAKE, None) == L.DSA_E_UNSUPPORTED
    assert lib.dsa_nsa_cmp_attn(1, FAKE, FAKE, FAKE, 1, 32, 2, S, 128, 32, 16, 64, 0.1, FAKE,
                                FAKE, None, None) == L.DSA_E_UNSUPPORTED
    L_ = 1 << 24                                  # 2^24 * 128 = 2^31
    ws = lib.dsa_sparse_attn_decode_workspace_size(1, 8, 8, 102, 64, 128)
    assert lib.dsa_sparse_attn_decode(1, FAKE, FAKE, FAKE, 1, 8, 8, L_, 128, FAKE, FAKE, 102, 64,
                                      0.1, FAKE, ws, FAKE, None) == L.DSA_E_UNSUPPORTED
    assert "2^31" in _err()


def test_bad_layouts_are_rejected():
    """Sizes that do not describe a valid dense layout fail validation: a
    cache length that is not a whole number of pages, a page list wider than
    the cache, summaries longer than the sequence, misaligned buffers."""
    lib = L.load()
    ws = lib.dsa_sparse_attn_decode_workspace_size(1, 8, 8, 4, 64, 128)
    dec = lib.dsa_sparse_attn_decode
    assert dec(1, FAKE, FAKE, FAKE, 1, 8, 8, 1000, 128, FAKE, FAKE, 4, 64, 0.1, FAKE, ws, FAKE,
               None) == L.DSA_E_ARG                                # L % page != 0
    assert dec(1, FAKE, FAKE, FAKE, 1, 8, 8, 256, 128, FAKE, FAKE, 5, 64, 0.1, FAKE, ws, FAKE,
               None) == L.DSA_E_ARG                                # 5 pages of a 4-page cache
    assert dec(1, FAKE, MISALIGNED, FAKE, 1, 8, 8, 256, 128, FAKE, FAKE, 4, 64, 0.1, FAKE, ws,
               FAKE, None) == L.DSA_E_ARG
    assert "aligned" in _err()
    assert lib.dsa_page_minmax(1, FAKE, 1, 8, 1000, 128, 64, FAKE, FAKE, None) == L.DSA_E_ARG
    assert lib.dsa_nsa_compress(1, FAKE, FAKE, 1, 4, 31, 128, 32, 16, FAKE, FAKE,
                                None) == L.DSA_E_ARG               # S < len


def test_read_stream_validation():
    lib = L.load()
    n = lib.dsa_read_stream_sink_words()
    assert n >= 256
    assert lib.dsa_read_stream(FAKE, 0, FAKE, n, None) == L.DSA_E_ARG
    assert lib.dsa_read_stream(FAKE, 24, FAKE, n, None) == L.DSA_E_ARG      # not 16-byte chunks
    assert lib.dsa_read_stream(MISALIGNED, 32, FAKE, n, None) == L.DSA_E_ARG
    assert lib.dsa_read_stream(FAKE, 32, None, n, None) == L.DSA_E_ARG
    assert lib.dsa_read_stream(FAKE, 32, FAKE, n - 1, None) == L.DSA_E_WORKSPACE


def test_decode_noalloc_validation():
    """The non-allocating decode validates like the workspace call and
    refuses a decode whose partial results exceed its scratch, before it
    touches the GPU."""
    lib = L.load()
    f = lib.dsa_sparse_attn_decode_noalloc
    args = [1, FAKE, FAKE, FAKE, 16, 32, 8, 131072, 128, FAKE, FAKE, 102, 64, 0.1, FAKE, None]
    limit = 16 << 20
    assert lib.dsa_sparse_attn_decode_workspace_size(16, 32, 8, 102, 64, 128) <= limit
    big = list(args); big[4] = 128                                  # 8x the batch
    assert lib.dsa_sparse_attn_decode_workspace_size(128, 32, 8, 102, 64, 128) > limit
    assert f(*big) == L.DSA_E_WORKSPACE
    assert "scratch" in _err()
    a = list(args); a[0] = 0
    assert f(*a) == L.DSA_E_UNSUPPORTED                             # float32
    a = list(args); a[12] = 96
    assert f(*a) == L.DSA_E_UNSUPPORTED                             # page 96
    a = list(args); a[11] = 5000
    assert f(*a) == L.DSA_E_ARG                                     # more pages than the cache
    a = list(args); a[9] = None
    assert f(*a) == L.DSA_E_ARG                                     # no page lists
    a = list(args); a[14] = MISALIGNED
    assert f(*a) == L.DSA_E_ARG
