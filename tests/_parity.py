"""Shared helpers for the GPU parity tests (not collected by pytest).

Acceptance rules (the bar every GPU result is held to):
  * indices: window blocks, counts and -1 padding identical; the top-k part
    must be *a* valid top-k under the oracle's scores up to a 1e-4 score gap:
    min over chosen of s >= max over unchosen candidates of s - 1e-4.  Where
    every gap is >= 1e-4 this forces bit-exact equality.
  * bf16 outputs: max-abs <= 2e-2 and mean-abs <= 2e-3 against the float64
    oracle evaluated at the GPU's accepted indices, and, because outputs can
    be far smaller than 2e-2, also max-abs <= 2^-6 * max|oracle| (eight bf16
    unit roundoffs: P and O are rounded to bf16 once each).
  * float32 outputs: max-abs <= 1e-4.
  * bf16 gradients (dq, dk, dv of the backward): max-abs <= 2^-6 * max|oracle|
    and ||gpu - oracle||_2 <= 2^-7 * ||oracle||_2.  P and dS enter the
    second products rounded to bf16 and the results are rounded to bf16,
    about three unit roundoffs (2^-9 each) per term; the norm bound leaves
    a factor ~5 over that and catches a systematic error that the max test
    alone could hide.  Gradient magnitudes (dq ~ 1e-4 at the 16K shape)
    make fixed absolute bounds meaningless, so both bounds are relative.
"""
from __future__ import annotations

import numpy as np
import torch

GAP = 1e-4
BF16_MAX_ABS, BF16_MEAN_ABS, BF16_REL_TO_MAX = 2e-2, 2e-3, 2.0 ** -6
F32_MAX_ABS = 1e-4


def to_np(t):
    return t.detach().to(torch.float64).cpu().numpy()


def check_index_row(s_row, gpu_row, gpu_cnt, k, n_local, causal, i, n_k):
    """Returns True when the GPU row equals the oracle's selection bit for bit;
    raises AssertionError when it is not an acceptable top-k."""
    if causal:
        last = i - n_local
        window = set(range(max(0, i - n_local + 1), i + 1))
    else:
        last = n_k - 1 - n_local
        window = set(range(n_k - n_local, n_k))
    cands = list(range(0, last + 1))
    n_top = min(k, len(cands))
    want_cnt = len(window) + n_top
    assert gpu_cnt == want_cnt, f"row {i}: count {gpu_cnt} != {want_cnt}"
    row = list(gpu_row[:gpu_cnt])
    assert row == sorted(row) and len(set(row)) == len(row), f"row {i}: not ascending/unique {row}"
    assert all(x == -1 for x in gpu_row[gpu_cnt:]), f"row {i}: bad padding"
    chosen = set(row)
    assert window <= chosen, f"row {i}: window {window} missing from {row}"
    top = chosen - window
    assert top <= set(cands), f"row {i}: non-candidate chosen {top - set(cands)}"
    assert len(top) == n_top
    rest = [j for j in cands if j not in top]
    if top and rest:
        lo = min(s_row[j] for j in top)
        hi = max(s_row[j] for j in rest)
        assert lo >= hi - GAP, f"row {i}: chosen min {lo} < unchosen max {hi} - {GAP}"
    oracle_top = sorted(cands, key=lambda j: (-s_row[j], j))[:n_top]
    return set(oracle_top) == top


def check_indices(scores, gpu_idx, gpu_cnt, k, n_local, causal, rows=None):
    """scores [..., nQ, nK] (oracle), gpu_idx [..., nQ, W], gpu_cnt [..., nQ].
    rows: the query-block index of each of the nQ rows when they are a slice
    (default 0..nQ-1).  Returns the fraction of rows that are bit-exact (all
    rows must be accepted)."""
    nQ, nK = scores.shape[-2:]
    rows = list(range(nQ)) if rows is None else list(rows)
    s = scores.reshape(-1, nQ, nK)
    gi = gpu_idx.reshape(-1, nQ, gpu_idx.shape[-1])
    gc = gpu_cnt.reshape(-1, nQ)
    exact = total = 0
    for r in range(s.shape[0]):
        for i in range(nQ):
            exact += check_index_row(s[r, i], gi[r, i], int(gc[r, i]), k, n_local, causal, rows[i], nK)
            total += 1
    return exact / total


def check_bf16(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ok = np.isfinite(ref)
    assert ok.any()
    err = np.abs(gpu[ok] - ref[ok])
    scale = np.abs(ref[ok]).max()
    assert np.isfinite(gpu[ok]).all(), f"{what}: non-finite GPU values"
    assert err.max() <= BF16_MAX_ABS, f"{what}: max-abs {err.max():.3e}"
    assert err.mean() <= BF16_MEAN_ABS, f"{what}: mean-abs {err.mean():.3e}"
    assert err.max() <= BF16_REL_TO_MAX * scale, f"{what}: max-abs {err.max():.3e} > 2^-6 * {scale:.3e}"
    return err.max(), err.mean()


GRAD_REL_TO_MAX, GRAD_REL_NORM = 2.0 ** -6, 2.0 ** -7


def check_grad(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref)
    scale = np.abs(ref).max()
    assert err.max() <= GRAD_REL_TO_MAX * scale, f"{what}: max-abs {err.max():.3e} > 2^-6 * {scale:.3e}"
    rel = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= GRAD_REL_NORM, f"{what}: relative norm error {rel:.3e}"
    return err.max() / scale, rel


def check_f32(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ok = np.isfinite(ref)
    err = np.abs(gpu[ok] - ref[ok])
    assert err.max() <= F32_MAX_ABS, f"{what}: max-abs {err.max():.3e}"
    return err.max()


def check_lse(gpu, ref, tol, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    assert (np.isneginf(gpu) == np.isneginf(ref)).all(), f"{what}: -inf pattern differs"
    assert np.abs(gpu[fin] - ref[fin]).max() <= tol, f"{what}: lse err {np.abs(gpu[fin]-ref[fin]).max()}"


def nsa_check_summaries(c, x, gck, gcv, groups=None):
    """The GPU's stored summaries against the oracle's (float64 mean rounded
    once to bf16): bit for bit.  Returns the oracle's (ck, cv) of the groups
    (all groups by default) as float64 arrays."""
    from oracle import nsa as On
    sl = slice(None) if groups is None else groups
    k, v = to_np(x["k"][:, sl]), to_np(x["v"][:, sl])
    ck = On.stored_summaries(k, c.cmp_len, c.cmp_stride, "bf16")
    cv = On.stored_summaries(v, c.cmp_len, c.cmp_stride, "bf16")
    gk, gv = to_np(gck[:, sl]), to_np(gcv[:, sl])
    assert np.array_equal(gk, ck), f"ck differs in {int((gk != ck).sum())} elements"
    assert np.array_equal(gv, cv), f"cv differs in {int((gv != cv).sum())} elements"
    return ck, cv
