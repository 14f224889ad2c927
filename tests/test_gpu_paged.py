"""GPU parity of the paged-cache serving decode: a pool of pages shared by a
batch of sequences of different lengths, filled partly in bulk and partly
token by token through dsa_paged_append (crossing page boundaries), then page
bounds through the page table, top pages, and attention — all against the
float64 oracle."""
import numpy as np
import pytest
import torch

from dynamic_block_sparse_head_amd import binding as L
from dynamic_block_sparse_head_amd.pipeline import PagedDecodePlan
from oracle import paged as Pg
from oracle import prefill as Op

from _parity import check_bf16, check_indices, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _build(full_pages, n_append, Hkv=8, G=4, D=128, page=64, spare=5, seed=0):
    """Pool with every sequence's first full_pages[b] pages written in bulk
    (summaries via dsa_page_minmax on the pool), then n_append tokens
    appended to every sequence one call at a time."""
    g = torch.Generator(device=DEV)
    g.manual_seed(1000 + seed)
    B = len(full_pages)
    lens = [f * page + n_append for f in full_pages]
    max_pages = max(-(-n // page) for n in lens) + 1
    n_pool = B * max_pages + spare
    rng = np.random.default_rng(seed)
    table = rng.permutation(n_pool)[:B * max_pages].reshape(B, max_pages).astype(np.int32)
    tok_k = torch.randn((B, max(lens), Hkv, D), generator=g, device=DEV).to(torch.bfloat16)
    tok_v = torch.randn((B, max(lens), Hkv, D), generator=g, device=DEV).to(torch.bfloat16)
    k_pool = torch.randn((n_pool, Hkv, page, D), generator=g, device=DEV).to(torch.bfloat16)  # stale data
    v_pool = torch.randn((n_pool, Hkv, page, D), generator=g, device=DEV).to(torch.bfloat16)
    for b in range(B):
        for p in range(full_pages[b]):
            phys = int(table[b, p])
            k_pool[phys] = tok_k[b, p * page:(p + 1) * page].transpose(0, 1)
            v_pool[phys] = tok_v[b, p * page:(p + 1) * page].transpose(0, 1)
    kmin = torch.empty((n_pool, Hkv, 1, D), dtype=torch.bfloat16, device=DEV)
    kmax = torch.empty_like(kmin)
    L.dsa_page_minmax(k_pool, page, kmin, kmax)        # pool viewed as [n_pool, Hkv, page, D]
    kmin, kmax = kmin[:, :, 0].contiguous(), kmax[:, :, 0].contiguous()
    table_d = torch.from_numpy(table).to(DEV)
    seq = torch.tensor([f * page for f in full_pages], dtype=torch.int32, device=DEV)
    plan = PagedDecodePlan(B, Hkv * G, Hkv, D, page, max_pages, 6, DEV)
    for t in range(n_append):
        cur = [f * page + t for f in full_pages]
        kn = torch.stack([tok_k[b, cur[b]] for b in range(B)]).contiguous()
        vn = torch.stack([tok_v[b, cur[b]] for b in range(B)]).contiguous()
        plan.append(kn, vn, table_d, seq, k_pool, v_pool, kmin, kmax)
    torch.cuda.synchronize()
    assert seq.cpu().tolist() == lens
    return dict(B=B, Hkv=Hkv, G=G, D=D, page=page, lens=np.array(lens), table=table, table_d=table_d,
                seq=seq, k_pool=k_pool, v_pool=v_pool, kmin=kmin, kmax=kmax, tok_k=tok_k,
                tok_v=tok_v, max_pages=max_pages, plan=plan)


@pytest.mark.parametrize("full_pages,n_append", [([10, 3, 0, 7], 101), ([4, 4], 64), ([2, 9, 1], 1),
                                                ([0, 5, 2], 0)])
def test_paged_decode_parity(full_pages, n_append):
    c = _build(full_pages, n_append)
    page, lens, table = c["page"], c["lens"], c["table"]
    kp, vp = to_np(c["k_pool"]), to_np(c["v_pool"])
    kn, kx = to_np(c["kmin"]), to_np(c["kmax"])
    tk, tv = to_np(c["tok_k"]), to_np(c["tok_v"])
    # the tokens sit where the table says, and every written page's summary
    # is the min/max of exactly its written tokens
    for b in range(c["B"]):
        assert np.array_equal(Pg.gather(kp, table, lens, b, page), tk[b, :lens[b]].transpose(1, 0, 2))
        assert np.array_equal(Pg.gather(vp, table, lens, b, page), tv[b, :lens[b]].transpose(1, 0, 2))
        for p in range(int(Pg.n_pages(lens[b], page))):
            rows = tk[b, p * page:min((p + 1) * page, lens[b])]
            assert np.array_equal(kn[table[b, p]], rows.min(axis=0))
            assert np.array_equal(kx[table[b, p]], rows.max(axis=0))
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    q = torch.randn((c["B"], c["Hkv"] * c["G"], c["D"]), generator=g, device=DEV).to(torch.bfloat16)
    plan = c["plan"]
    plan.run(q, c["k_pool"], c["v_pool"], c["kmin"], c["kmax"], c["table_d"], c["seq"])
    torch.cuda.synchronize()
    qn = to_np(q)
    s_ref = Pg.page_scores(qn, kn, kx, table, lens, page)
    s = to_np(plan.scores)[:, :, 0]
    assert (np.isneginf(s) == np.isneginf(s_ref)).all()
    fin = np.isfinite(s_ref)
    assert (np.abs(s[fin] - s_ref[fin]) <= 2.0 ** -23 * np.abs(s_ref[fin]) + 1e-30).all()
    gi, gc = plan.idx.cpu().numpy()[:, :, 0], plan.count.cpu().numpy()[:, :, 0]
    check_indices(s_ref[:, :, None], gi[:, :, None], gc[:, :, None], plan.topk, 0, False)
    ref = Pg.decode(qn, kp, vp, table, lens, gi, gc, plan.scale)
    check_bf16(to_np(plan.out), ref, "paged decode")


def test_paged_decode_out_of_range_pool_ids_are_skipped():
    """A page-table entry outside the pool names no page: appends to it are
    dropped and decode reads nothing there (no fault, the rest unchanged)."""
    c = _build([3, 2], 5)
    table = c["table"].copy()
    table[1, 2] = 10 ** 6                       # logical page 2 of sequence 1: beyond the pool
    table_d = torch.from_numpy(table).to(DEV)
    seq = c["seq"].clone()
    kn = torch.zeros((2, c["Hkv"], c["D"]), dtype=torch.bfloat16, device=DEV)
    c["plan"].append(kn, kn, table_d, seq, c["k_pool"], c["v_pool"], c["kmin"], c["kmax"])
    torch.cuda.synchronize()
    assert seq.cpu().tolist() == [3 * 64 + 6, 2 * 64 + 5]   # sequence 1 unchanged
