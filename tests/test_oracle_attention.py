"""Pins of the oracle's tree-masked verify attention (no GPU).

The independent reference is torch's scaled_dot_product_attention in float64
on the CPU: by the tree-mask argument of "把投机采样讲透" (4.3), each node's
output equals ordinary causal attention of the last query of the linear
sequence [history, root, ..., node] along that node's own path.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _tree(w):
    cfg = w.cfg
    return oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens,
                             cfg.topk, cfg.num_steps, cfg.num_draft_tokens)


def _run(w, mask, rows=None):
    cfg = w.cfg
    return oracle.verify_attention(w.q, w.k_pool[0], w.v_pool[0], w.page_table, w.seq_lens,
                                   w.out_cache_loc, mask, cfg.num_q_heads, cfg.num_kv_heads,
                                   cfg.page_size, cfg.dtype, rows=rows)


def _f64(w, x):
    return torch.from_numpy(W.decode(w.cfg, x).astype(np.float64))


def _path(parent, k):
    p = [k]
    while p[-1] != 0:
        p.append(int(parent[p[-1]]))
    return p[::-1]


def _cases():
    yield 1, W.CONFIGS[1]
    yield 2, W.shrink(W.CONFIGS[2], hist=("fixed", 40), vocab=64)
    yield 3, W.shrink(W.CONFIGS[3], batch=3, hist=("uniform", 1, 50), vocab=64)
    yield 4, W.shrink(W.CONFIGS[4], batch=3, hist=("fixed", 33), vocab=64)
    yield 5, W.shrink(W.CONFIGS[5], batch=2, hist=("fixed", 20), vocab=64)


@pytest.mark.parametrize("cid,cfg", list(_cases()), ids=lambda x: str(x) if isinstance(x, int) else "")
def test_path_equivalence_sdpa(cid, cfg):
    w = W.make_workload(cfg, 1000 * cid + 3)
    t = _tree(w)
    out = _run(w, t["mask"])
    n, G = cfg.num_draft_tokens, cfg.group
    q, K, V = _f64(w, w.q), _f64(w, w.k_pool[0]), _f64(w, w.v_pool[0])
    for r in range(cfg.batch):
        L = int(w.seq_lens[r])
        hist = [w.slot(r, p) for p in range(L)]
        for k in range(n):
            path = _path(t["parent"][r], k)
            slots = hist + [int(w.out_cache_loc[r * n + j]) for j in path]
            for h in range(cfg.num_q_heads):
                g = h // G
                qq = q[r * n + k, h].view(1, 1, 1, -1)
                kk = K[slots, g].unsqueeze(0).unsqueeze(0)
                vv = V[slots, g].unsqueeze(0).unsqueeze(0)
                ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[0, 0, 0]
                np.testing.assert_allclose(out[r * n + k, h], ref.numpy(), rtol=1e-11, atol=1e-12)


def test_chain_equals_causal_extend():
    cfg = W.shrink(W.CONFIGS[4], batch=2, hist=("fixed", 17), vocab=64)
    w = W.make_workload(cfg, 4242)
    t = _tree(w)
    out = _run(w, t["mask"])
    n, G = cfg.num_draft_tokens, cfg.group
    q, K, V = _f64(w, w.q), _f64(w, w.k_pool[0]), _f64(w, w.v_pool[0])
    for r in range(cfg.batch):
        L = int(w.seq_lens[r])
        slots = [w.slot(r, p) for p in range(L + n)]
        for h in range(cfg.num_q_heads):
            g = h // G
            qq = q[r * n:(r + 1) * n, h].unsqueeze(0).unsqueeze(0)
            kk = K[slots, g].unsqueeze(0).unsqueeze(0)
            vv = V[slots, g].unsqueeze(0).unsqueeze(0)
            # causal mask aligned to the end: query k sees keys < L + k + 1
            allow = torch.ones(n, L + n, dtype=torch.bool).tril(diagonal=L)
            ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=allow)[0, 0]
            np.testing.assert_allclose(out[r * n:(r + 1) * n, h], ref.numpy(), rtol=1e-11, atol=1e-12)


def test_page_relocation_invariance():
    """Moving pages to other physical slots (and the page table with them)
    leaves every output unchanged."""
    cfg = W.shrink(W.CONFIGS[3], batch=2, hist=("uniform", 20, 60), vocab=64)
    w = W.make_workload(cfg, 77)
    t = _tree(w)
    base = _run(w, t["mask"])
    ps = cfg.page_size
    npages = w.num_slots // ps
    perm = np.random.default_rng(5).permutation(npages)    # old page -> new page
    k2 = np.empty_like(w.k_pool)
    v2 = np.empty_like(w.v_pool)
    for old in range(npages):
        new = perm[old]
        k2[:, new * ps:(new + 1) * ps] = w.k_pool[:, old * ps:(old + 1) * ps]
        v2[:, new * ps:(new + 1) * ps] = w.v_pool[:, old * ps:(old + 1) * ps]
    pt2 = np.where(w.page_table >= 0, perm[np.maximum(w.page_table, 0)], -1).astype(np.int32)
    loc2 = np.array([perm[s // ps] * ps + s % ps for s in w.out_cache_loc], np.int32)
    moved = oracle.verify_attention(w.q, k2[0], v2[0], pt2, w.seq_lens, loc2, t["mask"],
                                    cfg.num_q_heads, cfg.num_kv_heads, ps, cfg.dtype)
    np.testing.assert_array_equal(base, moved)


def test_empty_history_and_row_subset():
    cfg = W.shrink(W.CONFIGS[1], hist=("fixed", 0))
    w = W.make_workload(cfg, 9)
    t = _tree(w)
    out = _run(w, t["mask"])
    # root row with no history attends only to itself: output = its own V row
    for r in range(cfg.batch):
        slot = int(w.out_cache_loc[r * cfg.num_draft_tokens])
        for h in range(cfg.num_q_heads):
            np.testing.assert_allclose(out[r * cfg.num_draft_tokens, h],
                                       W.decode(cfg, w.v_pool[0, slot, h // cfg.group]), rtol=0, atol=0)
    rows = [(1, 0), (7, 1), (3, 1)]
    sub = _run(w, t["mask"], rows=rows)
    for i, (row, h) in enumerate(rows):
        np.testing.assert_array_equal(sub[i], out[row, h])


def test_softmax_scale_default():
    # uniform scores (q = 0) average V over the visible set whatever the scale
    cfg = W.CONFIGS[1]
    w = W.make_workload(cfg, 12)
    t = _tree(w)
    w.q[:] = 0
    out = _run(w, t["mask"])
    n = cfg.num_draft_tokens
    r, k = 1, n - 1
    slots = [w.slot(r, p) for p in range(int(w.seq_lens[r]))]
    slots += [int(w.out_cache_loc[r * n + j]) for j in np.nonzero(t["mask"][r, k])[0]]
    want = W.decode(cfg, w.v_pool[0, slots, 0]).astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(out[r * n + k, 0], want, rtol=1e-12)
    assert math.isclose(1 / math.sqrt(cfg.head_dim), 0.125)


def _unit(w, mask, r, g):
    cfg = w.cfg
    return oracle.verify_attention_unit(w.q, w.k_pool[0], w.v_pool[0], w.page_table, w.seq_lens,
                                        w.out_cache_loc, mask, cfg.num_q_heads, cfg.num_kv_heads,
                                        cfg.page_size, cfg.dtype, r, g)


@pytest.mark.parametrize("cid,cfg", list(_cases()), ids=lambda x: str(x) if isinstance(x, int) else "")
def test_unit_form_path_equivalence_sdpa(cid, cfg):
    """The whole-unit evaluation (all n * G queries of one request and KV
    head as one score matrix) against torch's attention along each node's
    path, and against the per-vector evaluation."""
    w = W.make_workload(cfg, 1000 * cid + 5)
    t = _tree(w)
    per_vec = _run(w, t["mask"])
    n, G = cfg.num_draft_tokens, cfg.group
    q, K, V = _f64(w, w.q), _f64(w, w.k_pool[0]), _f64(w, w.v_pool[0])
    for r in range(cfg.batch):
        L = int(w.seq_lens[r])
        hist = [w.slot(r, p) for p in range(L)]
        for g in range(cfg.num_kv_heads):
            u = _unit(w, t["mask"], r, g)
            np.testing.assert_allclose(u.reshape(n, G, -1),
                                       per_vec[r * n:(r + 1) * n, g * G:(g + 1) * G],
                                       rtol=1e-11, atol=1e-12)
            for k in range(n):
                path = _path(t["parent"][r], k)
                slots = hist + [int(w.out_cache_loc[r * n + j]) for j in path]
                kk = K[slots, g].unsqueeze(0).unsqueeze(0)
                vv = V[slots, g].unsqueeze(0).unsqueeze(0)
                qq = q[r * n + k, g * G:(g + 1) * G].unsqueeze(0).unsqueeze(2)   # [1, G, 1, d]
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qq, kk.expand(1, G, -1, -1), vv.expand(1, G, -1, -1))[0, :, 0]
                np.testing.assert_allclose(u[k], ref.numpy(), rtol=1e-11, atol=1e-12)


def test_unit_form_planted_mask_error_fails():
    """A unit evaluation that lets every node see every tree key differs from
    the per-vector evaluation (the pin above would catch it)."""
    cfg = W.shrink(W.CONFIGS[5], batch=1, hist=("fixed", 10), vocab=64)
    w = W.make_workload(cfg, 31)
    t = _tree(w)
    full = np.ones_like(t["mask"])
    a = _unit(w, t["mask"], 0, 0)
    bad = _unit(w, full, 0, 0)
    assert np.abs(a - bad).max() > 1e-3
