"""Draft step (select_top_k_tokens) on the GPU against the oracle.

Every step of the draft loop is called with the inputs the oracle's previous
step produced (the generator's draft logits of the live branches, the
oracle's branch scores), so each call is compared on identical inputs; a
chained run then feeds the kernel its own outputs, in place, and compares
the finished lists.  Cases: the tiny float32 workload, shrunken copies of the
four bf16 workloads with several 8192-entry chunks and a ragged tail, a
vocabulary of exactly topk entries, 8192 entries, the largest vocabularies
of the one-launch and the two-launch forms, float32 over 50000 entries, the
four full-size workloads and more requests than one launch merges (sampled
requests, whole batch in one call).  The kernel picks 2048-entry chunks for
small grids and 8192-entry chunks for large ones; the cases cover both, and
chunks holding fewer than topk entries.

Bar: tokens, parents and next tokens bit-exact, scores and next scores
within 1e-6 relative, entries outside the step's blocks untouched; requests
whose rankings hold neighbours closer than 1e-6 relative (the oracle's
near_tie, equal logits of one branch excepted) are exempt.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import _gpu as G
    import speculative_decoding_build_amd as S

H8 = ("fixed", 8)
NEAR = 1e-6
RTOL = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = {
    "c1": W.CONFIGS[1],
    "c2_v20000": W.shrink(W.CONFIGS[2], hist=H8, vocab=20000),
    "c3_b5_v9000": W.shrink(W.CONFIGS[3], batch=5, hist=H8, vocab=9000),
    "chain_b64_v40000": W.shrink(W.CONFIGS[4], hist=H8, vocab=40000),
    "c5_b2_v16385": W.shrink(W.CONFIGS[5], batch=2, hist=H8, vocab=16385),
    "vocab_eq_topk": W.shrink(W.CONFIGS[2], batch=2, hist=H8, vocab=8),
    "v8192": W.shrink(W.CONFIGS[3], batch=3, hist=H8, vocab=8192),
    "f32_v50000": W.shrink(W.CONFIGS[1], batch=3, vocab=50000),
}


def _rows(w, step, topk, req=None):
    d = w.ctx_draft if req is None else w.ctx_draft[req]
    return d[:, 0:1] if step == 0 else d[:, 1 + (step - 1) * topk:1 + step * topk]


def _sentinel_lists(b, cfg):
    sc = torch.full((b, cfg.ncand), -3.0, dtype=torch.float32, device="cuda")
    tk = torch.full((b, cfg.ncand), -7, dtype=torch.int32, device="cuda")
    pa = torch.full((b, cfg.npar), -9, dtype=torch.int32, device="cuda")
    return sc, tk, pa


def _call(cfg, b, step, rows, bs, sc, tk, pa, ns, nt, ws=None):
    if ws is None:
        # any contents: start from a non-zero pattern
        ws = torch.full((max(1, S.spec_draft_step_workspace_size(b, cfg.topk, cfg.vocab)),), 0xA5,
                        dtype=torch.uint8, device="cuda")
    st = G.status()
    S.spec_draft_step(b, cfg.topk, cfg.num_steps, step, cfg.vocab, G.dtype_code(cfg),
                      G.dev(rows), bs, sc, tk, pa, ns, nt, workspace=ws, dev_status=st)
    torch.cuda.synchronize()
    return int(G.host(st)[0])


def _compare_step(o, g, cfg, step, exempt, label):
    """g: host copies of the kernel's lists and next arrays."""
    k = o["scores"].shape[1]
    s0, p0 = o["score_offset"], o["parent_offset"]
    b = o["scores"].shape[0]
    bad = []
    for r in range(b):
        # entries outside this step's blocks keep their sentinels
        assert np.all(np.delete(g["scores"][r], np.arange(s0, s0 + k)) == -3.0), (label, r)
        assert np.all(np.delete(g["tokens"][r], np.arange(s0, s0 + k)) == -7), (label, r)
        npb = o["parents"].shape[1] if o["write_parents"] else 0
        assert np.all(np.delete(g["parents"][r], np.arange(p0, p0 + npb)) == -9), (label, r)
        if exempt[r]:
            continue
        ok = (np.array_equal(g["tokens"][r, s0:s0 + k], o["tokens"][r])
              and np.array_equal(g["next_tokens"][r], o["next_tokens"][r])
              and (not o["write_parents"]
                   or np.array_equal(g["parents"][r, p0:p0 + npb], o["parents"][r])))
        ok = ok and np.allclose(g["scores"][r, s0:s0 + k], o["scores"][r], rtol=RTOL, atol=0)
        ok = ok and np.allclose(g["next_scores"][r], o["next_scores"][r], rtol=RTOL, atol=0)
        if not ok:
            bad.append(r)
    say(f"    {label} step {step}: exempt {int(np.sum(exempt))}/{b} mismatched {bad[:8]}")
    assert bad == []


def _host_lists(sc, tk, pa, ns, nt):
    return dict(scores=G.host(sc), tokens=G.host(tk), parents=G.host(pa), next_scores=G.host(ns),
                next_tokens=G.host(nt))


def _stepwise(cfg, w, req, label, steps=None):
    """Every step on the oracle's inputs; req = the requests checked."""
    b, topk = len(req), cfg.topk
    bs = None
    for step in range(cfg.num_steps if steps is None else steps):
        rows = _rows(w, step, topk, req)
        o = oracle.draft_step(rows, bs, step, topk, cfg.num_steps, cfg.dtype)
        sc, tk, pa = _sentinel_lists(b, cfg)
        ns = torch.full((b, topk), -3.0, dtype=torch.float32, device="cuda")
        nt = torch.full((b, topk), -7, dtype=torch.int32, device="cuda")
        gbs = None if bs is None else G.dev(np.asarray(bs, np.float32))
        st = _call(cfg, b, step, rows, gbs, sc, tk, pa, ns, nt)
        assert st == 0
        _compare_step(o, _host_lists(sc, tk, pa, ns, nt), cfg, step, o["near_tie"] < NEAR, label)
        bs = o["next_scores"]


@pytest.mark.parametrize("name", list(CASES))
def test_draft_step_cases(name):
    cfg = CASES[name]
    w = W.make_workload(cfg, 51, attention=False)
    say(f"[draft-step] {name} b={cfg.batch} topk={cfg.topk} steps={cfg.num_steps} V={cfg.vocab}")
    _stepwise(cfg, w, np.arange(cfg.batch), name)


def test_draft_step_largest_vocabulary():
    # step 0 over 1048576 entries: one row of 512 chunks of 2048, the most
    # one launch merges; then a later step over 2097152 entries: 8 branch
    # rows of 256 chunks of 8192, the most a separate merge launch takes
    # (one more entry is refused)
    say("[draft-step] largest vocabulary")
    for V, step in ((1048576, 0), (2097152, 1)):
        cfg = W.shrink(W.CONFIGS[2], hist=H8, vocab=V)
        rng = np.random.default_rng(52 + step)
        nrows = 1 if step == 0 else 8
        _, rows = W._logit_pair(cfg, rng, nrows)
        rows = rows[None]
        bs = None if step == 0 else np.sort(rng.random((1, 8), dtype=np.float32))[:, ::-1].copy()
        o = oracle.draft_step(rows, bs, step, 8, cfg.num_steps, cfg.dtype)
        sc, tk, pa = _sentinel_lists(1, cfg)
        ns = torch.full((1, 8), -3.0, dtype=torch.float32, device="cuda")
        nt = torch.full((1, 8), -7, dtype=torch.int32, device="cuda")
        assert _call(cfg, 1, step, rows, None if bs is None else G.dev(bs), sc, tk, pa, ns, nt) == 0
        _compare_step(o, _host_lists(sc, tk, pa, ns, nt), cfg, step, o["near_tie"] < NEAR,
                      f"v{V}")
    V1 = 2097153
    ws = torch.zeros(S.spec_draft_step_workspace_size(1, 8, V1), dtype=torch.uint8, device="cuda")
    with pytest.raises(S.SpecError):
        S.spec_draft_step(1, 8, cfg.num_steps, 1, V1, G.dtype_code(cfg),
                          torch.zeros(8 * V1, dtype=torch.int16, device="cuda"),
                          ns, sc, tk, pa, ns, nt, workspace=ws)


# the four full-size workloads; a batch large enough for 8192-entry chunks
# whose last chunk holds one entry (fewer than topk); more requests than one
# launch merges (a separate merge launch)
LARGE = {"cfg2": W.CONFIGS[2], "cfg3": W.CONFIGS[3], "cfg4": W.CONFIGS[4], "cfg5": W.CONFIGS[5],
         "b40_v16385": W.shrink(W.CONFIGS[5], batch=40, hist=H8, vocab=16385),
         "b1100_v5000": W.shrink(W.CONFIGS[4], batch=1100, hist=H8, vocab=5000)}


@pytest.mark.parametrize("name", list(LARGE))
def test_draft_step_full(name):
    cfg = LARGE[name]
    w = W.make_workload(cfg, 1000 * len(name) + cfg.batch, attention=False)
    b = cfg.batch
    req = np.unique(np.array([0, b // 2, b - 1]))
    cid = name
    say(f"[draft-step full] {name} b={b} topk={cfg.topk} V={cfg.vocab} requests {req.tolist()}")
    # the whole batch in one call; the sampled requests against the oracle
    topk = cfg.topk
    bs_o = None
    gbs = None
    for step in range(cfg.num_steps):
        rows_all = _rows(w, step, topk)
        o = oracle.draft_step(_rows(w, step, topk, req), bs_o, step, topk, cfg.num_steps,
                              cfg.dtype)
        sc, tk, pa = _sentinel_lists(b, cfg)
        ns = torch.full((b, topk), -3.0, dtype=torch.float32, device="cuda")
        nt = torch.full((b, topk), -7, dtype=torch.int32, device="cuda")
        if step > 0:
            full_bs = np.zeros((b, topk), np.float32)
            full_bs[req] = bs_o
            gbs = G.dev(full_bs)
        assert _call(cfg, b, step, rows_all, gbs, sc, tk, pa, ns, nt) == 0
        g = {k: v[req] for k, v in _host_lists(sc, tk, pa, ns, nt).items()}
        _compare_step(o, g, cfg, step, o["near_tie"] < NEAR, cid)
        bs_o = o["next_scores"]


@pytest.mark.parametrize("name", ["c1", "c3_b5_v9000", "c5_b2_v16385", "chain_b64_v40000"])
def test_draft_step_chained_in_place(name):
    """The kernel's own next scores feed the next call through one buffer;
    the finished lists match the generator's draft loop (which the oracle's
    draft step reproduces) for requests with no near tie on the way."""
    cfg = CASES[name]
    w = W.make_workload(cfg, 53, attention=False)
    b, topk = cfg.batch, cfg.topk
    sc, tk, pa = _sentinel_lists(b, cfg)
    ns = torch.zeros((b, topk), dtype=torch.float32, device="cuda")
    nt = torch.zeros((b, topk), dtype=torch.int32, device="cuda")
    ws = torch.zeros(S.spec_draft_step_workspace_size(b, topk, cfg.vocab), dtype=torch.uint8,
                     device="cuda")
    exempt = np.zeros(b, bool)
    bs = None
    for step in range(cfg.num_steps):
        rows = _rows(w, step, topk)
        o = oracle.draft_step(rows, bs, step, topk, cfg.num_steps, cfg.dtype)
        exempt |= o["near_tie"] < NEAR
        bs = o["next_scores"]
        assert _call(cfg, b, step, rows, ns if step else None, sc, tk, pa, ns, nt, ws=ws) == 0
    g = _host_lists(sc, tk, pa, ns, nt)
    keep = ~exempt
    say(f"    chained {name}: exempt {int(exempt.sum())}/{b}")
    np.testing.assert_array_equal(g["tokens"][keep], w.tokens[keep])
    np.testing.assert_array_equal(g["parents"][keep][:, :cfg.npar], w.parents[keep])
    np.testing.assert_allclose(g["scores"][keep], w.scores[keep], rtol=4 * RTOL, atol=0)


def test_draft_step_empty_batch():
    cfg = CASES["c1"]
    assert S.spec_draft_step(0, cfg.topk, cfg.num_steps, 0, cfg.vocab, S.SPEC_F32, None, None,
                             None, None, None, None, None) is None
