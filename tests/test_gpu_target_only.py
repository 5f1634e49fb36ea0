"""Target-only tree accept on the GPU against the oracle.

Cases: the tiny float32 workload, shrunken copies of the four bf16
workloads, one request over a 128256-entry vocabulary, low and high
temperature, a root-only tree, more requests than the one-launch form holds
at once (a second launch walks), the four full-size workloads, three
threshold settings, and three calls in a row on one workspace (each call
must leave it zero-filled).

Bar: bit-exact predict / accept_index / accept_length except for requests
the oracle marks exempt (a test within 1e-6 of its threshold, a
probability a float32 exponential may flush to zero, or a terminal draw
within 2e-8 of a CDF edge).
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


H8 = ("fixed", 8)
CASES = {
    "c1": W.CONFIGS[1],
    "c3s": W.shrink(W.CONFIGS[3], batch=3, hist=H8, vocab=9000),
    "c5s": W.shrink(W.CONFIGS[5], batch=2, hist=H8, vocab=8200),
    "chain_b64": W.shrink(W.CONFIGS[4], hist=H8, vocab=40000),
    "b1_v128256": W.shrink(W.CONFIGS[2], hist=H8),
    "f32_v50000": W.shrink(W.CONFIGS[1], batch=3, vocab=50000),
    "cold": W.shrink(W.CONFIGS[5], batch=3, hist=H8, vocab=12000, temperature=0.05),
    "hot": W.shrink(W.CONFIGS[5], batch=3, hist=H8, vocab=12000, temperature=2.5),
    "root_only": W.shrink(W.CONFIGS[3], batch=2, hist=H8, vocab=500, num_draft_tokens=1),
    "many_req": W.shrink(W.CONFIGS[4], batch=1100, hist=H8, vocab=5000),
    # peaked target rows: the children's mass is large, walks go deep
    "cold_b16": W.shrink(W.CONFIGS[3], batch=16, hist=H8, vocab=20000, temperature=0.1),
}
THRESHOLDS = [(1.0, 1.0), (0.6, 0.8), (0.25, 1.0)]


def _setup(cfg, seed):
    w = W.make_workload(cfg, seed, attention=False)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                          cfg.num_steps, cfg.num_draft_tokens)
    tl, _ = W.verify_logits(w, t["selected"])
    return w, t, tl


def _tree(t, b, n):
    return dict(draft_tokens=t["draft_tokens"].astype(np.int32),
                retrieve_index=t["retrieve_index"].reshape(-1).astype(np.int32),
                retrieve_next_token=t["retrieve_next_token"].reshape(-1).astype(np.int32),
                retrieve_next_sibling=t["retrieve_next_sibling"].reshape(-1).astype(np.int32))


def _check(w, t, tl, ts, ta, uniforms=None, final_uniforms=None, workspace=None, label="",
           accept_width=None):
    cfg = w.cfg
    b, n = cfg.batch, cfg.num_draft_tokens
    s1 = cfg.num_steps + 1 if accept_width is None else accept_width
    U = w.uniforms if uniforms is None else uniforms
    UF = w.final_uniforms if final_uniforms is None else final_uniforms
    o = oracle.accept_target_only(tl, w.temperature, ts, ta, U, UF, t["draft_tokens"],
                                  t["retrieve_index"], t["retrieve_next_token"],
                                  t["retrieve_next_sibling"], b, n, s1, cfg.dtype)
    g = G.accept_target_only(w, tl, _tree(t, b, n), ts, ta, uniforms=U, final_uniforms=UF,
                             workspace=workspace, accept_width=s1)
    bad = []
    for r in range(b):
        if o["exempt"][r]:
            continue
        same = (g["accept_length"][r] == o["accept_length"][r]
                and np.array_equal(g["accept_index"][r], o["accept_index"][r])
                and np.array_equal(g["predict"][r * n:(r + 1) * n], o["predict"][r * n:(r + 1) * n]))
        if not same:
            bad.append(r)
    say(f"    {label} thresholds ({ts}, {ta}): exempt {int(o['exempt'].sum())}/{b} "
        f"mismatched {bad[:8]} lengths {o['accept_length'].tolist()[:12]}")
    assert bad == []
    assert g["status"] == o["status"]
    return o


@pytest.mark.parametrize("name", list(CASES))
def test_target_only_cases(name):
    cfg = CASES[name]
    w, t, tl = _setup(cfg, 31)
    say(f"[target-only] {name} b={cfg.batch} n={cfg.num_draft_tokens} V={cfg.vocab} "
        f"T={cfg.temperature}")
    for ts, ta in THRESHOLDS:
        _check(w, t, tl, ts, ta, label=name)


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_target_only_full(cid):
    cfg = W.CONFIGS[cid]
    w, t, tl = _setup(cfg, 1000 * cid + 1)
    say(f"[target-only full] cfg{cid} b={cfg.batch} n={cfg.num_draft_tokens} V={cfg.vocab}")
    _check(w, t, tl, 1.0, 1.0, label=f"cfg{cid}")


def test_target_only_workspace_reused():
    cfg = W.shrink(W.CONFIGS[3], batch=5, hist=H8, vocab=20000)
    w, t, tl = _setup(cfg, 41)
    b, n = cfg.batch, cfg.num_draft_tokens
    ws = torch.zeros(G.S.spec_accept_target_only_workspace_size(b, n, cfg.vocab),
                     dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(3)
    for call in range(3):
        U = (rng.integers(0, 1 << 24, size=(b, n)) * 2.0 ** -24).astype(np.float32)
        UF = (rng.integers(0, 1 << 24, size=b) * 2.0 ** -24).astype(np.float32)
        _check(w, t, tl, 1.0, 1.0, uniforms=U, final_uniforms=UF, workspace=ws,
               label=f"call {call}")
        assert int(ws.count_nonzero()) == 0


def test_target_only_path_longer_than_accept_width():
    # accept_width 2 holds the root and one accepted node: deeper walks stop
    # with SPEC_ST_DEPTH and draw their terminal token at the second node,
    # as the oracle does
    cfg = CASES["cold_b16"]
    w, t, tl = _setup(cfg, 31)
    o = _check(w, t, tl, 1.0, 1.0, label="width 2", accept_width=2)
    assert o["status"] & oracle.ST_DEPTH
