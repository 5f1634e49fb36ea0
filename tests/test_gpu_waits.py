"""Bounded waits between workgroups, and the forms a graph records.

The eager accepts exchange partial results between workgroups through
slots in the workspace; every such wait gives up after SPEC_POLL_LIMIT
polls (an environment variable the library reads on every call) and raises
SPEC_ST_SYNC.  These tests force that path from the host with a limit of 0,
so that no wait is ever taken and every kernel still runs to its end:

* the co-resident sampled walk polls each exchange at least once, so with
  no polls allowed every call raises SPEC_ST_SYNC, and the next call on a
  re-zeroed workspace is exact again;
* the greedy accept never waits (its walk is a kernel of its own after the
  sweep): with no polls allowed a call is exact and raises nothing;
* the eager target-only walkers read the sweep's slots first and poll only
  for the ones still empty: with no polls allowed a call either raises
  SPEC_ST_SYNC or is exact;
* recorded into a graph, the target-only walk runs as its own kernel after
  the sweep (its slots are all written by then), and every
  request of the sampled walk whose wait gives up is walked again by a
  recovery kernel: a graph recorded with no polls allowed (so that every
  sampled request takes the recovery path) replays exactly and raises
  nothing.
"""
import os
import sys
from contextlib import contextmanager

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _bands import assert_only_ratio_band

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import _gpu as G
    import speculative_decoding_build_amd as S


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


H8 = ("fixed", 8)
CFG = W.shrink(W.CONFIGS[3], batch=3, hist=H8, vocab=30000, draft_noise=2.0)


@contextmanager
def poll_limit(value):
    old = os.environ.get("SPEC_POLL_LIMIT")
    os.environ["SPEC_POLL_LIMIT"] = str(value)
    try:
        yield
    finally:
        if old is None:
            del os.environ["SPEC_POLL_LIMIT"]
        else:
            os.environ["SPEC_POLL_LIMIT"] = old


def _setup(cfg, seed):
    w = W.make_workload(cfg, seed, attention=False)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                          cfg.num_steps, cfg.num_draft_tokens)
    tl, dl = W.verify_logits(w, t["selected"])
    tree = dict(draft_tokens=t["draft_tokens"].astype(np.int32),
                retrieve_index=t["retrieve_index"].reshape(-1).astype(np.int32),
                retrieve_next_token=t["retrieve_next_token"].reshape(-1).astype(np.int32),
                retrieve_next_sibling=t["retrieve_next_sibling"].reshape(-1).astype(np.int32))
    return w, t, tl, dl, tree


def _oracles(w, t, tl, dl):
    cfg = w.cfg
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    args = (t["draft_tokens"], t["retrieve_index"], t["retrieve_next_token"],
            t["retrieve_next_sibling"], b, n, s1, cfg.dtype)
    og = oracle.accept_greedy(tl, *args)
    os_ = oracle.accept_sample(tl, dl, w.temperature, w.uniforms, w.final_uniforms, *args)
    ot = oracle.accept_target_only(tl, w.temperature, 1.0, 1.0, w.uniforms, w.final_uniforms,
                                   *args)
    assert_only_ratio_band(os_, "sampled")
    return og, os_, ot


def _same(g, o, n, exempt=None):
    bad = []
    for r in range(len(o["accept_length"])):
        if exempt is not None and exempt[r]:
            continue
        if (g["accept_length"][r] != o["accept_length"][r]
                or not np.array_equal(g["accept_index"][r], o["accept_index"][r])
                or not np.array_equal(g["predict"][r * n:(r + 1) * n],
                                      o["predict"][r * n:(r + 1) * n])):
            bad.append(r)
    return bad


def test_sampled_wait_gives_up_then_recovers():
    w, t, tl, dl, tree = _setup(CFG, 61)
    b, n = CFG.batch, CFG.num_draft_tokens
    _, o, _ = _oracles(w, t, tl, dl)
    ws = torch.zeros(S.spec_accept_workspace_size(b, n, CFG.vocab, 1), dtype=torch.uint8,
                     device="cuda")
    say(f"[waits] sampled, no polls allowed: b={b} V={CFG.vocab}")
    with poll_limit(0):
        g = G.accept_sample(w, tl, dl, tree, workspace=ws)
    say(f"    status {g['status']}")
    assert g["status"] & S.SPEC_ST_SYNC
    ws.zero_()
    say("[waits] sampled, default limit, re-zeroed workspace")
    g = G.accept_sample(w, tl, dl, tree, workspace=ws)
    assert (g["status"] & ~S.SPEC_ST_ZERO_RESIDUAL) == 0
    assert _same(g, o, n, o["exempt"]) == []
    assert int(torch.count_nonzero(ws)) == 0


@pytest.mark.parametrize("which", ["greedy", "target_only"])
def test_sweep_walker_wait_gives_up_or_is_exact(which):
    w, t, tl, dl, tree = _setup(CFG, 62)
    b, n = CFG.batch, CFG.num_draft_tokens
    og, _, ot = _oracles(w, t, tl, dl)
    o = og if which == "greedy" else ot
    if which == "greedy":
        size = S.spec_accept_workspace_size(b, n, CFG.vocab, 0)
        call = lambda ws: G.accept_greedy(w, tl, tree, workspace=ws)
    else:
        size = S.spec_accept_target_only_workspace_size(b, n, CFG.vocab)
        call = lambda ws: G.accept_target_only(w, tl, tree, 1.0, 1.0, workspace=ws)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    say(f"[waits] {which}, no polls allowed")
    with poll_limit(0):
        g = call(ws)
    say(f"    status {g['status']}")
    assert g["status"] in ((0,) if which == "greedy" else (0, S.SPEC_ST_SYNC))
    if g["status"] == 0:
        assert _same(g, o, n, o.get("exempt")) == []
    ws.zero_()
    g = call(ws)
    assert g["status"] == 0
    assert _same(g, o, n, o.get("exempt")) == []
    assert int(torch.count_nonzero(ws)) == 0


def test_recorded_forms_complete_without_waits():
    """A graph recorded while no polls are allowed: every replay must still
    give the oracle's outputs, raise no SPEC_ST_SYNC and leave every
    workspace zero."""
    w, t, tl, dl, tree = _setup(CFG, 63)
    cfg = CFG
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    og, o, ot = _oracles(w, t, tl, dl)
    code = G.dtype_code(cfg)
    d = {k: G.dev(v) for k, v in tree.items()}
    x_tl, x_dl = G.dev(tl), G.dev(dl)
    temp = G.dev(np.asarray(w.temperature, np.float32))
    unif = G.dev(np.asarray(w.uniforms, np.float32))
    funif = G.dev(np.asarray(w.final_uniforms, np.float32))
    outs = {k: (G.i32(b * n), G.i32(b * s1), G.i32(b)) for k in ("greedy", "sample", "target")}
    st = G.status()
    ws = dict(greedy=torch.zeros(S.spec_accept_workspace_size(b, n, cfg.vocab, 0),
                                 dtype=torch.uint8, device="cuda"),
              sample=torch.zeros(S.spec_accept_workspace_size(b, n, cfg.vocab, 1),
                                 dtype=torch.uint8, device="cuda"),
              target=torch.zeros(S.spec_accept_target_only_workspace_size(b, n, cfg.vocab),
                                 dtype=torch.uint8, device="cuda"))

    def step():
        p, ai, al = outs["greedy"]
        S.spec_accept_greedy(b, n, s1, cfg.vocab, code, x_tl, d["draft_tokens"],
                             d["retrieve_index"], d["retrieve_next_token"],
                             d["retrieve_next_sibling"], p, ai, al, workspace=ws["greedy"],
                             dev_status=st)
        p, ai, al = outs["sample"]
        S.spec_accept_sample(b, n, s1, cfg.vocab, code, x_tl, x_dl, temp, unif, funif,
                             d["draft_tokens"], d["retrieve_index"], d["retrieve_next_token"],
                             d["retrieve_next_sibling"], p, ai, al, workspace=ws["sample"],
                             dev_status=st)
        p, ai, al = outs["target"]
        S.spec_accept_target_only(b, n, s1, cfg.vocab, code, x_tl, temp, 1.0, 1.0, unif, funif,
                                  d["draft_tokens"], d["retrieve_index"],
                                  d["retrieve_next_token"], d["retrieve_next_sibling"], p, ai,
                                  al, workspace=ws["target"], dev_status=st)

    say(f"[waits] recording greedy, sampled and target-only with no polls allowed")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with poll_limit(0):
        with torch.cuda.graph(g):
            step()
    for r in range(3):
        for v in outs.values():
            for x in v:
                x.fill_(-9)
        st.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        status = int(st.item())
        got = {k: dict(predict=G.host(v[0]), accept_index=G.host(v[1]).reshape(b, s1),
                       accept_length=G.host(v[2])) for k, v in outs.items()}
        bad = dict(greedy=_same(got["greedy"], og, n),
                   sample=_same(got["sample"], o, n, o["exempt"]),
                   target=_same(got["target"], ot, n, ot["exempt"]))
        say(f"    replay {r}: status {status} mismatched {bad}")
        assert status & ~S.SPEC_ST_ZERO_RESIDUAL == 0
        assert bad == dict(greedy=[], sample=[], target=[])
        for k, v in ws.items():
            assert int(torch.count_nonzero(v)) == 0, k
