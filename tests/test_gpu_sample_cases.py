"""Sampled tree accept on the GPU against the oracle: the cases that steer
the walk into its less common branches.

* one request over a 128256-entry vocabulary: the widest split of the
  vocabulary across workgroups;
* a noisy draft: many rejections per node, so F(c) reductions chain and the
  terminal draw reuses the last rejection's sums;
* low and high temperature;
* float32 logits on the multi-workgroup walk;
* a one-hot draft distribution (every other draft logit -inf): q(t) = 0 for
  the other children, whose ratio is then infinite, and a residual that
  drops exactly one token;
* three calls in a row on one workspace: each call must leave the workspace
  zero-filled, as the next call expects it (sampled and greedy);
* greedy accept with more requests than its one-launch form holds at once.

Same bar as the other sampled tests: bit-exact outputs except for requests
whose ratio test lies within 1e-6 of its threshold (the oracle's other
exemptions, a residual mass below 1e-6 or a terminal draw within 2e-8 of a
CDF edge, must not occur on these seeds).
"""
import sys

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
CASES = {
    "b1_v128256": W.shrink(W.CONFIGS[2], hist=H8),
    "noisy_draft": W.shrink(W.CONFIGS[3], batch=4, hist=H8, vocab=30000, draft_noise=3.0),
    "cold": W.shrink(W.CONFIGS[5], batch=3, hist=H8, vocab=12000, temperature=0.05),
    "hot": W.shrink(W.CONFIGS[5], batch=3, hist=H8, vocab=12000, temperature=2.5),
    "f32_v50000": W.shrink(W.CONFIGS[1], batch=3, vocab=50000),
    "chain_b64": W.shrink(W.CONFIGS[4], hist=H8, vocab=40000),
}


def _setup(cfg, seed):
    w = W.make_workload(cfg, seed, attention=False)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                          cfg.num_steps, cfg.num_draft_tokens)
    tl, dl = W.verify_logits(w, t["selected"])
    return w, t, tl, dl


def _tree(t):
    return dict(draft_tokens=t["draft_tokens"].astype(np.int32),
                retrieve_index=t["retrieve_index"].reshape(-1).astype(np.int32),
                retrieve_next_token=t["retrieve_next_token"].reshape(-1).astype(np.int32),
                retrieve_next_sibling=t["retrieve_next_sibling"].reshape(-1).astype(np.int32))


def _check(w, t, tl, dl, g, label):
    cfg = w.cfg
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    o = oracle.accept_sample(tl, dl, w.temperature, w.uniforms, w.final_uniforms,
                             t["draft_tokens"], t["retrieve_index"], t["retrieve_next_token"],
                             t["retrieve_next_sibling"], b, n, s1, cfg.dtype)
    assert (g["status"] & ~S.SPEC_ST_ZERO_RESIDUAL) == 0, g["status"]
    assert_only_ratio_band(o, label)
    ok = ~o["exempt"]
    bad = []
    for r in np.nonzero(ok)[0]:
        rows = slice(r * n, (r + 1) * n)
        if (g["accept_length"][r] != o["accept_length"][r]
                or not np.array_equal(g["accept_index"][r], o["accept_index"][r])
                or not np.array_equal(g["predict"][rows], o["predict"][rows])):
            bad.append(int(r))
    say(f"    {label}: exempt {int(o['exempt'].sum())}/{b} mismatched {bad} "
        f"lengths {o['accept_length'].tolist()[:12]}")
    assert bad == []
    return o


@pytest.mark.parametrize("name", list(CASES))
def test_sample_case(name):
    cfg = CASES[name]
    say(f"[sample case] {name} b={cfg.batch} n={cfg.num_draft_tokens} V={cfg.vocab} "
        f"T={cfg.temperature} {cfg.dtype}")
    w, t, tl, dl = _setup(cfg, 21)
    g = G.accept_sample(w, tl, dl, _tree(t))
    _check(w, t, tl, dl, g, name)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sample_one_hot_draft(dtype):
    cfg = W.shrink(W.CONFIGS[3], batch=4, hist=H8, vocab=9000, dtype=dtype)
    say(f"[sample one-hot draft] b={cfg.batch} V={cfg.vocab} {dtype}")
    w, t, tl, dl = _setup(cfg, 5)
    b, n = cfg.batch, cfg.num_draft_tokens
    rng = np.random.default_rng(3)
    nxt = t["retrieve_next_token"].reshape(b, n)
    neg = np.uint16(0xFF80) if dtype == "bf16" else np.float32(-np.inf)
    zero = np.uint16(0) if dtype == "bf16" else np.float32(0)
    dl = np.full_like(dl, neg)
    for r in range(b):
        for k in range(n):
            row = r * n + k
            c = nxt[r, k]
            # half the rows put the draft's whole mass on the first child's token
            tok = t["draft_tokens"][r * n + c] if (c >= 0 and rng.random() < 0.5) \
                else rng.integers(0, cfg.vocab)
            dl[row, tok] = zero
    g = G.accept_sample(w, tl, dl, _tree(t))
    _check(w, t, tl, dl, g, f"one-hot {dtype}")


def test_sample_workspace_reused():
    cfg = W.shrink(W.CONFIGS[3], batch=3, hist=H8, vocab=30000, draft_noise=2.0)
    b, n = cfg.batch, cfg.num_draft_tokens
    ws = torch.zeros(S.spec_accept_workspace_size(b, n, cfg.vocab, 1), dtype=torch.uint8,
                     device="cuda")
    for seed in (31, 32, 33):
        say(f"[sample reuse] seed {seed}")
        w, t, tl, dl = _setup(cfg, seed)
        g = G.accept_sample(w, tl, dl, _tree(t), workspace=ws)
        _check(w, t, tl, dl, g, f"seed {seed}")
        # the call leaves the workspace as it found it: zero
        assert int(torch.count_nonzero(ws)) == 0


def test_greedy_workspace_reused():
    """Three greedy accepts in a row on one workspace, each bit-exact against
    the oracle and each leaving the workspace zero (slots and counters of one
    call must not leak into the next)."""
    cfg = W.shrink(W.CONFIGS[5], batch=3, hist=H8, vocab=30000)
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    ws = torch.zeros(S.spec_accept_workspace_size(b, n, cfg.vocab, 0), dtype=torch.uint8,
                     device="cuda")
    for seed in (41, 42, 43):
        say(f"[greedy reuse] seed {seed}")
        w, t, tl, dl = _setup(cfg, seed)
        o = oracle.accept_greedy(tl, t["draft_tokens"], t["retrieve_index"],
                                 t["retrieve_next_token"], t["retrieve_next_sibling"], b, n, s1,
                                 cfg.dtype)
        g = G.accept_greedy(w, tl, _tree(t), workspace=ws)
        assert g["status"] == 0
        np.testing.assert_array_equal(g["target_predict"], o["target_predict"])
        np.testing.assert_array_equal(g["predict"], o["predict"])
        np.testing.assert_array_equal(g["accept_index"], o["accept_index"])
        np.testing.assert_array_equal(g["accept_length"], o["accept_length"])
        # the call leaves the workspace as it found it: zero
        assert int(torch.count_nonzero(ws)) == 0


def test_greedy_many_requests():
    """More requests than the device holds workgroups at once (2200 walk
    workgroups after 2200 x 5 sweep workgroups).  Bit-exact against the
    oracle; the workspace is left zero."""
    cfg = W.shrink(W.CONFIGS[4], batch=2200, hist=H8, vocab=300)
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    say(f"[greedy many requests] b={b} n={n} V={cfg.vocab}")
    w, t, tl, dl = _setup(cfg, 51)
    ws = torch.zeros(S.spec_accept_workspace_size(b, n, cfg.vocab, 0), dtype=torch.uint8,
                     device="cuda")
    o = oracle.accept_greedy(tl, t["draft_tokens"], t["retrieve_index"], t["retrieve_next_token"],
                             t["retrieve_next_sibling"], b, n, s1, cfg.dtype)
    g = G.accept_greedy(w, tl, _tree(t), workspace=ws)
    assert g["status"] == 0
    np.testing.assert_array_equal(g["target_predict"], o["target_predict"])
    np.testing.assert_array_equal(g["predict"], o["predict"])
    np.testing.assert_array_equal(g["accept_index"], o["accept_index"])
    np.testing.assert_array_equal(g["accept_length"], o["accept_length"])
    assert int(torch.count_nonzero(ws)) == 0
