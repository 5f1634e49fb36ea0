"""Pins of the oracle's draft step ([P1] select_top_k_tokens) against things
other than itself: a hand-worked two-step example (tests/golden), the list
lengths and offsets the page states, the tie rule, and the input
generator's own draft-loop record (an independent float32 implementation of
the same loop) on the shapes of every workload."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W


def _logits_for(probs):
    """float32 logits whose softmax is the given distribution."""
    return np.log(np.asarray(probs, np.float64)).astype(np.float32)


def test_hand_worked_two_steps(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "draft_step_tiny.json")))
    topk, S = g["topk"], g["num_steps"]
    s0 = g["step0"]
    o = oracle.draft_step(_logits_for(s0["probs"])[None], None, 0, topk, S, "f32")
    np.testing.assert_allclose(o["scores"][0], s0["scores"], rtol=1e-6)
    assert o["tokens"][0].tolist() == s0["tokens"]
    assert o["parents"][0].tolist() == s0["parents"]
    s1 = g["step1"]
    bs = np.asarray([s1["branch_scores"]], np.float32)
    o1 = oracle.draft_step(_logits_for(s1["probs"])[None], bs, 1, topk, S, "f32")
    np.testing.assert_allclose(o1["scores"][0], s1["scores"], rtol=1e-6)
    assert o1["tokens"][0].tolist() == s1["tokens"]
    assert o1["parents"][0].tolist() == s1["parents"]
    np.testing.assert_allclose(o1["next_scores"][0], s1["next_scores"], rtol=1e-6)
    assert o1["next_tokens"][0].tolist() == s1["next_tokens"]
    assert o1["score_offset"] == g["offsets"]["step1_scores"]
    assert o1["parent_offset"] == g["offsets"]["step1_parents"]
    o2 = oracle.draft_step(_logits_for(s1["probs"])[None], bs, 2, topk, S, "f32")
    assert o2["score_offset"] == g["offsets"]["step2_scores"]
    assert o2["parent_offset"] == g["offsets"]["step2_parents"]
    assert not o2["write_parents"]           # the last step's parents are dropped


@pytest.mark.parametrize("topk,steps", [(4, 5), (8, 6), (1, 4), (2, 3)])
def test_list_lengths_and_offsets(topk, steps):
    # the page: score rows 1 + (steps-1) topk (17 for 5 steps of topk 4),
    # token list topk + (steps-1) topk^2, parent list 1 + (steps-1) topk
    ncand = topk + (steps - 1) * topk * topk
    npar = 1 + (steps - 1) * topk
    if (topk, steps) == (4, 5):
        assert npar == 17
    end_s = end_p = 0
    for i in range(steps):
        logits = np.zeros((1, 1 if i == 0 else topk, max(topk + 1, 4)), np.float32)
        bs = None if i == 0 else np.full((1, topk), 0.5, np.float32)
        o = oracle.draft_step(logits, bs, i, topk, steps, "f32")
        assert o["score_offset"] == end_s
        end_s += o["scores"].shape[1]
        if o["write_parents"]:
            assert o["parent_offset"] == end_p
            end_p += o["parents"].shape[1]
    assert end_s == ncand and end_p == npar


def test_ties_take_the_lower_index():
    logits = np.zeros((1, 1, 10), np.float32)
    o = oracle.draft_step(logits, None, 0, 3, 2, "f32")
    assert o["tokens"][0].tolist() == [0, 1, 2]
    assert o["gap"][0] == 0.0
    # equal logits of one branch rank by index on any evaluation: no near tie
    assert o["near_tie"][0] == np.inf
    # equal products across branches: lower flat index first
    o1 = oracle.draft_step(np.zeros((1, 3, 10), np.float32), np.full((1, 3), 0.2, np.float32), 1,
                           3, 4, "f32")
    assert o1["parents"][0].tolist() == [3, 4, 5]          # flat 0, 1, 2 + 9*0 + 3
    # ... but the 3rd and 4th products come from different branches: a tie
    assert o1["near_tie"][0] == 0.0


def test_near_tie_measures_neighbours():
    # probabilities proportional to exp(logit): neighbours 3 and 2.5 differ by
    # 1 - e^-0.5 relative, 2.5 and 2.5 - 1e-6 by ~1e-6, the last pair is past k+1
    x = np.array([[[3.0, 2.5, 2.5 - 1e-6, 0.0, -5.0]]])
    o = oracle.draft_step(x, None, 0, 2, 2, "f32")
    assert o["tokens"][0].tolist() == [0, 1]
    assert abs(o["gap"][0] - 1e-6) < 2e-7
    assert abs(o["near_tie"][0] - 1e-6) < 2e-7
    o = oracle.draft_step(x, None, 0, 1, 2, "f32")
    assert abs(o["near_tie"][0] - (1 - np.exp(-0.5))) < 1e-6


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_reproduces_the_generators_draft_loop(cid):
    cfg = W.CONFIGS[cid]
    if cid != 1:
        cfg = W.shrink(cfg, batch=min(cfg.batch, 3), hist=("fixed", 8), vocab=3000)
    w = W.make_workload(cfg, 100 + cid, attention=False)
    b, topk, S = cfg.batch, cfg.topk, cfg.num_steps
    scores = np.zeros((b, cfg.ncand), np.float32)
    tokens = np.zeros((b, cfg.ncand), np.int64)
    parents = np.full((b, cfg.npar), -7, np.int64)
    bs = None
    for i in range(S):
        rows = w.ctx_draft[:, 0:1] if i == 0 else w.ctx_draft[:, 1 + (i - 1) * topk:1 + i * topk]
        o = oracle.draft_step(rows, bs, i, topk, S, cfg.dtype)
        k = o["scores"].shape[1]
        scores[:, o["score_offset"]:o["score_offset"] + k] = o["scores"]
        tokens[:, o["score_offset"]:o["score_offset"] + k] = o["tokens"]
        if o["write_parents"]:
            p = o["parents"].shape[1]
            parents[:, o["parent_offset"]:o["parent_offset"] + p] = o["parents"]
        bs = o["next_scores"]
    np.testing.assert_array_equal(tokens, w.tokens)
    np.testing.assert_array_equal(parents, w.parents)
    np.testing.assert_allclose(scores, w.scores, rtol=2e-6)


def _probs_f32(logits_row):
    """softmax of one row in float64, rounded to float32 (written out here)."""
    x = np.asarray(logits_row, np.float64)
    e = np.exp(x - x.max())
    return (e / e.sum()).astype(np.float32)


@pytest.mark.parametrize("topk,V,seed", [(4, 50, 1), (8, 200, 2), (2, 9, 3), (1, 30, 4)])
def test_next_branches_equal_brute_force_global_ranking(topk, V, seed):
    """The two-stage selection (each branch's top-k, then the top-k of the
    topk^2 products) must equal ranking every (branch, token) product of the
    whole vocabulary at once: a branch's (topk+1)-th token is beaten by its
    own topk better ones, so no global top-k entry is lost in stage one.
    Inputs are continuous random values (no ties)."""
    rng = np.random.default_rng(seed)
    steps = 3
    # step 0: the root distribution's top-k by a full sort
    root = rng.normal(0, 2, (1, 1, V)).astype(np.float32)
    o0 = oracle.draft_step(root, None, 0, topk, steps, "f32")
    p0 = _probs_f32(root[0, 0])
    order = sorted(range(V), key=lambda v: (-float(p0[v]), v))[:topk]
    assert o0["next_tokens"][0].tolist() == order
    np.testing.assert_array_equal(o0["next_scores"][0], p0[order])
    # later steps: every (branch, token) product ranked at once
    bs = o0["next_scores"]
    for step in (1, 2):
        logits = rng.normal(0, 2, (1, topk, V)).astype(np.float32)
        o = oracle.draft_step(logits, bs, step, topk, steps, "f32")
        probs = [_probs_f32(logits[0, j]) for j in range(topk)]
        prods = [(float(np.float32(bs[0, j] * probs[j][v])), j, v)
                 for j in range(topk) for v in range(V)]
        prods.sort(key=lambda e: (-e[0], e[1], e[2]))
        top = prods[:topk]
        assert len({e[0] for e in prods[:topk + 1]}) == topk + 1   # no ties at the cut
        assert o["next_tokens"][0].tolist() == [v for _, _, v in top]
        np.testing.assert_array_equal(o["next_scores"][0],
                                      np.array([s for s, _, _ in top], np.float32))
        # parents: flat index j*topk + (rank of v in branch j's top-k), offset
        # by topk^2 (step - 1) + topk
        par = []
        for _, j, v in top:
            rank = sorted(range(V), key=lambda u: (-float(probs[j][u]), u)).index(v)
            assert rank < topk
            par.append(j * topk + rank + topk * topk * (step - 1) + topk)
        assert o["parents"][0].tolist() == par
        bs = o["next_scores"]
