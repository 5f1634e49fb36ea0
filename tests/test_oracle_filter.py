"""Pins of the oracle's sampling-parameter pre-pass (top-k / top-p filtering
of the temperature-scaled target distribution, [P2] 四 eagle_sample)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "filter_tiny.json")) as f:
        return json.load(f)


def test_hand_worked_top_k_and_top_p(golden_dir):
    g = _golden(golden_dir)
    x = np.array([g["topk_logits"]], np.float32)
    for k, want in g["topk_cases"]:
        _, kept, _ = oracle.filter_logits(x, "f32", [1.0], [k], [1.0])
        assert np.flatnonzero(kept[0]).tolist() == want, k
    x = (np.array([g["topp_logits_times_ln2"]], np.float64) * math.log(2)).astype(np.float32)
    for tp, k, want in g["topp_cases"]:
        _, kept, near = oracle.filter_logits(x, "f32", [1.0], [k], [tp])
        assert np.flatnonzero(kept[0]).tolist() == want, (tp, k)
        assert not near[0]


def test_filtered_entries_are_minus_infinity_both_dtypes():
    x = np.array([[0.5, -1.0, 2.0, 2.0]], np.float32)
    out, kept, _ = oracle.filter_logits(x, "f32", [1.0], [2], [1.0])
    assert out.tolist() == [[-np.inf, -np.inf, 2.0, 2.0]]
    bits = W.f32_to_bf16_bits(x)
    outb, keptb, _ = oracle.filter_logits(bits, "bf16", [1.0], [2], [1.0])
    assert np.array_equal(keptb, kept)
    assert outb[0, 0] == 0xFF80 and outb[0, 2] == bits[0, 2]


def test_no_filter_is_identity():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 50)).astype(np.float32)
    out, kept, _ = oracle.filter_logits(x, "f32", [1.0] * 3, [0, 50, 99], [1.0] * 3)
    assert kept.all() and np.array_equal(out, x)


def test_all_masked_row_keeps_top_k_by_index():
    """A row of -inf logits has no distribution: top-p removes nothing, top_k
    keeps the entries of lowest index (equal logits rank by index)."""
    x = np.full((3, 10), -np.inf, np.float32)
    _, kept, near = oracle.filter_logits(x, "f32", [1.0] * 3, [4, 0, 1], [0.5, 0.1, 1.0])
    assert np.flatnonzero(kept[0]).tolist() == [0, 1, 2, 3]
    assert kept[1].all()
    assert np.flatnonzero(kept[2]).tolist() == [0]
    assert not near.any()


@pytest.mark.parametrize("seed", range(4))
def test_invariants_of_the_kept_set(seed):
    """Top-k keeps exactly k entries, none smaller than a removed one; top-p
    keeps a set whose mass reaches top_p while the set without its least
    likely entry does not (minimality), for several temperatures."""
    rng = np.random.default_rng(seed)
    V = 300
    x = np.round(rng.standard_normal((6, V)) * 2, 1).astype(np.float32)   # many ties
    T = np.array([1.0, 0.5, 2.0, 1.0, 0.7, 1.3])
    k = np.array([5, 0, 17, 1, 0, 40])
    tp = np.array([1.0, 0.9, 1.0, 1.0, 0.5, 0.95])
    _, kept, near = oracle.filter_logits(x, "f32", T, k, tp)
    for i in range(6):
        xi = x[i].astype(np.float64)
        p = np.exp((xi - xi.max()) / T[i])
        p /= p.sum()
        K = kept[i]
        if k[i] >= 1 and tp[i] >= 1:
            assert K.sum() == k[i]
        if K.sum() < V:
            assert xi[K].min() >= xi[~K].max()
        if tp[i] < 1 and not near[i] and (k[i] < 1 or K.sum() < k[i]):
            m = p[K].sum()
            assert m >= tp[i] - 1e-12
            # the least likely kept entry (highest index among the smallest)
            idx = np.flatnonzero(K)
            last = idx[np.lexsort((idx, -xi[idx]))][-1]
            assert m - p[last] < tp[i]


def test_lower_temperature_keeps_a_subset_under_top_p():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1, 400)).astype(np.float32)
    prev = None
    for T in (0.3, 0.6, 1.0, 2.0):
        _, kept, _ = oracle.filter_logits(x, "f32", [T], [0], [0.8])
        if prev is not None:
            assert np.all(kept[0][prev])          # the earlier (colder) set is contained
        prev = kept[0]


@pytest.mark.parametrize("cid", [1, 3])
def test_top1_sampled_accept_is_the_greedy_accept(cid):
    """A greedy request in a sampled batch: with top_k = 1 the target
    distribution is a point mass at the argmax, and the sampled rule then
    accepts exactly the child equal to the argmax and draws the argmax as the
    terminal token: the greedy accept's outputs."""
    cfg = W.CONFIGS[cid]
    if cid != 1:
        cfg = W.shrink(cfg, batch=4, hist=("fixed", 8), vocab=700)
    w = W.make_workload(cfg, 7, attention=False)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                          cfg.num_steps, cfg.num_draft_tokens)
    tl, dl = W.verify_logits(w, t["selected"])
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    rows = b * n
    ftl, _, _ = oracle.filter_logits(tl, cfg.dtype, np.repeat(w.temperature, n), [1] * rows,
                                     [1.0] * rows)
    args = (t["draft_tokens"], t["retrieve_index"], t["retrieve_next_token"],
            t["retrieve_next_sibling"], b, n, s1, cfg.dtype)
    g = oracle.accept_greedy(tl, *args)
    s = oracle.accept_sample(ftl, dl, w.temperature, w.uniforms, w.final_uniforms, *args)
    assert np.array_equal(s["accept_length"], g["accept_length"])
    assert np.array_equal(s["accept_index"], g["accept_index"])
    assert np.array_equal(s["predict"], g["predict"])
