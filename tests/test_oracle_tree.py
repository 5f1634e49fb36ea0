"""Pins of the oracle's tree build against the pages and against independent
constructions (no GPU)."""
import itertools

import numpy as np
import pytest

import oracle
import workloads as W
from _fixtures import draft_lists, load, tok


def _build(fx, prefix=0):
    scores, tokens, parents, bonus = draft_lists(fx)
    return oracle.build_tree(scores, tokens, parents, bonus, np.array([prefix]),
                             fx["topk"], fx["num_steps"], fx["num_draft_tokens"])


@pytest.mark.parametrize("name", ["p5_tree_table.json", "p2_tree_greedy.json"])
def test_page_pointer_tables(name):
    fx = load(name)
    t = _build(fx)
    exp = fx["expected"]
    assert t["status"] == 0
    assert t["retrieve_next_token"][0].tolist() == exp["retrieve_next_token"]
    assert t["retrieve_next_sibling"][0].tolist() == exp["retrieve_next_sibling"]
    assert t["draft_tokens"].tolist() == [tok(fx, x) for x in exp["row_tokens"]]
    n = fx["num_draft_tokens"]
    assert t["retrieve_index"][0].tolist() == list(range(n))


def test_positions_example():
    fx = load("p1_positions.json")
    t = _build(fx, prefix=fx["prefix_len"])
    assert t["depth"][0].tolist() == fx["expected"]["depth"]
    assert t["positions"].tolist() == fx["expected"]["positions"]


def test_p5_mask_siblings_isolated():
    # 4.3: siblings do not see each other; a node on another branch does not
    # see the earlier branch even though its index is larger.
    t = _build(load("p5_tree_table.json"))
    m = t["mask"][0]
    root, A, B, C, D, E = range(6)
    assert m[C, A] and m[D, A] and not m[C, D] and not m[D, C]
    assert not m[E, A] and not m[E, C] and m[E, B] and m[E, root]
    assert all(m[k, k] for k in range(6))


def test_count_identities():
    # organize_draft_results: 17 score rows for num_steps=5, topk=4; the flat
    # score and token spaces have the same length.
    cfg = W.shrink(W.CONFIGS[2], topk=4, num_steps=5, num_draft_tokens=20, vocab=64)
    assert cfg.npar == 17
    assert cfg.ncand == cfg.topk * 17 == cfg.topk + (cfg.num_steps - 1) * cfg.topk ** 2
    w = W.make_workload(cfg, 5, attention=False)
    assert w.scores.shape == w.tokens.shape == (cfg.batch, 68)


def test_chain_topk1():
    cfg = W.shrink(W.CONFIGS[4], batch=3, vocab=50)
    w = W.make_workload(cfg, 11, attention=False)
    n = cfg.num_draft_tokens
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens,
                          cfg.topk, cfg.num_steps, n)
    assert t["status"] == 0
    for r in range(cfg.batch):
        assert t["parent"][r].tolist() == [-1] + list(range(n - 1))
        assert np.array_equal(t["mask"][r], np.tril(np.ones((n, n), bool)))
        assert t["positions"][r * n:(r + 1) * n].tolist() == [int(w.seq_lens[r]) + k for k in range(n)]
        assert t["retrieve_next_token"][r].tolist() == list(range(1, n)) + [-1]
        assert t["retrieve_next_sibling"][r].tolist() == [-1] * n
    words = oracle.pack_mask(t["mask"], oracle.MASK_QLEN_BITS)
    assert words.dtype == np.uint8
    assert words[0].tolist() == [(1 << (k + 1)) - 1 for k in range(n)]


def _tree_cases():
    for cid in (1, 2, 3, 4, 5):
        cfg = W.CONFIGS[cid]
        yield W.shrink(cfg, batch=min(cfg.batch, 3), vocab=257)
    # extra tiny shapes
    yield W.shrink(W.CONFIGS[1], topk=3, num_steps=3, num_draft_tokens=7, vocab=40)
    yield W.shrink(W.CONFIGS[1], topk=2, num_steps=4, num_draft_tokens=5, vocab=40)
    yield W.shrink(W.CONFIGS[1], topk=4, num_steps=2, num_draft_tokens=21, vocab=40)
    yield W.shrink(W.CONFIGS[1], topk=1, num_steps=1, num_draft_tokens=2, vocab=40)
    yield W.shrink(W.CONFIGS[1], topk=3, num_steps=1, num_draft_tokens=1, vocab=40)


@pytest.mark.parametrize("cfg", list(_tree_cases()), ids=lambda c: f"k{c.topk}s{c.num_steps}n{c.num_draft_tokens}")
@pytest.mark.parametrize("seed", [0, 1])
def test_structure_against_draft_loop(cfg, seed):
    """The derived parent lookup agrees with the draft loop's own record of who
    expanded whom; the mask equals the root->node path found by walking the
    first-child / next-sibling lists; selection is ancestor-closed."""
    w = W.make_workload(cfg, 100 + seed, attention=False)
    n = cfg.num_draft_tokens
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens,
                          cfg.topk, cfg.num_steps, n)
    assert t["status"] == 0
    for r in range(cfg.batch):
        sel = t["selected"][r]
        node_of = {int(f): k + 1 for k, f in enumerate(sel)}
        for k in range(1, n):
            f = int(sel[k - 1])
            tp = int(w.truth_parent[r, f])
            want = 0 if tp < 0 else node_of[tp]
            assert t["parent"][r, k] == want
            assert want < k
            assert t["draft_tokens"][r * n + k] == w.tokens[r, f]
        assert t["depth"][r].max() <= cfg.num_steps
        # paths by DFS over the child / sibling lists
        nxt, sib = t["retrieve_next_token"][r], t["retrieve_next_sibling"][r]
        paths = {0: {0}}
        stack = [0]
        while stack:
            u = stack.pop()
            c = int(nxt[u])
            while c != -1:
                paths[c] = paths[u] | {c}
                stack.append(c)
                c = int(sib[c])
        assert sorted(paths) == list(range(n))
        for k in range(n):
            assert set(np.nonzero(t["mask"][r, k])[0].tolist()) == paths[k]
        # siblings carry distinct tokens (a branch's top-k are distinct tokens)
        for k in range(n):
            c, seen = int(nxt[k]), set()
            while c != -1:
                tk = int(t["draft_tokens"][r * n + c])
                assert tk not in seen
                seen.add(tk)
                c = int(sib[c])
        # sibling order is ascending index
        for k in range(n):
            c, prev = int(nxt[k]), -1
            while c != -1:
                assert c > prev
                prev = c
                c = int(sib[c])


@pytest.mark.parametrize("cid", [1, 2, 3, 5])
def test_selection_by_path_probability(cid):
    """Brute force: every kept candidate's path probability (product of the
    draft's local probabilities along the draft loop's parent record, in
    float64) is at least every dropped candidate's, up to float32 rounding."""
    cfg = W.shrink(W.CONFIGS[cid], batch=2, vocab=300)
    w = W.make_workload(cfg, 7, attention=False)
    n = cfg.num_draft_tokens
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens,
                          cfg.topk, cfg.num_steps, n)
    for r in range(cfg.batch):
        prob = np.zeros(cfg.ncand)
        for f in range(cfg.ncand):
            p, g = 1.0, f
            while g >= 0:
                p *= float(w.local_prob[r, g])
                g = int(w.truth_parent[r, g])
            prob[f] = p
        kept = set(t["selected"][r].tolist())
        lo = min(prob[f] for f in kept)
        hi = max([prob[f] for f in range(cfg.ncand) if f not in kept] or [0.0])
        assert lo >= hi * (1 - 1e-5)


def test_tie_break_lower_index():
    # equal scores: the lower flat index is kept
    scores = np.array([[0.5, 0.5, 0.5, 0.5]], np.float32)
    tokens = np.array([[1, 2, 3, 4]], np.int32)
    t = oracle.build_tree(scores, tokens, np.array([[-1]], np.int32), np.array([0]),
                          np.array([0]), 4, 1, 3)
    assert t["selected"][0].tolist() == [0, 1]


def test_not_closed_and_range_status():
    # topk=2, S=2: keep a step-1 child whose parent (flat 1) is dropped
    scores = np.array([[0.9, 0.1, 0.5, 0.4, 0.3, 0.2]], np.float32)
    tokens = np.arange(6, dtype=np.int32)[None]
    t = oracle.build_tree(scores, tokens, np.array([[-1, 0, 1]], np.int32), np.array([9]),
                          np.array([0]), 2, 2, 5)
    # kept flats 0, 2, 3, 4; flat 4's parent is flat 1 (not kept)
    assert t["selected"][0].tolist() == [0, 2, 3, 4]
    assert t["status"] & oracle.ST_NOT_CLOSED
    assert t["parent"][0].tolist() == [-1, 0, 1, 1, 0]
    bad = oracle.build_tree(scores, tokens, np.array([[-1, 0, 99]], np.int32), np.array([9]),
                            np.array([0]), 2, 2, 6)
    assert bad["status"] & oracle.ST_RANGE


def test_mask_word_width():
    # QLEN_ONLY_BITPACKING picks the dtype index ceil(log2(ceil(n / 8)))
    want = {1: 8, 8: 8, 9: 16, 16: 16, 17: 32, 24: 32, 32: 32, 33: 64, 64: 64}
    for n, bits in want.items():
        assert oracle.mask_word_bits(n) == bits


def test_pack_roundtrip_all_tiny_masks():
    # every lower-triangular-with-diagonal bit pattern up to n = 4 packs LSB first
    n = 4
    below = [(k, j) for k in range(n) for j in range(k)]
    for bits in itertools.product([False, True], repeat=len(below)):
        m = np.eye(n, dtype=bool)
        for (k, j), v in zip(below, bits):
            m[k, j] = v
        words = oracle.pack_mask(m[None], oracle.MASK_QLEN_BITS)[0]
        for k in range(n):
            assert int(words[k]) == sum(1 << j for j in range(n) if m[k, j])
        assert np.array_equal(oracle.unpack_mask(words, n), m)
