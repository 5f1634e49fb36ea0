"""Pins of the oracle's greedy accept, rejection-sampled accept and KV
compaction against the pages' worked examples, textbook special cases and a
chi-square test (no GPU)."""
import numpy as np
import pytest
from scipy import stats

import oracle
import workloads as W
from _fixtures import draft_lists, load, onehot_logits, tok, vocab_size


def _greedy_from_fixture(fx):
    scores, tokens, parents, bonus = draft_lists(fx)
    n = fx["num_draft_tokens"]
    prefix = fx.get("prefix_len", 0)
    t = oracle.build_tree(scores, tokens, parents, bonus, np.array([prefix]),
                          fx["topk"], fx["num_steps"], n)
    V = vocab_size(fx)
    logits = onehot_logits(fx, fx["target_argmax_by_row"], V)
    g = oracle.accept_greedy(logits, t["draft_tokens"], t["retrieve_index"],
                             t["retrieve_next_token"], t["retrieve_next_sibling"],
                             1, n, fx["num_steps"] + 1, "f32")
    return t, g


@pytest.mark.parametrize("name", ["p2_tree_greedy.json", "p5_tree_table.json",
                                  "p5_chain.json", "p2_dspark_chain.json"])
def test_greedy_worked_examples(name):
    fx = load(name)
    t, g = _greedy_from_fixture(fx)
    exp = fx["expected"]
    L = g["accept_length"][0]
    ai = g["accept_index"][0]
    assert ai[:L].tolist() == exp["accept_index"]
    assert (ai[L:] == -1).all()
    assert L == exp["accept_length"] == exp["num_correct_drafts"] + 1
    outs = [int(g["predict"][i]) for i in ai[:L]]
    assert outs == [tok(fx, x) for x in exp["outputs"]]
    if "predict" in exp:
        assert g["predict"].tolist() == [tok(fx, x) for x in exp["predict"]]
    if "committed_kv_rows" in exp:
        rows_in = [int(t["draft_tokens"][i]) for i in ai[:L]]
        assert rows_in == [tok(fx, x) for x in exp["committed_kv_rows"]]


def test_greedy_no_match_and_full_match():
    fx = load("p5_chain.json")
    # no child matches: one output, the root row's own prediction
    fx_none = dict(fx, target_argmax_by_row=["on", "cat", "cat", "cat"])
    _, g = _greedy_from_fixture(fx_none)
    assert g["accept_length"][0] == 1 and g["accept_index"][0].tolist() == [0, -1, -1, -1]
    assert g["predict"].tolist() == [tok(fx, "on"), 0, 0, 0]
    # every draft matches: the last row still yields a terminal token
    fx_all = dict(fx, target_argmax_by_row=["cat", "sat", "on", "the"])
    _, g = _greedy_from_fixture(fx_all)
    assert g["accept_length"][0] == 4 and g["accept_index"][0].tolist() == [0, 1, 2, 3]
    assert g["predict"].tolist() == [tok(fx, x) for x in ["cat", "sat", "on", "the"]]


def test_argmax_first_index_on_ties():
    x = np.array([[0.0, 3.0, 1.0, 3.0], [-1.0, -1.0, -2.0, -1.0], [-0.0, 0.0, -5.0, 0.0]], np.float32)
    assert oracle.argmax_rows(x, "f32").tolist() == [1, 0, 0]
    b = W.f32_to_bf16_bits(np.array([[1.0, 2.0, 2.0, 2.015625]], np.float32))
    # 2.015625 is one bf16 ulp above 2.0 and beats the tie; equal values keep the first
    assert oracle.argmax_rows(b, "bf16").tolist() == [3]
    b2 = W.f32_to_bf16_bits(np.array([[1.0, 2.0, 2.0, 2.0078125]], np.float32))
    assert oracle.argmax_rows(b2, "bf16").tolist() == [1]   # 2.0078125 rounds to 2.0


def _tree_and_logits(cfg, seed):
    w = W.make_workload(cfg, seed, attention=False)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens,
                          cfg.topk, cfg.num_steps, cfg.num_draft_tokens)
    tl, dl = W.verify_logits(w, t["selected"])
    return w, t, tl, dl


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_greedy_debug_invariants(cid):
    """[P2] 六: accept_length = valid accept_index entries = drafts + 1;
    predict[accept_index] = accepted drafts then the terminal token; the
    accepted input rows are the root followed by the accepted drafts."""
    cfg = W.shrink(W.CONFIGS[cid], batch=min(W.CONFIGS[cid].batch, 6), vocab=50)
    w, t, tl, dl = _tree_and_logits(cfg, 31 * cid)
    n, s1 = cfg.num_draft_tokens, cfg.num_steps + 1
    g = oracle.accept_greedy(tl, t["draft_tokens"], t["retrieve_index"], t["retrieve_next_token"],
                             t["retrieve_next_sibling"], cfg.batch, n, s1, cfg.dtype)
    tp = g["target_predict"]
    for r in range(cfg.batch):
        L = int(g["accept_length"][r])
        ai = g["accept_index"][r]
        assert 1 <= L <= s1 and (ai[:L] >= 0).all() and (ai[L:] == -1).all()
        assert ai[0] == r * n
        for j in range(1, L):
            # each accepted row's token is what the previous row predicted
            assert t["draft_tokens"][ai[j]] == g["predict"][ai[j - 1]] == tp[ai[j - 1]]
            # and it is a child of the previous accepted node
            assert t["parent"][r, ai[j] - r * n] == ai[j - 1] - r * n
        assert g["predict"][ai[L - 1]] == tp[ai[L - 1]]
        on_path = set(ai[:L].tolist())
        for k in range(n):
            if r * n + k not in on_path:
                assert g["predict"][r * n + k] == 0
        # the walk stopped: no child of the last node carries its prediction
        last = ai[L - 1] - r * n
        kids = [c for c in range(n) if t["parent"][r, c] == last]
        assert all(t["draft_tokens"][r * n + c] != tp[ai[L - 1]] for c in kids) or L == s1


# ---------------------------------------------------------------------------
# sampled accept
# ---------------------------------------------------------------------------

def _single_child(p, q, child_token, u, uf, T=1.0):
    """One request per (u, uf) pair: root (token 0) with one child."""
    b = len(u)
    V = len(p)
    n = 2
    with np.errstate(divide="ignore"):
        tl = np.tile(np.log(np.asarray(p, np.float64)), (b * n, 1)).astype(np.float32)
        dl = np.tile(np.log(np.asarray(q, np.float64)), (b * n, 1)).astype(np.float32)
    tl[~np.isfinite(tl)] = -1e4
    dl[~np.isfinite(dl)] = -1e4
    cand = np.tile([0, child_token], b)
    ri = np.arange(b * n).reshape(b, n)
    rn = np.tile([1, -1], (b, 1))
    rs = np.tile([-1, -1], (b, 1))
    unif = np.stack([np.zeros(b), np.asarray(u)], axis=1).astype(np.float32)
    res = oracle.accept_sample(tl, dl, np.full(b, T, np.float32), unif, np.asarray(uf, np.float32),
                               cand, ri, rn, rs, b, n, 2, "f32")
    return res


def _grid(m):
    return (np.arange(m) + 0.5) / m


def test_pq_table_exact():
    """[P2] 四 table: proposals drawn from q, accepted with min(1, p/q),
    rejections refilled from max(0, p - q)/Z, give exactly p."""
    fx = load("p2_pq_table.json")
    p, q = np.array(fx["p"]), np.array(fx["q"])
    exp = fx["expected"]
    m = 3000
    total = np.zeros(3)
    for x in range(3):
        acc = _single_child(p, q, x, _grid(m), np.full(m, 0.5))
        rate = np.mean(acc["accept_length"] == 2)
        if x == 0:
            assert rate == exp["accept_prob_when_A_proposed"]
        rej = _single_child(p, q, x, np.full(m, 0.999999), _grid(m))
        if rate < 1:
            assert (rej["accept_length"] == 1).all()
        hist = np.bincount(rej["predict"][0::2], minlength=3) / m
        if x == 0:
            np.testing.assert_allclose(hist, exp["residual_after_rejecting_A"], atol=1 / m)
        total[x] += q[x] * rate
        total += q[x] * (1 - rate) * hist
    np.testing.assert_allclose(total, exp["total"], atol=2 / m)


def test_point_mass_draft_is_inverse_cdf_sampling():
    """q = delta at the child's token: accept with p(t), else draw from p with
    t removed; the output law is exactly p."""
    rng = np.random.default_rng(3)
    p = rng.dirichlet(np.ones(6))
    t = 2
    q = np.zeros(6)
    q[t] = 1.0
    m = 4000
    acc = _single_child(p, q, t, _grid(m), np.full(m, 0.5))
    rate = np.mean(acc["accept_length"] == 2)
    assert abs(rate - p[t]) <= 1 / m
    rej = _single_child(p, q, t, np.full(m, 0.9999999), _grid(m))
    hist = np.bincount(rej["predict"][0::2], minlength=6) / m
    want = p.copy()
    want[t] = 0
    np.testing.assert_allclose(hist, want / want.sum(), atol=1 / m)
    law = rate * np.eye(6)[t] + (1 - rate) * hist
    np.testing.assert_allclose(law, p, atol=2 / m)


def test_p_equals_q_always_accepts():
    rng = np.random.default_rng(4)
    p = rng.dirichlet(np.ones(8))
    res = _single_child(p, p, 5, rng.random(500) * 0.9999, rng.random(500))
    assert (res["accept_length"] == 2).all()


def _iid_tree_trial(rng, logit_rows, shape, T=1.0):
    """Trees whose children are drawn i.i.d. from the parent row's draft law.

    ``shape`` is the number of children of the root and of each child.
    Returns the oracle result for a batch of independent requests.
    """
    b = logit_rows["b"]
    k1, k2 = shape
    n = 1 + k1 + k1 * k2
    V = logit_rows["V"]
    tl = np.tile(logit_rows["target"], (b, 1)).astype(np.float32)  # [b*n, V]
    dl = np.tile(logit_rows["draft"], (b, 1)).astype(np.float32)
    qrows = [oracle.softmax_t(logit_rows["draft"][i], T) for i in range(n)]
    cand = np.zeros((b, n), np.int64)
    parent = [-1] + [0] * k1 + [1 + i for i in range(k1) for _ in range(k2)]
    for k in range(1, n):
        cand[:, k] = rng.choice(V, size=b, p=qrows[parent[k]])
    rn = np.full((b, n), -1)
    rs = np.full((b, n), -1)
    for k in range(n):
        kids = [c for c in range(n) if parent[c] == k]
        if kids:
            rn[:, k] = kids[0]
            for a, c in zip(kids, kids[1:]):
                rs[:, a] = c
    ri = np.arange(b * n).reshape(b, n)
    unif = rng.random((b, n)).astype(np.float32)
    uf = rng.random(b).astype(np.float32)
    return oracle.accept_sample(tl, dl, np.full(b, T, np.float32), unif, uf, cand.reshape(-1),
                                ri, rn, rs, b, n, 3, "f32"), n


@pytest.mark.parametrize("shape", [(1, 0), (2, 0), (2, 2)])
def test_chi_square_32_vocab(shape):
    """The first output token follows the target law p of the root row."""
    rng = np.random.default_rng(20 + sum(shape))
    V = 32
    k1, k2 = shape
    n = 1 + k1 + k1 * k2
    target = rng.normal(0, 1, (n, V))
    draft = target + rng.normal(0, 1.0, (n, V))
    trials = 200000
    rows = dict(b=trials, V=V, target=target, draft=draft)
    res, n = _iid_tree_trial(rng, rows, shape)
    first = res["predict"][res["accept_index"][:, 0]]
    counts = np.bincount(first, minlength=V)
    p = oracle.softmax_t(target[0].astype(np.float32), 1.0)
    chi2 = ((counts - trials * p) ** 2 / (trials * p)).sum()
    assert chi2 < stats.chi2.ppf(1 - 1e-3, V - 1), chi2


def test_chi_square_detects_non_recursive_residual():
    """Control: keeping p unchanged across rejected siblings (a plausible
    mistake) is rejected by the same test, so the test has power."""
    rng = np.random.default_rng(99)
    V = 32
    target = rng.normal(0, 1, (3, V))
    draft = target + rng.normal(0, 1.0, (3, V))
    p = oracle.softmax_t(target[0].astype(np.float32), 1.0)
    q = oracle.softmax_t(draft[0].astype(np.float32), 1.0)
    # exact law of the wrong rule for two i.i.d. children: each rejection
    # refills from max(0, p - q) without updating p
    acc = np.minimum(1, p / q)
    rej_mass = 1 - (q * acc).sum()
    resid = np.maximum(p - q, 0)
    resid /= resid.sum()
    wrong = q * acc + rej_mass * (q * acc) + rej_mass ** 2 * resid
    trials = 60000
    counts = rng.multinomial(trials, wrong / wrong.sum())
    chi2 = ((counts - trials * p) ** 2 / (trials * p)).sum()
    assert chi2 > stats.chi2.ppf(1 - 1e-3, V - 1)


@pytest.mark.parametrize("cid", [1, 4])
def test_low_temperature_chain_matches_greedy(cid):
    """As T -> 0 a chain's sampled walk is the greedy walk: the one child (the
    draft's top token) passes iff it is the target's top token, and the
    residual collapses onto the target's top token.  (With several
    deterministic siblings the classic rule can accept a lower-ranked sibling
    whose target/draft ratio blows up, so the limit holds for chains only.)"""
    cfg = W.shrink(W.CONFIGS[cid], batch=min(W.CONFIGS[cid].batch, 6), vocab=50,
                   topk=1, num_draft_tokens=W.CONFIGS[cid].num_steps + 1)
    w, t, tl, dl = _tree_and_logits(cfg, 71 * cid)
    n, s1 = cfg.num_draft_tokens, cfg.num_steps + 1
    g = oracle.accept_greedy(tl, t["draft_tokens"], t["retrieve_index"], t["retrieve_next_token"],
                             t["retrieve_next_sibling"], cfg.batch, n, s1, cfg.dtype)
    # make every row's maximum unique so greedy has one answer
    tlf = W.decode(cfg, tl).astype(np.float32).copy()
    dlf = W.decode(cfg, dl).astype(np.float32).copy()
    tlf[np.arange(tlf.shape[0]), g["target_predict"]] += 0.5
    s = oracle.accept_sample(tlf, dlf, np.full(cfg.batch, 1e-3, np.float32), w.uniforms,
                             w.final_uniforms, t["draft_tokens"], t["retrieve_index"],
                             t["retrieve_next_token"], t["retrieve_next_sibling"],
                             cfg.batch, n, s1, "f32")
    assert np.array_equal(s["accept_length"], g["accept_length"])
    assert np.array_equal(s["accept_index"], g["accept_index"])
    assert np.array_equal(s["predict"], g["predict"])


# ---------------------------------------------------------------------------
# compaction
# ---------------------------------------------------------------------------

def _pool(slots, layers=2, hkv=2, d=4, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.integers(0, 2 ** 16, (layers, slots, hkv, d)).astype(np.uint16),
            rng.integers(0, 2 ** 16, (layers, slots, hkv, d)).astype(np.uint16))


def test_compact_p2_commits_root_and_accepted_rows():
    fx = load("p2_tree_greedy.json")
    t, g = _greedy_from_fixture(fx)
    n = fx["num_draft_tokens"]
    L = fx["prefix_len"]
    ps = 1
    page_table = np.arange(L + n, dtype=np.int32)[None]
    loc = np.arange(L, L + n, dtype=np.int32)          # verify rows written in place
    kp, vp = _pool(L + n)
    res = oracle.compact_kv(kp, vp, page_table, np.array([L]), loc, g["accept_index"],
                            g["accept_length"], 1, n, ps)
    assert res["new_seq_lens"].tolist() == [fx["expected"]["new_seq_len"]]
    # positions L, L+1, L+2 now hold rows R, A, C (verify rows 0, 1, 3)
    for j, row in enumerate([0, 1, 3]):
        np.testing.assert_array_equal(res["k_pool"][:, L + j], kp[:, L + row])
        np.testing.assert_array_equal(res["v_pool"][:, L + j], vp[:, L + row])
    # the slots of B and D beyond the committed prefix are freed: rows 3, 4's slots
    assert res["num_free"].tolist() == [2]
    assert res["free_slots"][:2].tolist() == [L + 3, L + 4]
    assert (res["free_slots"][2:] == -1).all()
    np.testing.assert_array_equal(res["k_pool"][:, :L], kp[:, :L])


def test_compact_overlap_read_before_write():
    # accepted rows [0, 2, 3] written in place: sources overlap targets
    n, L = 5, 4
    page_table = np.arange(L + n, dtype=np.int32)[None]
    loc = np.arange(L, L + n, dtype=np.int32)
    kp, vp = _pool(L + n, seed=2)
    ai = np.array([[0, 2, 3, -1]])
    res = oracle.compact_kv(kp, vp, page_table, np.array([L]), loc, ai, np.array([3]), 1, n, 1)
    for j, row in enumerate([0, 2, 3]):
        np.testing.assert_array_equal(res["k_pool"][:, L + j], kp[:, L + row])
    # the reversed order would need a buffer: rows [0, 3, 1] is not a valid
    # walk but exercises the simultaneous-assignment definition
    ai2 = np.array([[0, 3, 1, -1]])
    res2 = oracle.compact_kv(kp, vp, page_table, np.array([L]), loc, ai2, np.array([3]), 1, n, 1)
    for j, row in enumerate([0, 3, 1]):
        np.testing.assert_array_equal(res2["v_pool"][:, L + j], vp[:, L + row])


def test_compact_paged_slot_conservation():
    cfg = W.shrink(W.CONFIGS[3], batch=4, hist=("uniform", 3, 40), vocab=50)
    w, t, tl, dl = _tree_and_logits(cfg, 5)
    n, s1 = cfg.num_draft_tokens, cfg.num_steps + 1
    g = oracle.accept_greedy(tl, t["draft_tokens"], t["retrieve_index"], t["retrieve_next_token"],
                             t["retrieve_next_sibling"], cfg.batch, n, s1, cfg.dtype)
    kp, vp = _pool(w.num_slots, seed=3)
    res = oracle.compact_kv(kp, vp, w.page_table, w.seq_lens, w.out_cache_loc, g["accept_index"],
                            g["accept_length"], cfg.batch, n, cfg.page_size)
    for r in range(cfg.batch):
        L, m = int(w.seq_lens[r]), int(g["accept_length"][r])
        assert res["new_seq_lens"][r] == L + m
        kept = {w.slot(r, L + j) for j in range(m)}
        freed = set(res["free_slots"][r * n:r * n + res["num_free"][r]].tolist())
        verify = set(w.out_cache_loc[r * n:(r + 1) * n].tolist())
        assert kept.isdisjoint(freed) and kept | freed == verify
        for j in range(m):
            src = int(w.out_cache_loc[g["accept_index"][r, j]])
            np.testing.assert_array_equal(res["k_pool"][:, w.slot(r, L + j)], kp[:, src])


def test_compact_separate_verify_slots_all_freed():
    n, L = 3, 2
    page_table = np.array([[0, 1, 2, 3, 4]], np.int32)
    loc = np.array([10, 11, 12], np.int32)              # verify rows outside the sequence
    kp, vp = _pool(16, seed=4)
    res = oracle.compact_kv(kp, vp, page_table, np.array([L]), loc, np.array([[0, 2, -1]]),
                            np.array([2]), 1, n, 1)
    assert res["free_slots"].tolist() == [10, 11, 12] and res["num_free"].tolist() == [3]
    np.testing.assert_array_equal(res["k_pool"][:, 2], kp[:, 10])
    np.testing.assert_array_equal(res["k_pool"][:, 3], kp[:, 12])


# ---------------------------------------------------------------------------
# target-only sampled accept
# ---------------------------------------------------------------------------

def _links(parent, b):
    """retrieve arrays of b copies of the tree given by ``parent`` (node 0 the
    root, children in ascending node order)."""
    n = len(parent)
    rn = np.full((b, n), -1)
    rs = np.full((b, n), -1)
    for k in range(n):
        kids = [c for c in range(n) if parent[c] == k]
        if kids:
            rn[:, k] = kids[0]
            for a, c in zip(kids, kids[1:]):
                rs[:, a] = c
    return np.arange(b * n).reshape(b, n), rn, rs


def _target_only(rows_p, parent, tokens, u, uf, ts=1.0, ta=1.0, T=1.0):
    """One request per entry of ``uf``: tree ``parent``, node tokens
    ``tokens``, row k's target law rows_p[k] (given as logits log p), coins
    u[request, node]."""
    b = len(uf)
    n = len(parent)
    with np.errstate(divide="ignore"):
        logit = np.log(np.asarray(rows_p, np.float64))
    logit[~np.isfinite(logit)] = -np.inf
    tl = np.tile(logit, (b, 1)).astype(np.float32)
    cand = np.tile(np.asarray(tokens), b)
    ri, rn, rs = _links(parent, b)
    return oracle.accept_target_only(tl, np.full(b, T, np.float32), ts, ta,
                                     np.asarray(u, np.float32).reshape(b, n),
                                     np.asarray(uf, np.float32), cand, ri, rn, rs, b, n, n, "f32")


def test_target_only_thresholds_one_give_the_target_law():
    """Thresholds 1: child j is accepted iff the coin lies below the mass of
    children 1..j, and the terminal draw excludes the tried children, so the
    output law is exactly p (the children's tokens first, then the rest)."""
    rng = np.random.default_rng(7)
    V = 7
    p = rng.dirichlet(np.ones(V))
    kids = [4, 1, 6]
    parent = [-1, 0, 0, 0]
    tokens = [0] + kids
    m = 4000
    g = _grid(m)
    acc = _target_only([p] * 4, parent, tokens, np.stack([g] + [np.zeros(m)] * 3, 1),
                       np.full(m, 0.5))
    law = np.zeros(V)
    took = acc["accept_length"] == 2
    for r in np.nonzero(took)[0]:
        law[acc["predict"][4 * r]] += 1.0 / m
    rate = took.mean()
    assert abs(rate - p[kids].sum()) <= 1 / m
    rej = _target_only([p] * 4, parent, tokens, np.stack([np.full(m, 0.9999999)] + [np.zeros(m)] * 3, 1), g)
    assert (rej["accept_length"] == 1).all()
    hist = np.bincount(rej["predict"][0::4], minlength=V) / m
    assert hist[kids].sum() == 0
    law += (1 - rate) * hist
    np.testing.assert_allclose(law, p, atol=3 / m)


def test_target_only_two_level_chi_square():
    """Random coins on a 2 x 2 tree: the first output follows the root row's
    law, and after the first child is accepted the second output follows
    that child's row law (the accumulator and the coin are per level)."""
    rng = np.random.default_rng(11)
    V = 24
    parent = [-1, 0, 0, 1, 1, 2, 2]
    n = len(parent)
    logits = rng.normal(0, 1.2, (n, V))
    rows_p = [oracle.softmax_t(logits[k].astype(np.float32), 1.0) for k in range(n)]
    tokens = [0, 3, 9, 5, 7, 1, 2]
    trials = 60000
    res = _target_only(rows_p, parent, tokens, rng.random((trials, n)), rng.random(trials))
    first = res["predict"][res["accept_index"][:, 0]]
    counts = np.bincount(first, minlength=V)
    p0 = rows_p[0]
    chi2 = ((counts - trials * p0) ** 2 / (trials * p0)).sum()
    assert chi2 < stats.chi2.ppf(1 - 1e-3, V - 1), chi2
    via1 = res["accept_index"][:, 1] == np.arange(trials) * n + 1
    second = res["predict"][res["accept_index"][via1, 1]]
    c2 = np.bincount(second, minlength=V)
    m1 = int(via1.sum())
    p1 = rows_p[1]
    chi2 = ((c2 - m1 * p1) ** 2 / (m1 * p1)).sum()
    assert chi2 < stats.chi2.ppf(1 - 1e-3, V - 1), chi2


def test_target_only_accumulator_and_coin_per_level():
    """Root child (p = 0.6) accepted by the root's coin 0.5; its child
    (p = 0.2) is then tested against its own coin and a fresh accumulator:
    coin 0.3 rejects (an accumulator carried over, 0.8, would accept), coin
    0.1 accepts (the root's coin, 0.5, would reject)."""
    V = 4
    p = np.array([0.1, 0.6, 0.2, 0.1])
    parent = [-1, 0, 1]
    tokens = [0, 1, 2]
    for coin2, accepted in ((0.3, False), (0.1, True)):
        res = _target_only([p] * 3, parent, tokens, [[0.5, coin2, 0.0]], [0.5])
        assert res["accept_length"][0] == (3 if accepted else 2), coin2


def test_target_only_threshold_single_and_zero_guard():
    V = 5
    p = np.array([0.3, 0.35, 0.25, 0.1, 0.0])
    parent = [-1, 0, 0]
    # p >= threshold_single accepts whatever the coin
    res = _target_only([p] * 3, parent, [0, 1, 2], [[0.999, 0, 0]], [0.5], ts=0.3)
    assert res["accept_length"][0] == 2 and res["accept_index"][0, 1] == 1
    res = _target_only([p] * 3, parent, [0, 2, 3], [[0.999, 0, 0]], [0.5], ts=0.3)
    assert res["accept_length"][0] == 1
    # a zero-probability child is never accepted, not even with
    # threshold_single 0 or a coin of 0
    res = _target_only([p] * 3, parent, [0, 4, 3], [[0.0, 0, 0]], [0.5], ts=0.0)
    assert res["accept_index"][0, 1] == 2
    res = _target_only([p] * 2, [-1, 0], [0, 4], [[0.0, 0]], [0.5], ts=0.0)
    assert res["accept_length"][0] == 1 and res["predict"][0] != 4


def test_target_only_threshold_acc_scales_the_test():
    """threshold_acc = 0.5: the first child is accepted with probability
    min(1, 2 p(t))."""
    rng = np.random.default_rng(5)
    p = rng.dirichlet(np.ones(6))
    t = int(np.argsort(p)[2])
    m = 4000
    res = _target_only([p] * 2, [-1, 0], [0, t], np.stack([_grid(m), np.zeros(m)], 1),
                       np.full(m, 0.5), ta=0.5)
    rate = np.mean(res["accept_length"] == 2)
    assert abs(rate - min(1.0, 2 * p[t])) <= 1 / m
