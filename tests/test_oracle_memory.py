"""Pins of the oracle's memory-side functions: the FULL mask and the paged
draft-branch planning ([P1] 三种 mask 形态, prepare_for_draft)."""
import json
import os

import numpy as np
import pytest

import oracle


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_full_mask_hand_worked(golden_dir):
    g = _golden(golden_dir, "full_mask_tiny.json")
    tm = np.array(g["tree_mask"], bool)
    assert oracle.full_mask(g["seq_lens"], tm).tolist() == g["full"]
    prior = np.full(len(g["full"]), 7, np.uint8)
    assert oracle.full_mask(g["seq_lens"], tm, fill_prefix=False, prior=prior).tolist() == \
        g["tree_only_over_sevens"]


def test_full_mask_rows_are_prefix_plus_ancestors():
    # an independent construction: row k of request b, read as [prefix |
    # tree], must be all-true on the prefix and true exactly on the nodes of
    # k's root path (walked through the parent list)
    rng = np.random.default_rng(4)
    b, n = 3, 7
    L = rng.integers(0, 9, size=b)
    parent = [[-1] + [int(rng.integers(0, k)) for k in range(1, n)] for _ in range(b)]
    tm = np.zeros((b, n, n), bool)
    for r in range(b):
        for k in range(n):
            j = k
            while j >= 0:
                tm[r, k, j] = True
                j = parent[r][j]
    m = oracle.full_mask(L, tm)
    assert m.size == n * int((L + n).sum())
    off = 0
    for r in range(b):
        w = int(L[r]) + n
        block = m[off:off + n * w].reshape(n, w)
        assert np.all(block[:, :L[r]] == 1)
        for k in range(n):
            path = set()
            j = k
            while j >= 0:
                path.add(j)
                j = parent[r][j]
            assert set(np.flatnonzero(block[k, L[r]:])) == path
        off += n * w


def test_plan_draft_branches_hand_worked(golden_dir):
    g = _golden(golden_dir, "draft_branches_tiny.json")
    o = oracle.plan_draft_branches(g["seq_lens"], g["page_table"], g["branch_pages"], g["topk"],
                                   g["num_steps"], g["page_size"], 100)
    assert o["copies"] == [tuple(c) for c in g["copies"]]
    assert o["out_cache_loc"].tolist() == g["out_cache_loc"]
    assert o["status"] == 0


@pytest.mark.parametrize("ps,topk", [(4, 3), (16, 8), (1, 4), (8, 1), (16, 1)])
def test_branch_views_read_whole_pages_coherently(ps, topk):
    """Simulate what the pages say the duplication is for: after the copies
    and the draft writes, reading every position of a branch's view through
    whole pages (prefix pages, then the branch's region pages; or the
    prefix's own page table for topk 1) returns that position's KV: the
    prefix token's for prefix positions, the branch's draft token's after."""
    rng = np.random.default_rng(ps * 10 + topk)
    b, S = 3, 5
    L = rng.integers(1, 5 * ps + 3, size=b)
    num_pages = 200
    perm = rng.permutation(num_pages)
    maxp = (int(L.max()) + S) // ps + 2
    pt = perm[:b * maxp].reshape(b, maxp)
    per_branch = (ps - 1 + S) // ps + 1
    bp = perm[b * maxp:b * maxp + b * topk * per_branch].reshape(b, topk, per_branch)
    # pool: slot -> a marker of what it holds; prefix positions hold
    # (request, position), one layer, one head, d = 2
    pool = np.full((1, num_pages * ps, 1, 2), -1, np.int64)
    for r in range(b):
        for pos in range(int(L[r])):
            pool[0, pt[r, pos // ps] * ps + pos % ps, 0] = (r, pos)
    o = oracle.plan_draft_branches(L, pt, bp, topk, S, ps, num_pages)
    assert o["status"] == 0
    k2, _ = oracle.duplicate_prefix_tail(pool, pool, o["copies"])
    for r in range(b):
        for j in range(topk):
            for s in range(S):
                k2[0, o["out_cache_loc"][r, j, s], 0] = (r, 1000 * (j + 1) + s)
    for r in range(b):
        Lr = int(L[r])
        base = Lr - Lr % ps
        for j in range(topk):
            for pos in range(Lr + S):
                if topk == 1:
                    slot = pt[r, pos // ps] * ps + pos % ps
                elif pos < base:
                    slot = pt[r, pos // ps] * ps + pos % ps
                else:
                    t = pos - base
                    slot = bp[r, j, t // ps] * ps + t % ps
                want = (r, pos) if pos < Lr else (r, 1000 * (j + 1) + (pos - Lr))
                assert tuple(k2[0, slot, 0]) == want, (r, j, pos)
    if ps == 1 or topk == 1:
        assert o["copies"] == []


def test_plan_draft_branches_bad_page():
    o = oracle.plan_draft_branches([6], [[3, 7, 99]], [[[10, 500], [12, 13]]], 2, 3, 4, 100)
    assert o["status"] & oracle.ST_RANGE
    assert o["out_cache_loc"][0, 0].tolist() == [42, 43, -1]
