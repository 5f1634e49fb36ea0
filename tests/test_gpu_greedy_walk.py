"""The greedy walk on hand-made trees, against the oracle's walk.

The walk kernel finds every node's matching child in parallel (each node's
thread scans its own child list) and then follows those children from the
root; these cases pin the parts of that reading that random trees rarely
reach:

* two siblings holding the target's choice: the first in sibling order is
  taken ("把投机采样讲透", 5.3: the scan stops at the first match);
* a malformed child list on a node the walk never visits: nothing is raised
  and the outputs are the oracle's (the oracle never reads that list);
* a malformed child list on a visited node: SPEC_ST_RANGE, and the walk ends
  at that node with its own choice as the terminal token;
* paths longer than accept_width - 1 drafts: SPEC_ST_DEPTH, cut where the
  oracle cuts them, for every accept_width from 1 up.
"""
import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import _gpu as G
    import speculative_decoding_build_amd as S


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


V = 3000


def _tree():
    """Request 0 of 8 nodes, rows permuted:

        0 -> 1 (tok 5), 2 (tok 7), 3 (tok 7)        children of the root
        2 -> 4 (tok 9), 5 (tok 11)
        4 -> 6 (tok 13)
        6 -> 7 (tok 15)
    Node 3's child list points at node 6 (valid, unvisited: node 3 is never
    taken because node 2 holds the same token first)."""
    n = 8
    cand = np.array([100, 5, 7, 7, 9, 11, 13, 15], np.int32)
    nxt = np.array([1, -1, 4, 6, 6, -1, 7, -1], np.int32)
    sib = np.array([-1, 2, 3, -1, 5, -1, -1, -1], np.int32)
    rows = np.array([3, 0, 5, 1, 7, 2, 6, 4], np.int32)     # retrieve_index (request 0)
    return n, cand, nxt, sib, rows


def _logits(n, rows, choice, seed):
    """bf16 logits whose row rows[k] has its unique maximum at choice[k]."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, V)).astype(np.float32)
    for k in range(n):
        x[rows[k], choice[k]] = 8.0
    import workloads as W
    return W.f32_to_bf16_bits(x)


def _run(tl, cand, rows, nxt, sib, n, s1):
    b = 1
    predict, ai, al, tp, st = G.i32(b * n), G.i32(b * s1), G.i32(b), G.i32(b * n), G.status()
    ws = torch.zeros(S.spec_accept_workspace_size(b, n, V, 0), dtype=torch.uint8, device="cuda")
    S.spec_accept_greedy(b, n, s1, V, S.SPEC_BF16, G.dev(tl), G.dev(cand), G.dev(rows),
                         G.dev(nxt), G.dev(sib), predict, ai, al, target_predict=tp,
                         workspace=ws, dev_status=st)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws)) == 0
    return dict(predict=G.host(predict), accept_index=G.host(ai).reshape(b, s1),
                accept_length=G.host(al), target_predict=G.host(tp),
                status=int(G.host(st)[0]))


def _oracle(tl, cand, rows, nxt, sib, n, s1):
    return oracle.accept_greedy(tl, cand, rows.reshape(1, n), nxt.reshape(1, n),
                                sib.reshape(1, n), 1, n, s1, "bf16")


def _same(g, o):
    for k in ("predict", "accept_index", "accept_length", "target_predict"):
        np.testing.assert_array_equal(g[k], o[k], err_msg=k)


def test_first_matching_sibling_and_unvisited_bad_list():
    n, cand, nxt, sib, rows = _tree()
    # choices: root -> 7 (nodes 2 and 3 both hold it), 2 -> 9, 4 -> 13, 6 -> 15,
    # 7 (leaf) -> 42; the others arbitrary
    choice = np.array([7, 1, 9, 2, 13, 3, 15, 42])
    tl = _logits(n, rows, choice, 5)
    say("[greedy walk] duplicate sibling tokens, full path")
    g = _run(tl, cand, rows, nxt, sib, n, 6)
    o = _oracle(tl, cand, rows, nxt, sib, n, 6)
    assert g["status"] == 0 and o["status"] == 0
    _same(g, o)
    assert g["accept_index"][0].tolist() == [3, 5, 7, 6, 4, -1]
    # node 3's list made malformed: node 3 is never visited
    nxt_bad = nxt.copy()
    nxt_bad[3] = 40
    g = _run(tl, cand, rows, nxt_bad, sib, n, 6)
    assert g["status"] == 0
    _same(g, o)


def test_bad_list_on_the_path_raises_range():
    n, cand, nxt, sib, rows = _tree()
    choice = np.array([7, 1, 9, 2, 13, 3, 15, 42])
    tl = _logits(n, rows, choice, 6)
    # node 4's sibling link (scanned from node 2's list before node 5) points
    # past the tree; node 2's choice (9) is node 4's token, so the scan finds
    # node 4 first and never follows the bad link ...
    sib_bad = sib.copy()
    sib_bad[4] = 99
    g = _run(tl, cand, rows, nxt, sib_bad, n, 6)
    assert g["status"] == 0
    _same(g, _oracle(tl, cand, rows, nxt, sib, n, 6))
    # ... while a choice held by no child makes it scan on into the bad link
    choice2 = choice.copy()
    choice2[2] = 11 + 1000
    tl2 = _logits(n, rows, choice2, 7)
    g = _run(tl2, cand, rows, nxt, sib_bad, n, 6)
    say(f"    status {g['status']} path {g['accept_index'][0].tolist()}")
    assert g["status"] & S.SPEC_ST_RANGE
    # the walk ends at node 2: root, node 2; node 2's row takes its own choice
    assert g["accept_index"][0].tolist() == [3, 5, -1, -1, -1, -1]
    assert g["accept_length"].tolist() == [2]
    assert g["predict"][5] == choice2[2]


@pytest.mark.parametrize("s1", [1, 2, 3, 4, 5, 6])
def test_depth_cut_at_every_accept_width(s1):
    n, cand, nxt, sib, rows = _tree()
    choice = np.array([7, 1, 9, 2, 13, 3, 15, 42])
    tl = _logits(n, rows, choice, 8)
    g = _run(tl, cand, rows, nxt, sib, n, s1)
    o = _oracle(tl, cand, rows, nxt, sib, n, s1)
    say(f"[greedy walk] accept_width {s1}: status {g['status']} oracle {o['status']}")
    assert g["status"] == o["status"] == (S.SPEC_ST_DEPTH if s1 < 5 else 0)
    _same(g, o)
