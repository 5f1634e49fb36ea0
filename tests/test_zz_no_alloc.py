"""spec_accept_greedy_noalloc (row keys in the library's fixed device array)
against spec_accept_greedy (keys in a caller workspace): two calls in a row,
the second on a smaller input, each bit-exact against the workspace entry
point and the oracle.  The second call also checks that the array's
contents from the first call do not leak into it."""
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = [
    ("b4_n64_v128256", W.shrink(W.CONFIGS[5], hist=("fixed", 8))),
    ("b2_n32_v30000", W.shrink(W.CONFIGS[3], batch=2, hist=("fixed", 8), vocab=30000)),
]


def _run(name, cfg, seed):
    w = W.make_workload(cfg, seed, attention=False)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                          cfg.num_steps, cfg.num_draft_tokens)
    tl, _ = W.verify_logits(w, t["selected"])
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    say(f"[no-alloc greedy] {name} b={b} n={n} V={cfg.vocab}")
    o = oracle.accept_greedy(tl, t["draft_tokens"], t["retrieve_index"], t["retrieve_next_token"],
                             t["retrieve_next_sibling"], b, n, s1, cfg.dtype)
    tree = dict(draft_tokens=t["draft_tokens"].astype(np.int32),
                retrieve_index=t["retrieve_index"].reshape(-1).astype(np.int32),
                retrieve_next_token=t["retrieve_next_token"].reshape(-1).astype(np.int32),
                retrieve_next_sibling=t["retrieve_next_sibling"].reshape(-1).astype(np.int32))
    ref = G.accept_greedy(w, tl, tree)
    x_tl = G.dev(tl)
    d = {k: G.dev(v) for k, v in tree.items()}
    predict, ai, al, tp, st = G.i32(b * n), G.i32(b * s1), G.i32(b), G.i32(b * n), G.status()
    predict.fill_(-7)
    ai.fill_(-7)
    S.spec_accept_greedy_noalloc(b, n, s1, cfg.vocab, G.dtype_code(cfg), x_tl, d["draft_tokens"],
                                 d["retrieve_index"], d["retrieve_next_token"],
                                 d["retrieve_next_sibling"], predict, ai, al, target_predict=tp,
                                 dev_status=st)
    torch.cuda.synchronize()
    got = dict(predict=G.host(predict), accept_index=G.host(ai).reshape(b, s1),
               accept_length=G.host(al), target_predict=G.host(tp), status=int(G.host(st)[0]))
    say(f"    status {got['status']} lengths {got['accept_length'].tolist()}")
    assert got["status"] == ref["status"] == 0
    for k in ("predict", "accept_index", "accept_length", "target_predict"):
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
        np.testing.assert_array_equal(got[k], o[k], err_msg=k)


def test_noalloc_matches_workspace_entry_two_calls():
    for i, (name, cfg) in enumerate(CASES):
        _run(name, cfg, 71 + i)


def test_noalloc_refuses_more_keys_than_the_array_holds():
    # 513 requests x 64 nodes = 32832 row keys, more than the fixed array's
    # 32768: refused before any launch
    b, n, s1, V = 513, 64, 7, 300
    logits = torch.zeros(b * n * V, dtype=torch.int16, device="cuda")
    idx = torch.zeros(b * n, dtype=torch.int32, device="cuda")
    out = torch.zeros(b * s1, dtype=torch.int32, device="cuda")
    with pytest.raises(S.SpecError):
        S.spec_accept_greedy_noalloc(b, n, s1, V, S.SPEC_BF16, logits, idx, idx, idx, idx,
                                     idx, out, out[:b])


def test_noalloc_recorded_in_a_graph():
    """The entry point captured into a graph (no allocation during capture):
    three replays, with an eager call on another input between them, each
    equal to the oracle."""
    name, cfg = CASES[1]
    w = W.make_workload(cfg, 81, attention=False)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                          cfg.num_steps, cfg.num_draft_tokens)
    tl, _ = W.verify_logits(w, t["selected"])
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    o = oracle.accept_greedy(tl, t["draft_tokens"], t["retrieve_index"], t["retrieve_next_token"],
                             t["retrieve_next_sibling"], b, n, s1, cfg.dtype)
    d = dict(draft_tokens=G.dev(t["draft_tokens"].astype(np.int32)),
             retrieve_index=G.dev(t["retrieve_index"].reshape(-1).astype(np.int32)),
             retrieve_next_token=G.dev(t["retrieve_next_token"].reshape(-1).astype(np.int32)),
             retrieve_next_sibling=G.dev(t["retrieve_next_sibling"].reshape(-1).astype(np.int32)))
    x_tl = G.dev(tl)
    predict, ai, al, st = G.i32(b * n), G.i32(b * s1), G.i32(b), G.status()
    say(f"[no-alloc greedy, recorded] {name}")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.spec_accept_greedy_noalloc(b, n, s1, cfg.vocab, G.dtype_code(cfg), x_tl,
                                     d["draft_tokens"], d["retrieve_index"],
                                     d["retrieve_next_token"], d["retrieve_next_sibling"],
                                     predict, ai, al, dev_status=st)
    other_name, other_cfg = CASES[0]
    for r in range(3):
        # an eager call on the larger input shares (and refills) the array
        _run(other_name, other_cfg, 90 + r)
        predict.fill_(-7)
        ai.fill_(-7)
        al.fill_(-7)
        st.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"    replay {r}: status {int(st.item())}")
        assert int(st.item()) == 0
        np.testing.assert_array_equal(G.host(predict), o["predict"])
        np.testing.assert_array_equal(G.host(ai).reshape(b, s1), o["accept_index"])
        np.testing.assert_array_equal(G.host(al), o["accept_length"])
