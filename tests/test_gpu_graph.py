"""The whole path captured into a HIP graph: every replay must reproduce the
eager results bit for bit.

The five operations are captured once (torch.cuda.CUDAGraph on the stream
the binding launches on) and the graph is replayed three times.  Between
replays the program does its own eager work: it restores the KV pools that
compaction moved, refills every output with a marker, runs an eager tree
build on other buffers and synchronises.  Recorded, the accepts take their
graph forms (the greedy walk as a kernel of its own after the sweep; the
sampled walk's co-resident form as an ordinary launch followed by its
recovery kernel), so this also checks that those give the eager results.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import speculative_decoding_build_amd as S


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(a):
    a = np.ascontiguousarray(a)
    view = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32,
            np.dtype(np.uint64): np.int64}.get(a.dtype)
    if view is not None:
        a = a.view(view)
    return torch.from_numpy(a).to("cuda")


@pytest.mark.parametrize("name,cfg", [
    ("b2_v20000", W.shrink(W.CONFIGS[5], batch=2, hist=("fixed", 300), vocab=20000)),
    ("b1_v128256", W.shrink(W.CONFIGS[2], hist=("fixed", 200), accept=("greedy", "sample"))),
])
def test_graph_replay_matches_eager(name, cfg):
    say(f"[graph] {name} b={cfg.batch} n={cfg.num_draft_tokens} V={cfg.vocab}")
    w = W.make_workload(cfg, 7)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                          cfg.num_steps, cfg.num_draft_tokens)
    tl, dl = W.verify_logits(w, t["selected"])
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    code = S.SPEC_BF16 if cfg.dtype == "bf16" else S.SPEC_F32
    maxlen = int(w.seq_lens.max())
    i32 = lambda k: torch.zeros(k, dtype=torch.int32, device="cuda")
    inp = dict(scores=_dev(w.scores), tokens=_dev(w.tokens), parents=_dev(w.parents),
               bonus=_dev(w.bonus), seq_lens=_dev(w.seq_lens), q=_dev(w.q),
               page_table=_dev(w.page_table), out_cache_loc=_dev(w.out_cache_loc),
               tl=_dev(tl), dl=_dev(dl), temperature=_dev(w.temperature),
               uniforms=_dev(w.uniforms), final_uniforms=_dev(w.final_uniforms))
    k0, v0 = _dev(w.k_pool), _dev(w.v_pool)
    kp, vp = k0.clone(), v0.clone()
    out = dict(draft_tokens=i32(b * n), positions=i32(b * n), retrieve_index=i32(b * n),
               retrieve_next_token=i32(b * n), retrieve_next_sibling=i32(b * n),
               selected=i32(max(1, b * (n - 1))),
               tree_mask=torch.zeros(b * n * S.spec_mask_word_bytes(n), dtype=torch.uint8,
                                     device="cuda"),
               attn=torch.empty_like(inp["q"]), predict=i32(b * n), accept_index=i32(b * s1),
               accept_length=i32(b), target_predict=i32(b * n), spredict=i32(b * n),
               saccept_index=i32(b * s1), saccept_length=i32(b), new_seq_lens=i32(b),
               free_slots=i32(b * n), num_free=i32(b), status=i32(1))
    ws_a = torch.empty(max(1, S.spec_verify_attention_workspace_size(
        b, n, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, maxlen, code)),
        dtype=torch.uint8, device="cuda")
    ws_g = torch.zeros(S.spec_accept_workspace_size(b, n, cfg.vocab, 0), dtype=torch.uint8,
                       device="cuda")
    ws_s = torch.zeros(S.spec_accept_workspace_size(b, n, cfg.vocab, 1), dtype=torch.uint8,
                       device="cuda")

    def step():
        o = out
        S.spec_build_tree(b, cfg.topk, cfg.num_steps, n, S.SPEC_MASK_QLEN_BITS, inp["scores"],
                          inp["tokens"], inp["parents"], inp["bonus"], inp["seq_lens"],
                          o["draft_tokens"], o["positions"], o["tree_mask"],
                          o["retrieve_index"], o["retrieve_next_token"],
                          o["retrieve_next_sibling"], selected=o["selected"],
                          dev_status=o["status"])
        S.spec_verify_attention(b, n, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                                cfg.page_size, code, 0.0, inp["q"], kp, vp, kp.shape[1],
                                inp["page_table"], inp["page_table"].shape[1], inp["seq_lens"],
                                maxlen, inp["out_cache_loc"], o["tree_mask"], o["attn"],
                                workspace=ws_a, dev_status=o["status"])
        S.spec_accept_greedy(b, n, s1, cfg.vocab, code, inp["tl"], o["draft_tokens"],
                             o["retrieve_index"], o["retrieve_next_token"],
                             o["retrieve_next_sibling"], o["predict"], o["accept_index"],
                             o["accept_length"], target_predict=o["target_predict"],
                             workspace=ws_g, dev_status=o["status"])
        S.spec_accept_sample(b, n, s1, cfg.vocab, code, inp["tl"], inp["dl"],
                             inp["temperature"], inp["uniforms"], inp["final_uniforms"],
                             o["draft_tokens"], o["retrieve_index"], o["retrieve_next_token"],
                             o["retrieve_next_sibling"], o["spredict"], o["saccept_index"],
                             o["saccept_length"], workspace=ws_s, dev_status=o["status"])
        S.spec_compact_kv(b, n, s1, kp.shape[0], cfg.num_kv_heads, cfg.head_dim, cfg.page_size,
                          code, kp, vp, kp.shape[1], inp["page_table"],
                          inp["page_table"].shape[1], inp["seq_lens"], inp["out_cache_loc"],
                          o["saccept_index"], o["saccept_length"], o["new_seq_lens"],
                          o["free_slots"], o["num_free"], dev_status=o["status"])

    def reset():
        kp.copy_(k0)
        vp.copy_(v0)
        for v in out.values():
            v.fill_(-9 if v.dtype == torch.int32 else 0)
        out["status"].zero_()

    reset()
    step()
    torch.cuda.synchronize()
    assert int(out["status"][0]) & ~S.SPEC_ST_ZERO_RESIDUAL == 0
    ref = {k: v.clone() for k, v in out.items()}
    ref_k, ref_v = kp.clone(), vp.clone()

    g = torch.cuda.CUDAGraph()
    reset()
    with torch.cuda.graph(g):
        step()
    other = {k: torch.zeros_like(out[k]) for k in ("draft_tokens", "positions", "tree_mask",
                                                    "retrieve_index", "retrieve_next_token",
                                                    "retrieve_next_sibling")}
    for r in range(3):
        reset()
        # unrelated eager work between replays
        S.spec_build_tree(b, cfg.topk, cfg.num_steps, n, S.SPEC_MASK_QLEN_BITS, inp["scores"],
                          inp["tokens"], inp["parents"], inp["bonus"], inp["seq_lens"],
                          other["draft_tokens"], other["positions"], other["tree_mask"],
                          other["retrieve_index"], other["retrieve_next_token"],
                          other["retrieve_next_sibling"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bad = [k for k in ref if not torch.equal(ref[k], out[k])]
        say(f"    replay {r}: differing outputs {bad}")
        assert bad == []
        assert torch.equal(ref_k, kp) and torch.equal(ref_v, vp)
