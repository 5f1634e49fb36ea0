"""The next-row operations captured into a HIP graph: the target-only
accept, the draft loop (one draft-step call per step, path scores chained in
place), the top-k / top-p pre-pass, the FULL mask and the branch planning.
Each replay (three, with eager work and a refill of every output with a
marker between them) must reproduce the eager results bit for bit."""
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


def test_extra_operations_graph_replay():
    cfg = W.shrink(W.CONFIGS[5], batch=2, hist=("fixed", 300), vocab=20000)
    w = W.make_workload(cfg, 9, attention=False)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                          cfg.num_steps, cfg.num_draft_tokens)
    tl, _ = W.verify_logits(w, t["selected"])
    b, n, s1, k, V, S_ = (cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1, cfg.topk,
                          cfg.vocab, cfg.num_steps)
    code = S.SPEC_BF16
    d = G.dev
    i32 = lambda m: torch.zeros(m, dtype=torch.int32, device="cuda")
    tl_d = d(tl)
    T = d(np.asarray(w.temperature, np.float32))
    U, UF = d(np.asarray(w.uniforms, np.float32)), d(np.asarray(w.final_uniforms, np.float32))
    tree = {kk: d(np.ascontiguousarray(v).reshape(-1).astype(np.int32)) for kk, v in
            (("draft_tokens", t["draft_tokens"]), ("ri", t["retrieve_index"]),
             ("rn", t["retrieve_next_token"]), ("rs", t["retrieve_next_sibling"]))}
    words = d(oracle.pack_mask(t["mask"], oracle.MASK_QLEN_BITS))
    seq = d(np.asarray(w.seq_lens, np.int32))
    steps = [d(np.ascontiguousarray(w.ctx_draft[:, 0:1] if i == 0 else
                                    w.ctx_draft[:, 1 + (i - 1) * k:1 + i * k])) for i in range(S_)]
    ps, hkv, hd = 16, 2, 64
    per_branch = (ps - 1 + S_ + ps - 1) // ps
    pt = d(np.arange(b * 10, dtype=np.int32).reshape(b, 10))
    bp = d(np.arange(b * 10, b * 10 + b * k * per_branch, dtype=np.int32).reshape(b, k, per_branch))
    pages = b * 10 + b * k * per_branch
    lens = d(np.array([37, 50], np.int32))
    kpool = torch.randint(-30000, 30000, (pages * ps * hkv * hd,), dtype=torch.int16, device="cuda")
    vpool = torch.randint(-30000, 30000, (pages * ps * hkv * hd,), dtype=torch.int16, device="cuda")
    k0, v0 = kpool.clone(), vpool.clone()
    full_bytes = int(n * (np.sum(w.seq_lens) + n * b))
    out = dict(predict=i32(b * n), ai=i32(b * s1), al=i32(b),
               sc=torch.zeros(b * cfg.ncand, device="cuda"), tk=i32(b * cfg.ncand),
               pa=i32(b * cfg.npar), ns=torch.zeros(b * k, device="cuda"), nt=i32(b * k),
               filt=torch.empty_like(tl_d), mask=torch.zeros(full_bytes, dtype=torch.uint8,
                                                             device="cuda"),
               loc=i32(b * k * S_), st=i32(1))
    ws_to = torch.zeros(S.spec_accept_target_only_workspace_size(b, n, V), dtype=torch.uint8,
                        device="cuda")
    ws_ds = torch.empty(S.spec_draft_step_workspace_size(b, k, V), dtype=torch.uint8, device="cuda")
    ws_f = torch.empty(max(256, S.spec_sampling_filter_workspace_size(b, n, V)), dtype=torch.uint8,
                       device="cuda")
    topk_d, topp_d = d(np.array([30, 0], np.int32)), d(np.array([1.0, 0.9], np.float32))

    def run():
        S.spec_accept_target_only(b, n, s1, V, code, tl_d, T, 1.0, 1.0, U, UF,
                                  tree["draft_tokens"], tree["ri"], tree["rn"], tree["rs"],
                                  out["predict"], out["ai"], out["al"], workspace=ws_to,
                                  dev_status=out["st"])
        for i in range(S_):
            S.spec_draft_step(b, k, S_, i, V, code, steps[i], None if i == 0 else out["ns"],
                              out["sc"], out["tk"], out["pa"], out["ns"], out["nt"],
                              workspace=ws_ds, dev_status=out["st"])
        S.spec_sampling_filter(b, n, V, code, tl_d, T, topk_d, topp_d, out["filt"],
                               workspace=ws_f, dev_status=out["st"])
        S.spec_full_mask(b, n, seq, int(np.max(w.seq_lens)), words, True, out["mask"],
                         dev_status=out["st"])
        S.spec_plan_draft_branches(b, k, S_, ps, 1, hkv, hd, code, kpool, vpool, pages * ps,
                                   lens, pt, 10, bp, per_branch, out["loc"], dev_status=out["st"])

    run()
    torch.cuda.synchronize()
    ref = {kk: v.clone() for kk, v in out.items()}
    kref, vref = kpool.clone(), vpool.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for kk, v in out.items():
            # the status word is OR-ed into, so it starts at zero
            v.fill_(0 if kk == "st" else (0xA5 if v.dtype == torch.uint8 else -5))
        kpool.copy_(k0)
        vpool.copy_(v0)
        # eager work between replays
        S.spec_full_mask(b, n, seq, int(np.max(w.seq_lens)), words, False,
                         torch.zeros(full_bytes, dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for kk in out:
            assert torch.equal(out[kk], ref[kk]), (rep, kk)
        assert torch.equal(kpool, kref) and torch.equal(vpool, vref), rep
        say(f"    replay {rep}: all outputs equal the eager run")
