"""GPU-side helpers for the parity tests: upload seeded inputs, call the
C-ABI through the binding, download results.  No arithmetic of the path
lives here."""
import numpy as np
import torch

import speculative_decoding_build_amd as S
import workloads as W

DEV = "cuda"


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV)
    if a.dtype == np.uint64:
        return torch.from_numpy(a.view(np.int64)).to(DEV)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def host(t, dtype=None):
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def i32(n):
    return torch.zeros(n, dtype=torch.int32, device=DEV)


def status():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def dtype_code(cfg):
    return S.SPEC_BF16 if cfg.dtype == "bf16" else S.SPEC_F32


def build_tree(w, mask_mode=S.SPEC_MASK_QLEN_BITS):
    cfg = w.cfg
    b, n = cfg.batch, cfg.num_draft_tokens
    wb = S.spec_mask_word_bytes(n)
    out = dict(draft_tokens=i32(b * n), positions=i32(b * n), retrieve_index=i32(b * n),
               retrieve_next_token=i32(b * n), retrieve_next_sibling=i32(b * n),
               selected=i32(max(1, b * (n - 1))))
    if mask_mode == S.SPEC_MASK_QLEN_U8:
        out["tree_mask"] = torch.zeros(b * n * n, dtype=torch.uint8, device=DEV)
    else:
        out["tree_mask"] = torch.zeros(b * n * wb, dtype=torch.uint8, device=DEV)
    st = status()
    S.spec_build_tree(b, cfg.topk, cfg.num_steps, n, mask_mode, dev(w.scores), dev(w.tokens),
                      dev(w.parents), dev(w.bonus), dev(w.seq_lens), out["draft_tokens"],
                      out["positions"], out["tree_mask"], out["retrieve_index"],
                      out["retrieve_next_token"], out["retrieve_next_sibling"],
                      selected=out["selected"], dev_status=st)
    torch.cuda.synchronize()
    res = {k: host(v) for k, v in out.items()}
    res["status"] = int(host(st)[0])
    if mask_mode == S.SPEC_MASK_QLEN_BITS:
        words = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[wb]
        res["tree_mask"] = res["tree_mask"].view(words).reshape(b, n)
    else:
        res["tree_mask"] = res["tree_mask"].reshape(b, n, n)
    return res


def verify_attention(w, mask_words, layer=0, sm_scale=0.0):
    cfg = w.cfg
    b, n = cfg.batch, cfg.num_draft_tokens
    code = dtype_code(cfg)
    max_L = int(w.seq_lens.max())
    ws_bytes = S.spec_verify_attention_workspace_size(b, n, cfg.num_q_heads, cfg.num_kv_heads,
                                                      cfg.head_dim, max_L, code)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=DEV)
    q = dev(w.q)
    out = torch.empty_like(q)
    st = status()
    S.spec_verify_attention(b, n, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size,
                            code, sm_scale, q, dev(w.k_pool[layer]), dev(w.v_pool[layer]),
                            w.k_pool.shape[1], dev(w.page_table), w.page_table.shape[1],
                            dev(w.seq_lens), max_L, dev(w.out_cache_loc), dev(mask_words), out,
                            workspace=ws, dev_status=st)
    torch.cuda.synchronize()
    o = host(out)
    o = W.decode(cfg, o.view(np.uint16) if cfg.dtype == "bf16" else o)
    return o.reshape(b * n, cfg.num_q_heads, cfg.head_dim), int(host(st)[0])


def accept_greedy(w, tl, tree, workspace=None):
    cfg = w.cfg
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    ws = workspace
    if ws is None:
        ws = torch.zeros(S.spec_accept_workspace_size(b, n, cfg.vocab, 0), dtype=torch.uint8,
                         device=DEV)
    predict, ai, al, tp, st = i32(b * n), i32(b * s1), i32(b), i32(b * n), status()
    predict.fill_(-7)
    ai.fill_(-7)
    S.spec_accept_greedy(b, n, s1, cfg.vocab, dtype_code(cfg), dev(tl), dev(tree["draft_tokens"]),
                         dev(tree["retrieve_index"]), dev(tree["retrieve_next_token"]),
                         dev(tree["retrieve_next_sibling"]), predict, ai, al, target_predict=tp,
                         workspace=ws, dev_status=st)
    torch.cuda.synchronize()
    return dict(predict=host(predict), accept_index=host(ai).reshape(b, s1),
                accept_length=host(al), target_predict=host(tp), status=int(host(st)[0]))


def accept_sample(w, tl, dl, tree, temperature=None, uniforms=None, final_uniforms=None,
                  workspace=None):
    cfg = w.cfg
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    ws = workspace
    if ws is None:
        ws = torch.zeros(S.spec_accept_workspace_size(b, n, cfg.vocab, 1), dtype=torch.uint8,
                         device=DEV)
    predict, ai, al, st = i32(b * n), i32(b * s1), i32(b), status()
    predict.fill_(-7)
    ai.fill_(-7)
    T = w.temperature if temperature is None else temperature
    U = w.uniforms if uniforms is None else uniforms
    UF = w.final_uniforms if final_uniforms is None else final_uniforms
    S.spec_accept_sample(b, n, s1, cfg.vocab, dtype_code(cfg), dev(tl), dev(dl),
                         dev(np.asarray(T, np.float32)), dev(np.asarray(U, np.float32)),
                         dev(np.asarray(UF, np.float32)), dev(tree["draft_tokens"]),
                         dev(tree["retrieve_index"]), dev(tree["retrieve_next_token"]),
                         dev(tree["retrieve_next_sibling"]), predict, ai, al, workspace=ws,
                         dev_status=st)
    torch.cuda.synchronize()
    return dict(predict=host(predict), accept_index=host(ai).reshape(b, s1),
                accept_length=host(al), status=int(host(st)[0]))


def accept_target_only(w, tl, tree, threshold_single=1.0, threshold_acc=1.0, temperature=None,
                       uniforms=None, final_uniforms=None, workspace=None, accept_width=None):
    cfg = w.cfg
    b, n = cfg.batch, cfg.num_draft_tokens
    s1 = cfg.num_steps + 1 if accept_width is None else accept_width
    ws = workspace
    if ws is None:
        ws = torch.zeros(S.spec_accept_target_only_workspace_size(b, n, cfg.vocab),
                         dtype=torch.uint8, device=DEV)
    predict, ai, al, st = i32(b * n), i32(b * s1), i32(b), status()
    predict.fill_(-7)
    ai.fill_(-7)
    T = w.temperature if temperature is None else temperature
    U = w.uniforms if uniforms is None else uniforms
    UF = w.final_uniforms if final_uniforms is None else final_uniforms
    S.spec_accept_target_only(b, n, s1, cfg.vocab, dtype_code(cfg), dev(tl),
                              dev(np.asarray(T, np.float32)), threshold_single, threshold_acc,
                              dev(np.asarray(U, np.float32)), dev(np.asarray(UF, np.float32)),
                              dev(tree["draft_tokens"]), dev(tree["retrieve_index"]),
                              dev(tree["retrieve_next_token"]), dev(tree["retrieve_next_sibling"]),
                              predict, ai, al, workspace=ws, dev_status=st)
    torch.cuda.synchronize()
    return dict(predict=host(predict), accept_index=host(ai).reshape(b, s1),
                accept_length=host(al), status=int(host(st)[0]))


def compact_kv(cfg, k_pool, v_pool, page_table, seq_lens, out_cache_loc, accept_index,
               accept_length):
    """Pools are numpy [layers, slots, hkv, d] (uint16 bits or f32)."""
    b, n = cfg.batch, cfg.num_draft_tokens
    s1 = accept_index.shape[1]
    kp, vp = dev(k_pool), dev(v_pool)
    nsl, nf, fs, st = i32(b), i32(b), i32(b * n), status()
    S.spec_compact_kv(b, n, s1, k_pool.shape[0], k_pool.shape[2], k_pool.shape[3],
                      cfg.page_size, dtype_code(cfg), kp, vp, k_pool.shape[1], dev(page_table),
                      page_table.shape[1], dev(seq_lens), dev(out_cache_loc),
                      dev(accept_index.astype(np.int32)), dev(accept_length.astype(np.int32)),
                      nsl, fs, nf, dev_status=st)
    torch.cuda.synchronize()
    dt = np.uint16 if cfg.dtype == "bf16" else None
    return dict(k_pool=host(kp, dt), v_pool=host(vp, dt), new_seq_lens=host(nsl),
                free_slots=host(fs), num_free=host(nf), status=int(host(st)[0]))
