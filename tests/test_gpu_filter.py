"""Top-k / top-p pre-pass on the GPU against the oracle, and the sampled
accept on its output.

Cases: verify logits of the seeded workloads (bf16, many equal values) and
float32 rows; per-request parameter mixes (off, top_k 1, 20, 500, V-1,
top_p 0.5 / 0.9 / 0.99, both rules together, temperatures 0.3 to 2); rows
rounded to a few values so that the cutoff falls inside a run of equal
logits; vocabularies of 100, 8192, 50000, 128256 and 524288 entries; the
output written over the input.  Above 8192 entries the pre-pass works in
chunks and finishes a row from their candidates: rows built so that those
run short (ascending logits, all equal, a flat row under top_p alone) take
the whole-row search instead, next to rows that do not, at the smallest and
largest chunked vocabularies and the first one above; the workspace starts
filled with garbage.  Bar: the output logits bit-exact, except
rows the oracle flags near a top-p boundary (within 1e-6 of top_p).  Then
the sampled accept on the filtered logits equals the oracle's sampled accept
on its filtered logits, and requests with top_k 1 equal the greedy accept.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from _bands import assert_only_ratio_band
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import _gpu as G
    import speculative_decoding_build_amd as S

H8 = ("fixed", 8)
MIX = [  # (top_k, top_p, temperature)
    (0, 1.0, 1.0), (1, 1.0, 1.0), (20, 1.0, 0.7), (0, 0.9, 1.0), (50, 0.8, 1.3),
    (500, 0.99, 2.0), (0, 0.5, 0.3), (-1, 1.0, 1.0), (100000, 0.95, 1.0),
]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _params(b, V, seed):
    rng = np.random.default_rng(seed)
    pick = rng.integers(0, len(MIX), size=b)
    k = np.array([MIX[i][0] if MIX[i][0] != 100000 else V - 1 for i in pick], np.int32)
    p = np.array([MIX[i][1] for i in pick], np.float32)
    t = np.array([MIX[i][2] for i in pick], np.float32)
    return k, p, t


def _gpu_filter(logits, dtype, b, n, V, k, p, t, in_place=False):
    code = S.SPEC_BF16 if dtype == "bf16" else S.SPEC_F32
    x = G.dev(logits)
    out = x if in_place else torch.empty_like(x)
    st = G.status()
    ws = torch.full((max(16, S.spec_sampling_filter_workspace_size(b, n, V)),), 0xA5,
                    dtype=torch.uint8, device="cuda")
    S.spec_sampling_filter(b, n, V, code, x, G.dev(t), G.dev(k), G.dev(p), out, workspace=ws,
                           dev_status=st)
    torch.cuda.synchronize()
    res = G.host(out, np.uint16 if dtype == "bf16" else None)
    return res.reshape(b * n, V), int(G.host(st)[0])


def _check(logits, dtype, b, n, V, k, p, t, label, in_place=False):
    got, st = _gpu_filter(logits, dtype, b, n, V, k, p, t, in_place)
    want, kept, near = oracle.filter_logits(logits.reshape(b * n, V), dtype, np.repeat(t, n),
                                            np.repeat(k, n), np.repeat(p, n))
    # bit patterns: float compares would take -0 for +0
    gb = got.view(np.uint32) if got.dtype == np.float32 else got
    wb = np.ascontiguousarray(want).view(np.uint32) if want.dtype == np.float32 else want
    bad = [i for i in range(b * n) if not near[i] and not np.array_equal(gb[i], wb[i])]
    say(f"    {label}: rows {b * n} near {int(near.sum())} kept/row {kept.sum(1)[:6].tolist()} "
        f"mismatched {bad[:6]}")
    assert st == 0
    assert bad == []
    return got


CASES = {
    "c1_f32": W.CONFIGS[1],
    "c2_v128256": W.shrink(W.CONFIGS[2], hist=H8),
    "c3_b4_v50000": W.shrink(W.CONFIGS[3], batch=4, hist=H8, vocab=50000),
    "chain_b64_v8192": W.shrink(W.CONFIGS[4], hist=H8, vocab=8192),
    "c5_b2_v100": W.shrink(W.CONFIGS[5], batch=2, hist=H8, vocab=100),
    "f32_b3_v20000": W.shrink(W.CONFIGS[1], batch=3, vocab=20000),
}


@pytest.mark.parametrize("name", list(CASES))
def test_filter_workload_logits(name):
    cfg = CASES[name]
    w = W.make_workload(cfg, 81, attention=False)
    t0 = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                           cfg.num_steps, cfg.num_draft_tokens)
    tl, _ = W.verify_logits(w, t0["selected"])
    b, n, V = cfg.batch, cfg.num_draft_tokens, cfg.vocab
    k, p, t = _params(b, V, 5)
    say(f"[filter] {name} b={b} n={n} V={V} k={k.tolist()[:6]} p={p.tolist()[:6]}")
    _check(tl, cfg.dtype, b, n, V, k, p, t, name)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_filter_cut_inside_equal_values(dtype):
    # logits rounded to eight values: top-k and top-p cut inside runs of ties
    rng = np.random.default_rng(3)
    b, n, V = 6, 2, 30000
    x = np.round(rng.standard_normal((b * n, V)) * 1.5).astype(np.float32)
    logits = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
    k = np.array([7, 3000, 0, 12000, 1, 0], np.int32)
    p = np.array([1.0, 1.0, 0.3, 0.7, 1.0, 0.97], np.float32)
    t = np.array([1.0, 0.8, 1.0, 1.7, 1.0, 0.6], np.float32)
    _check(logits, dtype, b, n, V, k, p, t, f"ties {dtype}")


def test_filter_largest_vocabulary_in_place():
    rng = np.random.default_rng(4)
    b, n, V = 1, 2, 524288
    logits = W.f32_to_bf16_bits((rng.standard_normal((n, V)) * 2).astype(np.float32))
    k = np.array([300], np.int32)
    p = np.array([0.9], np.float32)
    t = np.array([1.0], np.float32)
    _check(logits, "bf16", b, n, V, k, p, t, "v524288 in place", in_place=True)


def _structured_rows(V, seed):
    """Rows whose chunk candidates run short next to rows whose do not, with
    the parameters of each (one row per request)."""
    rng = np.random.default_rng(seed)
    normal = rng.standard_normal(V) * 2
    peaked = rng.standard_normal(V)
    peaked[rng.integers(0, V, 3)] = [14.0, 13.0, 12.5]
    rows = [
        (np.linspace(-4, 4, V), 50, 1.0, 1.0),          # ascending: the last chunk's tops crowd one wave
        (np.full(V, 0.5), 20, 1.0, 1.0),                # all equal: ranked by index only
        (normal, 0, 0.6, 1.0),                          # top_p alone, cutoff far down the row
        (peaked, 0, 0.9, 1.0),                          # top_p alone, cutoff among the first entries
        (normal, 64, 1.0, 0.8),                         # the largest top_k ranked from the chunks
        (normal, 65, 0.95, 1.2),                        # just above it
        (normal, 1, 1.0, 1.0),                          # greedy
        (np.round(normal), 37, 0.9, 0.7),               # cut inside a run of equal logits
        (np.full(V, -np.inf), 5, 0.9, 1.0),             # every entry masked
    ]
    x = np.stack([r[0] for r in rows]).astype(np.float32)
    k = np.array([r[1] for r in rows], np.int32)
    p = np.array([r[2] for r in rows], np.float32)
    t = np.array([r[3] for r in rows], np.float32)
    return x, k, p, t


@pytest.mark.parametrize("V", [8193, 16385, 128256, 524288, 524289])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_filter_chunked_rows_and_whole_row_fallback(V, dtype):
    # 524288: the most chunks per row (64); 524289: one workgroup per row
    x, k, p, t = _structured_rows(V, 11)
    b = len(k)
    logits = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
    say(f"[filter] chunked V={V} {dtype} rows={b} ws={S.spec_sampling_filter_workspace_size(b, 1, V)}")
    _check(logits, dtype, b, 1, V, k, p, t, f"chunked V={V} {dtype}", in_place=(V == 16385))


KEPT_KEY_BYTES = 32 << 20   # 32 MiB = 33,554,432 bytes of logits per call


@pytest.mark.parametrize("dtype,b", [("bf16", 3), ("f32", 2)])
@pytest.mark.parametrize("in_place", [False, True])
def test_filter_above_32mb_writes_from_kept_keys(dtype, b, in_place):
    """Calls above 32 MiB (33,554,432 bytes) of logits take the output form
    that writes each row from its kept keys without reading the row again:
    3 requests x 64 rows x 128256 bf16 (49.3 MB) and 2 x 64 x 128256 float32
    (65.7 MB).  Requests: top_k 50 / top_p 0.9, top-p alone, and one whose
    rows keep only zeros of both signs (the key of -0 equals that of +0, so
    the written -0 must come from the input's bits)."""
    rng = np.random.default_rng(21)
    n, V = 64, 128256
    eb = 2 if dtype == "bf16" else 4
    assert b * n * V * eb > KEPT_KEY_BYTES
    x = (rng.standard_normal((b * n, V)) * 2).astype(np.float32)
    x[n // 2:n, :V // 3] = -np.inf                  # partly masked rows
    # last request: negative rows whose top entries are signed zeros
    z = slice((b - 1) * n, b * n)
    x[z] = -np.abs(x[z]) - 1.0
    cols = np.stack([rng.choice(V, size=6, replace=False) for _ in range(n)])
    for r in range(n):
        x[(b - 1) * n + r, cols[r, :3]] = -0.0
        x[(b - 1) * n + r, cols[r, 3:]] = 0.0
    logits = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
    # (top_k, top_p, temperature) per request; the zero rows' request is last
    par = [(50, 0.9, 1.0), (0, 0.5, 0.8), (4, 1.0, 1.0)]
    par = par if b == 3 else [par[0], par[2]]
    k = np.array([q[0] for q in par], np.int32)
    p = np.array([q[1] for q in par], np.float32)
    t = np.array([q[2] for q in par], np.float32)
    say(f"[filter] kept-key output {dtype} b={b} n={n} V={V} in_place={in_place}")
    got = _check(logits, dtype, b, n, V, k, p, t, "kept keys", in_place=in_place)
    # each zero row kept four of its six zeros (the lowest indices), so at
    # least one -0 per row, written with its sign
    bits = got.view(np.uint16 if dtype == "bf16" else np.uint32)[z]
    neg = 0x8000 if dtype == "bf16" else 0x80000000
    assert all((bits[r, cols[r, :3]] == neg).any() for r in range(n))
    k2 = np.array([1, 0, 1] if b == 3 else [1, 1], np.int32)
    p2 = np.ones(b, np.float32)                     # greedy rows, then rows kept whole
    _check(logits, dtype, b, n, V, k2, p2, t, "kept keys greedy / all", in_place=in_place)


def test_filter_workspace_size_and_refusals():
    # one chunk (<= 8192) and more than 64 chunks (> 524288) need none
    assert S.spec_sampling_filter_workspace_size(3, 4, 8192) == 0
    assert S.spec_sampling_filter_workspace_size(3, 4, 524289) == 0
    assert S.spec_sampling_filter_workspace_size(3, 4, 8193) > 0
    x = torch.zeros(2 * 9000, dtype=torch.int16, device="cuda")
    f = torch.ones(2, dtype=torch.float32, device="cuda")
    kk = torch.ones(2, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="workspace"):
        S.spec_sampling_filter(2, 1, 9000, S.SPEC_BF16, x, f, kk, f, x)


@pytest.mark.parametrize("cid", [1, 3])
def test_sampled_accept_on_filtered_logits(cid):
    cfg = W.CONFIGS[cid]
    if cid != 1:
        cfg = W.shrink(cfg, batch=6, hist=H8, vocab=20000)
    w = W.make_workload(cfg, 82, attention=False)
    t0 = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                           cfg.num_steps, cfg.num_draft_tokens)
    tl, dl = W.verify_logits(w, t0["selected"])
    b, n, V, s1 = cfg.batch, cfg.num_draft_tokens, cfg.vocab, cfg.num_steps + 1
    k = np.array([1, 40, 0, 1, 0, 5][:b], np.int32)
    p = np.array([1.0, 1.0, 0.9, 1.0, 1.0, 0.8][:b], np.float32)
    T = np.asarray(w.temperature, np.float32)
    ftl_gpu, _ = _gpu_filter(tl, cfg.dtype, b, n, V, k, p, T)
    ftl, _, near = oracle.filter_logits(tl, cfg.dtype, np.repeat(T, n), np.repeat(k, n),
                                        np.repeat(p, n))
    tree = dict(draft_tokens=t0["draft_tokens"].astype(np.int32),
                retrieve_index=t0["retrieve_index"].reshape(-1).astype(np.int32),
                retrieve_next_token=t0["retrieve_next_token"].reshape(-1).astype(np.int32),
                retrieve_next_sibling=t0["retrieve_next_sibling"].reshape(-1).astype(np.int32))
    g = G.accept_sample(w, ftl_gpu.reshape(tl.shape), dl, tree)
    args = (t0["draft_tokens"], t0["retrieve_index"], t0["retrieve_next_token"],
            t0["retrieve_next_sibling"], b, n, s1, cfg.dtype)
    o = oracle.accept_sample(ftl, dl, w.temperature, w.uniforms, w.final_uniforms, *args)
    greedy = oracle.accept_greedy(tl, *args)
    say(f"[filter+sample] cfg{cid}: lengths {o['accept_length'].tolist()} greedy "
        f"{greedy['accept_length'].tolist()}")
    assert_only_ratio_band(o, f"filtered cfg{cid}")
    for r in range(b):
        if o["exempt"][r] or near[r * n:(r + 1) * n].any():
            continue
        assert g["accept_length"][r] == o["accept_length"][r]
        assert np.array_equal(g["accept_index"][r], o["accept_index"][r])
        assert np.array_equal(g["predict"][r * n:(r + 1) * n], o["predict"][r * n:(r + 1) * n])
        if k[r] == 1:
            assert g["accept_length"][r] == greedy["accept_length"][r]
            assert np.array_equal(g["predict"][r * n:(r + 1) * n],
                                  greedy["predict"][r * n:(r + 1) * n])
