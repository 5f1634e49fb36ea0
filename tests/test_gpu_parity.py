"""Parity of the HIP path with the CPU oracle on the same seeded inputs.

Integer outputs (tree build, greedy accept, compaction) must match bit for
bit.  Sampled accept must match bit for bit except for requests whose
ratio test lies within 1e-6 of its threshold (no request of these seeds may
be exempt for another reason).  Attention must stay within
a max relative error (per output vector, inf-norm) of 1e-5 for f32 and 2e-2
for bf16.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _bands import assert_only_ratio_band

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import _gpu as G
    import speculative_decoding_build_amd as S


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


ATTN_TOL = {"f32": 1e-5, "bf16": 2e-2}

SMALL = {
    "c1": W.CONFIGS[1],
    "c1_long_f32": W.shrink(W.CONFIGS[1], hist=("fixed", 500), vocab=1001),
    "c2s": W.shrink(W.CONFIGS[2], hist=("fixed", 300), vocab=20000),
    "c3s": W.shrink(W.CONFIGS[3], batch=3, hist=("uniform", 0, 400), vocab=9000),
    "c4s": W.shrink(W.CONFIGS[4], batch=5, hist=("fixed", 130), vocab=17000),
    "c5s": W.shrink(W.CONFIGS[5], batch=2, hist=("fixed", 700), vocab=8200),
    "c5_L0mix": W.shrink(W.CONFIGS[5], batch=3, hist=("list", [0, 300, 5]), vocab=8200),
    "ps3_v1001": W.shrink(W.CONFIGS[3], batch=2, hist=("uniform", 50, 90), vocab=1001, page_size=3),
    "root_only": W.shrink(W.CONFIGS[3], batch=2, hist=("fixed", 40), vocab=500, num_draft_tokens=1),
    "d64_bf16": W.shrink(W.CONFIGS[3], batch=2, hist=("fixed", 200), vocab=700, head_dim=64),
    # more requests than the cooperative walk can hold at once: one
    # workgroup per request walks instead
    "many_req": W.shrink(W.CONFIGS[4], batch=1100, hist=("fixed", 8), vocab=5000),
}

_cache = {}


def workload(name, seed=11):
    key = (name, seed)
    if key not in _cache:
        cfg = SMALL[name] if name in SMALL else W.CONFIGS[int(name[-1])]
        _cache.clear()
        w = W.make_workload(cfg, seed)
        t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                              cfg.num_steps, cfg.num_draft_tokens)
        tl, dl = W.verify_logits(w, t["selected"])
        _cache[key] = (w, t, tl, dl)
    return _cache[key]


def _tree_for_gpu(t, b, n):
    return dict(draft_tokens=t["draft_tokens"].astype(np.int32),
                retrieve_index=t["retrieve_index"].reshape(-1).astype(np.int32),
                retrieve_next_token=t["retrieve_next_token"].reshape(-1).astype(np.int32),
                retrieve_next_sibling=t["retrieve_next_sibling"].reshape(-1).astype(np.int32))


@pytest.mark.parametrize("name", list(SMALL))
def test_build_tree_bit_exact(name):
    w, t, _, _ = workload(name)
    cfg = w.cfg
    b, n = cfg.batch, cfg.num_draft_tokens
    say(f"[build_tree] {name} b={b} topk={cfg.topk} S={cfg.num_steps} n={n}")
    for mode in (S.SPEC_MASK_QLEN_BITS, S.SPEC_MASK_QLEN_U8):
        g = G.build_tree(w, mode)
        assert g["status"] == t["status"] == 0
        np.testing.assert_array_equal(g["draft_tokens"], t["draft_tokens"])
        np.testing.assert_array_equal(g["positions"], t["positions"])
        np.testing.assert_array_equal(g["retrieve_index"].reshape(b, n), t["retrieve_index"])
        np.testing.assert_array_equal(g["retrieve_next_token"].reshape(b, n), t["retrieve_next_token"])
        np.testing.assert_array_equal(g["retrieve_next_sibling"].reshape(b, n), t["retrieve_next_sibling"])
        if n > 1:
            np.testing.assert_array_equal(g["selected"][:b * (n - 1)].reshape(b, n - 1), t["selected"])
        np.testing.assert_array_equal(g["tree_mask"], oracle.pack_mask(t["mask"], mode))


def _attn_err(got, ref):
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return float((num / np.maximum(den, 1e-30)).max())


# Trees whose every candidate is kept (n - 1 = ncand): the kernel skips the
# ranking; a full topk-2 step, a full 2-level topk-3 tree and a 7-node chain,
# each with both mask layouts.
ALL_KEPT = {
    "topk2_s1_n3": dict(topk=2, num_steps=1, num_draft_tokens=3),
    "topk3_s2_n13": dict(topk=3, num_steps=2, num_draft_tokens=13),
    "chain_s6_n7": dict(topk=1, num_steps=6, num_draft_tokens=7),
}


# Selection shapes: one ranking round shared by 1024/ceil64(ncand) threads
# per candidate (36 candidates: 16 ranges of keys; 114: 8; 968: 1) and
# several rounds above 1024 candidates (1032); plus scores floored to a
# coarse grid, so that the cut falls inside runs of equal scores (ranked by
# index).
SELECT = {
    "topk4_s3_n10": dict(topk=4, num_steps=3, num_draft_tokens=10),
    "topk6_s4_n40": dict(topk=6, num_steps=4, num_draft_tokens=40),
    "topk8_s16_n64": dict(topk=8, num_steps=16, num_draft_tokens=64),
    "topk8_s17_n64": dict(topk=8, num_steps=17, num_draft_tokens=64),
}


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("name", list(SELECT))
def test_build_tree_selection_shapes(name, ties):
    cfg = W.shrink(W.CONFIGS[3], batch=3, hist=("fixed", 8), vocab=500, **SELECT[name])
    w = W.make_workload(cfg, 6, attention=False)
    if ties:
        # flooring log2(score) to halves keeps a child's score <= its
        # parent's, and the parent has the smaller flat index, so the kept
        # set stays closed
        lg = np.floor(np.log2(np.maximum(w.scores, 1e-30)) * 2.0) / 2.0
        w.scores = np.exp2(lg).astype(np.float32)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                          cfg.num_steps, cfg.num_draft_tokens)
    b, n = cfg.batch, cfg.num_draft_tokens
    say(f"[build_tree] {name} ties={ties} ncand={cfg.ncand} n={n}")
    g = G.build_tree(w, mask_mode=S.SPEC_MASK_QLEN_BITS)
    assert g["status"] == t["status"]
    np.testing.assert_array_equal(g["selected"][:b * (n - 1)].reshape(b, n - 1), t["selected"])
    np.testing.assert_array_equal(g["draft_tokens"], t["draft_tokens"])
    np.testing.assert_array_equal(g["retrieve_next_token"].reshape(b, n), t["retrieve_next_token"])
    np.testing.assert_array_equal(g["retrieve_next_sibling"].reshape(b, n),
                                  t["retrieve_next_sibling"])
    np.testing.assert_array_equal(g["tree_mask"], oracle.pack_mask(t["mask"], S.SPEC_MASK_QLEN_BITS))


@pytest.mark.parametrize("name", list(ALL_KEPT))
def test_build_tree_all_kept(name):
    cfg = W.shrink(W.CONFIGS[3], batch=3, hist=("fixed", 8), vocab=500, **ALL_KEPT[name])
    w = W.make_workload(cfg, 5, attention=False)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                          cfg.num_steps, cfg.num_draft_tokens)
    b, n = cfg.batch, cfg.num_draft_tokens
    for mode in (S.SPEC_MASK_QLEN_BITS, S.SPEC_MASK_QLEN_U8):
        g = G.build_tree(w, mask_mode=mode)
        assert g["status"] == t["status"] == 0
        np.testing.assert_array_equal(g["draft_tokens"], t["draft_tokens"])
        np.testing.assert_array_equal(g["positions"], t["positions"])
        np.testing.assert_array_equal(g["retrieve_next_token"].reshape(b, n), t["retrieve_next_token"])
        np.testing.assert_array_equal(g["retrieve_next_sibling"].reshape(b, n),
                                      t["retrieve_next_sibling"])
        np.testing.assert_array_equal(g["selected"][:b * (n - 1)].reshape(b, n - 1), t["selected"])
        np.testing.assert_array_equal(g["tree_mask"], oracle.pack_mask(t["mask"], mode))


@pytest.mark.parametrize("name", list(SMALL))
def test_verify_attention_small(name):
    w, t, _, _ = workload(name)
    cfg = w.cfg
    say(f"[attention] {name} b={cfg.batch} n={cfg.num_draft_tokens} hq={cfg.num_q_heads} "
        f"hkv={cfg.num_kv_heads} d={cfg.head_dim} ps={cfg.page_size} L={w.seq_lens.tolist()}")
    words = oracle.pack_mask(t["mask"], oracle.MASK_QLEN_BITS)
    got, st = G.verify_attention(w, words)
    assert st == 0
    ref = oracle.verify_attention(w.q, w.k_pool[0], w.v_pool[0], w.page_table, w.seq_lens,
                                  w.out_cache_loc, t["mask"], cfg.num_q_heads, cfg.num_kv_heads,
                                  cfg.page_size, cfg.dtype)
    err = _attn_err(got, ref)
    say(f"    max rel err {err:.3e}")
    assert err <= ATTN_TOL[cfg.dtype]


def _compare_accept(g, o, b, n, exempt=None):
    bad = []
    for r in range(b):
        if exempt is not None and exempt[r]:
            continue
        same = (g["accept_length"][r] == o["accept_length"][r]
                and np.array_equal(g["accept_index"][r], o["accept_index"][r])
                and np.array_equal(g["predict"][r * n:(r + 1) * n], o["predict"][r * n:(r + 1) * n]))
        if not same:
            bad.append(r)
    return bad


@pytest.mark.parametrize("name", list(SMALL))
def test_accept_greedy_small(name):
    w, t, tl, _ = workload(name)
    cfg = w.cfg
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    say(f"[greedy] {name} b={b} n={n} V={cfg.vocab}")
    o = oracle.accept_greedy(tl, t["draft_tokens"], t["retrieve_index"], t["retrieve_next_token"],
                             t["retrieve_next_sibling"], b, n, s1, cfg.dtype)
    g = G.accept_greedy(w, tl, _tree_for_gpu(t, b, n))
    assert g["status"] == o["status"] == 0
    np.testing.assert_array_equal(g["target_predict"], o["target_predict"])
    assert _compare_accept(g, o, b, n) == []


@pytest.mark.parametrize("name", list(SMALL))
def test_accept_sample_small(name):
    w, t, tl, dl = workload(name)
    cfg = w.cfg
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    say(f"[sample] {name} b={b} n={n} V={cfg.vocab} T={cfg.temperature}")
    o = oracle.accept_sample(tl, dl, w.temperature, w.uniforms, w.final_uniforms,
                             t["draft_tokens"], t["retrieve_index"], t["retrieve_next_token"],
                             t["retrieve_next_sibling"], b, n, s1, cfg.dtype)
    g = G.accept_sample(w, tl, dl, _tree_for_gpu(t, b, n))
    assert (g["status"] & ~S.SPEC_ST_ZERO_RESIDUAL) == 0
    assert_only_ratio_band(o, name)
    bad = _compare_accept(g, o, b, n, o["exempt"])
    say(f"    exempt {int(o['exempt'].sum())}/{b}, mismatched {bad}")
    assert bad == []


@pytest.mark.parametrize("name", ["c1", "c3s", "c5s", "c5_L0mix", "ps3_v1001"])
@pytest.mark.parametrize("layers", [1, 3])
def test_compact_kv_small(name, layers):
    w, t, tl, _ = workload(name)
    cfg = w.cfg
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    say(f"[compact] {name} b={b} layers={layers}")
    o_acc = oracle.accept_greedy(tl, t["draft_tokens"], t["retrieve_index"], t["retrieve_next_token"],
                                 t["retrieve_next_sibling"], b, n, s1, cfg.dtype)
    rng = np.random.default_rng(5)
    shape = (layers,) + w.k_pool.shape[1:]
    if cfg.dtype == "bf16":
        kp = rng.integers(0, 2 ** 16, shape, dtype=np.uint16)
        vp = rng.integers(0, 2 ** 16, shape, dtype=np.uint16)
    else:
        kp = rng.standard_normal(shape, dtype=np.float32)
        vp = rng.standard_normal(shape, dtype=np.float32)
    # force a long accepted path on request 0 to exercise overlapping moves
    ai = o_acc["accept_index"].copy()
    al = o_acc["accept_length"].copy()
    o = oracle.compact_kv(kp, vp, w.page_table, w.seq_lens, w.out_cache_loc, ai, al, b, n,
                          cfg.page_size)
    g = G.compact_kv(cfg, kp, vp, w.page_table, w.seq_lens, w.out_cache_loc, ai, al)
    assert g["status"] == o["status"] == 0
    np.testing.assert_array_equal(g["new_seq_lens"], o["new_seq_lens"])
    np.testing.assert_array_equal(g["num_free"], o["num_free"])
    np.testing.assert_array_equal(g["free_slots"], o["free_slots"])
    assert np.array_equal(g["k_pool"].view(np.uint8), o["k_pool"].view(np.uint8))
    assert np.array_equal(g["v_pool"].view(np.uint8), o["v_pool"].view(np.uint8))


def test_compact_kv_overlap_in_place():
    """Accepted rows [0, 2, 3] of a request whose verify rows sit at its next
    positions: sources and targets overlap."""
    cfg = W.shrink(W.CONFIGS[1], batch=1, hist=("fixed", 4))
    L, n = 4, cfg.num_draft_tokens
    page_table = np.arange(L + n, dtype=np.int32)[None]
    loc = np.arange(L, L + n, dtype=np.int32)
    rng = np.random.default_rng(1)
    kp = rng.standard_normal((2, L + n, 1, 64), dtype=np.float32)
    vp = rng.standard_normal((2, L + n, 1, 64), dtype=np.float32)
    ai = np.array([[0, 2, 3, -1]])
    al = np.array([3])
    o = oracle.compact_kv(kp, vp, page_table, np.array([L], np.int32), loc, ai, al, 1, n, 1)
    g = G.compact_kv(cfg, kp, vp, page_table, np.array([L], np.int32), loc, ai, al)
    assert np.array_equal(g["k_pool"], o["k_pool"]) and np.array_equal(g["v_pool"], o["v_pool"])
    np.testing.assert_array_equal(g["free_slots"], o["free_slots"])


def test_batch_zero_is_noop():
    S.spec_build_tree(0, 2, 3, 6, S.SPEC_MASK_QLEN_BITS, *[torch.empty(0, device="cuda")] * 11)


# ---------------------------------------------------------------------------
# full-size workloads (the shapes the benchmark times)
# ---------------------------------------------------------------------------

_full = {}


def full(cid, attention):
    key = (cid, attention)
    if key not in _full:
        _full.clear()
        cfg = W.CONFIGS[cid]
        w = W.make_workload(cfg, 1000 * cid + 1, attention=attention)
        t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                              cfg.num_steps, cfg.num_draft_tokens)
        _full[key] = (w, t)
    return _full[key]


# Split-KV plans whose last key split holds 1, 2, 3 or 4 tiles, or ends in a
# part tile, or whose splits are 4 tiles long: every output vector against
# the oracle.  One-slot pages take the LDS-load form; 12-slot pages (not a
# power of two) keep the register-staged form with key halves.
SPLIT_CASES = {
    "L4160_last1_ps12": W.shrink(W.CONFIGS[2], hist=("fixed", 4160), vocab=1000, page_size=12),
    "L4288_last3_ps12": W.shrink(W.CONFIGS[2], hist=("fixed", 4288), vocab=1000, page_size=12),
    "L4100_part_ps12": W.shrink(W.CONFIGS[2], hist=("fixed", 4100), vocab=1000, page_size=12),
    "L4160_last1": W.shrink(W.CONFIGS[2], hist=("fixed", 4160), vocab=1000),
    "L4224_last2": W.shrink(W.CONFIGS[2], hist=("fixed", 4224), vocab=1000),
    "L4288_last3": W.shrink(W.CONFIGS[2], hist=("fixed", 4288), vocab=1000),
    "L4100_part": W.shrink(W.CONFIGS[2], hist=("fixed", 4100), vocab=1000),
    "L4032_4tile": W.shrink(W.CONFIGS[2], hist=("fixed", 4032), vocab=1000),
    "L2048": W.shrink(W.CONFIGS[2], hist=("fixed", 2048), vocab=1000),
    "b4_Lu": W.shrink(W.CONFIGS[3], batch=4, hist=("uniform", 1000, 3000), vocab=1000),
    # 560 query rows per KV head (n=35, 16 query heads per KV head): waves of
    # 64 rows, the last wave's second 32-row block cut at row 560
    "g16_n35_Lu": W.shrink(W.CONFIGS[5], batch=2, hist=("uniform", 300, 2500), vocab=1000,
                           num_draft_tokens=35, num_kv_heads=4),
}


@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_verify_attention_split_remainders(name):
    cfg = SPLIT_CASES[name]
    w = W.make_workload(cfg, 17)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                          cfg.num_steps, cfg.num_draft_tokens)
    say(f"[attention splits] {name} b={cfg.batch} L={w.seq_lens.tolist()}")
    words = oracle.pack_mask(t["mask"], oracle.MASK_QLEN_BITS)
    got, st = G.verify_attention(w, words)
    assert st == 0
    ref = oracle.verify_attention(w.q, w.k_pool[0], w.v_pool[0], w.page_table, w.seq_lens,
                                  w.out_cache_loc, t["mask"], cfg.num_q_heads, cfg.num_kv_heads,
                                  cfg.page_size, cfg.dtype)
    err = _attn_err(got, ref.reshape(got.shape))
    say(f"    max rel err {err:.3e} over all {got.shape[0] * got.shape[1]} vectors")
    assert err <= ATTN_TOL[cfg.dtype]


# Splits longer than the two 8-tile chunks of the slot ring the prologue
# fills, so chunks are refilled inside the loop, for waves of 64 rows (512
# rows per KV head) and of 32 rows: sampled vectors against the oracle.
LONG_SPLIT_CASES = {
    "rows512_L8700": W.shrink(W.CONFIGS[5], batch=4, hist=("fixed", 8700), vocab=1000),
    "rows128_Lu": W.shrink(W.CONFIGS[3], batch=12, hist=("uniform", 4000, 9000), vocab=1000),
}


# Shapes of the LDS-load form: one wave per 32-row block (KH = 1) and wave
# pairs taking key halves (KH = 2), pages of 1 to 64 slots (below 8 every
# lane looks its key's page up; from 8 on a wave's keys share one page id),
# static and length-balanced plans, and a row count (35) that leaves whole
# row blocks of the workgroup idle.
DMA_CASES = {
    "b4_Lu_ragged": W.shrink(W.CONFIGS[5], batch=4, hist=("uniform", 9001, 17003), vocab=1000),
    "b1_L50005": W.shrink(W.CONFIGS[5], batch=1, hist=("fixed", 50005), vocab=1000),
    "b3_L8195": W.shrink(W.CONFIGS[5], batch=3, hist=("fixed", 8195), vocab=1000),
    "kh1_b2_ps8_Lu": W.shrink(W.CONFIGS[5], batch=2, hist=("uniform", 5000, 9000), vocab=1000,
                              page_size=8),
    "kh2_b1_ps1_L3001": W.shrink(W.CONFIGS[2], hist=("fixed", 3001), vocab=1000),
    "kh2_b2_ps1_Lu": W.shrink(W.CONFIGS[2], batch=2, hist=("uniform", 600, 1900), vocab=1000),
    "kh2_b2_ps2_Lu": W.shrink(W.CONFIGS[3], batch=2, hist=("uniform", 300, 1900), vocab=1000,
                              page_size=2),
    "kh2_b3_ps4_Lu": W.shrink(W.CONFIGS[3], batch=3, hist=("uniform", 100, 2500), vocab=1000,
                              page_size=4),
    "kh2_b1_ps64_L2600": W.shrink(W.CONFIGS[2], hist=("fixed", 2600), vocab=1000, page_size=64),
    "kh2_b16_rows35": W.shrink(W.CONFIGS[4], batch=16, hist=("fixed", 700), vocab=1000),
    # 512 workgroups of 128 rows (two rounds): the key-half form one per CU
    "kh2_two_rounds_b16_Lu": W.shrink(W.CONFIGS[3], batch=16, hist=("uniform", 200, 1500),
                                      vocab=1000),
}


@pytest.mark.parametrize("name", list(DMA_CASES))
def test_verify_attention_lds_load_form(name):
    _attention_every_unit(DMA_CASES[name], name, "LDS-load form")


# Requests with no history (only the tree keys), alone and beside long ones:
# the static plan's one-split path, the length-balanced plan with a request
# of one tile, both kernel forms (one-slot and 16-slot pages: LDS-load form;
# 12-slot pages: register-staged form) and the f32 path.
ZERO_HIST_CASES = {
    "L0_all_g8_ps16": W.shrink(W.CONFIGS[5], batch=2, hist=("fixed", 0), vocab=1000),
    "L0_mixed_g8_ps16": W.shrink(W.CONFIGS[5], batch=3, hist=("list", [0, 20000, 5]), vocab=1000),
    "L0_mixed_g4_ps1": W.shrink(W.CONFIGS[2], batch=3, hist=("list", [3000, 0, 64]), vocab=1000),
    "L0_mixed_g8_ps12": W.shrink(W.CONFIGS[5], batch=3, hist=("list", [0, 9000, 1]), vocab=1000,
                                 page_size=12),
    "L0_all_f32": W.shrink(W.CONFIGS[1], hist=("fixed", 0), vocab=100),
    "L0_mixed_f32": W.shrink(W.CONFIGS[1], hist=("list", [0, 700]), vocab=100),
}


@pytest.mark.parametrize("name", list(ZERO_HIST_CASES))
def test_verify_attention_zero_history(name):
    _attention_every_unit(ZERO_HIST_CASES[name], name, "zero history")


def _attention_every_unit(cfg, name, label):
    w = W.make_workload(cfg, 29)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                          cfg.num_steps, cfg.num_draft_tokens)
    b, n, hq, hkv = cfg.batch, cfg.num_draft_tokens, cfg.num_q_heads, cfg.num_kv_heads
    G_ = hq // hkv
    say(f"[attention, {label}] {name} b={b} L={w.seq_lens.tolist()}")
    words = oracle.pack_mask(t["mask"], oracle.MASK_QLEN_BITS)
    got, st = G.verify_attention(w, words)
    assert st == 0
    assert np.isfinite(got).all()
    err = 0.0
    for r in range(b):
        for g in range(hkv):
            ref = oracle.verify_attention_unit(w.q, w.k_pool[0], w.v_pool[0], w.page_table,
                                               w.seq_lens, w.out_cache_loc, t["mask"], hq, hkv,
                                               cfg.page_size, cfg.dtype, r, g)
            mine = got[r * n:(r + 1) * n, g * G_:(g + 1) * G_]
            err = max(err, _attn_err(mine.reshape(-1, mine.shape[-1]),
                                     ref.reshape(-1, ref.shape[-1])))
    say(f"    max rel err {err:.3e} over {b * hkv * n * G_} vectors")
    assert err <= ATTN_TOL[cfg.dtype]


# One-slot pages around the LDS-load form's bound of 2048 page ids per split:
# at 131008 history keys the splits hold 32 tiles (2048 ids) and take that
# form; one key more makes them 33 tiles and the register-staged form runs.
# Every output vector, one (request, KV head) unit at a time.
PAGE_ID_BOUND_CASES = {
    "ps1_L131008_2048_ids": W.shrink(W.CONFIGS[2], hist=("fixed", 131008), vocab=1000),
    "ps1_L131009_register_staged": W.shrink(W.CONFIGS[2], hist=("fixed", 131009), vocab=1000),
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(PAGE_ID_BOUND_CASES))
def test_verify_attention_page_id_bound(name):
    cfg = PAGE_ID_BOUND_CASES[name]
    w = W.make_workload(cfg, 37)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                          cfg.num_steps, cfg.num_draft_tokens)
    b, n, hq, hkv = cfg.batch, cfg.num_draft_tokens, cfg.num_q_heads, cfg.num_kv_heads
    G_ = hq // hkv
    say(f"[attention, page-id bound] {name} b={b} L={w.seq_lens.tolist()}")
    words = oracle.pack_mask(t["mask"], oracle.MASK_QLEN_BITS)
    got, st = G.verify_attention(w, words)
    assert st == 0
    err = 0.0
    for r in range(b):
        for g in range(hkv):
            ref = oracle.verify_attention_unit(w.q, w.k_pool[0], w.v_pool[0], w.page_table,
                                               w.seq_lens, w.out_cache_loc, t["mask"], hq, hkv,
                                               cfg.page_size, cfg.dtype, r, g)
            mine = got[r * n:(r + 1) * n, g * G_:(g + 1) * G_]
            err = max(err, _attn_err(mine.reshape(-1, mine.shape[-1]),
                                     ref.reshape(-1, ref.shape[-1])))
    say(f"    max rel err {err:.3e} over {b * hkv * n * G_} vectors")
    assert err <= ATTN_TOL[cfg.dtype]


@pytest.mark.parametrize("name", list(LONG_SPLIT_CASES))
def test_verify_attention_long_splits_sampled(name):
    cfg = LONG_SPLIT_CASES[name]
    w = W.make_workload(cfg, 23)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                          cfg.num_steps, cfg.num_draft_tokens)
    b, n = cfg.batch, cfg.num_draft_tokens
    say(f"[attention long splits] {name} b={b} L={w.seq_lens.tolist()}")
    words = oracle.pack_mask(t["mask"], oracle.MASK_QLEN_BITS)
    got, st = G.verify_attention(w, words)
    assert st == 0
    rng = np.random.default_rng(5)
    rows = [(int(rng.integers(0, b * n)), int(rng.integers(0, cfg.num_q_heads))) for _ in range(48)]
    rows += [(b * n - 1, cfg.num_q_heads - 1), (0, 0), (n - 1, 0), (b * n - n, cfg.num_q_heads - 1)]
    ref = oracle.verify_attention(w.q, w.k_pool[0], w.v_pool[0], w.page_table, w.seq_lens,
                                  w.out_cache_loc, t["mask"], cfg.num_q_heads, cfg.num_kv_heads,
                                  cfg.page_size, cfg.dtype, rows=rows)
    err = _attn_err(np.stack([got[r, h] for r, h in rows]), ref)
    say(f"    max rel err {err:.3e} over {len(rows)} sampled vectors")
    assert err <= ATTN_TOL[cfg.dtype]
    assert np.isfinite(got).all()


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_full_tree_and_accept(cid):
    w, t = full(cid, False)
    cfg = w.cfg
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    say(f"[full tree+accept] cfg{cid} b={b} n={n} V={cfg.vocab}")
    g = G.build_tree(w)
    np.testing.assert_array_equal(g["draft_tokens"], t["draft_tokens"])
    np.testing.assert_array_equal(g["tree_mask"], oracle.pack_mask(t["mask"], oracle.MASK_QLEN_BITS))
    np.testing.assert_array_equal(g["retrieve_next_token"].reshape(b, n), t["retrieve_next_token"])
    np.testing.assert_array_equal(g["retrieve_next_sibling"].reshape(b, n), t["retrieve_next_sibling"])
    tl, dl = W.verify_logits(w, t["selected"])
    tree = _tree_for_gpu(t, b, n)
    if "greedy" in cfg.accept:
        o = oracle.accept_greedy(tl, t["draft_tokens"], t["retrieve_index"], t["retrieve_next_token"],
                                 t["retrieve_next_sibling"], b, n, s1, cfg.dtype)
        gg = G.accept_greedy(w, tl, tree)
        np.testing.assert_array_equal(gg["target_predict"], o["target_predict"])
        assert _compare_accept(gg, o, b, n) == []
        say(f"    greedy accept lengths {o['accept_length'].tolist()[:16]}")
    if "sample" in cfg.accept:
        o = oracle.accept_sample(tl, dl, w.temperature, w.uniforms, w.final_uniforms,
                                 t["draft_tokens"], t["retrieve_index"], t["retrieve_next_token"],
                                 t["retrieve_next_sibling"], b, n, s1, cfg.dtype)
        gs = G.accept_sample(w, tl, dl, tree)
        assert (gs["status"] & ~S.SPEC_ST_ZERO_RESIDUAL) == 0
        assert_only_ratio_band(o, f"cfg{cid}")
        bad = _compare_accept(gs, o, b, n, o["exempt"])
        say(f"    sample exempt {int(o['exempt'].sum())}/{b} mismatched {bad} "
            f"lengths {o['accept_length'].tolist()[:16]}")
        assert bad == []


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_full_attention_vector_complete(cid):
    """Every output vector of the full-size workload against the oracle, one
    (request, KV head) unit at a time: every tree node times every query
    head of the group, over the whole history (131072 keys at config 5)."""
    w, t = full(cid, True)
    cfg = w.cfg
    b, n, hq, hkv = cfg.batch, cfg.num_draft_tokens, cfg.num_q_heads, cfg.num_kv_heads
    G_ = hq // hkv
    units = [(r, g) for r in range(b) for g in range(hkv)]
    say(f"[full attention] cfg{cid} b={b} n={n} L={w.seq_lens.tolist()[:8]} "
        f"units {len(units)}")
    words = oracle.pack_mask(t["mask"], oracle.MASK_QLEN_BITS)
    got, st = G.verify_attention(w, words)
    assert st == 0
    assert np.isfinite(got).all()
    err = 0.0
    for r, g in units:
        ref = oracle.verify_attention_unit(w.q, w.k_pool[0], w.v_pool[0], w.page_table,
                                           w.seq_lens, w.out_cache_loc, t["mask"], hq, hkv,
                                           cfg.page_size, cfg.dtype, r, g)
        mine = got[r * n:(r + 1) * n, g * G_:(g + 1) * G_]
        err = max(err, _attn_err(mine.reshape(-1, mine.shape[-1]), ref.reshape(-1, ref.shape[-1])))
        if g == hkv - 1 and (b <= 8 or r % 8 == 7):
            say(f"    request {r} done, max rel err so far {err:.3e}")
    say(f"    max rel err {err:.3e} over {len(units) * n * G_} vectors")
    assert err <= ATTN_TOL[cfg.dtype]


@pytest.mark.parametrize("name,cfg", [
    ("lds_load_form", DMA_CASES["b3_L8195"]),
    ("lds_load_form_kh2_ps1", W.shrink(W.CONFIGS[2], batch=3, hist=("fixed", 700), vocab=1000)),
    # a page size that is not a power of two keeps the register-staged form
    ("register_staged", W.shrink(W.CONFIGS[3], batch=3, hist=("fixed", 2000), vocab=1000,
                                 page_size=12)),
])
def test_verify_attention_bad_slots(name, cfg):
    """Page ids and tree slots out of range in requests 1 and 2: the call
    raises SPEC_ST_RANGE, every kernel ends, and request 0 (untouched) is
    still exact."""
    w = W.make_workload(cfg, 31)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                          cfg.num_steps, cfg.num_draft_tokens)
    b, n, hq, hkv = cfg.batch, cfg.num_draft_tokens, cfg.num_q_heads, cfg.num_kv_heads
    say(f"[attention, bad slots] {name} b={b} L={w.seq_lens.tolist()}")
    nslots = w.k_pool.shape[1]
    w.page_table[1, 5] = -1
    w.page_table[2, 10] = nslots // cfg.page_size + 100
    w.out_cache_loc[2 * n + 3] = nslots + 7
    words = oracle.pack_mask(t["mask"], oracle.MASK_QLEN_BITS)
    got, st = G.verify_attention(w, words)
    say(f"    status {st}")
    assert st & S.SPEC_ST_RANGE
    G_ = hq // hkv
    err = 0.0
    for g in range(hkv):
        ref = oracle.verify_attention_unit(w.q, w.k_pool[0], w.v_pool[0], w.page_table,
                                           w.seq_lens, w.out_cache_loc, t["mask"], hq, hkv,
                                           cfg.page_size, cfg.dtype, 0, g)
        mine = got[0:n, g * G_:(g + 1) * G_]
        err = max(err, _attn_err(mine.reshape(-1, mine.shape[-1]), ref.reshape(-1, ref.shape[-1])))
    say(f"    request 0: max rel err {err:.3e}")
    assert err <= ATTN_TOL[cfg.dtype]
