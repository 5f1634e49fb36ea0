"""FULL mask and paged draft-branch planning on the GPU against the oracle.

FULL mask: trees of the seeded workloads (the oracle's tree build), the
prefix filled and not filled (over a buffer of 0xA5 bytes), lengths from 0
to 131072 (the 4 x 131072 workload's 33.6 MB mask, compared whole), and a
length above max_seq_len (status bit, nothing written outside the buffer).
Branch planning: page sizes 1, 4 and 16, topk 1, 3 and 8, aligned and
unaligned prefixes, two layers of bf16 and f32 pools, and a page id out of
range.  Bar: bit-exact (byte and index work).
"""
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


H8 = ("fixed", 8)
MASK_CASES = {
    "c1": W.CONFIGS[1],
    "c3_b5": W.shrink(W.CONFIGS[3], batch=5, vocab=500),
    "c2_n64": W.shrink(W.CONFIGS[2], vocab=500),
    "chain_b64": W.shrink(W.CONFIGS[4], vocab=500),
    "c5_full_len": W.shrink(W.CONFIGS[5], vocab=500),
}


def _tree(cfg, seed, lens=None):
    w = W.make_workload(cfg, seed, attention=False)
    L = w.seq_lens if lens is None else np.asarray(lens, np.int64)
    t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, L, cfg.topk, cfg.num_steps,
                          cfg.num_draft_tokens)
    return w, L, t["mask"]


def _run_full(cfg, L, mask, fill, max_len=None, nbytes=None):
    b, n = cfg.batch, cfg.num_draft_tokens
    words = oracle.pack_mask(mask, oracle.MASK_QLEN_BITS)
    total = int(n * (np.sum(L) + n * b))
    size = total if nbytes is None else nbytes
    out = torch.full((max(16, size),), 0xA5, dtype=torch.uint8, device="cuda")
    st = G.status()
    S.spec_full_mask(b, n, G.dev(np.asarray(L, np.int32)), int(np.max(L)) if max_len is None
                     else max_len, G.dev(words), fill, out[:size] if size else out[:16], dev_status=st)
    torch.cuda.synchronize()
    return G.host(out), int(G.host(st)[0]), total


@pytest.mark.parametrize("name", list(MASK_CASES))
@pytest.mark.parametrize("fill", [True, False])
def test_full_mask(name, fill):
    cfg = MASK_CASES[name]
    w, L, mask = _tree(cfg, 61)
    say(f"[full mask] {name} b={cfg.batch} n={cfg.num_draft_tokens} sum L={int(np.sum(L))} fill={fill}")
    got, st, total = _run_full(cfg, L, mask, fill)
    want = oracle.full_mask(L, mask, fill_prefix=fill,
                            prior=np.full(total, 0xA5, np.uint8))
    assert st == 0
    assert np.array_equal(got[:total], want)
    assert np.all(got[total:] == 0xA5)


def test_full_mask_zero_and_ragged_lengths():
    cfg = W.shrink(W.CONFIGS[3], batch=6, vocab=500)
    lens = [0, 1, 15, 16, 17, 4099]
    w, L, mask = _tree(cfg, 62, lens)
    got, st, total = _run_full(cfg, L, mask, True)
    assert st == 0
    assert np.array_equal(got[:total], oracle.full_mask(L, mask))


def test_full_mask_length_beyond_max_raises_and_stays_inside():
    cfg = W.shrink(W.CONFIGS[3], batch=3, vocab=500)
    lens = [10, 5000, 7]
    w, L, mask = _tree(cfg, 63, lens)
    total = int(cfg.num_draft_tokens * (np.sum(L) + cfg.num_draft_tokens * 3))
    got, st, _ = _run_full(cfg, L, mask, True, max_len=100, nbytes=total)
    assert st & oracle.ST_RANGE
    # request 0 is whole; nothing was written past the buffer
    n = cfg.num_draft_tokens
    want = oracle.full_mask(L, mask)
    assert np.array_equal(got[:n * (10 + n)], want[:n * (10 + n)])
    assert np.all(got[total:] == 0xA5)


PLAN_CASES = [  # (page_size, topk, num_steps, layers, dtype, aligned)
    (16, 8, 6, 2, "bf16", False),
    (4, 3, 5, 2, "bf16", False),
    (16, 4, 4, 1, "bf16", True),
    (1, 4, 5, 2, "bf16", False),
    (16, 1, 4, 2, "bf16", False),
    (8, 2, 7, 2, "f32", False),
]


def _plan_inputs(ps, topk, steps, layers, dtype, aligned, seed, b=5, hkv=2, d=64):
    rng = np.random.default_rng(seed)
    L = rng.integers(1, 6 * ps + 5, size=b)
    if aligned:
        L = (L // ps + 1) * ps
    maxp = (int(L.max()) + steps) // ps + 2
    per_branch = (ps - 1 + steps + ps - 1) // ps
    num_pages = b * maxp + b * topk * per_branch + 7
    perm = rng.permutation(num_pages)
    pt = perm[:b * maxp].reshape(b, maxp).astype(np.int32)
    bp = perm[b * maxp:b * maxp + b * topk * per_branch].reshape(b, topk, per_branch).astype(np.int32)
    shape = (layers, num_pages * ps, hkv, d)
    if dtype == "bf16":
        k = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
        v = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    else:
        k = rng.standard_normal(shape).astype(np.float32)
        v = rng.standard_normal(shape).astype(np.float32)
    return L, pt, bp, per_branch, num_pages, k, v


def _plan_gpu(L, pt, bp, per_branch, num_pages, k, v, ps, topk, steps, dtype):
    b = L.size
    layers, slots, hkv, d = k.shape
    kd, vd = G.dev(k), G.dev(v)
    ocl = torch.full((b * topk * steps,), -7, dtype=torch.int32, device="cuda")
    st = G.status()
    S.spec_plan_draft_branches(b, topk, steps, ps, layers, hkv, d,
                               S.SPEC_BF16 if dtype == "bf16" else S.SPEC_F32, kd, vd, slots,
                               G.dev(L.astype(np.int32)), G.dev(pt), pt.shape[1],
                               G.dev(bp) if topk > 1 else None, per_branch, ocl, dev_status=st)
    torch.cuda.synchronize()
    return (G.host(ocl).reshape(b, topk, steps), G.host(kd, k.dtype), G.host(vd, v.dtype),
            int(G.host(st)[0]))


@pytest.mark.parametrize("case", PLAN_CASES, ids=[f"ps{c[0]}_k{c[1]}_s{c[2]}_{c[4]}{'_al' if c[5] else ''}"
                                                  for c in PLAN_CASES])
def test_plan_draft_branches(case):
    ps, topk, steps, layers, dtype, aligned = case
    L, pt, bp, per_branch, num_pages, k, v = _plan_inputs(*case, seed=70 + ps + topk)
    say(f"[plan branches] ps={ps} topk={topk} steps={steps} L={L.tolist()}")
    ocl, k2, v2, st = _plan_gpu(L, pt, bp, per_branch, num_pages, k, v, ps, topk, steps, dtype)
    o = oracle.plan_draft_branches(L, pt, bp, topk, steps, ps, num_pages)
    kw, vw = oracle.duplicate_prefix_tail(k, v, o["copies"])
    assert st == o["status"] == 0
    assert np.array_equal(ocl, o["out_cache_loc"])
    assert np.array_equal(k2, kw) and np.array_equal(v2, vw)


def test_plan_draft_branches_bad_page():
    case = (4, 3, 5, 1, "bf16", False)
    L, pt, bp, per_branch, num_pages, k, v = _plan_inputs(*case, seed=90)
    bp[1, 2, 0] = num_pages + 3
    ocl, k2, v2, st = _plan_gpu(L, pt, bp, per_branch, num_pages, k, v, 4, 3, 5, "bf16")
    o = oracle.plan_draft_branches(L, pt, bp, 3, 5, 4, num_pages)
    kw, vw = oracle.duplicate_prefix_tail(k, v, o["copies"])
    assert st & oracle.ST_RANGE and o["status"] & oracle.ST_RANGE
    assert np.array_equal(ocl, o["out_cache_loc"])
    assert np.array_equal(k2, kw) and np.array_equal(v2, vw)
