"""Seeded synthetic inputs for the tree speculative-decoding hot path.

This module produces inputs only.  It holds none of the arithmetic of the
path's four steps (tree build, verify attention, accept, compaction): both the
CPU oracle and the HIP path consume what it produces, and it imports neither.

What it does compute is the *draft side* that sits before the path: a
simulation of the EAGLE draft loop that emits the per-step score / token /
parent lists, written from the description of ``select_top_k_tokens`` in
"SGLang 源码完全拆解(十一):投机解码" (section "organize_draft_results:三张表的归约").
Step 0 takes the top-k of the root's draft distribution; every later step
multiplies each branch's path score by its children's draft probabilities,
keeps the top-k of the topk*topk products, and records the kept entries'
flat positions shifted into the global candidate space.

Every random draw comes from ``numpy.random.Generator(PCG64)`` streams spawned
from ``SeedSequence(seed)`` in a fixed order, so each (config, seed) pair
reproduces the same bytes.  bf16 tensors are carried as uint16 bit patterns
(round-to-nearest-even of float32 draws).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# ---------------------------------------------------------------------------
# Workload shapes.  Sizes follow the five published workload descriptions:
# a tiny CPU-checkable case, a Llama-3-8B-shaped single request, a sampled
# mid-size batch, a large-batch chain, and a 70B-shaped long-context tree.
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    batch: int
    topk: int
    num_steps: int
    num_draft_tokens: int
    vocab: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str               # "f32" or "bf16": attention inputs and logits
    page_size: int
    hist_len: tuple          # ("fixed", L) or ("uniform", lo, hi)
    target_sigma: float      # target logits ~ N(0, target_sigma) (bf16 configs)
    draft_noise: float       # draft = target + N(0, draft_noise)
    temperature: float
    accept: tuple            # subset of ("greedy", "sample")
    compaction: bool
    num_layers: int = 1

    @property
    def ncand(self) -> int:
        return self.topk + (self.num_steps - 1) * self.topk * self.topk

    @property
    def npar(self) -> int:
        return 1 + (self.num_steps - 1) * self.topk

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


CONFIGS = {
    1: Config("tiny_b2_topk2_s3_n6_v32", 2, 2, 3, 6, 32, 2, 1, 64, "f32", 1,
              ("fixed", 64), 0.0, 0.5, 1.0, ("greedy", "sample"), True),
    2: Config("llama3_8b_b1_topk8_s5_n64_L4096", 1, 8, 5, 64, 128256, 32, 8, 128,
              "bf16", 1, ("fixed", 4096), 2.0, 1.0, 1.0, ("greedy",), False),
    3: Config("midbatch_b16_topk4_s4_n32_Lu1024_8192", 16, 4, 4, 32, 128256, 32, 8,
              128, "bf16", 16, ("uniform", 1024, 8192), 2.0, 1.0, 1.0, ("sample",),
              False),
    4: Config("chain_b64_topk1_s4_n5_L2048", 64, 1, 4, 5, 152064, 28, 4, 128, "bf16",
              16, ("fixed", 2048), 2.0, 1.5, 0.7, ("sample",), False),
    5: Config("llama70b_b4_topk8_s6_n64_L131072", 4, 8, 6, 64, 128256, 64, 8, 128,
              "bf16", 16, ("fixed", 131072), 2.0, 1.0, 1.0, ("greedy", "sample"),
              True),
}


def shrink(cfg: Config, *, batch=None, hist=None, vocab=None, **kw) -> Config:
    """A smaller copy of ``cfg`` with the same tree and head shapes."""
    upd = dict(kw)
    if batch is not None:
        upd["batch"] = batch
    if hist is not None:
        upd["hist_len"] = hist
    if vocab is not None:
        upd["vocab"] = vocab
    return dataclasses.replace(cfg, name=cfg.name + "_small", **upd)


# ---------------------------------------------------------------------------
# Encodings
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        v = flat_u[s:s + step].astype(np.uint64)
        v = (v + 0x7FFF + ((v >> 16) & 1)) >> 16
        flat_o[s:s + step] = v.astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def uniforms_from_u32(u32: np.ndarray) -> np.ndarray:
    """Exact float32 uniforms in [0, 1): the top 24 bits of a uint32 draw."""
    return ((u32 >> np.uint32(8)).astype(np.float64) * 2.0 ** -24).astype(np.float32)


# ---------------------------------------------------------------------------
# Draft-side helpers (input production only)
# ---------------------------------------------------------------------------

def _softmax_f32(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32)
    e = np.exp(x - x.max(axis=-1, keepdims=True), dtype=np.float32)
    return (e / e.sum(axis=-1, keepdims=True, dtype=np.float32)).astype(np.float32)


def _topk_desc(values: np.ndarray, k: int):
    """Indices of the k largest entries of a 1-D array, descending, lower
    index first among equal values.  Returns (values, indices)."""
    k = min(k, values.size)
    if values.size > 4 * k + 64:
        part = np.argpartition(-values, k - 1)[:k]
        thr = values[part].min()
        cand = np.nonzero(values >= thr)[0]
    else:
        cand = np.arange(values.size)
    order = np.lexsort((cand, -values[cand].astype(np.float64)))
    idx = cand[order[:k]]
    return values[idx], idx


@dataclasses.dataclass
class Workload:
    cfg: Config
    seed: int
    # tree-build inputs
    scores: np.ndarray        # [b, ncand] f32
    tokens: np.ndarray        # [b, ncand] i32
    parents: np.ndarray       # [b, npar] i32  (entry 0 is the -1 root sentinel)
    bonus: np.ndarray         # [b] i32
    seq_lens: np.ndarray      # [b] i32  history length before the tree
    truth_parent: np.ndarray  # [b, ncand] i64 flat index of each candidate's parent, -1 = root
    local_prob: np.ndarray    # [b, ncand] f32 the candidate's own draft probability
    ctx_of_flat: np.ndarray   # [b, ncand] i32 context row expanded from flat f, -1 if none
    ctx_target: np.ndarray    # [b, npar, V] logits (f32 or bf16 bits) of each draft context
    ctx_draft: np.ndarray     # [b, npar, V]
    # attention inputs
    q: np.ndarray             # [b*n, hq, d]  (f32 or bf16 bits)
    k_pool: np.ndarray        # [layers, slots, hkv, d]
    v_pool: np.ndarray        # [layers, slots, hkv, d]
    page_table: np.ndarray    # [b, max_pages] i32, unused entries -1
    out_cache_loc: np.ndarray  # [b*n] i32 slot of tree node k of request b
    # accept inputs
    temperature: np.ndarray   # [b] f32
    uniforms: np.ndarray      # [b, n] f32
    final_uniforms: np.ndarray  # [b] f32

    @property
    def num_slots(self) -> int:
        """Physical slots the page table addresses (the pool's row count)."""
        return (int(self.page_table.max()) + 1) * self.cfg.page_size

    def slot(self, b: int, pos: int) -> int:
        ps = self.cfg.page_size
        return int(self.page_table[b, pos // ps]) * ps + pos % ps


def _hist_lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    kind = cfg.hist_len[0]
    if kind == "fixed":
        return np.full(cfg.batch, cfg.hist_len[1], dtype=np.int32)
    if kind == "list":                     # explicit per-request lengths
        lens = np.asarray(cfg.hist_len[1], dtype=np.int32)
        assert lens.shape == (cfg.batch,)
        return lens.copy()
    lo, hi = cfg.hist_len[1], cfg.hist_len[2]
    return rng.integers(lo, hi + 1, size=cfg.batch).astype(np.int32)


def _logit_pair(cfg: Config, rng: np.random.Generator, rows: int):
    """(target, draft) logits of ``rows`` contexts, encoded per cfg.dtype."""
    V = cfg.vocab
    if cfg.dtype == "f32":
        draft = rng.standard_normal((rows, V), dtype=np.float32)
        target = (draft + np.float32(cfg.draft_noise) *
                  rng.standard_normal((rows, V), dtype=np.float32)).astype(np.float32)
        return target, draft
    target = np.float32(cfg.target_sigma) * rng.standard_normal((rows, V), dtype=np.float32)
    draft = target + np.float32(cfg.draft_noise) * rng.standard_normal((rows, V), dtype=np.float32)
    return f32_to_bf16_bits(target), f32_to_bf16_bits(draft)


def decode(cfg: Config, x: np.ndarray) -> np.ndarray:
    """Stored values as float32 (bf16 bits widened, f32 returned as is)."""
    return bf16_bits_to_f32(x) if cfg.dtype == "bf16" else np.asarray(x, dtype=np.float32)


def make_workload(cfg: Config, seed: int, *, attention=True, contiguous_pages=False,
                  num_layers=None) -> Workload:
    """Build every input of one iteration of the path for ``cfg``."""
    ss = np.random.SeedSequence(seed)
    (s_len, s_page, s_ctx, s_tok, s_q, s_k, s_v, s_unif) = [
        np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(8)]
    b, topk, S, n, V = cfg.batch, cfg.topk, cfg.num_steps, cfg.num_draft_tokens, cfg.vocab
    ncand, npar = cfg.ncand, cfg.npar
    layers = cfg.num_layers if num_layers is None else num_layers

    seq_lens = _hist_lengths(cfg, s_len)
    bonus = s_tok.integers(0, V, size=b).astype(np.int32)

    # ---- draft loop simulation -------------------------------------------
    scores = np.zeros((b, ncand), np.float32)
    tokens = np.zeros((b, ncand), np.int32)
    parents = np.full((b, npar), -1, np.int32)
    truth_parent = np.full((b, ncand), -1, np.int64)
    local_prob = np.zeros((b, ncand), np.float32)
    ctx_of_flat = np.full((b, ncand), -1, np.int32)
    tdtype = np.float32 if cfg.dtype == "f32" else np.uint16
    ctx_target = np.zeros((b, npar, V), tdtype)
    ctx_draft = np.zeros((b, npar, V), tdtype)
    for r in range(b):
        t_all, d_all = _logit_pair(cfg, s_ctx, npar)
        ctx_target[r], ctx_draft[r] = t_all, d_all
        dprob = _softmax_f32(decode(cfg, d_all))          # [npar, V]
        # step 0: the root context (row 0) spreads into topk children
        p0, i0 = _topk_desc(dprob[0], topk)
        scores[r, :topk] = p0
        tokens[r, :topk] = i0
        local_prob[r, :topk] = p0
        truth_parent[r, :topk] = -1
        parents[r, 0] = -1
        if S > 1:
            parents[r, 1:1 + topk] = np.arange(topk)
        branch_flat = np.arange(topk)                       # flat ids of the live branches
        branch_score = p0.astype(np.float32)
        for i in range(1, S):
            base = topk + (i - 1) * topk * topk
            exp_scores = np.zeros((topk, topk), np.float32)
            for j in range(topk):
                row = 1 + (i - 1) * topk + j                  # context row of branch j
                ctx_of_flat[r, branch_flat[j]] = row
                pj, ij = _topk_desc(dprob[row], topk)
                exp_scores[j] = branch_score[j] * pj          # fp32 path products
                f0 = base + j * topk
                tokens[r, f0:f0 + topk] = ij
                local_prob[r, f0:f0 + topk] = pj
                truth_parent[r, f0:f0 + topk] = branch_flat[j]
            scores[r, base:base + topk * topk] = exp_scores.reshape(-1)
            cs_p, cs_i = _topk_desc(exp_scores.reshape(-1), topk)
            if i < S - 1:
                parents[r, 1 + i * topk:1 + (i + 1) * topk] = cs_i + base
            branch_flat = cs_i + base
            branch_score = cs_p.astype(np.float32)

    # ---- attention inputs --------------------------------------------------
    hq, hkv, d, ps = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size
    pages_per = [(int(seq_lens[r]) + n + ps - 1) // ps for r in range(b)]
    total_pages = int(sum(pages_per))
    max_pages = max(pages_per)
    perm = np.arange(total_pages) if contiguous_pages else s_page.permutation(total_pages)
    page_table = np.full((b, max_pages), -1, np.int32)
    off = 0
    for r in range(b):
        page_table[r, :pages_per[r]] = perm[off:off + pages_per[r]]
        off += pages_per[r]
    num_slots = total_pages * ps
    out_cache_loc = np.zeros(b * n, np.int32)
    for r in range(b):
        for k in range(n):
            pos = int(seq_lens[r]) + k
            out_cache_loc[r * n + k] = page_table[r, pos // ps] * ps + pos % ps

    def normal(rng, shape):
        x = np.empty(shape, np.float32)
        flat = x.reshape(-1)
        step = 1 << 26
        for s in range(0, flat.size, step):
            flat[s:s + step] = rng.standard_normal(min(step, flat.size - s), dtype=np.float32)
        return x if cfg.dtype == "f32" else f32_to_bf16_bits(x)

    if attention:
        q = normal(s_q, (b * n, hq, d))
        k_pool = normal(s_k, (layers, num_slots, hkv, d))
        v_pool = normal(s_v, (layers, num_slots, hkv, d))
    else:
        q = np.zeros((0,), tdtype)
        k_pool = np.zeros((layers, 0, hkv, d), tdtype)
        v_pool = np.zeros((layers, 0, hkv, d), tdtype)

    temperature = np.full(b, cfg.temperature, np.float32)
    u32 = s_unif.integers(0, 2 ** 32, size=(b, n + 1), dtype=np.uint64).astype(np.uint32)
    unif = uniforms_from_u32(u32)
    return Workload(cfg, seed, scores, tokens, parents, bonus, seq_lens, truth_parent,
                    local_prob, ctx_of_flat, ctx_target, ctx_draft, q, k_pool, v_pool,
                    page_table, out_cache_loc, temperature,
                    np.ascontiguousarray(unif[:, :n]), np.ascontiguousarray(unif[:, n]))


def verify_logits(w: Workload, selected: np.ndarray):
    """Assemble the verify rows' (target, draft) logits [b*n, V] for a tree.

    ``selected[b, k-1]`` is the flat candidate index of tree node k (node 0 is
    the root).  Node k's row carries the logits of the context that ends in
    node k: the draft context the simulation expanded from that candidate, or
    a fresh pair (seeded per request and candidate) when the draft loop never
    expanded it.  The root row uses the root context.
    """
    cfg = w.cfg
    b, n, V = cfg.batch, cfg.num_draft_tokens, cfg.vocab
    tdtype = np.float32 if cfg.dtype == "f32" else np.uint16
    tgt = np.zeros((b * n, V), tdtype)
    dft = np.zeros((b * n, V), tdtype)
    for r in range(b):
        tgt[r * n], dft[r * n] = w.ctx_target[r, 0], w.ctx_draft[r, 0]
        for k in range(1, n):
            f = int(selected[r, k - 1])
            row = int(w.ctx_of_flat[r, f]) if 0 <= f < cfg.ncand else -1
            if row >= 0:
                tgt[r * n + k], dft[r * n + k] = w.ctx_target[r, row], w.ctx_draft[r, row]
            else:
                rng = np.random.Generator(np.random.PCG64(
                    np.random.SeedSequence([w.seed, 77, r, f])))
                t1, d1 = _logit_pair(cfg, rng, 1)
                tgt[r * n + k], dft[r * n + k] = t1[0], d1[0]
    return tgt, dft


def attention_bytes(cfg: Config, seq_lens: np.ndarray) -> int:
    """Algorithmic HBM bytes of one verify-attention call: every history and
    tree K/V row of each KV head once, Q in and O out once, the page-table
    entries, tree slots and mask words."""
    eb = 4 if cfg.dtype == "f32" else 2
    n, hq, hkv, d, ps = (cfg.num_draft_tokens, cfg.num_q_heads, cfg.num_kv_heads,
                         cfg.head_dim, cfg.page_size)
    mask_word = max(1, (8 << max(0, math.ceil(math.log2(max(1, (n + 7) // 8))))) // 8)
    total = 0
    for L in seq_lens.tolist():
        total += (L + n) * hkv * d * 2 * eb + 2 * n * hq * d * eb
        total += ((L + ps - 1) // ps) * 4 + n * (4 + mask_word)
    return int(total)


def attention_flops(cfg: Config, seq_lens: np.ndarray, depth: np.ndarray) -> int:
    """QK^T and PV multiply-adds (2 flops each) over the visible keys."""
    n, hq, d = cfg.num_draft_tokens, cfg.num_q_heads, cfg.head_dim
    total = 0
    for r, L in enumerate(seq_lens.tolist()):
        total += 4 * n * hq * d * L + 4 * hq * d * int((depth[r] + 1).sum())
    return int(total)
