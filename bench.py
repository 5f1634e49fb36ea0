"""Benchmark of the tree speculative-decoding hot path on one MI355X.

One step = one pass of every operation of the path over one batch of
synthetic input: tree build -> verify attention -> greedy accept -> sampled
accept -> accepted-KV compaction, all through the C-ABI library.  The
default workload is the largest one that fits one GPU: the long-context tree
at a 70B attention shape (batch 4, topk 8, 6 steps, 64 draft tokens, 64 query
/ 8 KV heads, head dim 128, bf16 paged KV with page size 16, 131072 cached
tokens per request, vocab 128256); ``--config`` picks another.

Inputs are resident in HBM before timing starts.  Several copies of them are
rotated through the steps and through each operation's own timing, so that
every HBM-bound operation (verify attention, the greedy vocabulary sweep)
reads at least twice the 256 MB last-level cache between two reads of the
same bytes.

Timing.  ``--mode graph`` (default) captures each copy's step once into a
HIP graph and times K replays, so the GPU runs the step's kernels back to
back as a serving loop would; ``--mode eager`` times K steps launched from
Python.  Either way the line also carries the eager step time and, per
operation, the GPU time of that operation alone: a graph holding the
operation for every copy, replayed between two HIP events on the stream the
kernels run on.

Five operations are timed the same way as extra operations
(``extra_op_ms``), not part of the step: the target-only tree accept (the
sibling-mass rule with thresholds 1, 1), the draft loop's selection (one
draft-step call per draft step over the workload's draft logits, the path
scores chained from call to call), the top-k / top-p pre-pass over the
verify logits (top_k 50, top_p 0.9), the FULL tree mask with its prefix
filled, and the paged draft-branch planning (prefix-tail duplication into
the branches' pages of a one-layer draft KV pool, draft write slots).

Prints one JSON line (rank 0).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

import workloads as W

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
MALL_BYTES = 256 << 20         # last-level cache (Infinity Cache) of the part
MAX_COPIES = 64
MAX_ROTATION_BYTES = 64 << 30  # device memory the input copies may take


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=5, choices=sorted(W.CONFIGS))
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured copy / GEMM peaks (profiler runs: keeps their "
                         "kernels out of traces and counter calibration)")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph",
                    help="graph: each input copy's step is captured once into a HIP graph and "
                         "the timed steps replay the graphs (no host launch cost between "
                         "kernels); eager: every step is launched from Python")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="before warm-up, run a plain device copy of this many MiB three times "
                         "(the reference kernel for scaling HBM byte counters)")
    return ap.parse_args()


class Inputs:
    """One resident copy of every input of a step, plus its outputs."""

    def __init__(self, torch, S, w, tl, dl):
        cfg = w.cfg
        d = lambda a: _dev(torch, a)
        b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
        self.scores, self.tokens, self.parents = d(w.scores), d(w.tokens), d(w.parents)
        self.bonus, self.seq_lens = d(w.bonus), d(w.seq_lens)
        self.q = d(w.q)
        self.k_pool, self.v_pool = d(w.k_pool), d(w.v_pool)
        self.page_table, self.out_cache_loc = d(w.page_table), d(w.out_cache_loc)
        self.tl, self.dl = d(tl), d(dl)
        self.temperature, self.uniforms, self.final_uniforms = (
            d(w.temperature), d(w.uniforms), d(w.final_uniforms))
        i32 = lambda k: torch.zeros(k, dtype=torch.int32, device="cuda")
        self.draft_tokens, self.positions = i32(b * n), i32(b * n)
        self.retrieve_index, self.retrieve_next_token, self.retrieve_next_sibling = (
            i32(b * n), i32(b * n), i32(b * n))
        self.selected = i32(max(1, b * (n - 1)))
        self.tree_mask = torch.zeros(b * n * S.spec_mask_word_bytes(n), dtype=torch.uint8,
                                     device="cuda")
        self.attn_out = torch.empty_like(self.q)
        self.predict, self.accept_index, self.accept_length = i32(b * n), i32(b * s1), i32(b)
        self.target_predict = i32(b * n)
        self.spredict, self.saccept_index, self.saccept_length = i32(b * n), i32(b * s1), i32(b)
        self.tpredict, self.taccept_index, self.taccept_length = i32(b * n), i32(b * s1), i32(b)
        self.new_seq_lens, self.free_slots, self.num_free = i32(b), i32(b * n), i32(b)
        self.status = i32(1)
        # the draft loop: each step's branch rows of draft logits, contiguous
        k = cfg.topk
        self.dsteps = [d(w.ctx_draft[:, 0:1] if i == 0 else w.ctx_draft[:, 1 + (i - 1) * k:1 + i * k])
                       for i in range(cfg.num_steps)]
        self.dscores = torch.zeros(b * cfg.ncand, dtype=torch.float32, device="cuda")
        self.dtokens, self.dparents = i32(b * cfg.ncand), i32(b * cfg.npar)
        self.dnext_scores = torch.zeros(b * k, dtype=torch.float32, device="cuda")
        self.dnext_tokens = i32(b * k)

    def clone(self, torch):
        other = object.__new__(Inputs)
        for k, v in self.__dict__.items():
            other.__dict__[k] = [t.clone() for t in v] if isinstance(v, list) else v.clone()
        return other

    def nbytes(self):
        return sum(sum(t.numel() * t.element_size() for t in v) if isinstance(v, list)
                   else v.numel() * v.element_size() for v in self.__dict__.values())


def _dev(torch, a):
    a = np.ascontiguousarray(a)
    view = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32,
            np.dtype(np.uint64): np.int64}.get(a.dtype)
    if view is not None:
        a = a.view(view)
    return torch.from_numpy(a).to("cuda")


def op_calls(S, cfg, x, ws_attn, ws_greedy, ws_sample, ws_target=None, ws_draft=None, mem=None):
    """The five operations of one step on input copy ``x``, as callables that
    enqueue their kernels on the current stream, then (timed on their own,
    not part of the step) the target-only accept and the draft loop's
    selection."""
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    code = S.SPEC_BF16 if cfg.dtype == "bf16" else S.SPEC_F32

    def build():
        S.spec_build_tree(b, cfg.topk, cfg.num_steps, n, S.SPEC_MASK_QLEN_BITS, x.scores,
                          x.tokens, x.parents, x.bonus, x.seq_lens, x.draft_tokens, x.positions,
                          x.tree_mask, x.retrieve_index, x.retrieve_next_token,
                          x.retrieve_next_sibling, selected=x.selected, dev_status=x.status)

    def attention():
        S.spec_verify_attention(b, n, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                                cfg.page_size, code, 0.0, x.q, x.k_pool, x.v_pool,
                                x.k_pool.shape[1], x.page_table, x.page_table.shape[1],
                                x.seq_lens, cfg_max_len(cfg), x.out_cache_loc, x.tree_mask,
                                x.attn_out, workspace=ws_attn, dev_status=x.status)

    def greedy():
        S.spec_accept_greedy(b, n, s1, cfg.vocab, code, x.tl, x.draft_tokens, x.retrieve_index,
                             x.retrieve_next_token, x.retrieve_next_sibling, x.predict,
                             x.accept_index, x.accept_length, target_predict=x.target_predict,
                             workspace=ws_greedy, dev_status=x.status)

    def sample():
        S.spec_accept_sample(b, n, s1, cfg.vocab, code, x.tl, x.dl, x.temperature, x.uniforms,
                             x.final_uniforms, x.draft_tokens, x.retrieve_index,
                             x.retrieve_next_token, x.retrieve_next_sibling, x.spredict,
                             x.saccept_index, x.saccept_length, workspace=ws_sample,
                             dev_status=x.status)

    def compact():
        ai, al = ((x.accept_index, x.accept_length) if "greedy" in cfg.accept
                  else (x.saccept_index, x.saccept_length))
        S.spec_compact_kv(b, n, s1, x.k_pool.shape[0], cfg.num_kv_heads, cfg.head_dim,
                          cfg.page_size, code, x.k_pool, x.v_pool, x.k_pool.shape[1],
                          x.page_table, x.page_table.shape[1], x.seq_lens, x.out_cache_loc, ai,
                          al, x.new_seq_lens, x.free_slots, x.num_free, dev_status=x.status)

    def target_only():
        S.spec_accept_target_only(b, n, s1, cfg.vocab, code, x.tl, x.temperature, 1.0, 1.0,
                                  x.uniforms, x.final_uniforms, x.draft_tokens, x.retrieve_index,
                                  x.retrieve_next_token, x.retrieve_next_sibling, x.tpredict,
                                  x.taccept_index, x.taccept_length, workspace=ws_target,
                                  dev_status=x.status)

    def draft_steps():
        for i in range(cfg.num_steps):
            S.spec_draft_step(b, cfg.topk, cfg.num_steps, i, cfg.vocab, code, x.dsteps[i],
                              None if i == 0 else x.dnext_scores, x.dscores, x.dtokens,
                              x.dparents, x.dnext_scores, x.dnext_tokens, workspace=ws_draft,
                              dev_status=x.status)

    def sampling_filter():
        S.spec_sampling_filter(b, n, cfg.vocab, code, x.tl, x.temperature, mem["top_k"],
                               mem["top_p"], mem["filtered"], workspace=mem["filter_ws"],
                               dev_status=x.status)

    def full_mask():
        S.spec_full_mask(b, n, x.seq_lens, cfg_max_len(cfg), x.tree_mask, True, mem["full_mask"],
                         dev_status=x.status)

    def plan_branches():
        S.spec_plan_draft_branches(b, cfg.topk, cfg.num_steps, cfg.page_size, 1, cfg.num_kv_heads,
                                   cfg.head_dim, code, mem["k"], mem["v"], mem["slots"],
                                   x.seq_lens, x.page_table, x.page_table.shape[1],
                                   mem["branch_pages"] if cfg.topk > 1 else None,
                                   mem["per_branch"], mem["draft_loc"], dev_status=x.status)

    return [build, attention, greedy, sample, compact, target_only, draft_steps, sampling_filter,
            full_mask, plan_branches]


def run_ops(S, cfg, x, ws_attn, ws_greedy, ws_sample):
    """Enqueue one step on the current stream."""
    for f in op_calls(S, cfg, x, ws_attn, ws_greedy, ws_sample)[:len(OPS)]:
        f()


_MAXLEN = {}


def memory_side_buffers(torch, S, cfg, w):
    """Buffers the pre-pass, FULL-mask and branch-planning extra operations
    share across input copies: the filtered logits and the pre-pass workspace, the mask output (n * sum(L + n) bytes) and a one-layer draft
    KV pool holding the target's page ids plus, per request and branch, the
    pages of a branch region (ids after the target's)."""
    b, n, ps, k = cfg.batch, cfg.num_draft_tokens, cfg.page_size, cfg.topk
    full_bytes = int(n * (int(w.seq_lens.sum()) + n * b))
    per_branch = (ps - 1 + cfg.num_steps + ps - 1) // ps
    used = int(w.page_table.max()) + 1
    pages = used + b * k * per_branch
    eb = 2 if cfg.dtype == "bf16" else 4
    mem = {
        "full_mask": torch.empty(max(16, full_bytes), dtype=torch.uint8, device="cuda"),
        "full_bytes": full_bytes,
        "k": torch.empty(pages * ps * cfg.num_kv_heads * cfg.head_dim * eb, dtype=torch.uint8, device="cuda"),
        "v": torch.empty(pages * ps * cfg.num_kv_heads * cfg.head_dim * eb, dtype=torch.uint8, device="cuda"),
        "slots": pages * ps,
        "per_branch": per_branch,
        "branch_pages": torch.arange(used, pages, dtype=torch.int32, device="cuda"),
        "draft_loc": torch.zeros(b * k * cfg.num_steps, dtype=torch.int32, device="cuda"),
        "top_k": torch.full((b,), 50, dtype=torch.int32, device="cuda"),
        "top_p": torch.full((b,), 0.9, dtype=torch.float32, device="cuda"),
        "filtered": torch.empty(b * n * cfg.vocab * eb, dtype=torch.uint8, device="cuda"),
        "filter_ws": torch.empty(max(256, S.spec_sampling_filter_workspace_size(b, n, cfg.vocab)),
                                 dtype=torch.uint8, device="cuda"),
    }
    return mem


def cfg_max_len(cfg):
    return _MAXLEN[cfg.name]


OPS = ("build_tree", "verify_attention", "accept_greedy", "accept_sample", "compact_kv")
EXTRA_OPS = ("accept_target_only", "draft_steps", "sampling_filter", "full_mask",
             "plan_draft_branches")


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, w, tl, dl, budget_s):
    """The CPU oracle as it stands, on the same host arrays.

    Tree build, both accepts and compaction run whole, once each, in one
    thread (they are KB- to MB-scale).  Verify attention, the bulk of the
    work, runs on a sample of (row, head) vectors: the (request, KV head)
    units are independent, so a pool of T threads (T = the cores this
    process may use) each takes one unit's sampled vectors, with one BLAS
    thread per worker.  The threaded figure is the median of three runs; a
    one-thread run of one unit's sample is reported beside it.  When the
    sample is not the whole batch, its time is scaled by the vector count.
    """
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    import oracle

    threads = len(os.sched_getaffinity(0))
    b, n, s1 = cfg.batch, cfg.num_draft_tokens, cfg.num_steps + 1
    G, hkv = cfg.group, cfg.num_kv_heads
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        t = oracle.build_tree(w.scores, w.tokens, w.parents, w.bonus, w.seq_lens, cfg.topk,
                              cfg.num_steps, n)
        t_build = time.perf_counter() - t0

        def attn(rows):
            oracle.verify_attention(w.q, w.k_pool[0], w.v_pool[0], w.page_table, w.seq_lens,
                                    w.out_cache_loc, t["mask"], cfg.num_q_heads, hkv,
                                    cfg.page_size, cfg.dtype, rows=rows)

        # units (request, KV head) and their vectors (row, head)
        units = [(r, g) for r in range(b) for g in range(hkv)]
        rng = np.random.default_rng(0)
        rng.shuffle(units)
        unit_vecs = lambda r, g: [(r * n + k, h) for k in range(n)
                                  for h in range(g * G, (g + 1) * G)]
        total_vecs = b * n * cfg.num_q_heads
        # probe: two vectors of one unit, one thread
        r0, g0 = units[0]
        probe = unit_vecs(r0, g0)[:2]
        t0 = time.perf_counter()
        attn(probe)
        per_vec = (time.perf_counter() - t0) / len(probe)
        # each threaded run should take about budget / 6 of wall time
        per_run = budget_s / 6.0
        nunits = min(threads, len(units))
        k = int(max(1, min(n * G, per_run / max(per_vec, 1e-9))))
        whole = per_vec * total_vecs / max(1, min(threads, len(units))) <= per_run
        if whole:
            work = [unit_vecs(r, g) for r, g in units]
        else:
            work = []
            for r, g in units[:nunits]:
                vecs = unit_vecs(r, g)
                pick = np.sort(rng.choice(len(vecs), size=k, replace=False))
                work.append([vecs[i] for i in pick])
        sampled = sum(len(x) for x in work)
        runs = []
        for _ in range(3):
            t0 = time.perf_counter()
            with ThreadPoolExecutor(max_workers=threads) as ex:
                list(ex.map(attn, work))
            runs.append(time.perf_counter() - t0)
        t_attn = float(np.median(runs)) * total_vecs / sampled
        t0 = time.perf_counter()
        attn(work[0])
        t_attn_1 = (time.perf_counter() - t0) * total_vecs / len(work[0])

        t0 = time.perf_counter()
        g = oracle.accept_greedy(tl, t["draft_tokens"], t["retrieve_index"],
                                 t["retrieve_next_token"], t["retrieve_next_sibling"], b, n, s1,
                                 cfg.dtype)
        t_greedy = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.accept_sample(tl, dl, w.temperature, w.uniforms, w.final_uniforms,
                             t["draft_tokens"], t["retrieve_index"], t["retrieve_next_token"],
                             t["retrieve_next_sibling"], b, n, s1, cfg.dtype)
        t_sample = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.compact_kv(w.k_pool, w.v_pool, w.page_table, w.seq_lens, w.out_cache_loc,
                          g["accept_index"], g["accept_length"], b, n, cfg.page_size)
        t_compact = time.perf_counter() - t0
    rest = t_build + t_greedy + t_sample + t_compact
    total = rest + t_attn
    if whole:
        sample = (f"whole step; verify attention over all {total_vecs} (row, head) vectors in "
                  f"{threads} threads (one per (request, KV head) unit at a time), median of 3; "
                  f"tree build, accepts and compaction whole in one thread; float64 numpy")
    else:
        sample = (f"tree build, both accepts and compaction whole in one thread; verify "
                  f"attention on {sampled} of {total_vecs} (row, head) vectors ({k} from each "
                  f"of {len(work)} (request, KV head) units, one unit per thread, {threads} "
                  f"threads), median of 3 runs, scaled by vector count; float64 numpy")
    return {
        "value": b * n / total,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": sample,
        "cpu_model": _cpu_model(),
        "value_1thread": b * n / (rest + t_attn_1),
        "attention_runs_s": runs,
        "op_seconds": {"build_tree": t_build, "verify_attention": t_attn,
                       "verify_attention_1thread": t_attn_1, "accept_greedy": t_greedy,
                       "accept_sample": t_sample, "compact_kv": t_compact},
    }


def _traffic(cfg):
    """HBM bytes per verify-attention call (both launches) from the committed
    counter summary of this workload, or None when there is none or it was
    taken on another version of the kernel source."""
    from rocprof_summary import read_traffic
    root = os.path.dirname(os.path.abspath(__file__))
    return read_traffic(os.path.join(root, "profiles", f"verify_attention_{cfg.name}_hbm.md"),
                        os.path.join(root, "speculative_decoding_build_amd", "csrc",
                                     "verify_attention.hip"))


def measured_peaks(torch):
    """Achievable peaks on this machine, reported beside the nominal ones: a plain
    device copy of 2 GiB (bytes read plus bytes written over its time) and a
    bf16 8192 x 8192 x 8192 matrix product through torch.matmul (the vendor
    BLAS on the matrix cores: 2 * 8192^3 FLOP over its time); best of five
    HIP-event timings each, after one untimed call."""
    def best(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts)
    nbytes = 2 << 30
    src = torch.ones(nbytes // 2, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    t_copy = best(lambda: dst.copy_(src))
    del src, dst
    m = 8192
    a = torch.randn(m, m, device="cuda").to(torch.bfloat16).contiguous()
    bm = torch.randn(m, m, device="cuda").to(torch.bfloat16).contiguous()
    t_mm = best(lambda: torch.matmul(a, bm))
    del a, bm
    torch.cuda.synchronize()
    return {"copy_gbs": 2 * nbytes / t_copy / 1e9, "bf16_gemm_tflops": 2 * m ** 3 / t_mm / 1e12,
            "how": "device copy of 2 GiB (read + write bytes); bf16 8192^3 torch.matmul; "
                   "best of 5"}


def _log(msg):
    """Progress of the run on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def rotation_copies(cfg, base_bytes, attn_bytes):
    """Input copies to rotate: enough that the smaller of the two HBM-bound
    operations' own inputs (the attention call's K/V stream, the greedy
    sweep's logits) spans twice the last-level cache, within the memory cap."""
    eb = 2 if cfg.dtype == "bf16" else 4
    own = min(attn_bytes, cfg.batch * cfg.num_draft_tokens * cfg.vocab * eb)
    want = math.ceil(2 * MALL_BYTES / max(1, own))
    fit = max(1, MAX_ROTATION_BYTES // max(1, base_bytes))
    return int(max(1, min(want, MAX_COPIES, fit)))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path "
              "would shard by request and by KV head with no exchange between GPUs.",
              file=sys.stderr)
        sys.exit(2)
    import gc
    import torch
    line = run(args)
    # Release every graph, input copy and workspace, and let the device
    # drain, before the interpreter tears down the runtime (and a profiler
    # attached to it): nothing of the library's is left to free at exit.
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    print(json.dumps(line), flush=True)


def run(args):
    import torch
    import speculative_decoding_build_amd as S

    cfg = W.CONFIGS[args.config]
    seed = args.seed if args.seed is not None else 1000 * args.config + 1
    _log(f"building workload {cfg.name} (seed {seed})")
    w = W.make_workload(cfg, seed)
    _MAXLEN[cfg.name] = int(w.seq_lens.max())
    b, n = cfg.batch, cfg.num_draft_tokens
    code = S.SPEC_BF16 if cfg.dtype == "bf16" else S.SPEC_F32

    torch.cuda.set_device(0)
    # the verify rows' logits follow the tree the GPU builds from these lists
    tl0 = np.zeros((b * n, cfg.vocab), np.uint16 if cfg.dtype == "bf16" else np.float32)
    base = Inputs(torch, S, w, tl0, tl0)
    ws_attn = torch.empty(max(1, S.spec_verify_attention_workspace_size(
        b, n, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, _MAXLEN[cfg.name], code)),
        dtype=torch.uint8, device="cuda")
    ws_greedy = torch.zeros(S.spec_accept_workspace_size(b, n, cfg.vocab, 0), dtype=torch.uint8,
                            device="cuda")
    ws_sample = torch.zeros(S.spec_accept_workspace_size(b, n, cfg.vocab, 1), dtype=torch.uint8,
                            device="cuda")
    ws_target = torch.zeros(S.spec_accept_target_only_workspace_size(b, n, cfg.vocab),
                            dtype=torch.uint8, device="cuda")
    ws_draft = torch.empty(S.spec_draft_step_workspace_size(b, cfg.topk, cfg.vocab),
                           dtype=torch.uint8, device="cuda")
    mem = memory_side_buffers(torch, S, cfg, w)
    S.spec_build_tree(b, cfg.topk, cfg.num_steps, n, S.SPEC_MASK_QLEN_BITS, base.scores,
                      base.tokens, base.parents, base.bonus, base.seq_lens, base.draft_tokens,
                      base.positions, base.tree_mask, base.retrieve_index,
                      base.retrieve_next_token, base.retrieve_next_sibling,
                      selected=base.selected, dev_status=base.status)
    sel = base.selected.cpu().numpy()[:b * (n - 1)].reshape(b, max(n - 1, 0))
    tl, dl = W.verify_logits(w, sel)
    base.tl, base.dl = _dev(torch, tl), _dev(torch, dl)

    if args.calibrate_copy_mb > 0:
        nbytes = args.calibrate_copy_mb << 20
        src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    attn_bytes = W.attention_bytes(cfg, w.seq_lens)
    copies = rotation_copies(cfg, base.nbytes(), attn_bytes)
    xs = [base] + [base.clone(torch) for _ in range(copies - 1)]
    torch.cuda.synchronize()
    _log(f"{copies} input copies resident ({copies * base.nbytes() / 1e9:.1f} GB)")

    for i in range(args.warmup):
        run_ops(S, cfg, xs[i % copies], ws_attn, ws_greedy, ws_sample)
    torch.cuda.synchronize()

    calls = [op_calls(S, cfg, x, ws_attn, ws_greedy, ws_sample, ws_target, ws_draft, mem)
             for x in xs]
    op_ms, extra_ms = {}, {}
    if args.mode == "graph":
        # per-operation GPU times: one graph per operation holding that
        # operation at least 16 times back to back (cycling through the input
        # copies), replayed between two events, so neither host time nor the
        # launch of a graph falls between the operations
        per_graph = max(16, copies)
        reps = max(2, math.ceil(64 / per_graph))
        for j, op in enumerate(OPS + EXTRA_OPS):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(per_graph):
                    calls[i % copies][j]()
            g.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            (op_ms if op in OPS else extra_ms)[op] = e0.elapsed_time(e1) / (reps * per_graph)
            del g
    else:
        # eager: events around every operation of eager steps (host launch
        # time between operations is included)
        k_ev = max(5, min(args.steps, 20))
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(k_ev)]
        for i in range(k_ev):
            c = calls[i % copies]
            for j in range(5):
                ev[i][j].record()
                c[j]()
            ev[i][5].record()
        torch.cuda.synchronize()
        for j, op in enumerate(OPS):
            op_ms[op] = float(np.mean([e[j].elapsed_time(e[j + 1]) for e in ev]))
        for j, op in enumerate(EXTRA_OPS):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(k_ev):
                calls[i % copies][len(OPS) + j]()
            e1.record()
            torch.cuda.synchronize()
            extra_ms[op] = e0.elapsed_time(e1) / k_ev

    _log("per-operation timing done")
    # eager steps (every launch from Python)
    k_e = max(5, min(args.steps, 20))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(k_e):
        run_ops(S, cfg, xs[i % copies], ws_attn, ws_greedy, ws_sample)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / k_e

    graph_check = None
    if args.mode == "graph":
        # one whole-step graph per input copy; the tree and accept outputs of a
        # replay must equal those of an eager step on the same copy (they do
        # not depend on the KV state that compaction changes)
        keys = ("draft_tokens", "retrieve_index", "retrieve_next_token", "retrieve_next_sibling",
                "predict", "accept_index", "accept_length", "spredict", "saccept_index",
                "saccept_length")
        run_ops(S, cfg, xs[0], ws_attn, ws_greedy, ws_sample)
        torch.cuda.synchronize()
        ref = {k: getattr(xs[0], k).clone() for k in keys}
        for k in keys:
            getattr(xs[0], k).fill_(-9)
        graphs = []
        for x in xs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_ops(S, cfg, x, ws_attn, ws_greedy, ws_sample)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % copies].replay()
        graphs[0].replay()
        torch.cuda.synchronize()
        graph_check = all(torch.equal(ref[k], getattr(xs[0], k)) for k in keys)
        step = lambda i: graphs[i % copies].replay()
    else:
        step = lambda i: run_ops(S, cfg, xs[i % copies], ws_attn, ws_greedy, ws_sample)

    # timed region: K steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = wall * 1e3 / args.steps
    status = int(base.status.cpu()[0])
    _log(f"timed {args.steps} steps: {step_ms:.4f} ms per step")

    acc_len = base.accept_length.cpu().numpy() if "greedy" in cfg.accept else \
        base.saccept_length.cpu().numpy()
    depth = (base.positions.cpu().numpy().reshape(b, n) - w.seq_lens[:, None]).astype(np.int64)
    eb = 2 if cfg.dtype == "bf16" else 4
    attn_flops = W.attention_flops(cfg, w.seq_lens, depth)
    sweep_g = b * n * cfg.vocab * eb
    draft_bytes = b * cfg.npar * cfg.vocab * eb
    t_attn = op_ms["verify_attention"] * 1e-3
    attn_gbs = attn_bytes / t_attn / 1e9
    attn_tflops = attn_flops / t_attn / 1e12
    greedy_gbs = sweep_g / (op_ms["accept_greedy"] * 1e-3) / 1e9
    # the sampled walk reads only the rows it visits: a request's root row and
    # each accepted node's row (accept_length rows), target and draft
    sample_fields = {}
    if "sample" in cfg.accept:
        visited = int(base.saccept_length.cpu().numpy().sum())
        vbytes = visited * 2 * cfg.vocab * eb
        sample_fields = {"accept_sample_visited_rows": visited,
                         "accept_sample_visited_bytes": vbytes,
                         "accept_sample_visited_gbs":
                             vbytes / (op_ms["accept_sample"] * 1e-3) / 1e9}
    accept_op = "accept_greedy" if "greedy" in cfg.accept else "accept_sample"
    # the binding roof: matrix cores when the call's flops per algorithmic
    # byte exceed the ridge (peak flops / peak bandwidth), else HBM
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    mfma_bound = cfg.dtype == "bf16" and attn_flops / attn_bytes > ridge
    traffic = _traffic(cfg)
    if mfma_bound:
        roof = {"kernel": "spec_verify_attention (split-KV MFMA + merge launches)",
                "bound": "mfma", "achieved": attn_tflops, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": attn_tflops / BF16_PEAK_TFLOPS, "traffic": traffic,
                "algorithmic_flops": attn_flops, "algorithmic_bytes": attn_bytes,
                "hbm_gbs": attn_gbs, "frac_hbm": attn_gbs / HBM_PEAK_GBS}
    else:
        roof = {"kernel": "spec_verify_attention (split-KV MFMA + merge launches)",
                "bound": "hbm", "achieved": attn_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": attn_gbs / HBM_PEAK_GBS, "traffic": traffic,
                "algorithmic_bytes": attn_bytes, "algorithmic_flops": attn_flops,
                "tflops": attn_tflops, "frac_mfma": attn_tflops / BF16_PEAK_TFLOPS}

    line = {
        "metric": "verified tree tokens/s (whole path per step)",
        "value": b * n / (step_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": b, "topk": cfg.topk,
                   "num_steps": cfg.num_steps, "num_draft_tokens": n, "vocab": cfg.vocab,
                   "q_heads": cfg.num_q_heads, "kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "page_size": cfg.page_size,
                   "cached_tokens": int(w.seq_lens.sum()), "temperature": cfg.temperature,
                   "input_copies_rotated": copies},
        "mode": args.mode,
        "op_timing": ("graph of the operation alone, events around the replays"
                      if args.mode == "graph" else "events around eager launches"),
        "graph_replay_matches_eager": graph_check,
        "ms_per_step_eager": eager_ms,
        "accept_steps_per_s": b / (op_ms[accept_op] * 1e-3),
        "accepted_tokens_per_s": float(acc_len.sum()) / (op_ms[accept_op] * 1e-3),
        "attention_tokens_per_s": b * n / t_attn,
        "op_ms": op_ms,
        "verify_attn_gbs": attn_gbs,
        "verify_attn_frac_hbm": attn_gbs / HBM_PEAK_GBS,
        "verify_attn_tflops": attn_tflops,
        "verify_attn_frac_mfma": attn_tflops / BF16_PEAK_TFLOPS,
        "accept_greedy_sweep_gbs": greedy_gbs,
        **sample_fields,
        "extra_op_ms": extra_ms,
        "accept_target_only_sweep_gbs": sweep_g / (extra_ms["accept_target_only"] * 1e-3) / 1e9,
        "draft_step_calls": cfg.num_steps,
        "sampling_filter_gbs": 2 * sweep_g / (extra_ms["sampling_filter"] * 1e-3) / 1e9,
        "full_mask_bytes": mem["full_bytes"],
        "full_mask_write_gbs": mem["full_bytes"] / (extra_ms["full_mask"] * 1e-3) / 1e9,
        "draft_steps_sweep_gbs": draft_bytes / (extra_ms["draft_steps"] * 1e-3) / 1e9,
        "mean_accept_length": float(acc_len.mean()),
        "dev_status": status,
        "roofline": roof,
        "roofline_accept_sweep": {"kernel": "spec_accept_greedy (vocabulary sweep + walk)",
                                  "bound": "hbm", "achieved": greedy_gbs,
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": greedy_gbs / HBM_PEAK_GBS,
                                  "algorithmic_bytes": sweep_g},
    }
    # fractions against what this box achieves, beside the nominal ones (not
    # in a counter-calibration run: its plain copy must be the largest one)
    if args.no_peaks or args.calibrate_copy_mb:
        peaks = None
    else:
        peaks = measured_peaks(torch)
        line["measured_peaks"] = peaks
    if peaks is None:
        pass
    elif mfma_bound:
        roof["measured_peak"] = peaks["bf16_gemm_tflops"]
        roof["frac_measured"] = attn_tflops / peaks["bf16_gemm_tflops"]
        roof["frac_hbm_measured"] = attn_gbs / peaks["copy_gbs"]
    else:
        roof["measured_peak"] = peaks["copy_gbs"]
        roof["frac_measured"] = attn_gbs / peaks["copy_gbs"]
    if peaks is not None:
        line["roofline_accept_sweep"]["measured_peak"] = peaks["copy_gbs"]
        line["roofline_accept_sweep"]["frac_measured"] = greedy_gbs / peaks["copy_gbs"]
        _log(f"measured peaks: copy {peaks['copy_gbs']:.0f} GB/s, "
             f"bf16 GEMM {peaks['bf16_gemm_tflops']:.0f} TFLOP/s")
    if not args.no_cpu_baseline:
        _log("CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline(cfg, w, tl, dl, args.cpu_budget_s)
    return line


if __name__ == "__main__":
    main()
