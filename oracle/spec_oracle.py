"""CPU oracle for the tree speculative-decoding hot path.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers; the library's product path
never imports, links or runs anything here, and this module imports nothing
from the library.

Plain numpy.  Every floating-point step runs in float64 on the stored input
values (float32 inputs widen exactly, bf16 bit patterns are widened here).
Loops follow the pages' own order; numpy's matmul, argmax, exp and sort are
used as library primitives for single steps, never to reorder the method.

Sources (web pages, cited by title and section):
  [P1] "SGLang 源码完全拆解(十一):投机解码——草稿生成、批量验证与 token 接受如何接进同一条前向"
  [P2] "投机解码 Accept:从 Verify 行到最终输出路径"
  [P4] "Speculative Decoding" (sglang-internals book, part 3, execution model)
  [P5] "把投机采样讲透:以 SGLang 中的 EAGLE-2 为例"

Readings where the pages are silent:
  * torch.topk's order among equal scores is unstated: rank by (score
    descending, flat index ascending).
  * A node's parent is found through the parent list as
    parents[f // topk] (the score row of flat index f holds the flat index of
    the token it was expanded from; -1 in row 0 is the root).
  * The tree mask includes the diagonal (a node attends to itself).
  * Bit-packed mask rows are LSB-first: bit j of row k set iff node j is
    visible to node k; word width 8 << ceil(log2(ceil(n / 8))).
  * Children and siblings are ordered by ascending node index.
  * Softmax scale is 1/sqrt(head_dim) unless the caller gives one.
  * Sampled accept: one uniform per tree node tests that node; one final
    uniform per request draws the terminal token by inverse CDF in vocabulary
    order; rejected siblings update the residual recursively.
  * Target-only sampled accept: the siblings under node k share the coin
    u[k] (the root's first, then each accepted node's); the terminal token
    is drawn like the sampled accept's, from relu(p - buffer).
  * Malformed trees: a node whose parent is not selected (or whose parent
    index is out of range) hangs off the root and raises a status bit.
  * Draft step: the draft distribution of a branch is softmax(logits) held at
    float32 (the draft's probability dtype), rounded once from float64; its
    top-k and the top-k over the path products rank by value descending,
    lower index first among equal values; path products are float32
    multiplications of float32 values (the page multiplies float32 tensors),
    so both sides take every integer decision from the same float32 values.

Status bits (OR-ed per call): 1 index out of range, 2 selection not closed
under ancestors, 4 accepted path longer than the accept_index row, 8 residual
mass exactly zero (informational).
"""
from __future__ import annotations

import math

import numpy as np

ST_RANGE = 1
ST_NOT_CLOSED = 2
ST_DEPTH = 4
ST_ZERO_RESIDUAL = 8

MASK_QLEN_U8 = 1
MASK_QLEN_BITS = 2


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values as float64.  bf16 arrives as uint16 bit patterns."""
    if dtype == "bf16":
        bits = np.ascontiguousarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# C1  Tree build
# ---------------------------------------------------------------------------

def select_nodes(scores_row: np.ndarray, count: int) -> np.ndarray:
    """[P1] organize_draft_results: take the ``count`` best flat candidates
    by path score, then sort the chosen flat indices ascending so every parent
    comes before its children."""
    s = np.asarray(scores_row, dtype=np.float64)
    order = sorted(range(s.size), key=lambda f: (-s[f], f))
    return np.array(sorted(order[:count]), dtype=np.int64)


def mask_word_bits(n: int) -> int:
    """[P1] 三种 mask 形态 (QLEN_ONLY_BITPACKING): the packed dtype index is
    ceil(log2(ceil(n/8))); the word is 8 << index bits wide."""
    idx = math.ceil(math.log2(max(1, (n + 7) // 8)))
    return 8 << idx


def build_tree(scores, tokens, parents, bonus, seq_lens, topk, num_steps, n):
    """[P1] build_tree_kernel_efficient and the retrieve_* adjacency lists;
    [P5] 4.3 tree mask and positions; [P2] 二 (first-child / next-sibling).

    Returns a dict of numpy arrays:
      draft_tokens [b*n], positions [b*n], mask bool [b, n, n],
      retrieve_index / next_token / next_sibling [b, n], selected [b, n-1],
      parent [b, n], depth [b, n], status int.
    """
    scores = np.asarray(scores)
    b = scores.shape[0]
    ncand = topk + (num_steps - 1) * topk * topk
    npar = 1 + (num_steps - 1) * topk
    assert scores.shape == (b, ncand) and np.shape(tokens) == (b, ncand)
    assert np.shape(parents) == (b, npar)
    assert 1 <= n and n - 1 <= ncand
    status = 0
    draft_tokens = np.zeros(b * n, np.int64)
    positions = np.zeros(b * n, np.int64)
    mask = np.zeros((b, n, n), bool)
    r_index = np.full((b, n), -1, np.int64)
    r_next = np.full((b, n), -1, np.int64)
    r_sib = np.full((b, n), -1, np.int64)
    selected = np.zeros((b, max(n - 1, 0)), np.int64)
    parent = np.full((b, n), -1, np.int64)
    depth = np.zeros((b, n), np.int64)
    for r in range(b):
        sel = select_nodes(scores[r], n - 1)
        selected[r] = sel
        # node 0 is the bonus token from the previous round; node k >= 1 is sel[k-1]
        draft_tokens[r * n] = bonus[r]
        for k in range(1, n):
            draft_tokens[r * n + k] = tokens[r, sel[k - 1]]
        where = {int(f): k for k, f in enumerate(sel, start=1)}
        for k in range(1, n):
            f = int(sel[k - 1])
            if f < topk:
                parent[r, k] = 0                      # step-0 candidates hang off the root
                continue
            g = int(parents[r, f // topk])            # flat index this score row expanded
            if g < 0 or g >= ncand:
                status |= ST_RANGE
                parent[r, k] = 0
            elif g not in where or where[g] >= k:
                status |= ST_NOT_CLOSED
                parent[r, k] = 0
            else:
                parent[r, k] = where[g]
        for k in range(1, n):
            depth[r, k] = depth[r, parent[r, k]] + 1
        for k in range(n):
            positions[r * n + k] = int(seq_lens[r]) + depth[r, k]
            # visible set of node k: itself and every ancestor up to the root
            j = k
            while True:
                mask[r, k, j] = True
                if j == 0:
                    break
                j = int(parent[r, j])
            r_index[r, k] = r * n + k
        for k in range(n):
            kids = [c for c in range(1, n) if parent[r, c] == k]
            r_next[r, k] = kids[0] if kids else -1
            if k > 0:
                later = [c for c in range(k + 1, n) if parent[r, c] == parent[r, k]]
                r_sib[r, k] = later[0] if later else -1
    return dict(draft_tokens=draft_tokens, positions=positions, mask=mask,
                retrieve_index=r_index, retrieve_next_token=r_next,
                retrieve_next_sibling=r_sib, selected=selected, parent=parent,
                depth=depth, status=status)


def pack_mask(mask: np.ndarray, mode: int) -> np.ndarray:
    """[P1] 三种 mask 形态: QLEN_ONLY as [b, n, n] bytes, or QLEN_ONLY bit-packed
    into one word per row (bit j = node j visible)."""
    b, n, _ = mask.shape
    if mode == MASK_QLEN_U8:
        return mask.astype(np.uint8)
    bits = mask_word_bits(n)
    dt = {8: np.uint8, 16: np.uint16, 32: np.uint32, 64: np.uint64}[bits]
    out = np.zeros((b, n), np.uint64)
    for j in range(n):
        out |= mask[:, :, j].astype(np.uint64) << np.uint64(j)
    return out.astype(dt)


def unpack_mask(words: np.ndarray, n: int) -> np.ndarray:
    w = np.asarray(words).astype(np.uint64)
    return ((w[..., None] >> np.arange(n, dtype=np.uint64)) & np.uint64(1)).astype(bool)


# ---------------------------------------------------------------------------
# C2  Tree-masked verify attention
# ---------------------------------------------------------------------------

def slot_of(page_table, page_size, r, pos):
    return int(page_table[r, pos // page_size]) * page_size + pos % page_size


def verify_attention(q, k_pool, v_pool, page_table, seq_lens, out_cache_loc, mask,
                     num_q_heads, num_kv_heads, page_size, dtype, sm_scale=None,
                     rows=None):
    """[P5] 4.2 / 4.3: each flattened tree node is a query over the cached
    history of its request plus the tree nodes its mask row allows (itself and
    its ancestors); [P1] the tree nodes' K/V sit at out_cache_loc.

    q [b*n, hq, d]; k_pool / v_pool [slots, hkv, d]; mask bool [b, n, n].
    Query head h reads KV head h // (hq / hkv).  Returns float64
    [b*n, hq, d], or, when ``rows`` lists (row, head) pairs, only those
    vectors as [len(rows), d].
    """
    b, n, _ = mask.shape
    d = q.shape[-1]
    G = num_q_heads // num_kv_heads
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    want = None
    if rows is not None:
        want = {}
        for i, (row, h) in enumerate(rows):
            want.setdefault((row // n, h // G), []).append((i, row, h))
        out = np.zeros((len(rows), d))
    else:
        out = np.zeros((b * n, num_q_heads, d))
    for r in range(b):
        L = int(seq_lens[r])
        hist = np.array([slot_of(page_table, page_size, r, p) for p in range(L)], np.int64)
        tree = np.asarray(out_cache_loc[r * n:(r + 1) * n], np.int64)
        for g in range(num_kv_heads):
            if want is not None and (r, g) not in want:
                continue
            K = widen(np.concatenate([k_pool[hist, g], k_pool[tree, g]]), dtype)
            V = widen(np.concatenate([v_pool[hist, g], v_pool[tree, g]]), dtype)
            pairs = (want[(r, g)] if want is not None else
                     [(None, r * n + k, h) for k in range(n) for h in range(g * G, (g + 1) * G)])
            for i, row, h in pairs:
                k = row - r * n
                visible = np.concatenate([np.ones(L, bool), mask[r, k]])
                s = scale * (K[visible] @ widen(q[row, h], dtype))
                p = np.exp(s - s.max())
                o = (p / p.sum()) @ V[visible]
                if i is None:
                    out[row, h] = o
                else:
                    out[i] = o
    return out


def verify_attention_unit(q, k_pool, v_pool, page_table, seq_lens, out_cache_loc, mask,
                          num_q_heads, num_kv_heads, page_size, dtype, r, g, sm_scale=None):
    """The same definition as verify_attention ([P5] 4.2 / 4.3), evaluated
    for every query of one (request r, KV head g) unit at once: the n tree
    nodes times the G query heads of the group form the rows of one score
    matrix against the request's keys (history, then tree nodes); a tree key
    a node's mask row does not allow scores -inf; each row's softmax weights
    V.  Matrix products stand in for the per-vector dot products; nothing is
    split or reordered beyond that.

    Returns float64 [n, G, d]: out[k, j] is query head g * G + j of node k.
    """
    b, n, _ = mask.shape
    d = q.shape[-1]
    G = num_q_heads // num_kv_heads
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    L = int(seq_lens[r])
    hist = np.array([slot_of(page_table, page_size, r, p) for p in range(L)], np.int64)
    tree = np.asarray(out_cache_loc[r * n:(r + 1) * n], np.int64)
    slots = np.concatenate([hist, tree])
    K = widen(k_pool[slots, g], dtype)                       # [L + n, d]
    V = widen(v_pool[slots, g], dtype)
    Q = widen(q[r * n:(r + 1) * n, g * G:(g + 1) * G], dtype).reshape(n * G, d)
    s = scale * (Q @ K.T)                                    # [n * G, L + n]
    allow = np.repeat(np.asarray(mask[r], bool), G, axis=0)  # row k * G + j: node k's mask row
    s[:, L:][~allow] = -np.inf
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return (p @ V).reshape(n, G, d)


# ---------------------------------------------------------------------------
# C3  Greedy accept
# ---------------------------------------------------------------------------

def argmax_rows(logits: np.ndarray, dtype: str) -> np.ndarray:
    """[P1] 三条判定路径: the target's choice per verify row is torch.argmax,
    which returns the first index among equal maxima."""
    x = widen(logits, dtype)
    return np.argmax(x, axis=-1).astype(np.int64)


def accept_greedy(target_logits, candidates, retrieve_index, retrieve_next_token,
                  retrieve_next_sibling, b, n, s1, dtype):
    """[P2] 三 (Greedy Accept 的行索引与输出) and [P5] 5.3: from the root,
    scan children by first-child / next-sibling for the candidate equal to
    the target's choice at the current node; descend on a match; the target's
    choice at the last node is the terminal token.  accept_index holds verify
    rows; accept_length counts accepted drafts plus the terminal token.
    """
    tp = argmax_rows(target_logits, dtype)
    predict = np.zeros(b * n, np.int64)
    accept_index = np.full((b, s1), -1, np.int64)
    accept_length = np.zeros(b, np.int64)
    status = 0
    cand = np.asarray(candidates).reshape(b, n)
    for r in range(b):
        cur = 0
        cnt = 0
        accept_index[r, 0] = retrieve_index[r, 0]
        while True:
            want = tp[retrieve_index[r, cur]]
            c = int(retrieve_next_token[r, cur])
            hit = -1
            while c != -1:
                if cand[r, c] == want:
                    hit = c
                    break
                c = int(retrieve_next_sibling[r, c])
            if hit < 0:
                break
            if cnt + 1 >= s1:
                status |= ST_DEPTH
                break
            predict[retrieve_index[r, cur]] = cand[r, hit]
            cnt += 1
            accept_index[r, cnt] = retrieve_index[r, hit]
            cur = hit
        predict[retrieve_index[r, cur]] = tp[retrieve_index[r, cur]]
        accept_length[r] = cnt + 1
    return dict(predict=predict, accept_index=accept_index, accept_length=accept_length,
                target_predict=tp, status=status)


# ---------------------------------------------------------------------------
# C4  Rejection-sampled accept
# ---------------------------------------------------------------------------

def softmax_t(logits_row: np.ndarray, temperature: float) -> np.ndarray:
    """[P2] 四: the target (and draft) distribution at temperature T,
    max-subtracted, float64."""
    x = np.asarray(logits_row, dtype=np.float64)
    e = np.exp((x - x.max()) / float(temperature))
    return e / e.sum()


def accept_sample(target_logits, draft_logits, temperature, uniforms, final_uniforms,
                  candidates, retrieve_index, retrieve_next_token, retrieve_next_sibling,
                  b, n, s1, dtype, band=1e-6, draw_band=2e-8):
    """[P4] 接受/拒绝 and [P2] 四 (Classic Rejection Sampling): at node cur
    the residual R starts as the target distribution p of row(cur); each child
    c (sibling order) with token t is accepted iff u[c] < min(1, R(t)/q(t)),
    q being the draft distribution of row(cur).  A rejection replaces R by
    max(0, R - q) renormalised.  When no child is accepted (or cur is a leaf)
    the terminal token is drawn from R by inverse CDF with the request's final
    uniform.  [P5] 5.6: the walk is the greedy walk's.

    Also returns, per request, how close each decision came to its
    boundary: ``ratio_margin`` = smallest |u - min(1, ratio)| over the tests
    made, ``z_min`` = the smallest residual mass Z, ``margin`` = the smaller
    of the two, ``draw_margin`` = the final uniform's distance to the nearest
    CDF edge, relative to the residual mass.  A
    request is ``exempt`` from bit-exact comparison when margin < ``band``
    (the 1e-6 band stated for the ratio test) or draw_margin < ``draw_band``
    (the terminal draw has no stated band; 2e-8 covers float32 evaluation of
    the exponentials with float64 accumulation, whose CDF error stays below
    about 5e-9 of the mass at vocabulary 128256).
    """
    tl = widen(target_logits, dtype)
    dl = widen(draft_logits, dtype)
    cand = np.asarray(candidates).reshape(b, n)
    predict = np.zeros(b * n, np.int64)
    accept_index = np.full((b, s1), -1, np.int64)
    accept_length = np.zeros(b, np.int64)
    margin = np.full(b, np.inf)
    ratio_margin = np.full(b, np.inf)
    z_min = np.full(b, np.inf)
    draw_margin = np.full(b, np.inf)
    status = 0
    for r in range(b):
        T = float(temperature[r])
        cur = 0
        cnt = 0
        accept_index[r, 0] = retrieve_index[r, 0]
        while True:
            row = int(retrieve_index[r, cur])
            R = softmax_t(tl[row], T)
            q = softmax_t(dl[row], T)
            c = int(retrieve_next_token[r, cur])
            hit = -1
            while c != -1:
                t = int(cand[r, c])
                if q[t] > 0:
                    ratio = R[t] / q[t]
                else:
                    ratio = math.inf if R[t] > 0 else 0.0
                thr = min(1.0, ratio)
                u = float(uniforms[r, c])
                margin[r] = min(margin[r], abs(u - thr))
                ratio_margin[r] = min(ratio_margin[r], abs(u - thr))
                if u < thr:
                    hit = c
                    break
                resid = np.maximum(R - q, 0.0)
                Z = resid.sum()
                margin[r] = min(margin[r], Z)
                z_min[r] = min(z_min[r], Z)
                if Z > 0:
                    R = resid / Z
                else:
                    status |= ST_ZERO_RESIDUAL
                c = int(retrieve_next_sibling[r, c])
            if hit < 0:
                break
            if cnt + 1 >= s1:
                status |= ST_DEPTH
                break
            predict[row] = cand[r, hit]
            cnt += 1
            accept_index[r, cnt] = retrieve_index[r, hit]
            cur = hit
        # terminal token: inverse CDF of the current residual in vocabulary order
        row = int(retrieve_index[r, cur])
        total = R.sum()
        target = float(final_uniforms[r]) * total
        cdf = np.cumsum(R)
        x = int(np.argmax(cdf > target)) if cdf[-1] > target else int(R.size - 1)
        lo = cdf[x - 1] if x > 0 else 0.0
        draw_margin[r] = min((target - lo) / total, (cdf[x] - target) / total)
        predict[row] = x
        accept_length[r] = cnt + 1
    return dict(predict=predict, accept_index=accept_index, accept_length=accept_length,
                margin=margin, ratio_margin=ratio_margin, z_min=z_min, draw_margin=draw_margin,
                exempt=(margin < band) | (draw_margin < draw_band), status=status)


def accept_target_only(target_logits, temperature, threshold_single, threshold_acc, uniforms,
                       final_uniforms, candidates, retrieve_index, retrieve_next_token,
                       retrieve_next_sibling, b, n, s1, dtype, band=1e-6, draw_band=2e-8,
                       tiny=1e-30):
    """[P2] 四 (Target-only Tree Sampling), with the two thresholds of [P1]
    三条判定路径: at node cur, p is the target distribution of row(cur) and the
    sibling accumulator starts at 0.  Each child c (sibling order) with token
    t adds p(t) to the accumulator and is accepted iff p(t) > 0 and (coin <
    accumulator / threshold_acc or p(t) >= threshold_single).  The coin of the
    siblings under cur is u[cur]: the pages switch to the accepted node's
    random number together with its distribution, starting from the root's.
    A rejected child's p(t) is written at token t into row(cur) of a work
    buffer that starts at zero (no draft distribution is used).  With no child
    accepted, or at a leaf, the terminal token is drawn from relu(p - buffer)
    of row(cur) by inverse CDF in vocabulary order with the request's final
    uniform (the draw of accept_sample).  [P5] 5.6: the walk is the greedy
    walk's.

    ``margin`` is the smallest distance of a test to its boundary: |coin -
    accumulator / threshold_acc|, |p(t) - threshold_single|, and p(t) itself
    when 0 < p(t) < ``tiny`` (a probability a float32 exponential may
    flush to zero); ``exempt`` as in accept_sample.
    """
    tl = widen(target_logits, dtype)
    cand = np.asarray(candidates).reshape(b, n)
    ts, ta = float(threshold_single), float(threshold_acc)
    predict = np.zeros(b * n, np.int64)
    accept_index = np.full((b, s1), -1, np.int64)
    accept_length = np.zeros(b, np.int64)
    margin = np.full(b, np.inf)
    ratio_margin = np.full(b, np.inf)
    z_min = np.full(b, np.inf)
    draw_margin = np.full(b, np.inf)
    status = 0
    for r in range(b):
        T = float(temperature[r])
        cur = 0
        cnt = 0
        accept_index[r, 0] = retrieve_index[r, 0]
        while True:
            row = int(retrieve_index[r, cur])
            p = softmax_t(tl[row], T)
            buf = np.zeros_like(p)
            coin = float(uniforms[r, cur])
            acc = 0.0
            c = int(retrieve_next_token[r, cur])
            hit = -1
            while c != -1:
                t = int(cand[r, c])
                pt = p[t]
                acc += pt
                margin[r] = min(margin[r], abs(coin - acc / ta), abs(pt - ts))
                if 0.0 < pt < tiny:
                    margin[r] = min(margin[r], pt)
                if pt > 0.0 and (coin < acc / ta or pt >= ts):
                    hit = c
                    break
                buf[t] = pt
                c = int(retrieve_next_sibling[r, c])
            if hit < 0:
                break
            if cnt + 1 >= s1:
                status |= ST_DEPTH
                break
            predict[row] = cand[r, hit]
            cnt += 1
            accept_index[r, cnt] = retrieve_index[r, hit]
            cur = hit
        # terminal token: inverse CDF of relu(p - buffer) in vocabulary order
        row = int(retrieve_index[r, cur])
        R = np.maximum(p - buf, 0.0)
        total = R.sum()
        if total <= 0.0:
            status |= ST_ZERO_RESIDUAL
        target = float(final_uniforms[r]) * total
        cdf = np.cumsum(R)
        x = int(np.argmax(cdf > target)) if cdf[-1] > target else int(R.size - 1)
        lo = cdf[x - 1] if x > 0 else 0.0
        if total > 0.0:
            draw_margin[r] = min((target - lo) / total, (cdf[x] - target) / total)
        predict[row] = x
        accept_length[r] = cnt + 1
    return dict(predict=predict, accept_index=accept_index, accept_length=accept_length,
                margin=margin, ratio_margin=ratio_margin, z_min=z_min, draw_margin=draw_margin,
                exempt=(margin < band) | (draw_margin < draw_band), status=status)


# ---------------------------------------------------------------------------
# Draft step (select_top_k_tokens)
# ---------------------------------------------------------------------------

def topk_desc(values, k):
    """The k largest entries of a 1-D array ranked by (value descending,
    index ascending): (values, indices).  [P1] fast_topk / torch.topk; the
    order among equal values is this reading's."""
    v = np.asarray(values)
    order = sorted(range(v.size), key=lambda i: (-float(v[i]), i))[:k]
    idx = np.array(order, dtype=np.int64)
    return v[idx], idx


def draft_probs(logits_row, dtype):
    """[P1] the draft distribution a step ranks: softmax of the branch's
    logits, float64 then rounded to float32."""
    x = widen(logits_row, dtype)
    e = np.exp(x - x.max())
    return (e / e.sum()).astype(np.float32)


def draft_step(draft_logits, branch_scores, step, topk, num_steps, dtype):
    """One call of [P1] select_top_k_tokens for a batch.

    draft_logits: [b, rows, V] logits of the live branches (rows = 1 at step
    0, topk later); branch_scores: [b, topk] float32 path scores of the live
    branches (unused at step 0).  Returns the step's blocks of the three
    lists organize_draft_results concatenates, with their offsets, and the
    next step's branch scores and input tokens:

      step 0 (_select_top_k_tokens_first): scores = tokens-ranked top-k of
        the root distribution, tokens = their ids, parents = arange(-1, topk);
      step i >= 1 (_select_top_k_tokens_later): expand[j, c] = branch
        score j x probability of branch j's c-th top-k token; scores =
        expand flattened, tokens = the top-k ids of every branch, and the
        top-k over the topk*topk products (cs) gives parents = cs + topk*topk
        * (i - 1) + topk, the next branch scores expand[cs], and the next
        input tokens tokens[cs].

    The score/token block of step i starts at 0 (i = 0) or topk + (i - 1) *
    topk^2 of the request's ncand entries; the parent block at 0 (i = 0) or
    topk + 1 + (i - 1) * topk of its npar entries, and the last step's parent
    block is not part of the list (organize_draft_results drops it).
    ``gap`` is the smallest relative distance between the k-th and the
    (k+1)-th value of any ranking the step made (inf when there is none).
    ``near_tie`` is the smallest relative distance between neighbours among
    the first k+1 entries of any ranking the step made, leaving out
    neighbours that are equal logits of one branch (every evaluation ranks
    those by index): where it is tiny, an evaluation whose probabilities
    differ from these by an ulp may order the entries otherwise.
    """
    dl = np.asarray(draft_logits)
    b, rows, _ = dl.shape
    tk2 = topk * topk
    out = []
    def rel(a, c):
        return (float(a) - float(c)) / float(a) if a > 0 else math.inf

    for r in range(b):
        gap = near = math.inf
        pv = np.zeros((rows, topk), np.float32)
        pi = np.zeros((rows, topk), np.int64)
        x = [widen(dl[r, j], dtype) for j in range(rows)]
        for j in range(rows):
            p = draft_probs(dl[r, j], dtype)
            vals, idx = topk_desc(p, topk + 1)
            pv[j], pi[j] = vals[:topk], idx[:topk]
            if vals.size > topk and vals[topk - 1] > 0:
                gap = min(gap, rel(vals[topk - 1], vals[topk]))
            for t in range(vals.size - 1):
                if x[j][idx[t]] != x[j][idx[t + 1]]:
                    near = min(near, rel(vals[t], vals[t + 1]))
        if step == 0:
            res = dict(scores=pv[0].copy(), tokens=pi[0].copy(),
                       parents=np.arange(-1, topk, dtype=np.int64),
                       next_scores=pv[0].copy(), next_tokens=pi[0].copy())
        else:
            bs = np.asarray(branch_scores[r], dtype=np.float32)
            expand = (bs[:, None] * pv).astype(np.float32)          # float32 products
            flat = expand.reshape(-1)
            tokens = pi.reshape(-1)
            vals, cs = topk_desc(flat, topk + 1)
            if vals.size > topk and vals[topk - 1] > 0:
                gap = min(gap, rel(vals[topk - 1], vals[topk]))
            for t in range(vals.size - 1):
                j1, j2 = cs[t] // topk, cs[t + 1] // topk
                if j1 != j2 or x[j1][tokens[cs[t]]] != x[j2][tokens[cs[t + 1]]]:
                    near = min(near, rel(vals[t], vals[t + 1]))
            cs = cs[:topk]
            res = dict(scores=flat.copy(), tokens=tokens.copy(),
                       parents=cs + tk2 * (step - 1) + topk,
                       next_scores=flat[cs].copy(), next_tokens=tokens[cs].copy())
        res["gap"] = gap
        res["near_tie"] = near
        out.append(res)
    off_s = 0 if step == 0 else topk + (step - 1) * tk2
    off_p = 0 if step == 0 else topk + 1 + (step - 1) * topk
    return dict(
        scores=np.stack([o["scores"] for o in out]), tokens=np.stack([o["tokens"] for o in out]),
        parents=np.stack([o["parents"] for o in out]),
        next_scores=np.stack([o["next_scores"] for o in out]),
        next_tokens=np.stack([o["next_tokens"] for o in out]),
        gap=np.array([o["gap"] for o in out]),
        near_tie=np.array([o["near_tie"] for o in out]), score_offset=off_s, parent_offset=off_p,
        write_parents=step < num_steps - 1)


# ---------------------------------------------------------------------------
# C5  Accepted-KV compaction
# ---------------------------------------------------------------------------

def compact_kv(k_pool, v_pool, page_table, seq_lens, out_cache_loc, accept_index,
               accept_length, b, n, page_size):
    """[P1] KV 回写 (move_accept_tokens_to_target_kvcache) and [P2] 六: the
    verify rows named by accept_index (root plus accepted drafts, not the
    terminal token) move from their verify slots to the request's sequence
    positions [L, L + accept_length); the sequence grows by accept_length and
    every verify slot that is not a target slot is returned free.

    Pools are [layers, slots, hkv, d] (any dtype; copied bit for bit).
    Returns new copies of the pools plus new_seq_lens [b], free_slots [b*n]
    (request r's list at r*n, padded with -1), num_free [b], status.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    nslots = k_out.shape[1]
    new_seq_lens = np.zeros(b, np.int64)
    free_slots = np.full(b * n, -1, np.int64)
    num_free = np.zeros(b, np.int64)
    status = 0
    for r in range(b):
        L = int(seq_lens[r])
        m = int(accept_length[r])
        src, tgt = [], []
        for j in range(m):
            row = int(accept_index[r, j])
            if row < 0:
                continue
            if row >= b * n:
                status |= 1
                continue
            s = int(out_cache_loc[row])
            pos = L + j
            page = int(page_table[r, pos // page_size])
            t = page * page_size + pos % page_size
            if not (0 <= s < nslots) or page < 0 or not (0 <= t < nslots):
                status |= 1
                continue
            src.append(s)
            tgt.append(t)
        # all source rows are read before any target row is written
        k_rows = k_out[:, src].copy()
        v_rows = v_out[:, src].copy()
        k_out[:, tgt] = k_rows
        v_out[:, tgt] = v_rows
        new_seq_lens[r] = L + m
        kept = set(tgt)
        cnt = 0
        for k in range(n):
            s = int(out_cache_loc[r * n + k])
            if s not in kept:
                free_slots[r * n + cnt] = s
                cnt += 1
        num_free[r] = cnt
    return dict(k_pool=k_out, v_pool=v_out, new_seq_lens=new_seq_lens,
                free_slots=free_slots, num_free=num_free, status=status)


# ---------------------------------------------------------------------------
# C7  Sampling-parameter pre-pass
# ---------------------------------------------------------------------------

def filter_logits(logits, dtype, temperature, top_k, top_p, band=1e-6):
    """[P2] 四 (eagle_sample: the target softmax at the request's temperature,
    then top-k / top-p filtering and renormalisation) and [P1] 三条判定路径
    (the sampled path renormalises top-k / top-p before the accept).

    Row i (request of row i given by the per-row parameters) has
    p = softmax(x / T) in float64.  Entries are ranked by p descending, lower
    index first; entry of rank r is kept iff r < top_k (when 1 <= top_k < V)
    and the mass of the entries ranked above it is < top_p (when top_p < 1),
    i.e. the smallest top set reaching mass top_p.  Both rules are decided on
    the same p, then one renormalisation: the kept logits are returned as
    they were and the others as -inf, so softmax(filtered / T) is the
    renormalised distribution.  A greedy request is top_k = 1.  A row whose
    logits are all -inf has no distribution: the top-p rule does nothing
    there and top_k alone decides.

    logits [rows, V] (float32 or bf16 bit patterns); temperature, top_k,
    top_p: per row.  Returns (filtered logits in the input's storage type,
    kept bool [rows, V], near bool [rows]: a top-p decision within `band` of
    top_p, where an evaluation whose masses are an ulp off may keep one entry
    more or less)."""
    x = widen(logits, dtype)
    rows, V = x.shape
    kept = np.zeros((rows, V), bool)
    near = np.zeros(rows, bool)
    for i in range(rows):
        xi = x[i]
        T = float(temperature[i])
        k = int(top_k[i])
        tp = float(top_p[i])
        order = np.lexsort((np.arange(V), -xi))     # x descending, index ascending
        if xi.max() == -np.inf:
            tp = 1.0                                # no distribution: top-p off
            p = np.zeros(V)
        else:
            e = np.exp((xi - xi.max()) / T)
            p = e / e.sum()
        before = 0.0
        for r, j in enumerate(order):
            keep = True
            if 1 <= k < V and r >= k:
                keep = False
            if tp < 1.0:
                if abs(before - tp) < band:
                    near[i] = True
                if before >= tp:
                    keep = False
            if not keep:
                break
            kept[i, j] = True
            before += p[j]
    if dtype == "bf16":
        out = np.where(kept, np.asarray(logits, np.uint16), np.uint16(0xFF80))
    else:
        out = np.where(kept, np.asarray(logits, np.float32), np.float32(-np.inf))
    return out, kept, near


# ---------------------------------------------------------------------------
# C6  Memory-side neighbours: FULL mask, paged draft-branch planning
# ---------------------------------------------------------------------------

def full_mask(seq_lens, tree_mask, fill_prefix=True, prior=None):
    """[P1] 三种 mask 形态 (FULL_MASK) with its fill_prefix_mask switch.

    Every verify row sees the whole committed prefix and, among the tree
    nodes, its QLEN_ONLY mask row.  Layout (the per-request blocks of the
    [rows, prefix + tree] mask, concatenated): request b's block starts at
    n * sum_{b' < b} (L_b' + n) bytes and holds n rows of L_b + n bytes; row
    k is L_b prefix bytes of 1, then tree_mask[b, k, :] as bytes.  With
    fill_prefix false the prefix bytes are not written: they keep the
    values of ``prior`` (same size; zeros when None).
    tree_mask: bool [b, n, n].  Returns uint8 [n * sum(L_b + n)]."""
    L = np.asarray(seq_lens, np.int64)
    tm = np.asarray(tree_mask, bool)
    b, n, _ = tm.shape
    total = int(n * (L.sum() + n * b))
    out = np.zeros(total, np.uint8) if prior is None else np.array(prior, np.uint8, copy=True)
    assert out.size == total
    off = 0
    for r in range(b):
        width = int(L[r]) + n
        for k in range(n):
            row = off + k * width
            if fill_prefix:
                out[row:row + int(L[r])] = 1
            out[row + int(L[r]):row + width] = tm[r, k].astype(np.uint8)
        off += n * width
    return out


def plan_draft_branches(seq_lens, page_table, branch_pages, topk, num_steps, page_size,
                        num_pages):
    """[P1] prepare_for_draft (KV slots for the draft writes) and
    duplicate_prefix_tail_to_draft_branches.

    Request b has L committed tokens; its prefix tail (the tokens on its last,
    partial page) is tail = L mod page_size tokens at slots
    page_table[b][L div page_size] * page_size + [0, tail).
      * topk > 1: branch j owns the pages branch_pages[b][j][0 ..), a
        page-aligned region whose slot t is page t div page_size, offset
        t mod page_size.  Its first `tail` slots are holes standing for the
        prefix tail: they receive a copy of the prefix tail's KV (every
        layer, K and V), so reading the branch's pages whole gives the right
        tokens.  Draft step s of branch j writes region slot tail + s.
      * topk == 1 (the contiguous case): the single branch continues the
        prefix in place: draft step s writes the slot of position L + s
        through page_table; nothing is copied.
    (page_size 1 makes tail 0: no copies in either case.)

    Returns out_cache_loc int64 [b, topk, num_steps] (-1 where a page id is
    out of range), copies: list of (src_slot, dst_slot), status (bit 1 on a
    page id outside [0, num_pages))."""
    L = np.asarray(seq_lens, np.int64)
    pt = np.asarray(page_table, np.int64)
    bp = np.asarray(branch_pages, np.int64)
    b = L.size
    ps = page_size
    out = np.full((b, topk, num_steps), -1, np.int64)
    copies = []
    status = 0

    def slot_of(page, off):
        nonlocal status
        if not (0 <= page < num_pages):
            status |= ST_RANGE
            return -1
        return int(page) * ps + off

    for r in range(b):
        tail = int(L[r]) % ps
        if topk == 1:
            for s in range(num_steps):
                pos = int(L[r]) + s
                out[r, 0, s] = slot_of(pt[r, pos // ps], pos % ps)
            continue
        src_page = pt[r, int(L[r]) // ps] if tail > 0 else 0
        for j in range(topk):
            for t in range(tail):
                src = slot_of(src_page, t)
                dst = slot_of(bp[r, j, t // ps], t % ps)
                if src >= 0 and dst >= 0:
                    copies.append((src, dst))
            for s in range(num_steps):
                t = tail + s
                out[r, j, s] = slot_of(bp[r, j, t // ps], t % ps)
    return dict(out_cache_loc=out, copies=copies, status=status)


def duplicate_prefix_tail(k_pool, v_pool, copies):
    """Apply the copies of plan_draft_branches to pools [layers, slots, hkv,
    d] (new arrays; every source is read before any destination is written)."""
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    if copies:
        src = np.array([c[0] for c in copies], np.int64)
        dst = np.array([c[1] for c in copies], np.int64)
        k_rows, v_rows = k_out[:, src].copy(), v_out[:, src].copy()
        k_out[:, dst] = k_rows
        v_out[:, dst] = v_rows
    return k_out, v_out
