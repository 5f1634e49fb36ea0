"""Tree speculative-decoding hot path for AMD MI355X (gfx950).

Thin Python binding of the C-ABI library ``libspecmi.so`` (declared in
``include/spec.h``).  Each function has the C name and argument order, takes
torch tensors where the C call takes device pointers, and only marshals
arguments: it checks that every tensor lives on the current GPU, is
contiguous and holds at least the elements the call will touch, then passes
``data_ptr()`` and the current HIP stream.  Every step runs in the library's
HIP kernels; there is no other code path.  Importing this package fails if
the library has not been built (``python
speculative_decoding_build_amd/build_lib.py``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecmi.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python speculative_decoding_build_amd/build_lib.py`")

_lib = ctypes.CDLL(LIB_PATH)

SPEC_OK = 0
SPEC_ERR_NULL = -1
SPEC_ERR_SHAPE = -2
SPEC_ERR_DTYPE = -3
SPEC_ERR_UNSUPPORTED = -4
SPEC_ERR_WORKSPACE = -5
SPEC_ERR_HIP = -6

SPEC_ST_RANGE = 1
SPEC_ST_NOT_CLOSED = 2
SPEC_ST_DEPTH = 4
SPEC_ST_ZERO_RESIDUAL = 8
SPEC_ST_SYNC = 16

SPEC_F32 = 0
SPEC_BF16 = 1
SPEC_MASK_QLEN_U8 = 1
SPEC_MASK_QLEN_BITS = 2

EXPORTS = ("spec_version", "spec_status_string", "spec_mask_word_bytes", "spec_build_tree",
           "spec_verify_attention_workspace_size", "spec_verify_attention",
           "spec_accept_workspace_size", "spec_accept_greedy", "spec_accept_greedy_noalloc",
           "spec_accept_sample",
           "spec_accept_target_only_workspace_size", "spec_accept_target_only",
           "spec_draft_step_workspace_size", "spec_draft_step",
           "spec_sampling_filter_workspace_size", "spec_sampling_filter", "spec_full_mask",
           "spec_plan_draft_branches",
           "spec_compact_kv")

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float


def _decl(name, restype, *argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)
    return f


_decl("spec_version", _I)
_decl("spec_status_string", ctypes.c_char_p, _I)
_decl("spec_mask_word_bytes", _I, _I)
_decl("spec_build_tree", _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
      _P, _P, _P)
_decl("spec_verify_attention_workspace_size", _SZ, _I, _I, _I, _I, _I, _I, _I)
_decl("spec_verify_attention", _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _I64, _P, _I,
      _P, _I, _P, _P, _P, _P, _SZ, _P, _P)
_decl("spec_accept_workspace_size", _SZ, _I, _I, _I64, _I)
_decl("spec_accept_greedy", _I, _I, _I, _I, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
      _SZ, _P, _P)
_decl("spec_accept_greedy_noalloc", _I, _I, _I, _I, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P,
      _P, _P, _P)
_decl("spec_accept_sample", _I, _I, _I, _I, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
      _P, _P, _P, _SZ, _P, _P)
_decl("spec_accept_target_only_workspace_size", _SZ, _I, _I, _I64)
_decl("spec_accept_target_only", _I, _I, _I, _I, _I64, _I, _P, _P, _F, _F, _P, _P, _P, _P, _P,
      _P, _P, _P, _P, _P, _SZ, _P, _P)
_decl("spec_draft_step_workspace_size", _SZ, _I, _I, _I64)
_decl("spec_draft_step", _I, _I, _I, _I, _I, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _P)
_decl("spec_sampling_filter_workspace_size", _SZ, _I, _I, _I64)
_decl("spec_sampling_filter", _I, _I, _I, _I64, _I, _P, _P, _P, _P, _P, _P, _SZ, _P, _P)
_decl("spec_full_mask", _I, _I, _I, _P, _I, _P, _I, _P, _I64, _P, _P)
_decl("spec_plan_draft_branches", _I, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _I64, _P, _P, _I, _P,
      _I, _P, _P, _P)
_decl("spec_compact_kv", _I, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _I64, _P, _I, _P, _P, _P,
      _P, _P, _P, _P, _P, _P)


class SpecError(RuntimeError):
    def __init__(self, call, code):
        super().__init__(f"{call}: {code} ({_lib.spec_status_string(code).decode()})")
        self.code = code


def _check(call, rc):
    if rc != SPEC_OK:
        raise SpecError(call, rc)


_ELEM = {SPEC_F32: 4, SPEC_BF16: 2}


def _device():
    """Index of the current GPU; ValueError when there is none (the calls
    take device tensors only)."""
    try:
        return torch.cuda.current_device()
    except (RuntimeError, AssertionError) as e:
        raise ValueError(f"no usable GPU: {e}") from None


def _ptr(t, what, dev, *, nbytes=None, optional=False):
    """Device pointer of tensor ``t`` after checking it is a contiguous tensor
    on GPU ``dev`` (the current one) with at least ``nbytes`` bytes."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{what}: tensor required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    if t.get_device() != dev:
        raise ValueError(f"{what}: must be on the current GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if nbytes is not None and t.nbytes < nbytes:
        raise ValueError(f"{what}: {t.nbytes} bytes, the call needs {nbytes}")
    return t.data_ptr() if t.numel() else None


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def spec_version() -> int:
    return _lib.spec_version()


def spec_status_string(status: int) -> str:
    return _lib.spec_status_string(status).decode()


def spec_mask_word_bytes(num_draft_tokens: int) -> int:
    return _lib.spec_mask_word_bytes(num_draft_tokens)


def spec_build_tree(batch, topk, num_steps, num_draft_tokens, mask_mode, scores, tokens,
                    parents, bonus, seq_lens, draft_tokens, positions, tree_mask,
                    retrieve_index, retrieve_next_token, retrieve_next_sibling,
                    selected=None, dev_status=None, stream=None):
    dev = _device()
    n = num_draft_tokens
    ncand = topk + (num_steps - 1) * topk * topk
    npar = 1 + (num_steps - 1) * topk
    bn = batch * n
    mbytes = batch * n * (n if mask_mode == SPEC_MASK_QLEN_U8 else max(1, spec_mask_word_bytes(n)))
    args = [
        _ptr(scores, "scores", dev, nbytes=batch * ncand * 4),
        _ptr(tokens, "tokens", dev, nbytes=batch * ncand * 4),
        _ptr(parents, "parents", dev, nbytes=batch * npar * 4, optional=num_steps == 1),
        _ptr(bonus, "bonus", dev, nbytes=batch * 4),
        _ptr(seq_lens, "seq_lens", dev, nbytes=batch * 4),
        _ptr(draft_tokens, "draft_tokens", dev, nbytes=bn * 4),
        _ptr(positions, "positions", dev, nbytes=bn * 4),
        _ptr(tree_mask, "tree_mask", dev, nbytes=mbytes),
        _ptr(retrieve_index, "retrieve_index", dev, nbytes=bn * 4),
        _ptr(retrieve_next_token, "retrieve_next_token", dev, nbytes=bn * 4),
        _ptr(retrieve_next_sibling, "retrieve_next_sibling", dev, nbytes=bn * 4),
        _ptr(selected, "selected", dev, nbytes=batch * (n - 1) * 4, optional=True),
        _ptr(dev_status, "dev_status", dev, nbytes=4, optional=True),
    ]
    _check("spec_build_tree", _lib.spec_build_tree(batch, topk, num_steps, n, mask_mode, *args,
                                                    _stream(stream)))


def spec_verify_attention_workspace_size(batch, num_draft_tokens, num_q_heads, num_kv_heads,
                                         head_dim, max_seq_len, dtype) -> int:
    return _lib.spec_verify_attention_workspace_size(batch, num_draft_tokens, num_q_heads,
                                                     num_kv_heads, head_dim, max_seq_len, dtype)


def spec_verify_attention(batch, num_draft_tokens, num_q_heads, num_kv_heads, head_dim,
                          page_size, dtype, sm_scale, q, k_pool, v_pool, num_slots, page_table,
                          max_pages, seq_lens, max_seq_len, out_cache_loc, tree_mask, out,
                          workspace=None, workspace_bytes=None, dev_status=None, stream=None):
    dev = _device()
    n = num_draft_tokens
    eb = _ELEM.get(dtype, 4)
    qbytes = batch * n * num_q_heads * head_dim * eb
    pool = num_slots * num_kv_heads * head_dim * eb
    need_ws = spec_verify_attention_workspace_size(batch, n, num_q_heads, num_kv_heads, head_dim,
                                                   max_seq_len, dtype)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [
        _ptr(q, "q", dev, nbytes=qbytes),
        _ptr(k_pool, "k_pool", dev, nbytes=pool),
        _ptr(v_pool, "v_pool", dev, nbytes=pool),
    ]
    args2 = [
        _ptr(page_table, "page_table", dev, nbytes=batch * max_pages * 4, optional=max_seq_len == 0),
        max_pages,
        _ptr(seq_lens, "seq_lens", dev, nbytes=batch * 4),
        max_seq_len,
        _ptr(out_cache_loc, "out_cache_loc", dev, nbytes=batch * n * 4),
        _ptr(tree_mask, "tree_mask", dev, nbytes=batch * n * max(1, spec_mask_word_bytes(n))),
        _ptr(out, "out", dev, nbytes=qbytes),
        _ptr(workspace, "workspace", dev, nbytes=need_ws, optional=need_ws == 0),
        workspace_bytes,
        _ptr(dev_status, "dev_status", dev, nbytes=4, optional=True),
    ]
    _check("spec_verify_attention", _lib.spec_verify_attention(
        batch, n, num_q_heads, num_kv_heads, head_dim, page_size, dtype, float(sm_scale), *args,
        num_slots, *args2, _stream(stream)))


def spec_accept_workspace_size(batch, num_draft_tokens, vocab, sampled) -> int:
    return _lib.spec_accept_workspace_size(batch, num_draft_tokens, vocab, int(bool(sampled)))


def spec_accept_greedy(batch, num_draft_tokens, accept_width, vocab, dtype, target_logits,
                       candidates, retrieve_index, retrieve_next_token, retrieve_next_sibling,
                       predict, accept_index, accept_length, target_predict=None,
                       workspace=None, workspace_bytes=None, dev_status=None, stream=None):
    dev = _device()
    n = num_draft_tokens
    bn = batch * n
    need_ws = spec_accept_workspace_size(batch, n, vocab, 0)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [
        _ptr(target_logits, "target_logits", dev, nbytes=bn * vocab * _ELEM.get(dtype, 4)),
        _ptr(candidates, "candidates", dev, nbytes=bn * 4),
        _ptr(retrieve_index, "retrieve_index", dev, nbytes=bn * 4),
        _ptr(retrieve_next_token, "retrieve_next_token", dev, nbytes=bn * 4),
        _ptr(retrieve_next_sibling, "retrieve_next_sibling", dev, nbytes=bn * 4),
        _ptr(predict, "predict", dev, nbytes=bn * 4),
        _ptr(accept_index, "accept_index", dev, nbytes=batch * accept_width * 4),
        _ptr(accept_length, "accept_length", dev, nbytes=batch * 4),
        _ptr(target_predict, "target_predict", dev, nbytes=bn * 4, optional=True),
        _ptr(workspace, "workspace", dev, nbytes=need_ws, optional=batch == 0),
        workspace_bytes,
        _ptr(dev_status, "dev_status", dev, nbytes=4, optional=True),
    ]
    _check("spec_accept_greedy", _lib.spec_accept_greedy(batch, n, accept_width, vocab, dtype,
                                                          *args, _stream(stream)))


def spec_accept_greedy_noalloc(batch, num_draft_tokens, accept_width, vocab, dtype,
                               target_logits, candidates, retrieve_index, retrieve_next_token,
                               retrieve_next_sibling, predict, accept_index, accept_length,
                               target_predict=None, dev_status=None, stream=None):
    dev = _device()
    n = num_draft_tokens
    bn = batch * n
    args = [
        _ptr(target_logits, "target_logits", dev, nbytes=bn * vocab * _ELEM.get(dtype, 4)),
        _ptr(candidates, "candidates", dev, nbytes=bn * 4),
        _ptr(retrieve_index, "retrieve_index", dev, nbytes=bn * 4),
        _ptr(retrieve_next_token, "retrieve_next_token", dev, nbytes=bn * 4),
        _ptr(retrieve_next_sibling, "retrieve_next_sibling", dev, nbytes=bn * 4),
        _ptr(predict, "predict", dev, nbytes=bn * 4),
        _ptr(accept_index, "accept_index", dev, nbytes=batch * accept_width * 4),
        _ptr(accept_length, "accept_length", dev, nbytes=batch * 4),
        _ptr(target_predict, "target_predict", dev, nbytes=bn * 4, optional=True),
        _ptr(dev_status, "dev_status", dev, nbytes=4, optional=True),
    ]
    _check("spec_accept_greedy_noalloc",
           _lib.spec_accept_greedy_noalloc(batch, n, accept_width, vocab, dtype, *args,
                                           _stream(stream)))


def spec_accept_sample(batch, num_draft_tokens, accept_width, vocab, dtype, target_logits,
                       draft_logits, temperature, uniforms, final_uniforms, candidates,
                       retrieve_index, retrieve_next_token, retrieve_next_sibling, predict,
                       accept_index, accept_length, workspace=None, workspace_bytes=None,
                       dev_status=None, stream=None):
    dev = _device()
    n = num_draft_tokens
    bn = batch * n
    lb = bn * vocab * _ELEM.get(dtype, 4)
    need_ws = spec_accept_workspace_size(batch, n, vocab, 1)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [
        _ptr(target_logits, "target_logits", dev, nbytes=lb),
        _ptr(draft_logits, "draft_logits", dev, nbytes=lb, optional=True),
        _ptr(temperature, "temperature", dev, nbytes=batch * 4),
        _ptr(uniforms, "uniforms", dev, nbytes=bn * 4),
        _ptr(final_uniforms, "final_uniforms", dev, nbytes=batch * 4),
        _ptr(candidates, "candidates", dev, nbytes=bn * 4),
        _ptr(retrieve_index, "retrieve_index", dev, nbytes=bn * 4),
        _ptr(retrieve_next_token, "retrieve_next_token", dev, nbytes=bn * 4),
        _ptr(retrieve_next_sibling, "retrieve_next_sibling", dev, nbytes=bn * 4),
        _ptr(predict, "predict", dev, nbytes=bn * 4),
        _ptr(accept_index, "accept_index", dev, nbytes=batch * accept_width * 4),
        _ptr(accept_length, "accept_length", dev, nbytes=batch * 4),
        _ptr(workspace, "workspace", dev, nbytes=need_ws, optional=batch == 0),
        workspace_bytes,
        _ptr(dev_status, "dev_status", dev, nbytes=4, optional=True),
    ]
    _check("spec_accept_sample", _lib.spec_accept_sample(batch, n, accept_width, vocab, dtype,
                                                          *args, _stream(stream)))


def spec_accept_target_only_workspace_size(batch, num_draft_tokens, vocab) -> int:
    return _lib.spec_accept_target_only_workspace_size(batch, num_draft_tokens, vocab)


def spec_accept_target_only(batch, num_draft_tokens, accept_width, vocab, dtype, target_logits,
                            temperature, threshold_single, threshold_acc, uniforms,
                            final_uniforms, candidates, retrieve_index, retrieve_next_token,
                            retrieve_next_sibling, predict, accept_index, accept_length,
                            workspace=None, workspace_bytes=None, dev_status=None, stream=None):
    dev = _device()
    n = num_draft_tokens
    bn = batch * n
    lb = bn * vocab * _ELEM.get(dtype, 4)
    need_ws = spec_accept_target_only_workspace_size(batch, n, vocab)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [
        _ptr(target_logits, "target_logits", dev, nbytes=lb),
        _ptr(temperature, "temperature", dev, nbytes=batch * 4),
        float(threshold_single),
        float(threshold_acc),
        _ptr(uniforms, "uniforms", dev, nbytes=bn * 4),
        _ptr(final_uniforms, "final_uniforms", dev, nbytes=batch * 4),
        _ptr(candidates, "candidates", dev, nbytes=bn * 4),
        _ptr(retrieve_index, "retrieve_index", dev, nbytes=bn * 4),
        _ptr(retrieve_next_token, "retrieve_next_token", dev, nbytes=bn * 4),
        _ptr(retrieve_next_sibling, "retrieve_next_sibling", dev, nbytes=bn * 4),
        _ptr(predict, "predict", dev, nbytes=bn * 4),
        _ptr(accept_index, "accept_index", dev, nbytes=batch * accept_width * 4),
        _ptr(accept_length, "accept_length", dev, nbytes=batch * 4),
        _ptr(workspace, "workspace", dev, nbytes=need_ws, optional=batch == 0),
        workspace_bytes,
        _ptr(dev_status, "dev_status", dev, nbytes=4, optional=True),
    ]
    _check("spec_accept_target_only", _lib.spec_accept_target_only(
        batch, n, accept_width, vocab, dtype, *args, _stream(stream)))


def spec_draft_step_workspace_size(batch, topk, vocab) -> int:
    return _lib.spec_draft_step_workspace_size(batch, topk, vocab)


def spec_draft_step(batch, topk, num_steps, step, vocab, dtype, draft_logits, branch_scores,
                    scores, tokens, parents, next_scores, next_tokens, workspace=None,
                    workspace_bytes=None, dev_status=None, stream=None):
    dev = _device()
    rows = 1 if step == 0 else topk
    ncand = topk + (num_steps - 1) * topk * topk
    npar = 1 + (num_steps - 1) * topk
    need_ws = spec_draft_step_workspace_size(batch, topk, vocab)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    none = batch == 0
    args = [
        _ptr(draft_logits, "draft_logits", dev, nbytes=batch * rows * vocab * _ELEM.get(dtype, 4),
             optional=none),
        _ptr(branch_scores, "branch_scores", dev, nbytes=batch * topk * 4,
             optional=none or step == 0),
        _ptr(scores, "scores", dev, nbytes=batch * ncand * 4, optional=none),
        _ptr(tokens, "tokens", dev, nbytes=batch * ncand * 4, optional=none),
        _ptr(parents, "parents", dev, nbytes=batch * npar * 4,
             optional=none or step >= num_steps - 1),
        _ptr(next_scores, "next_scores", dev, nbytes=batch * topk * 4, optional=none),
        _ptr(next_tokens, "next_tokens", dev, nbytes=batch * topk * 4, optional=none),
        _ptr(workspace, "workspace", dev, nbytes=need_ws, optional=batch == 0),
        workspace_bytes,
        _ptr(dev_status, "dev_status", dev, nbytes=4, optional=True),
    ]
    _check("spec_draft_step", _lib.spec_draft_step(batch, topk, num_steps, step, vocab, dtype,
                                                    *args, _stream(stream)))


def spec_sampling_filter_workspace_size(batch, num_draft_tokens, vocab) -> int:
    return _lib.spec_sampling_filter_workspace_size(batch, num_draft_tokens, vocab)


def spec_sampling_filter(batch, num_draft_tokens, vocab, dtype, logits, temperature, top_k,
                         top_p, out, workspace=None, workspace_bytes=None, dev_status=None,
                         stream=None):
    dev = _device()
    rows = batch * num_draft_tokens
    lb = rows * vocab * _ELEM.get(dtype, 4)
    none = batch == 0
    need_ws = spec_sampling_filter_workspace_size(batch, num_draft_tokens, vocab)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [
        _ptr(logits, "logits", dev, nbytes=lb, optional=none),
        _ptr(temperature, "temperature", dev, nbytes=batch * 4, optional=none),
        _ptr(top_k, "top_k", dev, nbytes=batch * 4, optional=none),
        _ptr(top_p, "top_p", dev, nbytes=batch * 4, optional=none),
        _ptr(out, "out", dev, nbytes=lb, optional=none),
        _ptr(workspace, "workspace", dev, nbytes=need_ws, optional=need_ws == 0),
        workspace_bytes,
        _ptr(dev_status, "dev_status", dev, nbytes=4, optional=True),
    ]
    _check("spec_sampling_filter", _lib.spec_sampling_filter(batch, num_draft_tokens, vocab, dtype,
                                                              *args, _stream(stream)))


def spec_full_mask(batch, num_draft_tokens, seq_lens, max_seq_len, tree_mask_bits, fill_prefix,
                   full_mask, dev_status=None, stream=None):
    dev = _device()
    n = num_draft_tokens
    wb = max(1, spec_mask_word_bytes(n))
    none = batch == 0
    args = [
        _ptr(seq_lens, "seq_lens", dev, nbytes=batch * 4, optional=none),
        max_seq_len,
        _ptr(tree_mask_bits, "tree_mask_bits", dev, nbytes=batch * n * wb, optional=none),
        1 if fill_prefix else 0,
        _ptr(full_mask, "full_mask", dev, optional=none),
        0 if full_mask is None else full_mask.numel() * full_mask.element_size(),
        _ptr(dev_status, "dev_status", dev, nbytes=4, optional=True),
    ]
    _check("spec_full_mask", _lib.spec_full_mask(batch, n, *args, _stream(stream)))


def spec_plan_draft_branches(batch, topk, num_steps, page_size, num_layers, num_kv_heads,
                             head_dim, dtype, k_pool, v_pool, num_slots, seq_lens, page_table,
                             max_pages, branch_pages, pages_per_branch, out_cache_loc,
                             dev_status=None, stream=None):
    dev = _device()
    pool = num_layers * num_slots * num_kv_heads * head_dim * _ELEM.get(dtype, 4)
    none = batch == 0
    args = [
        _ptr(k_pool, "k_pool", dev, nbytes=pool, optional=none),
        _ptr(v_pool, "v_pool", dev, nbytes=pool, optional=none),
        num_slots,
        _ptr(seq_lens, "seq_lens", dev, nbytes=batch * 4, optional=none),
        _ptr(page_table, "page_table", dev, nbytes=batch * max_pages * 4, optional=none),
        max_pages,
        _ptr(branch_pages, "branch_pages", dev, nbytes=batch * topk * pages_per_branch * 4,
             optional=none or topk == 1),
        pages_per_branch,
        _ptr(out_cache_loc, "out_cache_loc", dev, nbytes=batch * topk * num_steps * 4,
             optional=none),
        _ptr(dev_status, "dev_status", dev, nbytes=4, optional=True),
    ]
    _check("spec_plan_draft_branches", _lib.spec_plan_draft_branches(
        batch, topk, num_steps, page_size, num_layers, num_kv_heads, head_dim, dtype, *args,
        _stream(stream)))


def spec_compact_kv(batch, num_draft_tokens, accept_width, num_layers, num_kv_heads, head_dim,
                    page_size, dtype, k_pool, v_pool, num_slots, page_table, max_pages,
                    seq_lens, out_cache_loc, accept_index, accept_length, new_seq_lens,
                    free_slots, num_free, dev_status=None, stream=None):
    dev = _device()
    n = num_draft_tokens
    pool = num_layers * num_slots * num_kv_heads * head_dim * _ELEM.get(dtype, 4)
    args = [
        _ptr(k_pool, "k_pool", dev, nbytes=pool),
        _ptr(v_pool, "v_pool", dev, nbytes=pool),
    ]
    args2 = [
        _ptr(page_table, "page_table", dev, nbytes=batch * max_pages * 4),
        max_pages,
        _ptr(seq_lens, "seq_lens", dev, nbytes=batch * 4),
        _ptr(out_cache_loc, "out_cache_loc", dev, nbytes=batch * n * 4),
        _ptr(accept_index, "accept_index", dev, nbytes=batch * accept_width * 4),
        _ptr(accept_length, "accept_length", dev, nbytes=batch * 4),
        _ptr(new_seq_lens, "new_seq_lens", dev, nbytes=batch * 4),
        _ptr(free_slots, "free_slots", dev, nbytes=batch * n * 4),
        _ptr(num_free, "num_free", dev, nbytes=batch * 4),
        _ptr(dev_status, "dev_status", dev, nbytes=4, optional=True),
    ]
    _check("spec_compact_kv", _lib.spec_compact_kv(batch, n, accept_width, num_layers,
                                                    num_kv_heads, head_dim, page_size, dtype,
                                                    *args, num_slots, *args2, _stream(stream)))
