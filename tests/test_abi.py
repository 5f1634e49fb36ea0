"""The C-ABI library loads on a machine without a GPU, exports every entry
point include/spec.h declares, and rejects bad arguments on the host before
launching anything (no GPU)."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec.h")
LIB = os.path.join(ROOT, "speculative_decoding_build_amd", "libspecmi.so")


def _declared():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_five_calls():
    names = _declared()
    for call in ("spec_build_tree", "spec_verify_attention", "spec_accept_greedy",
                 "spec_accept_sample", "spec_compact_kv"):
        assert call in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_names_match_header():
    import speculative_decoding_build_amd as S
    assert set(S.EXPORTS) == set(_declared())
    for n in S.EXPORTS:
        assert callable(getattr(S, n))


def test_host_only_queries():
    import speculative_decoding_build_amd as S
    assert S.spec_version() >= 100
    for n in range(1, 65):
        assert S.spec_mask_word_bytes(n) * 8 == oracle.mask_word_bits(n)
    assert S.spec_mask_word_bytes(0) == 0 and S.spec_mask_word_bytes(65) == 0
    assert S.spec_accept_workspace_size(1, 64, 128256, 0) > 0
    # greedy: one 64-bit key per verify row
    assert S.spec_accept_workspace_size(5, 64, 128256, 0) == 5 * 64 * 8
    assert S.spec_accept_workspace_size(1, 64, 128256, 1) > S.spec_accept_workspace_size(1, 64, 128256, 0)
    # one (max, sum) pair of 64-bit words per verify row and 8192-entry chunk
    assert S.spec_accept_target_only_workspace_size(1, 64, 128256) == 64 * 16 * 16
    assert S.spec_accept_target_only_workspace_size(0, 64, 128256) == 0
    # 80 bytes (max, sum, up to 8 keys) per branch row and 2048-entry chunk,
    # rounded up to 256 bytes
    assert S.spec_draft_step_workspace_size(1, 8, 128256) == -(-8 * 63 * 80 // 256) * 256
    assert S.spec_draft_step_workspace_size(0, 8, 128256) == 0
    # a single split needs no workspace; a long history does
    assert S.spec_verify_attention_workspace_size(2, 6, 2, 1, 64, 64, S.SPEC_F32) >= 0
    assert S.spec_verify_attention_workspace_size(4, 64, 64, 8, 128, 131072, S.SPEC_BF16) > 0
    assert S.spec_verify_attention_workspace_size(1, 4, 6, 4, 128, 16, S.SPEC_BF16) == 0  # hq % hkv


def _c():
    lib = ctypes.CDLL(LIB)
    import speculative_decoding_build_amd  # noqa: F401  (declares argtypes on its own handle)
    return lib


P0 = ctypes.c_void_p(0)


def test_host_errors_before_launch():
    lib = ctypes.CDLL(LIB)
    I = ctypes.c_int
    bt = lib.spec_build_tree
    bt.restype = I
    # num_draft_tokens above 64, zero topk, bad mask mode, n-1 > ncand, batch 0
    assert bt(1, 2, 3, 65, 2, *([P0] * 14)) == -4
    assert bt(1, 0, 3, 6, 2, *([P0] * 14)) == -2
    assert bt(1, 2, 3, 6, 7, *([P0] * 14)) == -2
    assert bt(1, 1, 1, 3, 2, *([P0] * 14)) == -2
    assert bt(0, 2, 3, 6, 2, *([P0] * 14)) == 0
    assert bt(1, 2, 3, 6, 2, *([P0] * 14)) == -1
    va = lib.spec_verify_attention
    va.restype = I
    va.argtypes = [I, I, I, I, I, I, I, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, I, ctypes.c_void_p, I,
                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    args = dict(b=1, n=6, hq=2, hkv=1, d=64, ps=1, dt=1)

    def call(**kw):
        a = dict(args, **kw)
        return va(a["b"], a["n"], a["hq"], a["hkv"], a["d"], a["ps"], a["dt"], 0.0, P0, P0, P0,
                  100, P0, 70, P0, 64, P0, P0, P0, P0, 0, P0, P0)
    assert call(hq=3, hkv=2) == -2          # heads not grouped evenly
    assert call(d=96) == -4                 # head_dim unsupported
    assert call(n=65) == -4
    assert call(dt=5) == -3
    assert call(b=0) == 0
    assert call() == -1                     # null tensors
    ag = lib.spec_accept_greedy
    ag.restype = I
    ag.argtypes = [I, I, I, ctypes.c_int64, I] + [ctypes.c_void_p] * 10 + [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert ag(1, 6, 4, 32, 9, *([P0] * 10), 0, P0, P0) == -3
    assert ag(1, 6, 4, 32, 0, *([P0] * 10), 0, P0, P0) == -1
    assert ag(0, 6, 4, 32, 0, *([P0] * 10), 0, P0, P0) == 0
    na = lib.spec_accept_greedy_noalloc
    na.restype = I
    na.argtypes = [I, I, I, ctypes.c_int64, I] + [ctypes.c_void_p] * 11
    f10 = [ctypes.c_void_p(0x1000)] * 9 + [P0, P0]
    assert na(1, 6, 4, 32, 9, *f10) == -3
    assert na(1, 6, 4, 32, 0, *([P0] * 11)) == -1
    assert na(0, 6, 4, 32, 0, *([P0] * 11)) == 0
    # 513 requests x 64 nodes: more row keys than the library's fixed array
    # holds (32768)
    assert na(513, 64, 7, 128256, 1, *f10) == -5
    assert na(32769, 1, 2, 128256, 1, *f10) == -5
    asm = lib.spec_accept_sample
    asm.restype = I
    asm.argtypes = [I, I, I, ctypes.c_int64, I] + [ctypes.c_void_p] * 12 + [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    # missing draft distribution: the pages raise; here a NULL error code
    fake = ctypes.c_void_p(0x1000)
    ptrs = [fake] * 12
    ptrs[1] = P0
    assert asm(1, 6, 4, 32, 0, *ptrs, 1 << 20, fake, P0) == -1
    to = lib.spec_accept_target_only
    to.restype = I
    to.argtypes = ([I, I, I, ctypes.c_int64, I, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                    ctypes.c_float] + [ctypes.c_void_p] * 10 + [ctypes.c_size_t, ctypes.c_void_p,
                                                                ctypes.c_void_p])
    fake = ctypes.c_void_p(0x1000)
    big = 1 << 20
    assert to(1, 6, 4, 32, 0, fake, fake, 1.0, 0.0, *([fake] * 10), big, P0, P0) == -2   # threshold_acc <= 0
    assert to(1, 6, 4, 32, 9, fake, fake, 1.0, 1.0, *([fake] * 10), big, P0, P0) == -3
    assert to(1, 6, 4, 32, 0, P0, fake, 1.0, 1.0, *([fake] * 10), big, P0, P0) == -1
    assert to(1, 6, 4, 32, 0, fake, fake, 1.0, 1.0, *([fake] * 10), 8, P0, P0) == -5     # workspace small
    assert to(1, 99, 4, 32, 0, fake, fake, 1.0, 1.0, *([fake] * 10), big, P0, P0) == -4
    assert to(0, 6, 4, 32, 0, P0, P0, 1.0, 1.0, *([P0] * 10), 0, P0, P0) == 0
    ds = lib.spec_draft_step
    ds.restype = I
    ds.argtypes = ([I, I, I, I, ctypes.c_int64, I] + [ctypes.c_void_p] * 8
                   + [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p])
    f8 = [fake] * 8
    assert ds(1, 4, 3, 3, 1000, 0, *f8, big, P0, P0) == -2          # step >= num_steps
    assert ds(1, 4, 3, 1, 1000, 9, *f8, big, P0, P0) == -3
    assert ds(1, 9, 3, 1, 1000, 0, *f8, big, P0, P0) == -4          # topk > 8
    assert ds(1, 4, 3, 1, 3, 0, *f8, big, P0, P0) == -2             # vocab < topk
    assert ds(1, 8, 3, 1, (1 << 21) + 1, 0, *f8, big, P0, P0) == -4  # 8 rows x 257 chunks
    nb = list(f8)
    nb[1] = P0
    assert ds(1, 4, 3, 1, 1000, 0, *nb, big, P0, P0) == -1          # branch scores at step 1
    npr = list(f8)
    npr[4] = P0
    assert ds(1, 4, 3, 1, 1000, 0, *npr, big, P0, P0) == -1         # parents before the last step
    assert ds(1, 4, 3, 1, 1000, 0, *f8, 8, P0, P0) == -5            # workspace small
    assert ds(0, 4, 3, 1, 1000, 0, *([P0] * 8), 0, P0, P0) == 0
    sf = lib.spec_sampling_filter
    sf.restype = I
    sf.argtypes = ([I, I, ctypes.c_int64, I] + [ctypes.c_void_p] * 6
                   + [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p])
    f5 = [ctypes.c_void_p(0x1000)] * 5
    assert sf(1, 4, 1000, 9, *f5, P0, 0, P0, P0) == -3
    assert sf(1, 4, 1 << 31, 0, *f5, P0, 0, P0, P0) == -4
    assert sf(1, 0, 1000, 0, *f5, P0, 0, P0, P0) == -2
    n5 = list(f5)
    n5[2] = P0
    assert sf(1, 4, 1000, 0, *n5, P0, 0, P0, P0) == -1
    assert sf(0, 4, 1000, 0, *([P0] * 5), P0, 0, P0, P0) == 0
    sfw = lib.spec_sampling_filter_workspace_size
    sfw.restype = ctypes.c_size_t
    sfw.argtypes = [I, I, ctypes.c_int64]
    need = sfw(1, 4, 128256)      # 16 chunks of 8016 entries per row
    assert need == 256 + 4 * 16 * 16 + 4 * 16 * 64 * 8 + 4 * 64 * 8
    assert sfw(1, 4, 8192) == 0 and sfw(1, 4, 524289) == 0 and sfw(0, 4, 128256) == 0
    assert sfw(1, 4, 8193) > 0 and sfw(1, 4, 524288) > 0
    assert sf(1, 4, 128256, 0, *f5, P0, 0, P0, P0) == -5                 # no workspace
    assert sf(1, 4, 128256, 0, *f5, ctypes.c_void_p(0x1000), need - 1, P0, P0) == -5
    assert sf(1, 4, 128256, 0, *f5, ctypes.c_void_p(0x1008), need, P0, P0) == -5   # misaligned
    fm = lib.spec_full_mask
    fm.restype = I
    fm.argtypes = [I, I, ctypes.c_void_p, I, ctypes.c_void_p, I, ctypes.c_void_p, ctypes.c_int64,
                   ctypes.c_void_p, ctypes.c_void_p]
    al16 = ctypes.c_void_p(0x1000)
    assert fm(1, 65, al16, 8, al16, 1, al16, 1 << 20, P0, P0) == -4        # n > 64
    assert fm(1, 0, al16, 8, al16, 1, al16, 1 << 20, P0, P0) == -2
    assert fm(1, 8, P0, 8, al16, 1, al16, 1 << 20, P0, P0) == -1
    assert fm(1, 8, al16, 8, al16, 1, ctypes.c_void_p(0x1001), 1 << 20, P0, P0) == -2
    assert fm(0, 8, P0, 8, P0, 1, P0, 0, P0, P0) == 0
    pb = lib.spec_plan_draft_branches
    pb.restype = I
    pb.argtypes = ([I] * 8 + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                              ctypes.c_void_p, I, ctypes.c_void_p, I, ctypes.c_void_p,
                              ctypes.c_void_p, ctypes.c_void_p])
    a6 = [al16] * 2
    assert pb(1, 2, 5, 4, 1, 8, 128, 1, *a6, 1024, al16, al16, 8, al16, 1, al16, P0, P0) == -2  # region small
    assert pb(1, 2, 5, 4, 1, 8, 128, 9, *a6, 1024, al16, al16, 8, al16, 2, al16, P0, P0) == -3
    assert pb(1, 2, 5, 4, 1, 1, 6, 0, *a6, 1024, al16, al16, 8, al16, 2, al16, P0, P0) == -4  # 24-byte rows
    assert pb(1, 2, 5, 4, 1, 8, 128, 1, *a6, 1024, al16, al16, 8, P0, 2, al16, P0, P0) == -1
    assert pb(0, 2, 5, 4, 1, 8, 128, 1, P0, P0, 1024, P0, P0, 8, P0, 2, P0, P0, P0) == 0
    assert pb(1, 2, 5, 4, 1, 8, 128, 1, *a6, 1 << 31, al16, al16, 8, al16, 2, al16, P0, P0) == -4
    ck = lib.spec_compact_kv
    ck.restype = I
    ck.argtypes = [I] * 8 + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, I] + [ctypes.c_void_p] * 9 + [ctypes.c_void_p]
    assert ck(1, 6, 4, 1, 1, 64, 1, 0, P0, P0, 100, P0, 8, *([P0] * 9), P0) == -1
    assert ck(1, 6, 99, 1, 1, 64, 1, 0, P0, P0, 100, P0, 8, *([P0] * 9), P0) == -4
    assert ck(1, 6, 4, 1, 1, 6, 1, 1, P0, P0, 100, P0, 8, *([P0] * 9), P0) == -4   # 12-byte rows


def test_binding_rejects_host_tensors():
    import torch
    import speculative_decoding_build_amd as S
    x = torch.zeros(16, dtype=torch.int32)
    with pytest.raises(ValueError):
        S.spec_build_tree(1, 1, 1, 2, S.SPEC_MASK_QLEN_BITS, x, x, x, x, x, x, x, x, x, x, x)
