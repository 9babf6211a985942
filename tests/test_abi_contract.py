"""C-ABI contract on the CPU: the library loads, exports every declared symbol, and
rejects every invalid argument with the documented status before any HIP call.
No kernel is launched here (validation happens on the host first)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from block_diffusion_sparse_herald_amd import herald as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "herald.h")

# a fake device address: validation never dereferences seq_start_dev or tensor pointers
FAKE = 0x10000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(herald_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return H.load()


def prob(**kw):
    base = dict(seq_start=[0, 4096, 9000], B=32, Hq=8, Hkv=2, head_dim=128, C=512, topk=128, dtype=H.HERALD_BF16)
    base.update(kw)
    return H.make_problem(base.pop("seq_start"), seq_start_dev=FAKE, **base)


def status_of(fn, *args):
    with pytest.raises(H.HeraldError) as e:
        fn(*args)
    assert H.herald_last_error(), "error message must not be empty"
    return e.value.status


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(H.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", H.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (herald_\w+)", out))
    assert set(names) <= exported, set(names) - exported


def test_load_fails_loudly_when_missing():
    saved = H._lib
    H._lib = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            H.load("/nonexistent/libherald.so")
    finally:
        H._lib = saved


def test_workspace_sizes(lib):
    p = prob()
    for op in (H.HERALD_OP_SELECT, H.HERALD_OP_REFINE, H.HERALD_OP_GATHER_HOST):
        assert H.herald_workspace_size(p, op) > 0
    assert H.herald_workspace_size(p, H.HERALD_OP_ATTN) >= 0
    big = prob(seq_start=[0, 8192, 20000])
    assert H.herald_workspace_size(big, H.HERALD_OP_SELECT) > H.herald_workspace_size(p, H.HERALD_OP_SELECT)
    assert H.herald_workspace_size(prob(seq_start=[0]), H.HERALD_OP_SELECT) == 0
    assert status_of(H.herald_workspace_size, p, 99) == H.HERALD_ERR_INVALID_ARG


def test_workspace_bytes_matches_workspace_size(lib):
    """herald_workspace_bytes returns what herald_workspace_size writes, SIZE_MAX on error."""
    for p in (prob(), prob(seq_start=[0, 32768], Hq=32, Hkv=8, C=4096, topk=1024), prob(dtype=H.HERALD_F32),
              prob(seq_start=[0])):
        for op in (H.HERALD_OP_SELECT, H.HERALD_OP_REFINE, H.HERALD_OP_ATTN, H.HERALD_OP_GATHER_HOST,
                   H.HERALD_OP_SELECT_COMPRESSED):
            assert H.herald_workspace_bytes(p, op) == H.herald_workspace_size(p, op)
    assert H.herald_workspace_bytes(prob(), 99) == H.SIZE_MAX
    assert "unknown op" in H.herald_last_error()
    assert H.herald_workspace_bytes(prob(Hq=9), H.HERALD_OP_REFINE) == H.SIZE_MAX
    big = prob(C=30000, topk=30000, seq_start=[0, 30000, 61000])
    assert H.herald_workspace_bytes(big, H.HERALD_OP_SELECT) == H.SIZE_MAX  # selection takes C <= 16384


def test_subset_and_work_split_bounds(lib):
    """Subsets beyond 2^24 keys and attention work splits beyond the kernel's 32-bit
    workgroup numbering are refused on the host, before any launch."""
    n = 1 << 24
    ok = prob(seq_start=[0, n], B=1, Hq=8, Hkv=8, C=n, topk=n)
    assert H.herald_workspace_size(ok, H.HERALD_OP_ATTN) > 0
    over = prob(seq_start=[0, n + 1], B=1, Hq=8, Hkv=8, C=n + 1, topk=n + 1)
    assert status_of(H.herald_workspace_size, over, H.HERALD_OP_ATTN) == H.HERALD_ERR_UNSUPPORTED
    assert status_of(H.herald_block_attn, over, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, 0) == \
        H.HERALD_ERR_UNSUPPORTED
    assert status_of(H.herald_gather_kv, over, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None, None, None, 0, 0, None) == \
        H.HERALD_ERR_UNSUPPORTED
    # 200 sequences x 8 KV heads, 8193 key ranges each: 13.1M workgroups, beyond the decode
    wide = prob(seq_start=[i * n for i in range(201)], B=1, Hq=8, Hkv=8, C=n, topk=n)
    assert status_of(H.herald_workspace_size, wide, H.HERALD_OP_ATTN) == H.HERALD_ERR_UNSUPPORTED
    assert H.herald_workspace_bytes(wide, H.HERALD_OP_ATTN) == H.SIZE_MAX
    assert status_of(H.herald_block_attn, wide, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, 0) == \
        H.HERALD_ERR_UNSUPPORTED
    assert H.herald_workspace_size(wide, H.HERALD_OP_REFINE) > 0  # the other calls are not limited by it


def test_block_attn_static_contract(lib):
    """The allocation-free attention validates like herald_block_attn and refuses, before any
    HIP call, a problem whose attention workspace exceeds its static scratch."""
    p = prob()
    assert status_of(H.herald_block_attn_static, p, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0) == H.HERALD_ERR_INVALID_ARG
    assert status_of(H.herald_block_attn_static, p, FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, 0) == \
        H.HERALD_ERR_INVALID_ARG
    assert status_of(H.herald_block_attn_static, prob(Hq=9), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0) == \
        H.HERALD_ERR_INVALID_ARG
    H.herald_block_attn_static(prob(seq_start=[0]), None, None, None, None, None, None, 0)  # empty batch: no-op
    # dense attention over whole 32K caches: the split partials outgrow the static buffer
    n = 1
    while True:
        big = prob(seq_start=[32768 * i for i in range(n + 1)], Hq=32, Hkv=8, C=32768, topk=32768)
        if H.herald_workspace_size(big, H.HERALD_OP_ATTN) > H.HERALD_STATIC_SCRATCH_BYTES:
            break
        n += 1
    assert status_of(H.herald_block_attn_static, big, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0) == \
        H.HERALD_ERR_UNSUPPORTED
    assert "static" in H.herald_last_error()


def test_gather_status_word_checks(lib):
    """The device and GPU-read gathers take an optional 4-byte status word in ws."""
    p = prob()
    assert status_of(H.herald_gather_kv, p, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None, None, FAKE, 3, 0, None) == \
        H.HERALD_ERR_WORKSPACE
    assert status_of(H.herald_gather_kv, p, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None, None, FAKE + 2, 4, 0, None) == \
        H.HERALD_ERR_INVALID_ARG
    assert status_of(H.herald_gather_kv, p, FAKE, FAKE, 2, FAKE, FAKE, FAKE, None, None, FAKE, 3, 0, None) == \
        H.HERALD_ERR_WORKSPACE


def test_vsel_ld(lib):
    assert H.herald_vsel_ld(1) == 64
    assert H.herald_vsel_ld(64) == 64
    assert H.herald_vsel_ld(65) == 128
    assert H.herald_vsel_ld(1024) == 1024


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=9, Hkv=2), H.HERALD_ERR_INVALID_ARG),            # Hq % Hkv != 0
    (dict(Hq=1, Hkv=2), H.HERALD_ERR_INVALID_ARG),            # Hq < Hkv
    (dict(Hkv=0), H.HERALD_ERR_INVALID_ARG),
    (dict(Hq=18, Hkv=2), H.HERALD_ERR_UNSUPPORTED),           # G = 9 > 8
    (dict(B=64, Hq=16, Hkv=2), H.HERALD_ERR_UNSUPPORTED),     # B*G = 512 > 256
    (dict(B=0), H.HERALD_ERR_INVALID_ARG),
    (dict(B=65), H.HERALD_ERR_UNSUPPORTED),
    (dict(head_dim=96), H.HERALD_ERR_UNSUPPORTED),
    (dict(topk=513), H.HERALD_ERR_INVALID_ARG),               # topk > C
    (dict(topk=0), H.HERALD_ERR_INVALID_ARG),
    (dict(C=0, topk=0), H.HERALD_ERR_INVALID_ARG),
    (dict(C=5000, topk=10), H.HERALD_ERR_INVALID_ARG),        # C > L_0 = 4096
    (dict(dtype=7), H.HERALD_ERR_INVALID_ARG),
    (dict(seq_start=[1, 5000]), H.HERALD_ERR_INVALID_ARG),    # seq_start[0] != 0
    (dict(seq_start=[0, 5000, 4000]), H.HERALD_ERR_INVALID_ARG),  # negative length
    (dict(softmax_scale=-1.0), H.HERALD_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), H.HERALD_ERR_INVALID_ARG),
])
def test_invalid_problem(lib, kw, status):
    p = prob(**kw)
    assert status_of(H.herald_workspace_size, p, H.HERALD_OP_SELECT) == status
    assert status_of(H.herald_select_merged, p, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, 0) == status
    assert status_of(H.herald_select_query, p, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, 0) == status
    assert status_of(H.herald_select_compressed, p, FAKE, FAKE, 16, FAKE, None, FAKE, 1 << 40, 0) == status
    assert status_of(H.herald_compress_keys, p, FAKE, 32, 16, FAKE, 0) == status
    assert H.herald_compressed_rows(p, 16) == -1
    assert status_of(H.herald_refine_topk, p, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, 0) == status
    assert status_of(H.herald_block_attn, p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, 0) == status
    assert status_of(H.herald_gather_kv, p, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None, None, None, 0, 0, None) == status


def test_candidate_limit_is_the_selections_only(lib):
    """C > 16384 is refused by the merged-query selection (its emission keeps C in LDS) and
    accepted by the other calls: refine over a whole sequence, attention over the whole cache."""
    p = prob(C=30000, topk=30000, seq_start=[0, 30000, 61000])
    assert status_of(H.herald_workspace_size, p, H.HERALD_OP_SELECT) == H.HERALD_ERR_UNSUPPORTED
    assert status_of(H.herald_select_merged, p, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, 0) == H.HERALD_ERR_UNSUPPORTED
    assert H.herald_workspace_size(p, H.HERALD_OP_REFINE) > 0
    assert H.herald_workspace_size(p, H.HERALD_OP_ATTN) > 0
    assert H.herald_workspace_size(p, H.HERALD_OP_GATHER_HOST) > 0
    assert H.herald_attn_splits(p) > 1


def test_compressed_keys_contract(lib):
    p = prob()  # lengths 4096 and 4904
    assert H.herald_compressed_rows(p, 16) == 256 + 307
    assert H.herald_compressed_rows(p, 4096) == 1 + 2
    assert H.herald_compressed_rows(p, 1) == -1
    n = H.herald_workspace_size(p, H.HERALD_OP_SELECT_COMPRESSED)
    assert n > 0
    for stride, ksize in [(1, 8), (0, 8), (65537, 8), (16, 0), (16, 65537)]:
        assert status_of(H.herald_compress_keys, p, FAKE, ksize, stride, FAKE, 0) == H.HERALD_ERR_INVALID_ARG
    assert status_of(H.herald_select_compressed, p, FAKE, FAKE, 1, FAKE, None, FAKE, n, 0) == H.HERALD_ERR_INVALID_ARG
    assert status_of(H.herald_select_compressed, p, FAKE, None, 16, FAKE, None, FAKE, n, 0) == H.HERALD_ERR_INVALID_ARG
    assert status_of(H.herald_select_compressed, p, FAKE, FAKE, 16, FAKE, None, FAKE, n - 1, 0) == H.HERALD_ERR_WORKSPACE
    assert status_of(H.herald_compress_keys, p, None, 32, 16, FAKE, 0) == H.HERALD_ERR_INVALID_ARG
    big = prob(C=20000, topk=10, seq_start=[0, 30000])
    assert status_of(H.herald_workspace_size, big, H.HERALD_OP_SELECT_COMPRESSED) == H.HERALD_ERR_UNSUPPORTED


def test_negative_nseq_and_reserved(lib):
    p = prob()
    p.c.nseq = -1
    assert status_of(H.herald_workspace_size, p, H.HERALD_OP_SELECT) == H.HERALD_ERR_INVALID_ARG
    p = prob()
    p.c.reserved = 1
    assert status_of(H.herald_workspace_size, p, H.HERALD_OP_SELECT) == H.HERALD_ERR_INVALID_ARG
    p = prob()
    p.c.seq_start_dev = None
    assert status_of(H.herald_workspace_size, p, H.HERALD_OP_SELECT) == H.HERALD_ERR_INVALID_ARG
    with pytest.raises(H.HeraldError):
        H._check(H.load().herald_workspace_size(None, 0, ctypes.byref(ctypes.c_size_t())), "x")


def test_pointer_checks(lib):
    p = prob()
    ws = H.herald_workspace_size(p, H.HERALD_OP_SELECT)
    # NULL and misaligned operands
    assert status_of(H.herald_select_merged, p, None, FAKE, FAKE, None, FAKE, ws, 0) == H.HERALD_ERR_INVALID_ARG
    assert status_of(H.herald_select_merged, p, FAKE + 8, FAKE, FAKE, None, FAKE, ws, 0) == H.HERALD_ERR_INVALID_ARG
    assert status_of(H.herald_select_merged, p, FAKE, FAKE, FAKE, FAKE + 4, FAKE, ws, 0) == H.HERALD_ERR_INVALID_ARG
    assert status_of(H.herald_select_query, p, None, FAKE, FAKE, None, FAKE, ws, 0) == H.HERALD_ERR_INVALID_ARG
    assert status_of(H.herald_select_query, p, FAKE + 8, FAKE, FAKE, None, FAKE, ws, 0) == H.HERALD_ERR_INVALID_ARG
    assert status_of(H.herald_select_query, p, FAKE, FAKE, FAKE, None, FAKE, ws - 1, 0) == H.HERALD_ERR_WORKSPACE
    # workspace too small / missing
    assert status_of(H.herald_select_merged, p, FAKE, FAKE, FAKE, None, FAKE, ws - 1, 0) == H.HERALD_ERR_WORKSPACE
    assert status_of(H.herald_select_merged, p, FAKE, FAKE, FAKE, None, None, ws, 0) == H.HERALD_ERR_WORKSPACE
    rws = H.herald_workspace_size(p, H.HERALD_OP_REFINE)
    assert status_of(H.herald_refine_topk, p, FAKE, FAKE, FAKE, FAKE, None, FAKE, rws - 1, 0) == H.HERALD_ERR_WORKSPACE
    assert status_of(H.herald_refine_topk, p, FAKE, FAKE, None, FAKE, None, FAKE, rws, 0) == H.HERALD_ERR_INVALID_ARG
    assert status_of(H.herald_block_attn, p, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, 0) == \
        H.HERALD_ERR_INVALID_ARG
    # gather: bad flag, host path without staging / event / workspace
    assert status_of(H.herald_gather_kv, p, FAKE, FAKE, 2, FAKE, FAKE, FAKE, None, None, None, 0, 0, None) == \
        H.HERALD_ERR_INVALID_ARG
    assert status_of(H.herald_gather_kv, p, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, 0, FAKE) == \
        H.HERALD_ERR_INVALID_ARG
    assert status_of(H.herald_gather_kv, p, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 0, None) == \
        H.HERALD_ERR_INVALID_ARG
    gws = H.herald_workspace_size(p, H.HERALD_OP_GATHER_HOST)
    assert status_of(H.herald_gather_kv, p, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, gws - 1, 0, FAKE) == \
        H.HERALD_ERR_WORKSPACE


def test_empty_batch_is_a_noop(lib):
    p = prob(seq_start=[0])
    H.herald_select_merged(p, None, None, None, None, None, 0, 0)
    H.herald_refine_topk(p, None, None, None, None, None, None, 0, 0)
    H.herald_gather_kv(p, None, None, 0, None, None, None, None, None, None, 0, 0, None)
    H.herald_block_attn(p, None, None, None, None, None, None, None, 0, 0)
    assert H.herald_last_error() == ""


def test_kernel_events_argument_checks(lib):
    assert status_of(H.herald_set_kernel_events, len(H.KERNEL_IDS), None, None) == H.HERALD_ERR_INVALID_ARG
    for kid in H.KERNEL_IDS.values():
        H.herald_set_kernel_events(kid, None, None)
    assert status_of(H.herald_set_kernel_events, -1, None, None) == H.HERALD_ERR_INVALID_ARG
    assert status_of(H.herald_set_kernel_events, 0, FAKE, None) == H.HERALD_ERR_INVALID_ARG
    H.herald_set_kernel_events(0, None, None)


def test_attn_splits_reported(lib):
    assert 1 <= H.herald_attn_splits(prob()) <= 32
    assert H.herald_attn_splits(prob(seq_start=[0])) >= 1  # empty batch: host geometry must not divide by zero
    assert H.herald_workspace_size(prob(seq_start=[0]), H.HERALD_OP_ATTN) == 0
    assert H.herald_attn_splits(prob(dtype=H.HERALD_F32)) == 1


@pytest.mark.parametrize("kw,splits", [
    # 1 x 32K, 32/8/128: few (sequence, KV head) pairs, 17 blocks in ranges of 3
    (dict(seq_start=[0, 32768], Hq=32, Hkv=8, C=4096, topk=1024), 6),
    # 16 x 32K: 256 workgroups without a split
    (dict(seq_start=[32768 * i for i in range(17)], Hq=32, Hkv=8, C=4096, topk=1024), 1),
    # 4 x 128K: aimed at one workgroup per compute unit, 17 blocks in 4 ranges
    (dict(seq_start=[131072 * i for i in range(5)], Hq=32, Hkv=8, C=8192, topk=1024), 4),
    # 8 ragged sequences, 28/4/128, K = 2048: 33 blocks, at most 32 per range
    (dict(seq_start=[0, 16384, 40000, 65536, 90000, 120000, 150000, 200000, 240000], Hq=28, Hkv=4, C=4096,
          topk=2048), 2),
    # dense attention over a whole 32K cache: 513 blocks, at most 32 per range
    (dict(seq_start=[0, 32768], Hq=32, Hkv=8, C=32768, topk=32768), 17),
])
def test_attn_split_geometry(lib, kw, splits):
    """Key ranges the attention call splits each (sequence, KV head) into, for the
    benchmark workloads' shapes (host-side geometry only)."""
    assert H.herald_attn_splits(prob(**kw)) == splits


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "block_diffusion_sparse_herald_amd")
    pat = re.compile(r"^\s*(import\s+oracle|from\s+oracle|from\s+\.+\s*import\s+oracle)|herald_oracle|#include.*oracle",
                     re.M)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not pat.search(text), f
