"""GPU parity of the compressed-key path: herald_compress_keys against the oracle's
mean-pooled windows, and herald_select_compressed against the oracle's block-granular
selection (band test on the token scores, candidate scores, and whole blocks taken
from their lowest token up)."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle.herald_oracle as orc
from block_diffusion_sparse_herald_amd import herald as H
from block_diffusion_sparse_herald_amd.inputs import WORKLOADS, Workload, bf16_bits_to_f32, make_batch
from block_diffusion_sparse_herald_amd.runner import BlockRunner, batch_to_device
from parity import band_check

pytestmark = pytest.mark.gpu

BASE = WORKLOADS["gqa32x8_L32768_b1"]
CASES = {
    # (workload, ksize, stride)
    "overlap_32_16": (BASE.with_(name="cmp_overlap", L=5000, nseq=2, C=1000, topk=300, T=1), 32, 16),
    "ragged_g7_24_8": (WORKLOADS["gqa28x4_ragged16k-64k_b8"].with_(name="cmp_ragged", L=6000, L_min=1500, nseq=3,
                                                                  C=1024, topk=333, T=1), 24, 8),
    "f32_8_4": (WORKLOADS["tiny_f32_L4096"], 8, 4),
    "d64_gaps_4_6": (Workload("cmp_d64", nseq=2, L=3000, Hq=8, Hkv=2, d=64, dtype="bf16", B=16, C=600, topk=130,
                              T=1, planted=8, seed_base=9400), 4, 6),
    # longer than the LDS top-C: the radix passes and the bitmap emission
    "long_16_16": (Workload("cmp_long", nseq=1, L=50000, Hq=8, Hkv=2, d=128, dtype="bf16", B=4, C=2000, topk=100,
                            T=1, planted=8, seed_base=9500), 16, 16),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def widen(a: np.ndarray) -> np.ndarray:
    return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


@pytest.fixture(scope="module", autouse=True)
def _lib(gpu_lib):
    yield


@pytest.mark.parametrize("name", list(CASES))
def test_compressed_selection(name):
    wl, ksize, stride = CASES[name]
    batch = make_batch(wl)
    dev = batch_to_device(batch)
    r = BlockRunner(batch.seq_start, wl.B, wl.Hq, wl.Hkv, wl.d, wl.C, wl.topk, wl.dtype)
    rows = H.herald_compressed_rows(r.problem, stride)
    k_comp = torch.empty((rows, wl.Hkv, wl.d), dtype=torch.float32, device="cuda")
    H.herald_compress_keys(r.problem, dev["k_cache"], ksize, stride, k_comp)
    ws = torch.empty((H.herald_workspace_size(r.problem, H.HERALD_OP_SELECT_COMPRESSED),), dtype=torch.uint8,
                     device="cuda")
    H.herald_select_compressed(r.problem, dev["q0"], k_comp, stride, r.cand, r.cand_score, ws)
    torch.cuda.synchronize()
    kc = k_comp.cpu().numpy().astype(np.float64)
    cand = r.cand.cpu().numpy().astype(np.int64)
    cscore = r.cand_score.cpu().numpy()
    scale = orc.default_scale(wl.d)
    off = 0
    for s in range(wl.nseq):
        a, e = int(batch.seq_start[s]), int(batch.seq_start[s + 1])
        L = e - a
        k = widen(batch.k_cache[a:e])
        want_kc = orc.compress_keys(k, ksize, stride)
        M = want_kc.shape[0]
        np.testing.assert_allclose(kc[off:off + M], want_kc, rtol=1e-5, atol=1e-6, err_msg=f"{name} s{s} k_comp")
        off += M
        _, S_tok, _ = orc.select_compressed(widen(batch.q0[s]), k, wl.C, scale, ksize, stride)
        band = 0
        for g in range(wl.Hkv):
            band += band_check(cand[s, g], S_tok[g], wl.C, what=f"{name} s{s} g{g} compressed candidates")
            np.testing.assert_allclose(cscore[s, g], S_tok[g][cand[s, g]], rtol=1e-4, atol=1e-30)
            # every block contributes a prefix of its tokens (ties go to the lower index)
            blocks = cand[s, g] // stride
            for m in np.unique(blocks):
                toks = cand[s, g][blocks == m]
                assert toks.tolist() == list(range(m * stride, m * stride + toks.size)), (name, s, g, m)
            partial = [m for m in np.unique(blocks)
                       if (blocks == m).sum() < min(stride, L - m * stride)]
            assert len(partial) <= 1, f"{name} s{s} g{g}: more than one partly selected block"
        log(f"  {name} s{s}: {M} blocks, band {band}")
    assert off == rows
