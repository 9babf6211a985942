"""GPU parity of the exact layer baselines the library expresses through the same calls.

  MAGE-exact selection: herald_refine_topk over every key of the sequence (candidate
  set = 0..L-1, so C = L), then gather and attention over the top-K. Checked with the
  band test against the oracle's refine scores over all keys (the exact top-K of the
  real queries), and the attention against the oracle on the GPU's subset.
  Dense attention: herald_block_attn with topk = L over the gathered whole cache,
  against the oracle's attention over every key.
Sizes put the candidate set on both sides of 16384 (the LDS-staged top-K and the
global-memory one) and the dense subset over several key ranges.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle.herald_oracle as orc
from block_diffusion_sparse_herald_amd.inputs import Workload, bf16_bits_to_f32, make_batch
from block_diffusion_sparse_herald_amd.runner import BlockRunner, batch_to_device
from parity import ATOL, band_check, max_abs

pytestmark = pytest.mark.gpu

CASES = {
    "exact_L3000_bf16": Workload("exact_L3000_bf16", nseq=2, L=3000, Hq=8, Hkv=2, d=128, dtype="bf16", B=4, C=3000,
                                 topk=300, T=1, planted=4, seed_base=9100),
    "exact_L20000_bf16": Workload("exact_L20000_bf16", nseq=2, L=20000, Hq=8, Hkv=2, d=64, dtype="bf16", B=4,
                                  C=20000, topk=700, T=1, planted=4, seed_base=9200),
    "exact_L2500_f32": Workload("exact_L2500_f32", nseq=1, L=2500, Hq=4, Hkv=1, d=64, dtype="f32", B=8, C=2500,
                                topk=256, T=1, planted=4, seed_base=9300),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def widen(a: np.ndarray) -> np.ndarray:
    return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def iota(nseq: int, Hkv: int, n: int) -> torch.Tensor:
    return torch.arange(n, dtype=torch.int32, device="cuda").repeat(nseq, Hkv, 1).contiguous()


@pytest.fixture(scope="module", autouse=True)
def _lib(gpu_lib):
    yield


@pytest.mark.parametrize("name", list(CASES))
def test_mage_exact_selection(name):
    wl = CASES[name]
    batch = make_batch(wl)
    dev = batch_to_device(batch)
    L = wl.L
    r = BlockRunner(batch.seq_start, wl.B, wl.Hq, wl.Hkv, wl.d, L, wl.topk, wl.dtype)
    r.refine(dev["q0"], dev["k_cache"], cand=iota(wl.nseq, wl.Hkv, L))
    r.gather(dev["k_cache"], dev["v_cache"])
    out = torch.empty_like(r.out)
    r.attn(dev["q_steps"][0], dev["kb_steps"][0], dev["vb_steps"][0], out=out)
    torch.cuda.synchronize()
    sel, sel_score, got = to_np(r.sel).astype(np.int64), to_np(r.sel_score), to_np(out)
    scale = orc.default_scale(wl.d)
    for s in range(wl.nseq):
        a, e = int(batch.seq_start[s]), int(batch.seq_start[s + 1])
        q0, k, v = widen(batch.q0[s]), widen(batch.k_cache[a:e]), widen(batch.v_cache[a:e])
        all_keys = np.tile(np.arange(L), (wl.Hkv, 1))
        R = orc.refine_scores(q0, k, all_keys, scale)
        band = 0
        for g in range(wl.Hkv):
            band += band_check(sel[s, g], R[g], wl.topk, what=f"{name} s{s} g{g} exact top-K")
            np.testing.assert_allclose(sel_score[s, g], R[g][sel[s, g]], rtol=1e-4, atol=1e-30)
            assert set(batch.planted[s][g].tolist()) <= set(sel[s, g].tolist()), f"{name}: planted key dropped"
        ks, vs = orc.gather_kv(k, v, sel[s])
        want = orc.block_attention(widen(batch.q_steps[0, s]), widen(batch.kb_steps[0, s]),
                                   widen(batch.vb_steps[0, s]), ks, vs, scale)
        err = max_abs(widen(got[s]), want)
        assert err <= ATOL[wl.dtype], f"{name} s{s}: attention max abs error {err}"
        log(f"  {name} s{s}: band {band}, attention max abs err {err:.3g}")


@pytest.mark.parametrize("name", list(CASES))
def test_dense_attention(name):
    wl = CASES[name]
    batch = make_batch(wl)
    dev = batch_to_device(batch)
    L = wl.L
    r = BlockRunner(batch.seq_start, wl.B, wl.Hq, wl.Hkv, wl.d, L, L, wl.dtype)
    r.gather(dev["k_cache"], dev["v_cache"], sel=iota(wl.nseq, wl.Hkv, L))
    out = torch.empty_like(r.out)
    r.attn(dev["q_steps"][0], dev["kb_steps"][0], dev["vb_steps"][0], out=out)
    torch.cuda.synchronize()
    got = to_np(out)
    scale = orc.default_scale(wl.d)
    for s in range(wl.nseq):
        a, e = int(batch.seq_start[s]), int(batch.seq_start[s + 1])
        k, v = widen(batch.k_cache[a:e]), widen(batch.v_cache[a:e])
        ks = np.transpose(k, (1, 0, 2))
        vs = np.transpose(v, (1, 0, 2))
        want = orc.block_attention(widen(batch.q_steps[0, s]), widen(batch.kb_steps[0, s]),
                                   widen(batch.vb_steps[0, s]), ks, vs, scale)
        err = max_abs(widen(got[s]), want)
        assert err <= ATOL[wl.dtype], f"{name} s{s}: dense attention max abs error {err}"
        log(f"  {name} s{s}: dense attention over {L} + {wl.B} keys, max abs err {err:.3g} "
            f"({r.attn_splits} key ranges)")
