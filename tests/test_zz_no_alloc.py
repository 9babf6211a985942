"""The allocation-free attention entry point (herald_block_attn_static, static device
scratch) against herald_block_attn with a caller workspace, through the C ABI: two calls
in a row, the second with a smaller input, both splitting the keys so that the scratch
holds the partial results. Outputs must be bit-identical, and within the attention
tolerance of the oracle on the same subset."""

import numpy as np
import pytest
import torch

import oracle.herald_oracle as orc
from block_diffusion_sparse_herald_amd import herald as H
from block_diffusion_sparse_herald_amd.inputs import Workload, bf16_bits_to_f32, make_batch
from block_diffusion_sparse_herald_amd.runner import BlockRunner, batch_to_device
from parity import ATOL, max_abs

pytestmark = pytest.mark.gpu

CASES = [
    Workload("static_1x32k_g4", nseq=1, L=32768, Hq=32, Hkv=8, d=128, dtype="bf16", B=32, C=4096, topk=1024, T=1,
             seed_base=9100),
    Workload("static_2x3k_d64", nseq=2, L=3000, Hq=8, Hkv=2, d=64, dtype="bf16", B=16, C=600, topk=300, T=1,
             seed_base=9200),
]


def widen(a):
    return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def test_block_attn_static_matches_block_attn(gpu_lib):
    for wl in CASES:
        batch = make_batch(wl)
        dev = batch_to_device(batch)
        r = BlockRunner(batch.seq_start, wl.B, wl.Hq, wl.Hkv, wl.d, wl.C, wl.topk, wl.dtype)
        need = H.herald_workspace_size(r.problem, H.HERALD_OP_ATTN)
        assert 0 < need <= H.HERALD_STATIC_SCRATCH_BYTES, need
        rng = np.random.default_rng(wl.seed_base)
        L = batch.lengths
        sel = np.stack([np.stack([np.sort(rng.choice(int(L[s]), wl.topk, replace=False)) for _ in range(wl.Hkv)])
                        for s in range(wl.nseq)]).astype(np.int32)
        r.gather(dev["k_cache"], dev["v_cache"], sel=torch.from_numpy(sel).cuda())
        q, kb, vb = dev["q_steps"][0], dev["kb_steps"][0], dev["vb_steps"][0]
        want = torch.empty_like(r.out)
        got = torch.full_like(r.out, 7.0)
        H.herald_block_attn(r.problem, q, kb, vb, r.k_sel, r.v_sel, want, r.ws["attn"])
        H.herald_block_attn_static(r.problem, q, kb, vb, r.k_sel, r.v_sel, got)
        torch.cuda.synchronize()
        assert torch.equal(want.view(torch.int16), got.view(torch.int16)), f"{wl.name}: outputs differ"
        out = widen(got.cpu().view(torch.int16).numpy().view(np.uint16))
        scale = orc.default_scale(wl.d)
        for s in range(wl.nseq):
            a, e = int(batch.seq_start[s]), int(batch.seq_start[s + 1])
            ks, vs = orc.gather_kv(widen(batch.k_cache[a:e]), widen(batch.v_cache[a:e]), sel[s].astype(np.int64))
            ref = orc.block_attention(widen(batch.q_steps[0, s]), widen(batch.kb_steps[0, s]),
                                      widen(batch.vb_steps[0, s]), ks, vs, scale)
            err = max_abs(out[s], ref)
            assert err <= ATOL[wl.dtype], f"{wl.name} s{s}: {err}"
