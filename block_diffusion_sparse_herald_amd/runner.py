"""Device buffers and the per-block call sequence, on top of the C ABI.

PyTorch provides device memory and streams only; all compute happens in
libherald.so. ``BlockRunner`` owns the outputs and workspaces of one batch shape
and issues, per block: herald_select_merged, herald_refine_topk,
herald_gather_kv, then herald_block_attn once per denoising step.
"""

from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import herald as H


def device_tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy input (uint16 bf16 bits or float32) -> torch device tensor of the same bits."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def batch_to_device(batch, device="cuda") -> dict:
    return {n: device_tensor(getattr(batch, n), device)
            for n in ["q0", "k_cache", "v_cache", "q_steps", "kb_steps", "vb_steps"]}


class BlockRunner:
    """Outputs and workspaces for one (workload shape, sequence offsets)."""

    def __init__(self, seq_start, B, Hq, Hkv, d, C, topk, dtype: str, softmax_scale: float = 0.0, device="cuda"):
        self.dtype = H.HERALD_BF16 if dtype == "bf16" else H.HERALD_F32
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.problem = H.make_problem(seq_start, B, Hq, Hkv, d, C, topk, self.dtype, softmax_scale=softmax_scale,
                                      device=device)
        nseq = len(seq_start) - 1
        self.nseq, self.B, self.Hq, self.Hkv, self.d, self.C, self.topk = nseq, B, Hq, Hkv, d, C, topk
        dev = device
        self.cand = torch.empty((nseq, Hkv, C), dtype=torch.int32, device=dev)
        self.cand_score = torch.empty((nseq, Hkv, C), dtype=torch.float32, device=dev)
        self.sel = torch.empty((nseq, Hkv, topk), dtype=torch.int32, device=dev)
        self.sel_score = torch.empty((nseq, Hkv, topk), dtype=torch.float32, device=dev)
        self.ldv = H.herald_vsel_ld(topk)
        self.k_sel = torch.empty((nseq, Hkv, topk, d), dtype=self.tdtype, device=dev)
        self.v_sel = torch.empty((nseq, Hkv, d, self.ldv), dtype=self.tdtype, device=dev)
        self.out = torch.empty((nseq, B, Hq, d), dtype=self.tdtype, device=dev)
        self.ws = {}
        for name, op in [("select", H.HERALD_OP_SELECT), ("refine", H.HERALD_OP_REFINE), ("attn", H.HERALD_OP_ATTN)]:
            n = H.herald_workspace_size(self.problem, op)
            self.ws[name] = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        self.attn_splits = H.herald_attn_splits(self.problem)

    def select(self, q_merge, k_cache, stream=None):
        H.herald_select_merged(self.problem, q_merge, k_cache, self.cand, self.cand_score, self.ws["select"],
                               stream=stream)

    def refine(self, q_refine, k_cache, cand=None, stream=None):
        H.herald_refine_topk(self.problem, q_refine, k_cache, self.cand if cand is None else cand, self.sel,
                             self.sel_score, self.ws["refine"], stream=stream)

    def gather(self, k_cache, v_cache, sel=None, stream=None):
        H.herald_gather_kv(self.problem, k_cache, v_cache, 0, self.sel if sel is None else sel, self.k_sel,
                           self.v_sel, stream=stream)

    def attn(self, q, k_blk, v_blk, out: Optional[torch.Tensor] = None, stream=None):
        H.herald_block_attn(self.problem, q, k_blk, v_blk, self.k_sel, self.v_sel, self.out if out is None else out,
                            self.ws["attn"], stream=stream)

    def run_block(self, q0, k_cache, v_cache, q_steps, kb_steps, vb_steps, outs=None, stream=None):
        """select -> refine -> gather -> T attention steps; outs[t] receives step t (default self.out)."""
        self.select(q0, k_cache, stream)
        self.refine(q0, k_cache, stream=stream)
        self.gather(k_cache, v_cache, stream=stream)
        for t in range(q_steps.shape[0]):
            self.attn(q_steps[t], kb_steps[t], vb_steps[t], None if outs is None else outs[t], stream)
