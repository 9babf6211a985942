"""Device buffers and the per-block call sequence, on top of the C ABI.

The caller's allocator provides device memory (PyTorch by default, or the plain
HIP runtime of ``hiprt``); all compute happens in libherald.so. ``BlockRunner``
owns the outputs and workspaces of one batch shape and issues, per block:
herald_select_merged, herald_refine_topk, herald_gather_kv, then
herald_block_attn once per denoising step.
"""

from __future__ import annotations

import inspect
from typing import Callable, Optional

import numpy as np

from . import herald as H


def device_tensor(a: np.ndarray, device="cuda"):
    """numpy input (uint16 bf16 bits or float32) -> torch device tensor of the same bits."""
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def batch_to_device(batch, device="cuda") -> dict:
    return {n: device_tensor(getattr(batch, n), device)
            for n in ["q0", "k_cache", "v_cache", "q_steps", "kb_steps", "vb_steps"]}


def _takes_keyword(fn: Callable, name: str) -> bool:
    """Whether `fn` accepts keyword `name` (allocators written before the placement hint do not)."""
    try:
        params = inspect.signature(fn).parameters
    except (TypeError, ValueError):
        return False
    return name in params or any(p.kind is inspect.Parameter.VAR_KEYWORD for p in params.values())


def torch_alloc(device="cuda") -> Callable:
    import torch

    def alloc(shape, dtype, zero=False, contiguous=False):  # the caching allocator places its own blocks
        dt = {np.dtype(np.int32): torch.int32, np.dtype(np.float32): torch.float32,
              np.dtype(np.uint16): torch.bfloat16, np.dtype(np.uint8): torch.uint8}[np.dtype(dtype)]
        return (torch.zeros if zero else torch.empty)(tuple(shape), dtype=dt, device=device)

    return alloc


class BlockRunner:
    """Outputs and workspaces for one (workload shape, sequence offsets).

    `alloc(shape, numpy_dtype, zero=False[, contiguous=False])` returns device memory exposing
    data_ptr() and nbytes (uint16 stands for bf16), zero-filled when asked (the attention
    workspace); `contiguous` asks for physically contiguous memory where the allocator can
    place it (the attention workspace, whose split partial results are written and read back
    within one call, runs faster from it; the full-cache scan writes its logits faster to
    scattered pages, so the other buffers do not ask);
    `seq_start_dev` is the device copy of the offsets (made with the allocator's
    framework when omitted).
    """

    def __init__(self, seq_start, B, Hq, Hkv, d, C, topk, dtype: str, softmax_scale: float = 0.0, device="cuda",
                 alloc: Optional[Callable] = None, seq_start_dev=None):
        self.dtype = H.HERALD_BF16 if dtype == "bf16" else H.HERALD_F32
        alloc = torch_alloc(device) if alloc is None else alloc
        self.problem = H.make_problem(seq_start, B, Hq, Hkv, d, C, topk, self.dtype, softmax_scale=softmax_scale,
                                      device=device, seq_start_dev=seq_start_dev)
        nseq = len(seq_start) - 1
        self.nseq, self.B, self.Hq, self.Hkv, self.d, self.C, self.topk = nseq, B, Hq, Hkv, d, C, topk
        el = np.uint16 if dtype == "bf16" else np.float32
        self.cand = alloc((nseq, Hkv, C), np.int32)
        self.cand_score = alloc((nseq, Hkv, C), np.float32)
        self.sel = alloc((nseq, Hkv, topk), np.int32)
        self.sel_score = alloc((nseq, Hkv, topk), np.float32)
        self.ldv = H.herald_vsel_ld(topk)
        self.k_sel = alloc((nseq, Hkv, topk, d), el)
        self.v_sel = alloc((nseq, Hkv, d, self.ldv), el)
        self.out = alloc((nseq, B, Hq, d), el)
        self.ws = {}
        for name, op in [("select", H.HERALD_OP_SELECT), ("refine", H.HERALD_OP_REFINE), ("attn", H.HERALD_OP_ATTN)]:
            try:
                n = H.herald_workspace_size(self.problem, op)
            except H.HeraldError as e:
                # the merged-query selection takes at most 16384 candidates; larger sets (the
                # exact baselines: every key a candidate) use the other three calls only
                if name == "select" and e.status == H.HERALD_ERR_UNSUPPORTED:
                    self.ws[name] = None
                    continue
                raise
            hint = {"contiguous": True} if name == "attn" and _takes_keyword(alloc, "contiguous") else {}
            self.ws[name] = alloc((max(n, 256),), np.uint8, zero=name == "attn", **hint)
        self.attn_splits = H.herald_attn_splits(self.problem)

    def select(self, q_merge, k_cache, stream=None):
        H.herald_select_merged(self.problem, q_merge, k_cache, self.cand, self.cand_score, self.ws["select"],
                               stream=stream)

    def select_query(self, q_sel, k_cache, stream=None):
        """Stage one from one query per head (q_sel [nseq][Hq][d]) instead of the block mean."""
        H.herald_select_query(self.problem, q_sel, k_cache, self.cand, self.cand_score, self.ws["select"],
                              stream=stream)

    def refine(self, q_refine, k_cache, cand=None, stream=None):
        H.herald_refine_topk(self.problem, q_refine, k_cache, self.cand if cand is None else cand, self.sel,
                             self.sel_score, self.ws["refine"], stream=stream)

    def gather(self, k_cache, v_cache, sel=None, stream=None):
        H.herald_gather_kv(self.problem, k_cache, v_cache, 0, self.sel if sel is None else sel, self.k_sel,
                           self.v_sel, stream=stream)

    def attn(self, q, k_blk, v_blk, out=None, stream=None):
        H.herald_block_attn(self.problem, q, k_blk, v_blk, self.k_sel, self.v_sel, self.out if out is None else out,
                            self.ws["attn"], stream=stream)

    def run_block(self, q0, k_cache, v_cache, q_steps, kb_steps, vb_steps, outs=None, stream=None):
        """select -> refine -> gather -> T attention steps; outs[t] receives step t (default self.out)."""
        self.select(q0, k_cache, stream)
        self.refine(q0, k_cache, stream=stream)
        self.gather(k_cache, v_cache, stream=stream)
        for t in range(q_steps.shape[0]):
            self.attn(q_steps[t], kb_steps[t], vb_steps[t], None if outs is None else outs[t], stream)


def _pick(x, i: int):
    """Copy i % len(x) of a list of copies, or x itself."""
    return x[i % len(x)] if isinstance(x, (list, tuple)) else x


class StreamOps:
    """Streams and events of the caller's runtime: new_event() -> event,
    record(event, stream), wait(stream, event) (the stream waits for the event's work)."""

    def __init__(self, new_event: Callable, record: Callable, wait: Callable):
        self.new_event, self.record, self.wait = new_event, record, wait

    @staticmethod
    def torch() -> "StreamOps":
        import torch

        return StreamOps(torch.cuda.Event, lambda ev, st: ev.record(st), lambda st, ev: st.wait_event(ev))

    @staticmethod
    def hip(hip) -> "StreamOps":
        return StreamOps(hip.event, lambda ev, st: hip.record(ev, st), lambda st, ev: hip.wait(st, ev))


class SpeculativePipeline:
    """The per-block path as a two-stream pipeline over two sparse KV pools.

    Block i's candidates come from the previous block's queries merged into one per head
    (the speculative search; block 0 searches with its own), its final subset from
    refining those candidates with block i's own queries, gathered into pool i % 2; then
    its T attention steps read that pool. The `search` stream runs block i+1's search
    while the `denoise` stream runs block i's steps. With overlap_refine False, block
    i+1's refine and gather wait for block i's last step (in a decoder the next block's
    queries exist only then); with True they follow its search on the search stream (the
    next block's queries taken as given), so the fetch into the other pool also overlaps
    block i. A pool is refilled only after the steps of the block two before are done.
    """

    def __init__(self, r: BlockRunner, alloc: Callable, ops: StreamOps, src_is_host: int = 0,
                 overlap_refine: bool = False):
        self.r, self.ops, self.src_is_host, self.overlap_refine = r, ops, src_is_host, overlap_refine
        el = np.uint16 if r.dtype == H.HERALD_BF16 else np.float32
        self.sel = [r.sel, alloc((r.nseq, r.Hkv, r.topk), np.int32)]
        self.pools = [(r.k_sel, r.v_sel), (alloc((r.nseq, r.Hkv, r.topk, r.d), el), alloc((r.nseq, r.Hkv, r.d, r.ldv), el))]
        self.fetched = [ops.new_event(), ops.new_event()]   # pool p holds its block's subset
        self.consumed = [ops.new_event(), ops.new_event()]  # pool p's block finished its steps

    def run(self, blocks, k_cache, k_src, v_src, denoise, search, outs=None, cands=None, sels=None):
        """blocks[i]: dict of device tensors or addresses "q0" [nseq][B][Hq][d] and lists
        "q_steps", "kb_steps", "vb_steps" (one per step). k_cache: device K cache for the
        search and refine; k_src, v_src: where the gather reads the subset (the device cache,
        or a pinned host pool when src_is_host = 2); each may also be a list of copies, block
        i using copy i % len. outs[i][t] receives block i's step t (default: the runner's
        output); cands[i] / sels[i], when given, receive block i's candidates / final subset
        (default: the runner's buffers, reused)."""
        r, ops, n = self.r, self.ops, len(blocks)

        def search_block(i):
            cand = r.cand if cands is None else cands[i]
            H.herald_select_merged(r.problem, blocks[max(i - 1, 0)]["q0"], _pick(k_cache, i), cand, r.cand_score,
                                   r.ws["select"], stream=search)

        def refine_fetch(i):
            p = i % 2
            cand = r.cand if cands is None else cands[i]
            sel = self.sel[p] if sels is None else sels[i]
            H.herald_refine_topk(r.problem, blocks[i]["q0"], _pick(k_cache, i), cand, sel, r.sel_score,
                                 r.ws["refine"], stream=search)
            if i >= 2:
                ops.wait(search, self.consumed[p])  # block i-2 is done with this pool
            H.herald_gather_kv(r.problem, _pick(k_src, i), _pick(v_src, i), self.src_is_host, sel, self.pools[p][0],
                               self.pools[p][1], stream=search)
            ops.record(self.fetched[p], search)

        def denoise_block(i):
            p = i % 2
            ops.wait(denoise, self.fetched[p])
            b = blocks[i]
            for t in range(len(b["q_steps"])):
                out = r.out if outs is None else outs[i][t]
                H.herald_block_attn(r.problem, b["q_steps"][t], b["kb_steps"][t], b["vb_steps"][t], self.pools[p][0],
                                    self.pools[p][1], out, r.ws["attn"], stream=denoise)
            ops.record(self.consumed[p], denoise)

        search_block(0)
        refine_fetch(0)
        for i in range(n):
            denoise_block(i)
            if i + 1 < n:
                search_block(i + 1)  # overlaps block i's steps
                if not self.overlap_refine:
                    ops.wait(search, self.consumed[i % 2])
                refine_fetch(i + 1)

    def run_serial(self, blocks, k_cache, k_src, v_src, stream, outs=None, cands=None, sels=None):
        """The same calls, in the same order per block, on one stream (the reference schedule)."""
        r, n = self.r, len(blocks)
        for i in range(n):
            p = i % 2
            cand = r.cand if cands is None else cands[i]
            sel = self.sel[p] if sels is None else sels[i]
            H.herald_select_merged(r.problem, blocks[max(i - 1, 0)]["q0"], _pick(k_cache, i), cand, r.cand_score,
                                   r.ws["select"], stream=stream)
            H.herald_refine_topk(r.problem, blocks[i]["q0"], _pick(k_cache, i), cand, sel, r.sel_score,
                                 r.ws["refine"], stream=stream)
            H.herald_gather_kv(r.problem, _pick(k_src, i), _pick(v_src, i), self.src_is_host, sel, self.pools[p][0],
                               self.pools[p][1], stream=stream)
            b = blocks[i]
            for t in range(len(b["q_steps"])):
                out = r.out if outs is None else outs[i][t]
                H.herald_block_attn(r.problem, b["q_steps"][t], b["kb_steps"][t], b["vb_steps"][t], self.pools[p][0],
                                    self.pools[p][1], out, r.ws["attn"], stream=stream)
