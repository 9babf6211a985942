"""Thin Python binding of libherald.so (include/herald.h).

Argument marshalling only: every step of the path runs in the HIP kernels of the
library. Functions keep the C names; tensors are passed as torch tensors (device
memory from PyTorch's allocator) or raw integer addresses, streams as torch
streams or raw handles. A missing library raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libherald.so")

HERALD_OK = 0
HERALD_ERR_INVALID_ARG = 1
HERALD_ERR_UNSUPPORTED = 2
HERALD_ERR_WORKSPACE = 3
HERALD_ERR_HIP = 4

HERALD_F32 = 0
HERALD_BF16 = 1

HERALD_OP_SELECT = 0
HERALD_OP_REFINE = 1
HERALD_OP_ATTN = 2
HERALD_OP_GATHER_HOST = 3
HERALD_OP_SELECT_COMPRESSED = 4

KERNEL_IDS = {
    "scan": 0, "score_hist": 1, "radix": 2, "emit": 3, "refine_stats": 4, "refine_scores": 5,
    "refine_select": 6, "gather": 7, "attn": 8, "attn_combine": 9,
}

EXPORTED = [
    "herald_workspace_size", "herald_workspace_bytes", "herald_vsel_ld", "herald_select_merged", "herald_select_query", "herald_refine_topk",
    "herald_gather_kv", "herald_block_attn", "herald_block_attn_static", "herald_last_error", "herald_set_kernel_events",
    "herald_attn_splits", "herald_compressed_rows", "herald_compress_keys", "herald_select_compressed",
]


class HeraldError(RuntimeError):
    def __init__(self, status: int, func: str, message: str):
        super().__init__(f"{func} failed with status {status}: {message}")
        self.status = status
        self.message = message


class herald_problem(ctypes.Structure):
    _fields_ = [
        ("nseq", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_candidates", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("reserved", ctypes.c_int32),
        ("seq_start_host", ctypes.c_void_p),
        ("seq_start_dev", ctypes.c_void_p),
    ]


_lib: Optional[ctypes.CDLL] = None
_vp = ctypes.c_void_p


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m block_diffusion_sparse_herald_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(herald_problem)
    sig = {
        "herald_workspace_size": ([P, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
        "herald_workspace_bytes": ([P, ctypes.c_int], ctypes.c_size_t),
        "herald_vsel_ld": ([ctypes.c_int32], ctypes.c_int64),
        "herald_select_merged": ([P, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp], ctypes.c_int),
        "herald_select_query": ([P, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp], ctypes.c_int),
        "herald_compressed_rows": ([P, ctypes.c_int32], ctypes.c_int64),
        "herald_compress_keys": ([P, _vp, ctypes.c_int32, ctypes.c_int32, _vp, _vp], ctypes.c_int),
        "herald_select_compressed": ([P, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp, ctypes.c_size_t, _vp], ctypes.c_int),
        "herald_refine_topk": ([P, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp], ctypes.c_int),
        "herald_gather_kv": ([P, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp, _vp],
                             ctypes.c_int),
        "herald_block_attn": ([P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp], ctypes.c_int),
        "herald_block_attn_static": ([P, _vp, _vp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
        "herald_last_error": ([], ctypes.c_char_p),
        "herald_set_kernel_events": ([ctypes.c_int32, _vp, _vp], ctypes.c_int),
        "herald_attn_splits": ([P], ctypes.c_int32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _ptr(x) -> Optional[int]:
    """Address of a tensor / array / raw int (None stays NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def _nbytes(x) -> int:
    if x is None or isinstance(x, int):
        return 0
    if hasattr(x, "nbytes"):
        return int(x.nbytes)
    raise TypeError(f"pass workspace sizes explicitly for {type(x)}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, func: str) -> None:
    if status != HERALD_OK:
        raise HeraldError(status, func, load().herald_last_error().decode())


@dataclass
class Problem:
    """A herald_problem plus the buffers it points to (kept alive here)."""

    c: herald_problem
    seq_start_host: np.ndarray
    seq_start_dev: object

    @property
    def ref(self):
        return ctypes.byref(self.c)


def make_problem(seq_start: Sequence[int], B: int, Hq: int, Hkv: int, head_dim: int, C: int, topk: int,
                 dtype: int, seq_start_dev=None, softmax_scale: float = 0.0, device: str = "cuda") -> Problem:
    """Build a problem. The device copy of the offsets is made with torch unless given."""
    host = np.ascontiguousarray(np.asarray(seq_start, dtype=np.int64))
    if seq_start_dev is None:
        import torch

        seq_start_dev = torch.from_numpy(host.copy()).to(device)
    c = herald_problem(nseq=len(host) - 1, block_size=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=head_dim,
                       num_candidates=C, topk=topk, dtype=dtype, softmax_scale=softmax_scale, reserved=0,
                       seq_start_host=host.ctypes.data, seq_start_dev=_ptr(seq_start_dev))
    return Problem(c, host, seq_start_dev)


def herald_workspace_size(problem: Problem, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().herald_workspace_size(problem.ref, op, ctypes.byref(n)), "herald_workspace_size")
    return n.value


SIZE_MAX = ctypes.c_size_t(-1).value


def herald_workspace_bytes(problem: Problem, op: int) -> int:
    """The workspace size as the C call returns it: SIZE_MAX on error (no exception)."""
    return int(load().herald_workspace_bytes(problem.ref, op))


def herald_vsel_ld(topk: int) -> int:
    return int(load().herald_vsel_ld(topk))


def herald_attn_splits(problem: Problem) -> int:
    return int(load().herald_attn_splits(problem.ref))


def herald_select_merged(problem: Problem, q_merge, k_cache, cand_idx, cand_score, ws, ws_bytes=None,
                         stream=None) -> None:
    _check(load().herald_select_merged(problem.ref, _ptr(q_merge), _ptr(k_cache), _ptr(cand_idx), _ptr(cand_score),
                                       _ptr(ws), _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream)),
           "herald_select_merged")


def herald_select_query(problem: Problem, q_sel, k_cache, cand_idx, cand_score, ws, ws_bytes=None,
                        stream=None) -> None:
    _check(load().herald_select_query(problem.ref, _ptr(q_sel), _ptr(k_cache), _ptr(cand_idx), _ptr(cand_score),
                                      _ptr(ws), _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream)),
           "herald_select_query")


def herald_compressed_rows(problem: Problem, stride: int) -> int:
    return int(load().herald_compressed_rows(problem.ref, stride))


def herald_compress_keys(problem: Problem, k_cache, ksize: int, stride: int, k_comp, stream=None) -> None:
    _check(load().herald_compress_keys(problem.ref, _ptr(k_cache), ksize, stride, _ptr(k_comp), _stream(stream)),
           "herald_compress_keys")


def herald_select_compressed(problem: Problem, q_merge, k_comp, stride: int, cand_idx, cand_score, ws,
                             ws_bytes=None, stream=None) -> None:
    _check(load().herald_select_compressed(problem.ref, _ptr(q_merge), _ptr(k_comp), stride, _ptr(cand_idx),
                                           _ptr(cand_score), _ptr(ws), _nbytes(ws) if ws_bytes is None else ws_bytes,
                                           _stream(stream)),
           "herald_select_compressed")


def herald_refine_topk(problem: Problem, q_refine, k_cache, cand_idx, topk_idx, topk_score, ws, ws_bytes=None,
                       stream=None) -> None:
    _check(load().herald_refine_topk(problem.ref, _ptr(q_refine), _ptr(k_cache), _ptr(cand_idx), _ptr(topk_idx),
                                     _ptr(topk_score), _ptr(ws), _nbytes(ws) if ws_bytes is None else ws_bytes,
                                     _stream(stream)),
           "herald_refine_topk")


def herald_gather_kv(problem: Problem, k_src, v_src, src_is_host: int, topk_idx, k_sel, v_sel, host_staging=None,
                     host_idx=None, ws=None, ws_bytes=None, stream=None, done=None) -> None:
    _check(load().herald_gather_kv(problem.ref, _ptr(k_src), _ptr(v_src), int(src_is_host), _ptr(topk_idx),
                                   _ptr(k_sel), _ptr(v_sel), _ptr(host_staging), _ptr(host_idx), _ptr(ws),
                                   _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream),
                                   None if done is None else _event(done)),
           "herald_gather_kv")


def herald_block_attn(problem: Problem, q, k_blk, v_blk, k_sel, v_sel, out, ws, ws_bytes=None, stream=None) -> None:
    _check(load().herald_block_attn(problem.ref, _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_sel), _ptr(v_sel),
                                    _ptr(out), _ptr(ws), _nbytes(ws) if ws_bytes is None else ws_bytes,
                                    _stream(stream)),
           "herald_block_attn")


HERALD_STATIC_SCRATCH_BYTES = 16 << 20


def herald_block_attn_static(problem: Problem, q, k_blk, v_blk, k_sel, v_sel, out, stream=None) -> None:
    """herald_block_attn with its partial results in the library's static device scratch."""
    _check(load().herald_block_attn_static(problem.ref, _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_sel), _ptr(v_sel),
                                           _ptr(out), _stream(stream)),
           "herald_block_attn_static")


def herald_last_error() -> str:
    return load().herald_last_error().decode()


def _event(ev) -> Optional[int]:
    if ev is None or isinstance(ev, int):
        return ev
    return ev.cuda_event  # torch.cuda.Event handle


def herald_set_kernel_events(kernel: str | int, start=None, stop=None) -> None:
    kid = KERNEL_IDS[kernel] if isinstance(kernel, str) else int(kernel)
    _check(load().herald_set_kernel_events(kid, _event(start), _event(stop)), "herald_set_kernel_events")
