"""Host-side pieces of the benchmark runtime that need no GPU: sub-range views of device
allocations and the attention-workspace placement step's early exits."""

import types

import numpy as np
import pytest

import bench
from block_diffusion_sparse_herald_amd import herald as H
from block_diffusion_sparse_herald_amd.hiprt import DevView


def _parent(ptr=0x10000, nbytes=4096):
    return types.SimpleNamespace(ptr=ptr, nbytes=nbytes)


def test_devview_addresses_and_size():
    v = DevView(_parent(), 1024, 2048)
    assert v.data_ptr() == 0x10000 + 1024 and v.nbytes == 2048
    assert DevView(_parent(), 0, 4096).data_ptr() == 0x10000  # the whole allocation


@pytest.mark.parametrize("offset,nbytes", [(-1, 16), (0, 4097), (4000, 200), (16, -1)])
def test_devview_rejects_ranges_outside_the_allocation(offset, nbytes):
    with pytest.raises(ValueError):
        DevView(_parent(), offset, nbytes)


def test_placement_skips_runs_without_a_split_workspace():
    # no workspace, or an unsplit attention: nothing to place, nothing touched on the device
    hip = object()
    for ws, splits in (({"attn": None}, 2), ({"attn": _parent()}, 1)):
        r = types.SimpleNamespace(ws=dict(ws), attn_splits=splits)
        assert bench.place_attn_workspace(hip, r, None, [], [], [], 8) is None
        assert r.ws == ws


class _FakeBuf:
    """Stands in for device memory: an address and a size, never dereferenced here."""

    def __init__(self, shape, dtype):
        self.shape = tuple(shape)
        self.nbytes = int(np.prod(shape)) * np.dtype(dtype).itemsize
        self.ptr = 0x100000

    def data_ptr(self):
        return self.ptr


def _runner(alloc):
    from block_diffusion_sparse_herald_amd.runner import BlockRunner

    # the 1 x 32K shape splits its attention keys, so it has an attention workspace
    return BlockRunner([0, 32768], 32, 32, 8, 128, 4096, 1024, "bf16", alloc=alloc,
                       seq_start_dev=_FakeBuf((2,), np.int64))


def test_runner_asks_for_contiguous_attention_workspace_only():
    H.load()
    calls = []

    def alloc(shape, dt, zero=False, contiguous=False):
        calls.append((tuple(shape), np.dtype(dt), zero, contiguous))
        return _FakeBuf(shape, dt)

    r = _runner(alloc)
    assert r.attn_splits > 1
    contiguous = [c for c in calls if c[3]]
    assert len(contiguous) == 1 and contiguous[0][2] and contiguous[0][1] == np.uint8  # the zeroed attention workspace
    assert r.ws["attn"].nbytes == contiguous[0][0][0]


def test_runner_accepts_allocators_without_the_placement_hint():
    H.load()
    calls = []

    def alloc(shape, dt, zero=False):  # the protocol before the hint
        calls.append(tuple(shape))
        return _FakeBuf(shape, dt)

    r = _runner(alloc)
    assert r.ws["attn"] is not None and len(calls) >= 8
