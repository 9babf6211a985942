"""Host-side pieces of the benchmark runtime that need no GPU: sub-range views of device
allocations and the attention-workspace placement step's early exits."""

import types

import pytest

import bench
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
