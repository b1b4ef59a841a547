"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching a device.  No
compute call runs here (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

import bit_quantized_moe_router_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    names = _header_functions()
    assert {"moe_pack_weights", "moe_route", "moe_forward_prefill", "moe_forward_decode"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def _desc(**kw):
    base = dict(hidden=2048, n_experts=256, top_k=8, inter=512, shared_inter=512)
    base.update(kw)
    return moe.make_desc(**base)


TRAILER = 256  # the blob's last bytes: the small-scale flag of the grouped GEMM's rebuild


def test_packed_bytes_is_0p5625_bytes_per_param():
    d = _desc()
    params = 3 * 2048 * 512 * (256 + 1)
    assert moe.moe_packed_bytes(d) == params * 9 // 16 + TRAILER == 257 * 1769472 + TRAILER
    d0 = _desc(shared_inter=0)
    assert moe.moe_packed_bytes(d0) == 256 * 1769472 + TRAILER
    tiny = _desc(hidden=256, n_experts=16, top_k=2, inter=128, shared_inter=128)
    assert moe.moe_packed_bytes(tiny) == 17 * 3 * 256 * 128 * 9 // 16 + TRAILER


def test_workspace_and_tile_bounds():
    d = _desc(tile_rows=64)
    assert moe.moe_max_tiles(d, 2048) == (2048 * 8 + 63) // 64 + 256 + 2048 // 64
    assert moe.moe_max_tiles(d, 1) == 1 + 8 + 1
    w1 = moe.moe_workspace_bytes(d, 1)
    w2 = moe.moe_workspace_bytes(d, 2048)
    w3 = moe.moe_workspace_bytes(d, 4096)  # two chunk areas: two chunks in flight
    w4 = moe.moe_workspace_bytes(d, 1 << 20)  # still bounded by max_chunk
    assert 0 < w1 < w2 < w3 == w4 == 2 * w2


@pytest.mark.parametrize("kw,status", [
    (dict(group_size=32), 2), (dict(hidden=1028), 2), (dict(inter=772), 2), (dict(shared_inter=100), 2),
    (dict(top_k=9, n_experts=8), 1), (dict(top_k=0), 1), (dict(n_experts=0), 2), (dict(n_experts=1024), 2),
    (dict(tile_rows=48), 1), (dict(tile_rows=256), 1), (dict(max_chunk=0), 1), (dict(gemv_max_rows=9), 1),
    (dict(host_sync_routing=2), 1), (dict(dequant_pass=-1), 1),
])
def test_invalid_desc_rejected(kw, status):
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_packed_bytes(_desc(**kw))
    assert ei.value.status == status


class _FakeTensor:
    """Stands in for a device tensor: only pointer and size are ever read."""

    def __init__(self, nbytes, ptr=0x1000):
        self._n, self._p = nbytes, ptr

    def data_ptr(self):
        return self._p

    def numel(self):
        return self._n

    def element_size(self):
        return 1


def test_errors_before_any_device_work():
    d = _desc()
    t = _FakeTensor(16)
    # T = 0 is a no-op, even with null pointers.
    moe.moe_forward_prefill(d, None, None, None, None, 0, None, _FakeTensor(0, 0), stream=0)
    # Workspace too small.
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward_prefill(d, t, t, None, t, 16, t, _FakeTensor(100), stream=0)
    assert ei.value.status == 3
    # Null pointers.
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward_prefill(d, None, t, None, t, 16, t, _FakeTensor(1 << 30), stream=0)
    assert ei.value.status == 1
    # The GEMV path takes at most 8 rows: a row threshold above 8 is refused.
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward_decode(_desc(gemv_max_rows=9), t, t, None, t, 9, t, _FakeTensor(1 << 30), stream=0)
    assert ei.value.status == 1
    # Route: T above max_chunk.
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_route(_desc(max_chunk=16), t, 17, t, None, {n: t for n, _ in moe.Routing._fields_},
                      _FakeTensor(1 << 30), stream=0)
    assert ei.value.status == 1
    # Packed blob too small.
    q = (t, t, t)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_pack_weights(d, q, q, q, q, q, q, _FakeTensor(1000), stream=0)
    assert ei.value.status == 3
    assert b"required" in moe.lib().moe_last_error()


def test_status_strings():
    L = moe.lib()
    for code, name in moe.STATUS.items():
        assert L.moe_status_str(code).decode() == name
