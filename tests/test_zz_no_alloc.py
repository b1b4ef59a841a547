"""moe_forward_decode_static, the decode entry point without a workspace
argument (its workspace is a fixed device array inside the library), against
moe_forward_decode with a caller-owned workspace: same kernels, so the same
bits.  Two calls in a row on the fixed array, the second with fewer rows, on
both decode paths (row-parallel GEMV and grouped GEMM)."""
import numpy as np
import pytest

import moe_inputs as mi
import bit_quantized_moe_router_amd as moe
from oracle import oracle as orc


def test_static_decode_rejects_oversized_layers():
    """Host-side limit check, before any device call: a layer whose decode
    workspace exceeds the fixed array is refused with a clear message."""
    d = moe.make_desc(4096, 256, 8, 1024, 1024)
    assert moe.moe_workspace_bytes(d, 8) > moe_static_limit()
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward_decode_static(d, _Fake(), _Fake(), None, _Fake(), 8, _Fake(), stream=0)
    assert ei.value.status == 3 and "static scratch" in str(ei.value)
    d2 = moe.make_desc(2048, 256, 8, 512, 512, dequant_pass=1)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward_decode_static(d2, _Fake(), _Fake(), None, _Fake(), 1, _Fake(), stream=0)
    assert ei.value.status == 1


class _Fake:
    """Stands in for a tensor in host-only checks: a non-null address that is never dereferenced."""

    def data_ptr(self):
        return 0x1000


def moe_static_limit():
    return 16 << 20


@pytest.mark.gpu
@pytest.mark.parametrize("gemv,bi", [(8, 0), (0, 0), (8, 1)])
def test_static_decode_matches_workspace_decode(gemv, bi):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_quantized_moe_router_amd.layer import MoELayer, to_dev

    case = mi.make_case("decode")
    H = case["cfg"]["H"]
    lay = MoELayer(case["w"], case["k"], device="cuda", max_tokens=8, gemv_max_rows=gemv)
    lay.set_desc(batch_invariant=bi)  # 1: the GEMV with the grouped GEMM's arithmetic
    assert moe.moe_workspace_bytes(lay.desc, 8) <= moe_static_limit()
    rows = mi.gen_x(8, H, 5150 + gemv)
    xs = {8: to_dev(rows, "cuda"), 3: to_dev(rows[5:8], "cuda")}
    # Two calls in a row on the fixed array: 8 rows, then 3 rows.
    ys = {}
    for T in (8, 3):
        ys[T] = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        moe.moe_forward_decode_static(lay.desc, lay.packed, lay.router_w, None, xs[T], T, ys[T])
    torch.cuda.synchronize()
    for T in (8, 3):
        ref = lay.forward_decode(xs[T], None)
        torch.cuda.synchronize()
        assert torch.equal(ys[T], ref), (gemv, bi, T)
    # And the oracle, within the layer tolerance, for the second (smaller) call.
    want, _ = orc.forward(case["w"], case["k"], rows[5:8], None, 2048, 64)
    got = ys[3].cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    mx = np.abs(got - want).max() / np.sqrt(np.mean(want ** 2))
    print(f"[parity] static decode T=3 gemv_max_rows={gemv} batch_invariant={bi}: rel_l2={rel:.3e} "
          f"max_abs/rms={mx:.3e}", flush=True)
    assert rel <= 5e-3 and mx <= 2e-2
