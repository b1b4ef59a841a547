"""Python binding of libmoe.so, the MI355X 4-bit group-affine MoE layer.

Argument marshalling only: every function forwards device pointers (taken
from torch tensors with ``.data_ptr()``) and the current HIP stream to the C
ABI declared in include/moe.h, and raises MoEError on a non-OK status.  All
computation happens in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_UNSUPPORTED_SHAPE",
          3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_HIP", 5: "MOE_ERR_DEVICE_UNSUPPORTED"}

# Kernel ids of moe_profile_read.
(K_LOGITS, K_TOPK, K_META, K_GATEUP_GEMM, K_DOWN_GEMM, K_GATEUP_GEMV, K_DOWN_GEMV, K_COMBINE, K_DEQUANT,
 K_PROBE_READ, K_PROBE_MFMA) = range(11)
KERNEL_NAMES = {K_LOGITS: "k_screen|k_logits_small", K_TOPK: "k_route_exact", K_META: "k_meta|k_topk_meta",
                K_GATEUP_GEMM: "k_gateup_gemm", K_DOWN_GEMM: "k_down_gemm",
                K_GATEUP_GEMV: "k_gemv_experts", K_DOWN_GEMV: "k_gemv_reduce", K_COMBINE: "k_combine",
                K_DEQUANT: "k_dequant_active", K_PROBE_READ: "k_stream_read", K_PROBE_MFMA: "k_mfma_rate"}


class MoEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class LayerDesc(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("hidden", "n_experts", "top_k", "inter", "shared_inter",
                                         "group_size", "gemv_max_rows", "max_chunk", "tile_rows",
                                         "host_sync_routing", "dequant_pass", "batch_invariant")]


class QMatrix(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("biases", C.c_void_p)]


class Routing(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("topk_ids", "topk_weights", "expert_counts",
                                          "expert_offsets", "sorted_assign", "tile_map", "n_tiles")]


_lib = None


def lib():
    """Load libmoe.so (built by bit_quantized_moe_router_amd/build.py); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python bit_quantized_moe_router_amd/build.py`")
        # torch carries its own HIP runtime (same soname as ROCm's).  Loading it
        # first makes libmoe.so bind to that one; loaded the other way round the
        # process would hold two HIP runtimes, and the second to open the GPU
        # finds no device.
        import torch  # noqa: F401
        L = C.CDLL(LIB_PATH)
        P, vp, i32, sz = C.POINTER, C.c_void_p, C.c_int32, C.c_size_t
        D = P(LayerDesc)
        L.moe_packed_bytes.argtypes = [D, P(sz)]
        L.moe_workspace_bytes.argtypes = [D, i32, P(sz)]
        L.moe_max_tiles.argtypes = [D, i32, P(i32)]
        L.moe_pack_weights.argtypes = [D, QMatrix, QMatrix, QMatrix, QMatrix, QMatrix, QMatrix, vp, sz, vp]
        L.moe_route.argtypes = [D, vp, i32, vp, vp, P(Routing), vp, sz, vp]
        L.moe_forward_prefill.argtypes = [D, vp, vp, vp, vp, i32, vp, vp, sz, vp]
        L.moe_forward_decode.argtypes = [D, vp, vp, vp, vp, i32, vp, vp, sz, vp]
        L.moe_forward_decode_static.argtypes = [D, vp, vp, vp, vp, i32, vp, vp]
        L.moe_default_gemv_max_rows.argtypes = []
        L.moe_default_gemv_max_rows.restype = i32
        L.moe_status_str.argtypes = [C.c_int]
        L.moe_status_str.restype = C.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = C.c_char_p
        L.moe_probe_stream_read.argtypes = [vp, sz, vp, i32, vp]
        L.moe_probe_mfma_rate.argtypes = [i32, i32, vp, vp, vp]
        L.moe_profile_enable.argtypes = [i32]
        L.moe_profile_reset.argtypes = []
        L.moe_profile_read.argtypes = [i32, P(C.c_double), P(i32)]
        for name in ("moe_packed_bytes", "moe_workspace_bytes", "moe_max_tiles", "moe_pack_weights",
                     "moe_route", "moe_forward_prefill", "moe_forward_decode", "moe_forward_decode_static",
                     "moe_probe_stream_read", "moe_probe_mfma_rate", "moe_profile_enable",
                     "moe_profile_reset", "moe_profile_read"):
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise MoEError(status, lib().moe_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_desc(hidden, n_experts, top_k, inter, shared_inter, gemv_max_rows=-1, max_chunk=2048,
              tile_rows=0, group_size=64, host_sync_routing=0, dequant_pass=0, batch_invariant=0) -> LayerDesc:
    return LayerDesc(hidden, n_experts, top_k, inter, shared_inter, group_size, gemv_max_rows,
                     max_chunk, tile_rows, host_sync_routing, dequant_pass, batch_invariant)


def moe_packed_bytes(desc: LayerDesc) -> int:
    n = C.c_size_t()
    _check(lib().moe_packed_bytes(C.byref(desc), C.byref(n)))
    return n.value


def moe_workspace_bytes(desc: LayerDesc, max_tokens: int) -> int:
    n = C.c_size_t()
    _check(lib().moe_workspace_bytes(C.byref(desc), max_tokens, C.byref(n)))
    return n.value


def moe_max_tiles(desc: LayerDesc, T: int) -> int:
    n = C.c_int32()
    _check(lib().moe_max_tiles(C.byref(desc), T, C.byref(n)))
    return n.value


def moe_default_gemv_max_rows() -> int:
    return lib().moe_default_gemv_max_rows()


def _qm(m):
    if m is None:
        return QMatrix(None, None, None)
    codes, scales, biases = m
    return QMatrix(_ptr(codes), _ptr(scales), _ptr(biases))


def moe_pack_weights(desc, gate, up, down, sh_gate, sh_up, sh_down, packed, stream=None):
    """gate/up/down/sh_* are (codes, scales, biases) device tensors; packed a device byte tensor."""
    _check(lib().moe_pack_weights(C.byref(desc), _qm(gate), _qm(up), _qm(down), _qm(sh_gate),
                                  _qm(sh_up), _qm(sh_down), _ptr(packed),
                                  packed.numel() * packed.element_size(), _stream(stream)))


def moe_route(desc, x, T, router_w, logit_bias, routing: dict, ws, stream=None):
    """routing: dict of device tensors keyed like the moe_routing fields."""
    r = Routing(*(_ptr(routing[n]) for n, _ in Routing._fields_))
    _check(lib().moe_route(C.byref(desc), _ptr(x), T, _ptr(router_w), _ptr(logit_bias), C.byref(r),
                           _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_forward_prefill(desc, packed, router_w, logit_bias, x, T, y, ws, stream=None):
    _check(lib().moe_forward_prefill(C.byref(desc), _ptr(packed), _ptr(router_w), _ptr(logit_bias),
                                     _ptr(x), T, _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)))


def moe_forward_decode(desc, packed, router_w, logit_bias, x, T, y, ws, stream=None):
    _check(lib().moe_forward_decode(C.byref(desc), _ptr(packed), _ptr(router_w), _ptr(logit_bias),
                                    _ptr(x), T, _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)))


def moe_forward_decode_static(desc, packed, router_w, logit_bias, x, T, y, stream=None):
    """moe_forward_decode on the library's fixed device scratch (no workspace argument)."""
    _check(lib().moe_forward_decode_static(C.byref(desc), _ptr(packed), _ptr(router_w), _ptr(logit_bias),
                                           _ptr(x), T, _ptr(y), _stream(stream)))


def moe_probe_stream_read(src, nbytes, sink, max_workgroups, stream=None):
    """Streaming read of nbytes of src (16-byte pieces per lane); sink holds max_workgroups words."""
    _check(lib().moe_probe_stream_read(_ptr(src), nbytes, _ptr(sink), max_workgroups, _stream(stream)))


def moe_probe_mfma_rate(iters, workgroups, clocks, sink, stream=None):
    """MFMA-only kernel: workgroups x 4 waves x iters x 8 MFMAs of 32x32x16 (32768 flop each)."""
    _check(lib().moe_probe_mfma_rate(iters, workgroups, _ptr(clocks), _ptr(sink), _stream(stream)))


def moe_profile_enable(mask: int):
    """Bit i set = record events around kernel id i (0 = off)."""
    _check(lib().moe_profile_enable(int(mask)))


def moe_profile_reset():
    _check(lib().moe_profile_reset())


def moe_profile_read(kernel_id: int):
    ms = C.c_double()
    n = C.c_int32()
    _check(lib().moe_profile_read(kernel_id, C.byref(ms), C.byref(n)))
    return ms.value, n.value
