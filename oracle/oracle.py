"""ctypes wrapper over the C oracle (test infrastructure only).

Every function here forwards numpy arrays to oracle/moe_oracle.c; the only
Python-side logic is argument marshalling and the chunk loop (a chunk is an
independent slice of tokens, as in the chunked prefill section of the
"Optimizing on-device inference for Apple Silicon" page).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_ORACLE_LIB selects another build of the same source (the sanitizer
# build that tests/test_oracle_sanitized.py loads in a child process).
LIB_PATH = os.environ.get("MOE_ORACLE_LIB", os.path.join(HERE, "liboracle.so"))

_lib = None


class _QMat(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("biases", C.c_void_p)]


class _Layer(C.Structure):
    _fields_ = [("H", C.c_int32), ("E", C.c_int32), ("k", C.c_int32), ("I", C.c_int32),
                ("Is", C.c_int32),
                ("gate", _QMat), ("up", _QMat), ("down", _QMat),
                ("sh_gate", _QMat), ("sh_up", _QMat), ("sh_down", _QMat)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            if "MOE_ORACLE_LIB" in os.environ:
                raise ImportError(f"MOE_ORACLE_LIB={LIB_PATH} does not exist")
            from . import build as _b
            _b.build()
        L = C.CDLL(LIB_PATH)
        vp, i32 = C.c_void_p, C.c_int
        L.oracle_dequant.argtypes = [vp, vp, vp, i32, i32, vp]
        L.oracle_router_logits.argtypes = [vp, i32, i32, vp, vp, i32, vp]
        L.oracle_topk.argtypes = [vp, i32, i32, i32, vp, vp]
        L.oracle_route_meta.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_ffn_tokens.argtypes = [C.POINTER(_Layer), vp, vp, vp, vp, i32, vp]
        for f in (L.oracle_dequant, L.oracle_router_logits, L.oracle_topk,
                  L.oracle_route_meta, L.oracle_ffn_tokens):
            f.restype = None
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def dequant(codes, scales, biases) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint16)
    biases = _c(biases, np.uint16)
    N, K2 = codes.shape
    out = np.empty((N, 2 * K2), dtype=np.float64)
    lib().oracle_dequant(_p(codes), _p(scales), _p(biases), N, 2 * K2, _p(out))
    return out


def router_logits(x, router_w, bias=None) -> np.ndarray:
    x = _c(x, np.uint16)
    router_w = _c(router_w, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    T, H = x.shape
    E = router_w.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    lib().oracle_router_logits(_p(x), T, H, _p(router_w), _p(b), E, _p(out))
    return out


def topk(logits, k):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    lib().oracle_topk(_p(logits), T, E, k, _p(ids), _p(w))
    return ids, w


def route_meta(ids, E, BM, with_shared=True) -> dict:
    ids = _c(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    sorted_assign = np.empty(T * k, dtype=np.int32)
    max_tiles = max_tiles_for(T, k, E, BM)
    tiles = np.zeros((max_tiles, 3), dtype=np.int32)
    n_tiles = np.zeros(1, dtype=np.int32)
    lib().oracle_route_meta(_p(ids), T, k, E, BM, 1 if with_shared else 0, _p(counts),
                            _p(offsets), _p(sorted_assign), _p(tiles), _p(n_tiles))
    n = int(n_tiles[0])
    return dict(counts=counts, offsets=offsets, sorted_assign=sorted_assign,
                tiles=tiles[:n].copy(), n_tiles=n)


def max_tiles_for(T, k, E, BM) -> int:
    """Upper bound on the number of tiles for one chunk (routed + shared)."""
    if T == 0:
        return 1
    return (T * k + BM - 1) // BM + min(E, T * k) + (T + BM - 1) // BM


def route(x, router_w, bias, k, BM, with_shared=True) -> dict:
    """Full routing of one chunk: logits, top-k, weights and metadata."""
    logits = router_logits(x, router_w, bias)
    ids, w = topk(logits, k)
    r = route_meta(ids, router_w.shape[0], BM, with_shared)
    r.update(logits=logits, topk_ids=ids, topk_weights=w)
    return r


def _layer_struct(w: dict, k: int):
    keep = []

    def qm(m):
        if m is None:
            return _QMat(None, None, None)
        arrs = (_c(m["codes"], np.uint8), _c(m["scales"], np.uint16), _c(m["biases"], np.uint16))
        keep.extend(arrs)
        return _QMat(*(a.ctypes.data for a in arrs))

    Is = w["Is"]
    L = _Layer(w["H"], w["E"], k, w["I"], Is,
               qm(w["gate"]), qm(w["up"]), qm(w["down"]),
               qm(w.get("sh_gate") if Is else None), qm(w.get("sh_up") if Is else None),
               qm(w.get("sh_down") if Is else None))
    return L, keep


def ffn_tokens(w: dict, k: int, x, topk_ids, topk_weights, tokens) -> np.ndarray:
    """float64 layer output rows for the listed tokens (indices into x)."""
    x = _c(x, np.uint16)
    ids = _c(topk_ids, np.int32)
    tw = _c(topk_weights, np.float32)
    tokens = _c(tokens, np.int32)
    y = np.empty((len(tokens), w["H"]), dtype=np.float64)
    L, keep = _layer_struct(w, k)
    lib().oracle_ffn_tokens(C.byref(L), _p(x), _p(ids), _p(tw), _p(tokens), len(tokens), _p(y))
    del keep
    return y


def forward(w: dict, k: int, x, bias, chunk: int, BM: int, tokens=None):
    """Layer output, chunk by chunk.  Returns (y rows, list of per-chunk routing).

    With `tokens` given, only those rows of y are evaluated (routing is still
    computed for every chunk that holds one of them).
    """
    x = _c(x, np.uint16)
    T = x.shape[0]
    want = np.arange(T, dtype=np.int32) if tokens is None else _c(tokens, np.int32)
    y = np.zeros((len(want), w["H"]), dtype=np.float64)
    routes = []
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        sel = np.nonzero((want >= c0) & (want < c1))[0]
        if tokens is not None and len(sel) == 0:
            routes.append(None)
            continue
        r = route(x[c0:c1], w["router_w"], bias, k, BM)
        routes.append(r)
        if len(sel):
            y[sel] = ffn_tokens(w, k, x[c0:c1], r["topk_ids"], r["topk_weights"], want[sel] - c0)
    return y, routes
