"""Pins of the CPU oracle against values fixed by the pages or by mathematics.

None of these tests runs the HIP path.  Each check is independent of the
oracle's own code: hand-computed groups, numpy library routines (matmul,
stable argsort, bincount, cumsum), a dense all-experts brute force written
here in numpy, and special cases that reduce to a textbook gated MLP.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import moe_inputs as mi
from oracle import oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---- independent numpy helpers (written from the definitions, not the oracle) ----

def np_bf16(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def np_dequant(m, e=0):
    codes = np.asarray(m["codes"][e])
    q = np.empty((codes.shape[0], codes.shape[1] * 2), np.float64)
    q[:, 0::2] = codes & 0x0F
    q[:, 1::2] = codes >> 4
    s = np.repeat(np_bf16(m["scales"][e]), 64, axis=1)
    b = np.repeat(np_bf16(m["biases"][e]), 64, axis=1)
    return s * q + b


def np_gated_mlp(wg, wu, wd, x):
    g = x @ wg.T
    u = x @ wu.T
    h = g * (1.0 / (1.0 + np.exp(-g))) * u
    return h @ wd.T


def np_route(x_bits, router_w, bias, k):
    xf = np_bf16(x_bits)
    logits = (xf @ router_w.astype(np.float64).T).astype(np.float32)
    if bias is not None:
        logits = (logits + bias.astype(np.float32)).astype(np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, order, 1).astype(np.float64)
    p = np.exp(sel - sel[:, :1])
    return logits, order.astype(np.int32), (p / p.sum(1, keepdims=True)).astype(np.float32)


def pack_codes(q):
    q = np.asarray(q, np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


# ---- dequant and nibble order -------------------------------------------------

def test_dequant_hand_group():
    g = _gold("hand_dequant.json")
    K = 128
    q = (np.arange(K) % 16)[None, :]
    s = mi.f32_to_bf16_bits(np.array([[1 / 16, 1 / 8]], np.float32))
    b = mi.f32_to_bf16_bits(np.array([[-0.5, 0.25]], np.float32))
    w = orc.dequant(pack_codes(q), s, b)
    sums = [w[0, :64].sum(), w[0, 64:].sum()]
    assert sums == g["expected_group_sums_with_x_ones"]
    assert list(w[0, :4]) == g["expected_first_weights"]
    # Ramp dot: sum_k k*w_k in exact rational arithmetic (catches a swapped
    # nibble order, a wrong group index and a dropped bias).
    exact = sum(Fraction(kk) * (Fraction(1, 16 if kk < 64 else 8) * (kk % 16)
                                + (Fraction(-1, 2) if kk < 64 else Fraction(1, 4)))
                for kk in range(K))
    assert Fraction(float((np.arange(K) * w[0]).sum())) == exact


def test_dequant_zero_scale_gives_bias_and_random_matches_definition():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (8, 64), dtype=np.uint8)
    s = np.zeros((8, 2), np.uint16)
    b = mi.f32_to_bf16_bits(rng.uniform(-1, 1, (8, 2)).astype(np.float32))
    w = orc.dequant(codes, s, b)
    assert np.array_equal(w, np.repeat(np_bf16(b), 64, axis=1))
    s = mi.f32_to_bf16_bits(rng.uniform(0.005, 0.02, (8, 2)).astype(np.float32))
    w = orc.dequant(codes, s, b)
    assert np.array_equal(w, np_dequant(dict(codes=codes[None], scales=s[None], biases=b[None])))


# ---- storage closed form --------------------------------------------------------

def test_storage_bytes_per_param():
    g = _gold("pages_storage.json")
    H, I = 2048, 512
    w = mi.gen_weights(H, 1, I, 0, seed=3)
    nbytes = sum(w[m][a].nbytes for m in ("gate", "up", "down") for a in ("codes", "scales", "biases"))
    params = 3 * H * I
    assert params == g["expert_params_h2048_i512"]
    assert nbytes == g["expert_bytes_h2048_i512"]
    assert nbytes / params == g["bytes_per_param"] == g["bits"] / 8 + 4 / g["group"]


# ---- router logits ----------------------------------------------------------------

@pytest.mark.parametrize("T,H,E", [(64, 256, 16), (16, 2048, 256)])
def test_router_logits_vs_numpy_float64(T, H, E):
    rng = np.random.default_rng(T + H)
    x = mi.gen_x(T, H, seed=T)
    wr = rng.normal(0, 0.02, (E, H)).astype(np.float32)
    bias = mi.zipf_logit_bias(E, seed=7)
    got = orc.router_logits(x, wr, bias)
    ref, _, _ = np_route(x, wr, bias, 1)
    ulps = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1
    assert (ulps == 0).mean() > 0.999


def test_router_zero_weights_with_decreasing_bias():
    T, H, E, k = 10, 128, 12, 3
    x = mi.gen_x(T, H, 1)
    wr = np.zeros((E, H), np.float32)
    bias = -np.arange(E, dtype=np.float32)
    r = orc.route(x, wr, bias, k, BM=4)
    assert np.array_equal(r["topk_ids"], np.tile(np.arange(k, dtype=np.int32), (T, 1)))
    assert np.array_equal(r["counts"][:k], np.full(k, T, np.int32))
    assert r["counts"][k:].sum() == 0


# ---- top-k and weights --------------------------------------------------------------

def test_topk_matches_stable_sort_with_ties():
    rng = np.random.default_rng(11)
    logits = (rng.integers(0, 6, (200, 32)) * 0.25).astype(np.float32)  # many ties
    for k in (1, 2, 5, 8):
        ids, w = orc.topk(logits, k)
        ref = np.argsort(-logits, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref)
        sel = np.take_along_axis(logits, ref, 1).astype(np.float64)
        p = np.exp(sel - sel[:, :1])
        assert np.array_equal(w, (p / p.sum(1, keepdims=True)).astype(np.float32))


def test_equal_logits_give_uniform_weights():
    logits = np.zeros((5, 16), np.float32)
    for k in (1, 2, 4, 8):
        ids, w = orc.topk(logits, k)
        assert np.array_equal(ids, np.tile(np.arange(k), (5, 1)))
        assert np.all(w == np.float32(1.0 / k))


# ---- routing metadata ----------------------------------------------------------------

@pytest.mark.parametrize("T,E,k,BM", [(64, 16, 2, 16), (300, 64, 8, 32), (1, 256, 8, 64), (7, 8, 8, 4)])
def test_meta_matches_library_routines(T, E, k, BM):
    rng = np.random.default_rng(T * E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    m = orc.route_meta(ids, E, BM)
    flat = ids.reshape(-1)
    assert np.array_equal(m["counts"], np.bincount(flat, minlength=E))
    assert m["counts"].sum() == T * k
    assert np.array_equal(m["offsets"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(m["sorted_assign"], np.argsort(flat, kind="stable"))
    c = m["counts"]
    n_expected = int(sum((int(ci) + BM - 1) // BM for ci in c)) + (T + BM - 1) // BM
    assert m["n_tiles"] == n_expected
    tiles = m["tiles"]
    assert tiles[:, 2].min() >= 1 and tiles[:, 2].max() <= BM
    assert tiles[:, 2].sum() == T * k + T
    keys = tiles[:, 0].astype(np.int64) * (1 << 32) + tiles[:, 1]
    assert np.all(np.diff(keys) > 0)
    for e, r0, rows in tiles:
        lim = T if e == E else c[e]
        assert r0 % BM == 0 and r0 + rows <= lim


def test_pages_routing_load_2k_chunk():
    """2048 tokens, top-8 of 256: 16,384 assignments, mean 64 rows, uneven."""
    g = _gold("pages_routing_load.json")
    case = mi.make_case("prefill512", cache=False)
    x = mi.gen_x(g["tokens"], 2048, seed=9)
    r = orc.route(x, case["w"]["router_w"], None, g["top_k"], BM=64)
    assert r["counts"].sum() == g["assignments"]
    assert r["counts"].sum() / g["experts"] == g["mean_rows_per_expert"]
    assert r["counts"].max() > g["mean_rows_per_expert"] > r["counts"].min()


# ---- FFN and combine ---------------------------------------------------------------------

def _dense_bruteforce(case):
    """All experts evaluated for every token, masked by the top-k weights."""
    w, x, k = case["w"], case["x"], case["k"]
    xf = np_bf16(x)
    _, ids, tw = np_route(x, w["router_w"], case["bias"], k)
    T, E = xf.shape[0], w["E"]
    gate_mat = np.zeros((T, E))
    np.put_along_axis(gate_mat, ids, tw.astype(np.float64), 1)
    y = np.zeros((T, w["H"]))
    for e in range(E):
        out_e = np_gated_mlp(np_dequant(w["gate"], e), np_dequant(w["up"], e), np_dequant(w["down"], e), xf)
        y += gate_mat[:, e:e + 1] * out_e
    if w["Is"]:
        y += np_gated_mlp(np_dequant(w["sh_gate"]), np_dequant(w["sh_up"]), np_dequant(w["sh_down"]), xf)
    return y, ids, tw


def test_ffn_matches_dense_bruteforce_tiny():
    case = mi.make_case("tiny")
    y_ref, ids_ref, tw_ref = _dense_bruteforce(case)
    y, routes = orc.forward(case["w"], case["k"], case["x"], case["bias"], chunk=2048, BM=16)
    assert np.array_equal(routes[0]["topk_ids"], ids_ref)
    assert np.array_equal(routes[0]["topk_weights"], tw_ref)
    rel = np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref)
    assert rel < 1e-12


def test_ffn_matches_dense_bruteforce_with_bias_and_ragged():
    case = mi.small_layer(T=37, H=128, E=8, k=3, I=64, Is=128, seed=21, zipf_seed=22)
    y_ref, _, _ = _dense_bruteforce(case)
    y, _ = orc.forward(case["w"], case["k"], case["x"], case["bias"], chunk=16, BM=8)
    assert np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref) < 1e-12


def test_single_expert_reduces_to_gated_mlp():
    case = mi.small_layer(T=9, H=192, E=1, k=1, I=128, Is=0, seed=31)
    w = case["w"]
    y, routes = orc.forward(w, 1, case["x"], None, chunk=64, BM=4)
    assert np.all(routes[0]["topk_weights"] == 1.0)
    ref = np_gated_mlp(np_dequant(w["gate"]), np_dequant(w["up"]), np_dequant(w["down"]), np_bf16(case["x"]))
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 1e-12


def test_zero_up_projection_leaves_shared_only():
    case = mi.small_layer(T=12, H=128, E=6, k=2, I=64, Is=64, seed=41)
    w = case["w"]
    for a in ("codes", "scales", "biases"):
        w["up"][a][...] = 0
    y, _ = orc.forward(w, 2, case["x"], None, chunk=64, BM=4)
    ref = np_gated_mlp(np_dequant(w["sh_gate"]), np_dequant(w["sh_up"]), np_dequant(w["sh_down"]), np_bf16(case["x"]))
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 1e-12


def test_chunking_does_not_change_output():
    case = mi.make_case("tiny")
    y1, r1 = orc.forward(case["w"], case["k"], case["x"], case["bias"], chunk=64, BM=16)
    y2, r2 = orc.forward(case["w"], case["k"], case["x"], case["bias"], chunk=16, BM=16)
    assert np.array_equal(y1, y2)
    assert len(r1) == 1 and len(r2) == 4
    assert np.array_equal(np.concatenate([r["topk_ids"] for r in r2]), r1[0]["topk_ids"])


def test_token_subset_equals_full_rows():
    case = mi.make_case("tiny")
    y, _ = orc.forward(case["w"], case["k"], case["x"], case["bias"], chunk=32, BM=16)
    sub = np.array([0, 5, 31, 32, 63], np.int32)
    ys, _ = orc.forward(case["w"], case["k"], case["x"], case["bias"], chunk=32, BM=16, tokens=sub)
    assert np.array_equal(ys, y[sub])


def test_zipf_workload_load_range():
    """The skewed prefill recipe gives expert loads from 0 to more than 400 rows per 2048-token chunk."""
    case = mi.make_case("prefill512", cache=False)
    x = mi.gen_x(2048, 2048, 400)
    r = orc.route(x, case["w"]["router_w"], mi.zipf_logit_bias(256, 401), 8, BM=64)
    assert r["counts"].min() == 0 and r["counts"].max() > 400
