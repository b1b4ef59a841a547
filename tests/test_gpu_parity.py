"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars: routing indices, counts, offsets, permutation and block map bit-exact;
routing weights within 1e-5; layer outputs within relative L2 <= 5e-3 and
max-abs <= 2e-2 * RMS(reference) of the float64 oracle.
"""
import numpy as np
import pytest

import conftest
import moe_inputs as mi
from oracle import oracle as orc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL_L2 = 5e-3
MAXABS_RMS = 2e-2
W_TOL = 1e-5


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def M():
    _need_gpu()
    from bit_quantized_moe_router_amd import layer as L
    return L


_LAYERS = {}


def get_layer(M, case, **kw):
    key = (case["cfg"]["H"], case["cfg"]["E"], case["cfg"]["I"], case["cfg"]["Is"], case["cfg"]["wseed"],
           case["k"], tuple(sorted(kw.items())))
    if key not in _LAYERS:
        bi = kw.pop("batch_invariant", 0)
        _LAYERS[key] = M.MoELayer(case["w"], case["k"], max_tokens=kw.pop("max_tokens", 2048), **kw)
        _LAYERS[key].set_desc(batch_invariant=bi)
    return _LAYERS[key]


def dev(M, a):
    return None if a is None else M.to_dev(a, "cuda")


def check_close(y, ref, label):
    y = np.asarray(y, np.float64)
    err = y - ref
    rel = np.linalg.norm(err) / np.linalg.norm(ref)
    rms = np.sqrt(np.mean(ref ** 2))
    maxabs = np.abs(err).max()
    print(f"[parity] {label}: rel_l2={rel:.3e} max_abs/rms={maxabs / rms:.3e}", flush=True)
    conftest.PARITY_LOG.append((label, float(rel), float(maxabs / rms)))
    assert np.all(np.isfinite(y)), label
    assert rel <= REL_L2, (label, rel)
    assert maxabs <= MAXABS_RMS * rms, (label, maxabs / rms)


def check_route(r_gpu, r_ref, label):
    g = {k: v.cpu().numpy() for k, v in r_gpu.items()}
    assert np.array_equal(g["topk_ids"], r_ref["topk_ids"]), label
    assert np.array_equal(g["expert_counts"], r_ref["counts"]), label
    assert np.array_equal(g["expert_offsets"], r_ref["offsets"]), label
    assert np.array_equal(g["sorted_assign"], r_ref["sorted_assign"]), label
    n = int(g["n_tiles"][0])
    assert n == r_ref["n_tiles"], label
    assert np.array_equal(g["tile_map"][:n], r_ref["tiles"]), label
    dw = np.abs(g["topk_weights"].astype(np.float64) - r_ref["topk_weights"]).max()
    assert dw <= W_TOL, (label, dw)
    print(f"[route] {label}: bit-exact, max|dw|={dw:.2e}", flush=True)


# ---- packer -------------------------------------------------------------------

def unpack_matrix(blob, base, N, K, stride_nb, stride_g, stride_blk=1152):
    """Inverse of the documented blob layout, written from the layout description."""
    NBn, G = N // 32, K // 64
    idx = (base + np.arange(NBn)[:, None, None] * stride_nb + np.arange(G)[None, :, None] * stride_g
           + np.arange(1152)[None, None, :])
    blk = blob[idx]  # [NBn][G][1152]
    d = np.ascontiguousarray(blk[..., :1024]).view(np.uint32).reshape(NBn, G, 2, 32, 4)
    nib = (d[..., None] >> (4 * np.arange(8, dtype=np.uint32))) & 15  # [NBn][G][h][row][c][p]
    koff = np.array([0, 2, 4, 6, 1, 3, 5, 7])
    q = np.empty((NBn, 32, G, 2, 4, 8), np.uint8)
    q[..., koff] = nib.transpose(0, 3, 1, 2, 4, 5)
    q = q.reshape(N, K)
    sb = np.ascontiguousarray(blk[..., 1024:]).view(np.uint32).reshape(NBn, G, 32).transpose(0, 2, 1).reshape(N, G)
    return q, (sb & 0xFFFF).astype(np.uint16), (sb >> 16).astype(np.uint16)


def bf16_as_f16_bits(a):
    """The packer's conversion of bf16 scale/bias bits to fp16 bits (round to nearest even)."""
    f = (np.asarray(a, np.uint32) << 16).view(np.float32)
    return f.astype(np.float16).view(np.uint16)


def canon_q(codes):
    q = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.uint8)
    q[..., 0::2] = codes & 15
    q[..., 1::2] = codes >> 4
    return q


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_pack_roundtrip(M, name):
    case = mi.make_case(name)
    w = case["w"]
    lay = get_layer(M, case)
    blob = lay.packed.cpu().numpy()
    H, E, I, Is = w["H"], w["E"], w["I"], w["Is"]
    gu = (I // 32) * (H // 64) * 2 * 1152
    ex = gu + (H // 32) * (I // 64) * 1152
    assert blob.size == E * ex + 3 * H * Is * 9 // 16 + 256
    # The trailer: the small-scale flag (every scale of these layers is below 2^-4), then zeros.
    trailer = blob[-256:].view(np.int32)
    assert trailer[0] == 1 and not trailer[1:].any()
    experts = range(E) if E <= 16 else [0, 1, 77, E - 1]
    for e in experts:
        for which, m in ((0, "gate"), (1, "up")):
            q, s, b = unpack_matrix(blob, e * ex + which * 1152, I, H, (H // 64) * 2 * 1152, 2 * 1152)
            assert np.array_equal(q, canon_q(w[m]["codes"][e])), (e, m)
            assert np.array_equal(s, bf16_as_f16_bits(w[m]["scales"][e]))
            assert np.array_equal(b, bf16_as_f16_bits(w[m]["biases"][e]))
        q, s, b = unpack_matrix(blob, e * ex + gu, H, I, (I // 64) * 1152, 1152)
        assert np.array_equal(q, canon_q(w["down"]["codes"][e]))
        assert np.array_equal(s, bf16_as_f16_bits(w["down"]["scales"][e]))
        assert np.array_equal(b, bf16_as_f16_bits(w["down"]["biases"][e]))
    sgu = (Is // 32) * (H // 64) * 2 * 1152
    q, s, b = unpack_matrix(blob, E * ex + 1152, Is, H, (H // 64) * 2 * 1152, 2 * 1152)
    assert np.array_equal(q, canon_q(w["sh_up"]["codes"][0]))
    q, s, b = unpack_matrix(blob, E * ex + sgu, H, Is, (Is // 64) * 1152, 1152)
    assert np.array_equal(q, canon_q(w["sh_down"]["codes"][0]))
    assert np.array_equal(b, bf16_as_f16_bits(w["sh_down"]["biases"][0]))
    # In fp16's normal range the conversion is exact; below it (small biases)
    # it is off by less than half the fp16 subnormal step, 2^-25.
    for m in ("gate", "up", "down"):
        for a in (w[m]["scales"], w[m]["biases"]):
            f = (np.asarray(a, np.uint32) << 16).view(np.float32)
            g = f.astype(np.float16).astype(np.float32)
            normal = np.abs(f) >= 2.0 ** -14
            assert np.array_equal(g[normal], f[normal])
            assert np.all(np.abs(g - f) <= 2.0 ** -25)


def _with_scales_times(w, factor, mats=("gate", "up", "down")):
    """A copy of layer weights with the listed matrices' scales multiplied by factor (bf16 bits)."""
    w2 = dict(w)
    for m in mats:
        q = dict(w[m])
        q["scales"] = mi.f32_to_bf16_bits(mi.bf16_bits_to_f32(q["scales"]) * factor)
        w2[m] = q
    return w2


def test_pack_clears_small_scale_flag(M):
    """A layer with scales of 2^-4 and more: the packer clears the trailer's
    flag, the grouped GEMM rebuilds weights with the general form, and the
    output matches the oracle."""
    case = mi.small_layer(300, 256, 16, 4, 128, 128, 71, 72)
    case["w"] = _with_scales_times(case["w"], 8.0, ("up", "down"))  # U(0.04, 0.16)
    lay = M.MoELayer(case["w"], case["k"], max_tokens=300)
    assert lay.packed[-256:].cpu().numpy().view(np.int32)[0] == 0
    y = lay.forward_prefill(dev(M, case["x"]), dev(M, case["bias"]))
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), oracle_rows(case), "scales up to 0.16 (general rebuild)")


@pytest.mark.parametrize("name,T", [("tiny", 64), ("prefill4096", 2048)])
def test_rebuild_forms_same_bits(M, name, T):
    """The grouped GEMM's two weight rebuilds (the subnormal form taken when
    every scale is below 2^-4, and the general form) give the same bits: the
    same blob with its trailer flag cleared by hand takes the general form."""
    case = mi.make_case(name)
    lay = get_layer(M, case)
    assert lay.packed[-256:].cpu().numpy().view(np.int32)[0] == 1
    x, b = dev(M, case["x"])[:T].contiguous(), dev(M, case["bias"])
    y_small = lay.forward_prefill(x, b).clone()
    saved = lay.packed.clone()
    try:
        lay.packed[-256:-252].zero_()
        y_general = lay.forward_prefill(x, b).clone()
        torch.cuda.synchronize()
    finally:
        lay.packed.copy_(saved)
        torch.cuda.synchronize()
    assert torch.equal(y_small, y_general)


def test_rebuild_forms_same_bits_edge_scales(M):
    """Scales at the edges of the subnormal rebuild's range (just below 2^-4,
    negative, zero, fp16-subnormal after the packer's conversion) and biases of
    many magnitudes: the packer keeps the small-scale flag, both rebuild forms
    give the same bits, and the output matches the oracle."""
    case = mi.small_layer(300, 256, 16, 4, 128, 128, 73, 74)
    rng = np.random.default_rng(75)
    edge = np.array([0.0625 - 2.0 ** -12, -(0.0625 - 2.0 ** -12), 0.0, 2.0 ** -15, -(2.0 ** -18), 2.0 ** -24,
                     0.03, -0.011, 1e-4], np.float32)
    w = dict(case["w"])
    for m in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
        q = dict(w[m])
        sc = mi.bf16_bits_to_f32(q["scales"]).copy()
        pick = rng.random(sc.shape) < 0.5
        sc[pick] = rng.choice(edge, size=int(pick.sum()))
        q["scales"] = mi.f32_to_bf16_bits(sc)
        bi = mi.bf16_bits_to_f32(q["biases"]).copy()
        pick = rng.random(bi.shape) < 0.3
        bi[pick] *= rng.choice(np.array([1e-5, 1e-3, 30.0, -30.0], np.float32), size=int(pick.sum()))
        q["biases"] = mi.f32_to_bf16_bits(bi)
        w[m] = q
    case["w"] = w
    lay = M.MoELayer(w, case["k"], max_tokens=300)
    assert lay.packed[-256:].cpu().numpy().view(np.int32)[0] == 1
    x, b = dev(M, case["x"]), dev(M, case["bias"])
    y_small = lay.forward_prefill(x, b).clone()
    lay.packed[-256:-252].zero_()
    y_general = lay.forward_prefill(x, b).clone()
    torch.cuda.synchronize()
    assert torch.equal(y_small, y_general)
    check_close(y_small.cpu().numpy(), oracle_rows(case), "edge scales (subnormal rebuild)")


# ---- routing ------------------------------------------------------------------

ROUTE_CASES = ["tiny", "decode", "smallrow2", "smallrow3", "smallrow4", "smallrow5", "smallrow8", "prefill512",
               "prefill4096"]


@pytest.mark.parametrize("name", ROUTE_CASES)
def test_route_bitexact(M, name):
    case = mi.make_case(name)
    lay = get_layer(M, case)
    BM = lay.desc.tile_rows or 128  # library default
    x, bias = case["x"], case["bias"]
    for c0 in range(0, case["T"], mi.CHUNK):
        xc = x[c0:c0 + mi.CHUNK]
        r = lay.route(dev(M, xc), dev(M, bias))
        torch.cuda.synchronize()
        ref = orc.route(xc, case["w"]["router_w"], bias, case["k"], BM)
        check_route(r, ref, f"{name}[{c0}:]")


@pytest.mark.parametrize("spread", [1e-7, 3e-3])
def test_route_near_ties(M, spread):
    """Router rows that all differ from one shared row by a relative `spread`:
    every logit of a token lies within a few times the screen's error bound
    of the others, so the exact step recomputes most or all experts (up to
    256 candidates, ranked through LDS past 64) and must still give the
    oracle's top-k exactly."""
    case = mi.make_case("prefill512")
    rng = np.random.default_rng(4711)
    H, E = case["cfg"]["H"], case["cfg"]["E"]
    base = rng.standard_normal(H).astype(np.float32) * np.float32(0.02)
    wr = (base[None, :] * (1 + spread * rng.standard_normal((E, H)))).astype(np.float32)
    w = dict(case["w"], router_w=wr)
    lay = M.MoELayer(w, case["k"], max_tokens=256)
    x = case["x"][:256]
    r = lay.route(dev(M, x), None)
    torch.cuda.synchronize()
    ref = orc.route(x, wr, None, case["k"], lay.desc.tile_rows or 128)
    logits = ref["logits"].astype(np.float64)
    kth = -np.sort(-logits, axis=1)[:, case["k"] - 1]
    close = (logits >= kth[:, None] - 1e-3).sum(axis=1)  # experts within 1e-3 of the k-th logit
    print(f"[route] near ties spread={spread}: median experts within 1e-3 of the k-th: {int(np.median(close))}",
          flush=True)
    check_route(r, ref, f"near ties spread={spread}")


@pytest.mark.parametrize("bm", [16, 32, 128])
def test_route_tile_rows(M, bm):
    case = mi.make_case("prefill512")
    lay = get_layer(M, case, tile_rows=bm)
    r = lay.route(dev(M, case["x"]), None)
    torch.cuda.synchronize()
    check_route(r, orc.route(case["x"], case["w"]["router_w"], None, case["k"], bm), f"prefill512 BM={bm}")


# ---- full layer -----------------------------------------------------------------

def oracle_rows(case, tokens=None, chunk=mi.CHUNK):
    y, _ = orc.forward(case["w"], case["k"], case["x"], case["bias"], chunk, 64, tokens=tokens)
    return y


@pytest.mark.parametrize("bm,chunk", [(0, 2048), (16, 2048), (32, 16), (128, 64), (64, 7)])
def test_tiny_prefill_all_rows(M, bm, chunk):
    case = mi.make_case("tiny")
    lay = get_layer(M, case, tile_rows=bm, max_chunk=chunk)
    y = lay.forward_prefill(dev(M, case["x"]), dev(M, case["bias"]))
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), oracle_rows(case), f"tiny prefill BM={bm} chunk={chunk}")


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("gemv", [8, 0])
def test_tiny_decode_both_paths(M, T, gemv):
    case = mi.make_case("tiny")
    lay = get_layer(M, case, gemv_max_rows=gemv)
    x = case["x"][:T]
    y = lay.forward_decode(dev(M, x), None)
    torch.cuda.synchronize()
    sub = dict(case, x=x, T=T)
    check_close(y.cpu().numpy(), oracle_rows(sub), f"tiny decode T={T} gemv_max_rows={gemv}")


@pytest.mark.parametrize("T", [9, 20])
def test_decode_above_gemv_rows_takes_gemm_path(M, T):
    """moe_forward_decode with more rows than the GEMV takes runs the grouped-GEMM
    path (checked by which kernels ran) and matches the oracle."""
    from bit_quantized_moe_router_amd import (K_DOWN_GEMM, K_GATEUP_GEMV, moe_profile_enable, moe_profile_read,
                                              moe_profile_reset)
    case = mi.make_case("decode")
    lay = get_layer(M, case)
    x = mi.gen_x(T, case["cfg"]["H"], 6100 + T)
    moe_profile_reset()
    moe_profile_enable((1 << K_GATEUP_GEMV) | (1 << K_DOWN_GEMM))
    try:
        y = lay.forward_decode(dev(M, x), None)
        torch.cuda.synchronize()
        ran = (moe_profile_read(K_GATEUP_GEMV)[1], moe_profile_read(K_DOWN_GEMM)[1])
    finally:
        moe_profile_enable(0)
        moe_profile_reset()
    assert ran == (0, 1), ran
    check_close(y.cpu().numpy(), oracle_rows(dict(case, x=x, T=T)), f"decode T={T} (grouped GEMM)")


def test_decode_T1(M):
    case = mi.make_case("decode")
    lay = get_layer(M, case)
    y = lay.forward_decode(dev(M, case["x"]), None)
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), oracle_rows(case), "decode T=1 (GEMV)")


@pytest.mark.parametrize("T", mi.SMALLROW_TS)
@pytest.mark.parametrize("gemv", [8, 0])
def test_smallrow_both_paths(M, T, gemv):
    case = mi.make_case(f"smallrow{T}")
    lay = get_layer(M, case, gemv_max_rows=gemv)
    y = lay.forward_decode(dev(M, case["x"]), None)
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), oracle_rows(case), f"smallrow T={T} gemv_max_rows={gemv}")


EDGE_DECODE = [  # T, H, E, k, I, Is, seed, zipf
    (5, 64, 4, 4, 64, 64, 61, None),      # k == E
    (8, 192, 1, 1, 128, 0, 31, None),     # one expert, no shared expert
    (7, 128, 8, 3, 64, 128, 21, 22),      # Is != I, zipf bias
    (8, 320, 16, 8, 192, 64, 71, None),   # k == 8 of 16, odd group counts
    (8, 4096, 64, 8, 256, 256, 91, None), # T * H at the GEMV's LDS limit, 64 groups per row
    (4, 8192, 32, 4, 128, 64, 93, None),  # widest hidden the GEMV takes, 128 groups per row
]


@pytest.mark.parametrize("T,H,E,k,I,Is,seed,zipf", EDGE_DECODE)
def test_decode_gemv_edge_shapes(M, T, H, E, k, I, Is, seed, zipf):
    """The GEMV path (forced for all T <= 8) on odd shapes; checks that it is the path that ran."""
    from bit_quantized_moe_router_amd import (K_DOWN_GEMM, K_GATEUP_GEMV, moe_profile_enable, moe_profile_read,
                                              moe_profile_reset)
    case = mi.small_layer(T, H, E, k, I, Is, seed, zipf)
    lay = M.MoELayer(case["w"], k, max_tokens=T, gemv_max_rows=8)
    moe_profile_reset()
    moe_profile_enable((1 << K_GATEUP_GEMV) | (1 << K_DOWN_GEMM))
    try:
        y = lay.forward_decode(dev(M, case["x"]), dev(M, case["bias"]))
        torch.cuda.synchronize()
        ran = (moe_profile_read(K_GATEUP_GEMV)[1], moe_profile_read(K_DOWN_GEMM)[1])
    finally:
        moe_profile_enable(0)
        moe_profile_reset()
    assert ran == (1, 0), ran
    check_close(y.cpu().numpy(), oracle_rows(case), f"edge {case['name']} GEMV decode")


@pytest.mark.parametrize("gemv,scale", [(8, 1.0 / 32), (8, 256.0), (0, 1.0 / 32), (0, 16.0)])
def test_decode_activation_scale(M, gemv, scale):
    """Both decode paths keep activations as fp16(x / 256) for their MFMAs:
    small activations (many of them fp16 subnormals after the scaling) and
    large ones stay within tolerance of the oracle.  The grouped-GEMM path
    also keeps h as fp16(h / 256), so |h| must stay below about 1.7e7; h
    grows with the square of the activations' scale, and x * 16 (|x| up to
    about 70) is well inside it.  The GEMV path keeps h in bf16 and takes
    x * 256 (|x| up to about 1000)."""
    case = mi.small_layer(3, 1024, 32, 4, 256, 128, 97, None)
    x = mi.bf16_bits_to_f32(case["x"]) * np.float32(scale)
    case["x"] = mi.f32_to_bf16_bits(x)
    lay = M.MoELayer(case["w"], case["k"], max_tokens=8, gemv_max_rows=gemv)
    y = lay.forward_decode(dev(M, case["x"]), None)
    torch.cuda.synchronize()
    yn = y.cpu().numpy()
    assert np.all(np.isfinite(yn))
    check_close(yn, oracle_rows(case), f"decode x*{scale} gemv_max_rows={gemv}")


def _sample_tokens(case, n, seed):
    """Seeded random sample of the tokens, plus the first and the last token."""
    rng = np.random.default_rng(seed)
    T = case["T"]
    toks = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    toks.update([0, T - 1])
    return np.array(sorted(toks), np.int32)


@pytest.mark.parametrize("name", ["prefill512", "prefill4096"])
def test_prefill_sampled_rows(M, name):
    case = mi.make_case(name)
    lay = get_layer(M, case)
    y = lay.forward_prefill(dev(M, case["x"]), dev(M, case["bias"]))
    torch.cuda.synchronize()
    yn = y.cpu().numpy()
    assert np.all(np.isfinite(yn))
    toks = _sample_tokens(case, 40, seed=7)
    check_close(yn[toks], oracle_rows(case, toks), f"{name} sampled {len(toks)} rows")


def test_prefill_full_layer_ragged_second_chunk(M):
    """The full-size layer at T = 2048 + 37: a whole 2048-token chunk and a
    37-token chunk in flight together (the second on the library's stream).
    Every token of the short chunk and a sample of the long one against the
    oracle."""
    base = mi.make_case("prefill4096")
    T = mi.CHUNK + 37
    case = dict(base, x=base["x"][:T], T=T)
    lay = get_layer(M, base)
    y = lay.forward_prefill(dev(M, case["x"]), dev(M, case["bias"]))
    torch.cuda.synchronize()
    yn = y.cpu().numpy()
    assert yn.shape == (T, base["w"]["H"]) and np.all(np.isfinite(yn))
    toks = np.union1d(_sample_tokens(case, 24, seed=11), np.arange(mi.CHUNK, T)).astype(np.int32)
    check_close(yn[toks], oracle_rows(case, toks), f"prefill4096[:{T}] sampled {len(toks)} rows")


# ---- edge cases -------------------------------------------------------------------

EDGE = [
    # T, H, E, k, I, Is, seed, zipf, chunk, bm
    (37, 128, 8, 3, 64, 128, 21, 22, 16, 16),   # ragged chunks, zipf bias, Is != I
    (9, 192, 1, 1, 128, 0, 31, None, 64, 32),   # one expert, no shared expert
    (50, 256, 32, 8, 192, 64, 51, 52, 2048, 64),  # k=8 of 32, I not a multiple of 128
    (5, 64, 4, 4, 64, 64, 61, None, 2, 16),     # k == E, tiny chunks
    (300, 256, 32, 8, 64, 64, 91, 92, 2048, 128),  # 2400 assignments: three metadata segments, the last partial
]


@pytest.mark.parametrize("T,H,E,k,I,Is,seed,zipf,chunk,bm", EDGE)
def test_edge_layers(M, T, H, E, k, I, Is, seed, zipf, chunk, bm):
    case = mi.small_layer(T, H, E, k, I, Is, seed, zipf)
    lay = M.MoELayer(case["w"], k, max_tokens=T, max_chunk=chunk, tile_rows=bm)
    y = lay.forward_prefill(dev(M, case["x"]), dev(M, case["bias"]))
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), oracle_rows(case, chunk=chunk), f"edge {case['name']} prefill")
    if T <= 8:
        for gemv in (8, 0):
            lay.set_desc(gemv_max_rows=gemv)
            y = lay.forward_decode(dev(M, case["x"]), dev(M, case["bias"]))
            torch.cuda.synchronize()
            check_close(y.cpu().numpy(), oracle_rows(case, chunk=chunk), f"edge {case['name']} decode {gemv}")
    # routing of the first chunk
    xc = case["x"][:chunk]
    r = lay.route(dev(M, xc), dev(M, case["bias"]))
    torch.cuda.synchronize()
    ref = orc.route(xc, case["w"]["router_w"], case["bias"], k, bm, with_shared=Is > 0)
    check_route(r, ref, f"edge {case['name']}")


def test_prefill_cut_long_tiles(M):
    """Wide experts (8 gate/up column tiles each, so 32 long tiles stay whole on
    256 compute units) with 48 long tiles: the schedule cuts 16 of them in two;
    every output row is checked."""
    case = mi.small_layer(2048, 64, 2, 2, 2048, 2048, 81, None)
    lay = M.MoELayer(case["w"], 2, max_tokens=2048, tile_rows=128)
    y = lay.forward_prefill(dev(M, case["x"]), None)
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), oracle_rows(case), "cut long tiles")


def test_repeat_calls_bit_identical(M):
    """No atomics touch the outputs (the histogram's integer counts do not
    depend on order), so two calls on the same inputs agree bit for bit:
    prefill output, routing outputs, decode output."""
    case = mi.make_case("prefill512")
    lay = get_layer(M, case)
    x, b = dev(M, case["x"]), dev(M, case["bias"])
    y1 = lay.forward_prefill(x, b).clone()
    y2 = lay.forward_prefill(x, b).clone()
    r1 = {k: v.clone() for k, v in lay.route(x[:300], b).items()}
    r2 = lay.route(x[:300], b)
    d1 = lay.forward_decode(x[:3], b).clone()
    d2 = lay.forward_decode(x[:3], b).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    for key in r1:
        assert torch.equal(r1[key], r2[key]), key
    assert torch.equal(d1, d2)


@pytest.mark.parametrize("T,bi", [(1, 0), (3, 0), (2, 1)])
def test_decode_graph_replays_match_eager(M, T, bi):
    """Decode captured in a HIP graph (the calls enqueue kernels only: no
    allocation, copy, memset or host synchronisation), replayed several times
    with other eager work in between; every replay equals the eager call on
    the same rows bit for bit, and the oracle within tolerance.  bi = 1: the
    GEMV with the grouped GEMM's arithmetic."""
    case = mi.make_case("decode")
    lay = get_layer(M, case, batch_invariant=bi)
    H = case["cfg"]["H"]
    rows = [mi.gen_x(T, H, 9000 + r) for r in range(3)]
    eager = []
    for r in rows:
        eager.append(lay.forward_decode(dev(M, r), None).clone())
    torch.cuda.synchronize()
    x_static = dev(M, rows[0]).clone()
    y_static = torch.empty((T, H), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lay.forward_decode(x_static, None, y_static)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lay.forward_decode(x_static, None, y_static)
    other = dev(M, mi.gen_x(2, H, 9100))
    for rep in range(2):
        for i, r in enumerate(rows):
            x_static.copy_(dev(M, r))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y_static, eager[i]), (rep, i)
            lay.forward_decode(other, None)  # eager work between replays
            torch.cuda.synchronize()
    sub = dict(case, x=rows[-1], T=T)
    check_close(y_static.cpu().numpy(), oracle_rows(sub), f"decode graph replay T={T}" + (" batch-invariant" if bi else ""))


def test_prefill4096_two_chunks_in_flight_same_bits(M):
    """A workspace sized for the whole call (two chunk areas) runs the second
    2048-token chunk on the library's second stream beside the first; the output
    equals the one-area (serial) call bit for bit, and sampled rows match the
    oracle."""
    case = mi.make_case("prefill4096")
    ser = get_layer(M, case)
    two = get_layer(M, case, max_tokens=case["T"])
    assert two.ws.numel() > ser.ws.numel()
    x, b = dev(M, case["x"]), dev(M, case["bias"])
    y0 = ser.forward_prefill(x, b).clone()
    y1 = two.forward_prefill(x, b).clone()
    y2 = two.forward_prefill(x, b)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    assert torch.equal(y1, y2)
    toks = _sample_tokens(case, 40, seed=13)
    check_close(y1.cpu().numpy()[toks], oracle_rows(case, toks), "prefill4096 two chunks in flight")


@pytest.mark.parametrize("T,chunk", [(300, 64), (129, 64), (200, 100)])
def test_two_chunks_in_flight_many_chunks(M, T, chunk):
    """3-5 chunks, the last one ragged, alternating between the caller's stream
    and the second stream (chunk c + 2 reuses chunk c's area on the same
    stream).  Every row against the oracle, and the same bits as the serial
    call; then the call captured in a HIP graph and replayed with eager work in
    between, each replay equal to the eager result."""
    case = mi.small_layer(T, 256, 32, 8, 128, 64, 71, 72)
    ser = M.MoELayer(case["w"], 8, max_tokens=chunk, max_chunk=chunk)
    two = M.MoELayer(case["w"], 8, max_tokens=T, max_chunk=chunk)
    assert two.ws.numel() > ser.ws.numel()
    x, b = dev(M, case["x"]), dev(M, case["bias"])
    y0 = ser.forward_prefill(x, b).clone()
    y1 = two.forward_prefill(x, b).clone()
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    check_close(y1.cpu().numpy(), oracle_rows(case, chunk=chunk), f"two chunks in flight T={T} chunk={chunk}")
    x_static = x.clone()
    y_static = torch.empty_like(y1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        two.forward_prefill(x_static, b, y_static)
    other = dev(M, mi.gen_x(T, 256, 7300))
    y_other = two.forward_prefill(other, b).clone()
    for rep in range(3):
        y_static.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_static, y1), rep
        y_o = two.forward_prefill(other, b)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y_o, y_other), rep


def test_two_chunks_in_flight_from_two_threads(M):
    """Two host threads, each with its own layer workspace and torch stream,
    enqueue multi-chunk calls at the same time: they share the library's second
    stream and event pool, and every output equals the one-chunk-at-a-time
    result bit for bit."""
    import threading
    T, chunk = 300, 64
    case = mi.small_layer(T, 256, 32, 8, 128, 64, 75, 76)
    ser = M.MoELayer(case["w"], 8, max_tokens=chunk, max_chunk=chunk)
    lays = [M.MoELayer(case["w"], 8, max_tokens=T, max_chunk=chunk) for _ in range(2)]
    xs = [dev(M, mi.gen_x(T, 256, 7400 + i)) for i in range(2)]
    b = dev(M, case["bias"])
    refs = [ser.forward_prefill(x, b).clone() for x in xs]
    torch.cuda.synchronize()
    outs = [[None] * 6 for _ in range(2)]
    errs = []

    def work(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for r in range(6):
                    outs[i][r] = lays[i].forward_prefill(xs[i], b).clone()
            st.synchronize()
        except Exception as e:  # reported below
            errs.append(e)

    th = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t_ in th:
        t_.start()
    for t_ in th:
        t_.join()
    torch.cuda.synchronize()
    assert not errs, errs
    for i in range(2):
        for r in range(6):
            assert torch.equal(outs[i][r], refs[i]), (i, r)


@pytest.mark.parametrize("name", ["tiny", "prefill512"])
def test_host_sync_routing_same_result(M, name):
    """The host-synchronised routing measurement (schedule size read back,
    GEMM grids sized on the host) runs the same kernels: same bits as the
    normal path."""
    case = mi.make_case(name)
    lay = get_layer(M, case)
    x, b = dev(M, case["x"]), dev(M, case["bias"])
    y0 = lay.forward_prefill(x, b).clone()
    lay.set_desc(host_sync_routing=1)
    try:
        y1 = lay.forward_prefill(x, b)
        torch.cuda.synchronize()
    finally:
        lay.set_desc(host_sync_routing=0)
    assert torch.equal(y0, y1)
    toks = _sample_tokens(case, 24, seed=11)
    check_close(y1.cpu().numpy()[toks], oracle_rows(case, toks), f"{name} host-synchronised routing")


def test_batch_invariant_gemm_path(M):
    """With the row threshold at 0 the grouped-GEMM path serves every row
    count, and a row's output does not depend on the other rows of the call:
    the same rows decoded 1..8 at a time, and inside a 300-row prefill, give
    the same bits (routing is exact, each output element's K reduction runs
    in one fixed order, and the combine adds a token's rows in top-k order)."""
    case = mi.make_case("decode")
    lay = get_layer(M, case, gemv_max_rows=0, max_tokens=512)
    H = case["cfg"]["H"]
    big = mi.gen_x(300, H, 7700)
    pos = [0, 17, 64, 127, 128, 200, 256, 299]
    y_big = lay.forward_prefill(dev(M, big), None)
    torch.cuda.synchronize()
    for T in range(1, 9):
        y = lay.forward_decode(dev(M, big[pos[:T]]), None)
        torch.cuda.synchronize()
        for i in range(T):
            assert torch.equal(y[i], y_big[pos[i]]), (T, i)


def test_batch_invariant_gemm_path_large_tiles(M):
    """The same invariance across tile sizes for routed experts: in one
    skewed 2048-token chunk (Zipf logit bias) the popular experts fill
    128-row tiles, long ones cut into pieces, while the same rows decoded a
    few at a time sit in one-fragment tiles; the bits must agree."""
    case = mi.make_case("prefill4096")
    lay = get_layer(M, case, gemv_max_rows=0, max_tokens=2048)
    x = case["x"][:2048]
    bias = dev(M, case["bias"])
    y_big = lay.forward_prefill(dev(M, x), bias)
    torch.cuda.synchronize()
    pos = [0, 1, 511, 1024, 1500, 2047]
    for T in (1, 3, 6):
        y = lay.forward_decode(dev(M, x[pos[:T]]), bias)
        torch.cuda.synchronize()
        for i in range(T):
            assert torch.equal(y[i], y_big[pos[i]]), (T, i)


def test_fixed_tile_heights_same_bits(M):
    """The tile-height ablation's legs compute the same layer: one skewed
    2048-token chunk with the metadata's tiles fixed at 16, 32 or 64 rows gives
    the bits of the default (128-row tiles with row fragments following each
    expert's load, long tiles cut)."""
    case = mi.make_case("prefill4096")
    x, bias = dev(M, case["x"][:2048]), dev(M, case["bias"])
    y0 = get_layer(M, case, max_tokens=2048).forward_prefill(x, bias).clone()
    for bm in (16, 32, 64):
        y = get_layer(M, case, max_tokens=2048, tile_rows=bm).forward_prefill(x, bias)
        torch.cuda.synchronize()
        assert torch.equal(y, y0), bm


def test_batch_invariant_gemv_path(M):
    """Within the GEMV path a row's output does not depend on the other rows
    either (per-row dot products, fixed-order partial sums)."""
    case = mi.make_case("decode")
    lay = get_layer(M, case, gemv_max_rows=8)
    H = case["cfg"]["H"]
    rows = mi.gen_x(8, H, 7701)
    y1 = [lay.forward_decode(dev(M, rows[i:i + 1]), None).clone() for i in range(8)]
    for T in range(2, 9):
        y = lay.forward_decode(dev(M, rows[:T]), None)
        torch.cuda.synchronize()
        for i in range(T):
            assert torch.equal(y[i], y1[i][0]), (T, i)


@pytest.mark.parametrize("name", ["tiny", "prefill512"])
def test_dequant_pass_same_result(M, name):
    """The separate-dequant measurement (active experts rebuilt as fp16 into
    the workspace, GEMMs reading them) rounds every weight as the fused path
    does: same bits, and the dequant kernel is the one that ran."""
    from bit_quantized_moe_router_amd import K_DEQUANT, moe_profile_enable, moe_profile_read, moe_profile_reset
    case = mi.make_case(name)
    lay = get_layer(M, case)
    x, b = dev(M, case["x"]), dev(M, case["bias"])
    y0 = lay.forward_prefill(x, b).clone()
    lay.set_desc(dequant_pass=1)
    moe_profile_reset()
    moe_profile_enable(1 << K_DEQUANT)
    try:
        y1 = lay.forward_prefill(x, b)
        torch.cuda.synchronize()
        ran = moe_profile_read(K_DEQUANT)[1]
    finally:
        moe_profile_enable(0)
        moe_profile_reset()
        lay.set_desc(dequant_pass=0)
    assert ran >= 1
    assert torch.equal(y0, y1)
    toks = _sample_tokens(case, 24, seed=12)
    check_close(y1.cpu().numpy()[toks], oracle_rows(case, toks), f"{name} separate dequant pass")


def test_zero_tokens_is_noop(M):
    case = mi.make_case("tiny")
    lay = get_layer(M, case)
    y = torch.full((4, case["cfg"]["H"]), 7.0, device="cuda")
    x = dev(M, case["x"][:0])
    from bit_quantized_moe_router_amd import moe_forward_prefill
    moe_forward_prefill(lay.desc, lay.packed, lay.router_w, None, x, 0, y, lay.ws)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


# ---- routing corner cases: exact ties and degenerate router weights ---------------

@pytest.mark.parametrize("T", [4, 64, 300])
def test_route_exact_ties(M, T):
    """Pairs of identical router rows give exactly equal logits; the lower expert must win."""
    case = mi.small_layer(T, 256, 32, 4, 64, 64, seed=71)
    w = case["w"]
    w["router_w"][1::2] = w["router_w"][0::2]
    lay = M.MoELayer(w, 4, max_tokens=T, max_chunk=2048, tile_rows=16)
    r = lay.route(dev(M, case["x"]), None)
    torch.cuda.synchronize()
    ref = orc.route(case["x"], w["router_w"], None, 4, 16)
    check_route(r, ref, f"ties T={T}")
    assert np.all(ref["topk_ids"][:, 0] % 2 == 0)


def test_route_widest_hidden(M):
    """H = 8192, the largest hidden size: the screen's slices hold 32 groups
    each, and the error bound scales with them; routing stays bit-exact."""
    case = mi.small_layer(200, 8192, 16, 4, 64, 64, seed=91, zipf_seed=92)
    lay = M.MoELayer(case["w"], 4, max_tokens=200, tile_rows=32)
    r = lay.route(dev(M, case["x"]), dev(M, case["bias"]))
    torch.cuda.synchronize()
    ref = orc.route(case["x"], case["w"]["router_w"], case["bias"], 4, 32, with_shared=True)
    check_route(r, ref, "H=8192")


@pytest.mark.parametrize("T", [3, 40])
def test_route_zero_router_with_bias(M, T):
    case = mi.small_layer(T, 128, 24, 5, 64, 0, seed=81)
    w = case["w"]
    w["router_w"][...] = 0
    bias = np.linspace(1.0, -1.0, 24).astype(np.float32)
    lay = M.MoELayer(w, 5, max_tokens=T, max_chunk=2048, tile_rows=16)
    r = lay.route(dev(M, case["x"]), dev(M, bias))
    torch.cuda.synchronize()
    ref = orc.route(case["x"], w["router_w"], bias, 5, 16, with_shared=False)
    check_route(r, ref, f"zero router T={T}")
    assert np.array_equal(ref["topk_ids"], np.tile(np.arange(5, dtype=np.int32), (T, 1)))


# ---- decode with the grouped-GEMM path's arithmetic (batch_invariant = 1) ----------

def test_batch_invariant_decode_equals_gemm_path(M):
    """With batch_invariant = 1 the GEMV path computes every output element with
    the grouped-GEMM path's operations in the same order: decoding T = 1..8 rows
    through the GEMV path (row threshold 8) and through the grouped-GEMM path
    (row threshold 0) gives the same bits, and the same rows inside a 300-row
    prefill too, so the row threshold cannot change a row's output.  The
    library's default threshold in this mode (4) gives the same bits again."""
    case = mi.make_case("decode")
    H = case["cfg"]["H"]
    gv = get_layer(M, case, gemv_max_rows=8, batch_invariant=1, max_tokens=512)
    gm = get_layer(M, case, gemv_max_rows=0, batch_invariant=1, max_tokens=512)
    gd = get_layer(M, case, gemv_max_rows=-1, batch_invariant=1, max_tokens=512)
    big = mi.gen_x(300, H, 7702)
    pos = [3, 40, 64, 128, 129, 200, 257, 299]
    y_big = gm.forward_prefill(dev(M, big), None)
    torch.cuda.synchronize()
    for T in range(1, 9):
        x = dev(M, big[pos[:T]])
        y1 = gv.forward_decode(x, None).clone()
        y0 = gm.forward_decode(x, None).clone()
        yd = gd.forward_decode(x, None)
        torch.cuda.synchronize()
        assert torch.equal(y1, y0), T
        assert torch.equal(yd, y0), T
        for i in range(T):
            assert torch.equal(y1[i], y_big[pos[i]]), (T, i)
    check_close(y1.cpu().numpy(), oracle_rows(dict(case, x=big[pos], T=8)), "batch-invariant decode T=8")


def test_batch_invariant_decode_zipf_large_tiles(M):
    """The same against rows of a skewed 2048-token chunk (Zipf logit bias),
    where the grouped GEMM serves the popular experts in 128-row and cut tiles."""
    case = mi.make_case("prefill4096")
    gm = get_layer(M, case, gemv_max_rows=0, max_tokens=2048)
    gv = get_layer(M, case, gemv_max_rows=8, batch_invariant=1, max_tokens=2048)
    x = case["x"][:2048]
    bias = dev(M, case["bias"])
    y_big = gm.forward_prefill(dev(M, x), bias)
    torch.cuda.synchronize()
    pos = [0, 1, 511, 1024, 1500, 1777, 2000, 2047]
    for T in (1, 2, 5, 8):
        y = gv.forward_decode(dev(M, x[pos[:T]]), bias)
        torch.cuda.synchronize()
        for i in range(T):
            assert torch.equal(y[i], y_big[pos[i]]), (T, i)


@pytest.mark.parametrize("T,H,E,k,I,Is,seed,zipf", [
    (5, 64, 4, 4, 64, 64, 61, None),       # k == E, one group along H
    (8, 192, 1, 1, 128, 0, 31, None),      # one expert, no shared expert, 3 groups (padded to 4)
    (7, 128, 8, 3, 64, 128, 21, 22),       # Is != I, zipf bias
    (8, 320, 16, 8, 192, 64, 71, None),    # odd group counts along H and I
    (4, 8192, 32, 4, 128, 64, 93, None),   # 128 groups: four passes of the wave chain
    (2, 128, 32, 16, 64, 64, 97, None),    # k = 16: 17 rows per token, more than the 16 down waves
])
def test_batch_invariant_decode_edge_shapes(M, T, H, E, k, I, Is, seed, zipf):
    case = mi.small_layer(T, H, E, k, I, Is, seed, zipf)
    gv = M.MoELayer(case["w"], k, max_tokens=T, gemv_max_rows=8)
    gv.set_desc(batch_invariant=1)
    gm = M.MoELayer(case["w"], k, max_tokens=T, gemv_max_rows=0)
    x, b = dev(M, case["x"]), dev(M, case["bias"])
    y1 = gv.forward_decode(x, b).clone()
    y0 = gm.forward_decode(x, b)
    torch.cuda.synchronize()
    assert torch.equal(y1, y0)
    check_close(y1.cpu().numpy(), oracle_rows(case), f"edge {case['name']} batch-invariant decode")
