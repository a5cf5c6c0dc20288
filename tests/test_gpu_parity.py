"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars: packed words, codes and fp16 scales bit-exact given the same fp32
scale vector; candidate errors within 1e-3 relative; chosen alpha index equal
unless the oracle's errors tie within 1e-4 relative; x_mean within 1e-6
relative; candidate scales within 2 ulp (fp64 pow may differ in its last bit
before the single rounding to fp32); per-row clip errors within 1e-3
relative and the chosen clip ratio equal unless the oracle's errors tie within
1e-4 relative.
"""
import numpy as np
import pytest

from oracle import awq_oracle as O
import workloads as WL
from tests._util import argmin_ok, dev_f16, dev_f32, dev_x, host, say, ulp_dist

pytestmark = pytest.mark.gpu

F32 = np.float32


@pytest.fixture(scope="module")
def A():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import post_weight_quantization_awq_amd as A
    A.lib()
    return A


# ---------------------------------------------------------------------------
# A1 act_stats
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,d_in,dtype,pad", [
    (64, 512, "f16", 0),        # single linear, fp16 activations
    (4096, 4096, "bf16", 0),    # q_proj calibration
    (37, 520, "bf16", 0),       # ragged token count
    (53, 515, "f16", 0),        # d_in not a multiple of 8 (scalar path)
    (77, 256, "bf16", 40),      # leading dimension > d_in (strided rows)
    (1, 64, "bf16", 0),
    (16400, 4096, "bf16", 0),   # 128-row splits (>= 1024 blocks) + a 16-row tail
    (32831, 2048, "f16", 0),    # 128-row splits on 4 column strips, a 63-row tail
    # the persistent lean kernel (128-row splits): blocks loop over several
    # splits, the last column block ragged (lanes past d_in), rows strided
    (65613, 1000, "bf16", 0),   # 512 splits on 2 column blocks (128 per block row), a 77-row tail
    (20480, 3080, "f16", 8),    # 160 splits on 7 column blocks, ld = 3088
])
def test_act_stats(A, T, d_in, dtype, pad):
    import torch
    say(f"act_stats T={T} d_in={d_in} {dtype} pad={pad}")
    X = WL.make_activations(10 + T, T, d_in + pad, dtype)
    Xd = dev_x(X)[:, :d_in] if pad else dev_x(X)
    got = host(A.act_stats(Xd))
    ref = O.act_stats(X[:, :d_in])
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=0)


def test_act_stats_empty_and_chunked(A):
    import torch
    say("act_stats T=0 and chunked accumulate")
    d_in = 384
    Xe = torch.empty((0, d_in), dtype=torch.bfloat16, device="cuda")
    xm = torch.full((d_in,), 3.0, device="cuda")
    A.act_stats(Xe, x_mean=xm, inv_count=0.0)
    assert np.all(host(xm) == 0.0)
    X = WL.make_activations(99, 300, d_in, "bf16")
    Xd = dev_x(X)
    xm = A.act_stats(Xd[:128], inv_count=1.0 / 300)
    A.act_stats(Xd[128:250], x_mean=xm, inv_count=1.0 / 300, accumulate=True)
    A.act_stats(Xd[250:], x_mean=xm, inv_count=1.0 / 300, accumulate=True)
    np.testing.assert_allclose(host(xm), O.act_stats(X), rtol=2e-6)


# ---------------------------------------------------------------------------
# A2 candidate scales
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d_in,n_grid", [(512, 20), (4096, 20), (12288, 20), (100, 7)])
def test_candidate_scales(A, d_in, n_grid):
    say(f"candidate_scales d_in={d_in} n_grid={n_grid}")
    xm = O.act_stats(WL.make_activations(5 + d_in, 64, d_in, "bf16"))
    xm[3] = 0.0                      # a dead channel: clamp to s_min for alpha > 0
    got = host(A.candidate_scales(dev_f32(xm), n_grid))
    ref = O.candidate_scales(xm, n_grid)
    assert np.all(got[0] == 1.0)
    assert ulp_dist(got, ref) <= 2


# ---------------------------------------------------------------------------
# A3 + A5 weight-score search
# ---------------------------------------------------------------------------
def _search_case(A, parts, X, G, n_grid=20):
    import torch
    xm = O.act_stats(X)
    res = A.search_scales([dev_f16(p) for p in parts], dev_f32(xm), group_size=G, n_grid=n_grid)
    errs, k, s = O.search_scales(parts, xm, G, n_grid)
    g_err = host(res.err).astype(np.float64)
    g_k = int(host(res.best_idx)[0])
    g_s = host(res.best_s)
    return g_err, g_k, g_s, errs, k, s, xm


@pytest.mark.parametrize("name,parts,d_in,T,G,xdt", [
    ("single_linear_256x512", [256], 512, 64, 128, "f16"),
    ("q_proj_4096x4096", [4096], 4096, 4096, 128, "bf16"),
    ("qkv_parts_ragged", [96, 40, 64], 256, 50, 64, "bf16"),
    ("g32_ragged_rows", [200], 384, 33, 32, "bf16"),
    ("one_row", [1], 128, 9, 128, "bf16"),
    # all eight parts, one empty, blocks straddling part boundaries
    ("eight_parts_one_empty", [130, 8, 0, 120, 1, 64, 70, 7], 256, 40, 128, "bf16"),
    ("eight_parts_g64", [33, 0, 95, 2, 128, 17, 5, 60], 192, 21, 64, "bf16"),
])
def test_search_weight(A, name, parts, d_in, T, G, xdt):
    say(f"search weight {name} parts={parts} d_in={d_in} G={G}")
    Ws = [WL.make_weight(7000 + 13 * i + d_in, r, d_in) for i, r in enumerate(parts)]
    X = WL.make_activations(8000 + d_in, T, d_in, xdt)
    g_err, g_k, g_s, errs, k, s, _ = _search_case(A, Ws, X, G)
    np.testing.assert_allclose(g_err, errs, rtol=1e-3, atol=0)
    assert argmin_ok(g_k, errs, k), (g_k, k)
    assert g_err[g_k] <= g_err[0]                         # never worse than RTN
    assert ulp_dist(g_s, O.candidate_scales(O.act_stats(X), 20)[g_k]) <= 2


@pytest.mark.parametrize("n_grid", [2, 33, 64])
def test_search_weight_grid_sizes(A, n_grid):
    """Smallest and largest grids, and one just past the 32 candidates whose
    scales the selection loads together with the partial errors."""
    say(f"search weight n_grid={n_grid}")
    Ws = [WL.make_weight(7300 + n_grid, 300, 512)]
    X = WL.make_activations(8300 + n_grid, 70, 512, "bf16")
    g_err, g_k, g_s, errs, k, s, xm = _search_case(A, Ws, X, 128, n_grid=n_grid)
    np.testing.assert_allclose(g_err, errs, rtol=1e-3, atol=0)
    assert argmin_ok(g_k, errs, k), (g_k, k)
    assert ulp_dist(g_s, O.candidate_scales(xm, n_grid)[g_k]) <= 2


def test_search_worked_example_embedded(A):
    """The page-4 worked example row inside a 128-wide group: x_mean [16,1,1,...]
    makes candidate 10 scale channel 0 by 2 and the rest by 1/2 (= [4,1,1,1]/2)."""
    say("search weight worked example")
    W = np.zeros((8, 128), dtype=np.float16)
    W[:, :4] = np.array([0.5, -0.3, 0.8, 0.1], dtype=np.float16)
    xm = np.ones(128, dtype=F32)
    xm[0] = 16.0
    res = A.search_scales([dev_f16(W)], dev_f32(xm), group_size=128)
    errs, k, _ = O.search_scales([W], xm, 128)
    np.testing.assert_allclose(host(res.err), errs, rtol=1e-5)
    # oracle pins (fp16-rounded weights): per row 0.4746856 (RTN) and 0.01348827 (alpha=0.5)
    assert errs[0] / 8 == pytest.approx(0.4746856, rel=1e-6)
    assert errs[10] / 8 == pytest.approx(0.01348827, rel=1e-6)


# ---------------------------------------------------------------------------
# A7 quantize + pack, A8 unpack + dequant
# ---------------------------------------------------------------------------
def _pack_compare(A, W, G, s=None, clip=None):
    import torch
    qw, sc, qz = A.quantize_pack(dev_f16(W), G, None if s is None else dev_f32(s),
                                 None if clip is None else dev_f32(clip))
    rqw, rsc, rqz, rq, rstep = O.quantize_pack(W, s, G, clip)
    assert np.array_equal(host(qw), rqw)
    assert np.array_equal(host(sc).view(np.uint16), rsc.view(np.uint16))
    assert np.array_equal(host(qz), rqz)
    return qw, sc, qz, rq, rstep


@pytest.mark.parametrize("d_out,d_in,G,with_s,with_clip", [
    (256, 512, 128, True, False),
    (4096, 4096, 128, True, False),
    (4096, 4096, 128, False, False),
    (264, 384, 64, True, True),
    (1032, 256, 32, True, True),
    (8, 128, 128, True, False),
])
def test_quantize_pack_bit_exact(A, d_out, d_in, G, with_s, with_clip):
    say(f"pack d_out={d_out} d_in={d_in} G={G} s={with_s} clip={with_clip}")
    W = WL.make_weight(9000 + d_out + G, d_out, d_in)
    W[3, :G] = 0                                   # an all-zero group: step 0, codes 7
    s = (np.exp(np.random.default_rng(d_in).standard_normal(d_in) * 0.8)).astype(F32) if with_s else None
    clip = None
    if with_clip:
        r = O.clip_ratios(20, 0.5)
        clip = r[np.random.default_rng(d_out).integers(0, 20, d_out)]
    _pack_compare(A, W, G, s, clip)


def test_pack_worked_example_codes(A):
    """Page-4 row padded into a 128-group: AWQ codes [7,-1,3,0] -> unsigned [14,6,10,7];
    RTN codes [4,-3,7,1] -> [11,4,14,8]."""
    say("pack worked example")
    W = np.zeros((8, 128), dtype=np.float16)
    W[:, :4] = np.array([0.5, -0.3, 0.8, 0.1], dtype=np.float16)
    s = np.ones(128, dtype=F32)
    s[0] = 4.0
    for sv, want in [(s, [14, 6, 10, 7]), (None, [11, 4, 14, 8])]:
        qw, sc, qz = A.quantize_pack(dev_f16(W), 128, None if sv is None else dev_f32(sv))
        u = O.unpack_codes(host(qw), 8)
        assert u[:, :4].tolist() == [want] * 8
        assert np.all(u[:, 4:] == 7)


@pytest.mark.parametrize("d_out", [136, 256])   # one word per thread; four (d_out % 32 == 0)
@pytest.mark.parametrize("G,out_f16,with_s", [(128, False, True), (64, True, False), (32, False, False)])
def test_unpack_roundtrip(A, G, out_f16, with_s, d_out):
    import torch
    say(f"unpack G={G} f16={out_f16} s={with_s} d_out={d_out}")
    d_in = 512
    W = WL.make_weight(31 + G, d_out, d_in)
    s = (np.exp(np.random.default_rng(G).standard_normal(d_in) * 0.5)).astype(F32)
    qw, sc, qz, rq, rstep = _pack_compare(A, W, G, s)
    sdev = dev_f32(s) if with_s else None
    out = A.unpack_dequant(qw, sc, qz, d_out, G, sdev, torch.float16 if out_f16 else torch.float32)
    ref = O.unpack_dequant(host(qw), host(sc), host(qz), d_out, G, s if with_s else None)
    got = host(out)
    if out_f16:
        assert np.array_equal(got.view(np.uint16), ref.astype(np.float16).view(np.uint16))
    else:
        assert np.array_equal(got, ref)
    # zeros NULL means 7
    out2 = A.unpack_dequant(qw, sc, None, d_out, G, sdev, torch.float16 if out_f16 else torch.float32)
    assert np.array_equal(host(out2).view(np.uint16 if out_f16 else np.uint32),
                          got.view(np.uint16 if out_f16 else np.uint32))


@pytest.mark.parametrize("d_in,G,d_out", [(96, 32, 160), (192, 64, 288), (384, 128, 160)])
@pytest.mark.parametrize("out_f16,with_s", [(False, True), (True, False), (True, True)])
def test_unpack_partial_tiles(A, d_in, G, d_out, out_f16, with_s):
    """The tiled unpack (64 inputs x 128 outputs through LDS, for d_out % 32 == 0)
    on its ragged edges: d_in not a multiple of 64 and d_out not a multiple of 128."""
    import torch
    say(f"unpack partial tiles d_in={d_in} G={G} d_out={d_out} f16={out_f16} s={with_s}")
    W = WL.make_weight(61 + d_in + d_out, d_out, d_in)
    s = (np.exp(np.random.default_rng(d_in + G).standard_normal(d_in) * 0.5)).astype(F32)
    qw, sc, qz, rq, rstep = _pack_compare(A, W, G, s)
    sdev = dev_f32(s) if with_s else None
    odt = torch.float16 if out_f16 else torch.float32
    got = host(A.unpack_dequant(qw, sc, qz, d_out, G, sdev, odt))
    ref = O.unpack_dequant(host(qw), host(sc), host(qz), d_out, G, s if with_s else None)
    if out_f16:
        assert np.array_equal(got.view(np.uint16), ref.astype(np.float16).view(np.uint16))
    else:
        assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# A4 output score, A6 clip search (matrix cores)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("parts,d_in,T,G,xdt", [
    ([64], 256, 300, 128, "bf16"),
    ([96, 40, 64], 256, 129, 64, "bf16"),
    ([136], 512, 200, 128, "f16"),
    ([72], 384, 77, 32, "bf16"),
    ([40], 96, 70, 32, "bf16"),            # K padded to the 64-wide GEMM step
    ([300, 220], 512, 600, 128, "bf16"),   # several token and row tiles, ragged edges
    ([40, 0, 24, 8, 16, 33, 7, 16], 256, 90, 64, "bf16"),  # eight parts, one empty
    ([300], 256, 384, 128, "bf16"),        # exactly one 384-token tile
    ([64, 200], 128, 385, 64, "f16"),      # one token past it: a second tile of one row
    ([260], 192, 769, 64, "bf16"),         # three token tiles, one row in the last
])
def test_search_output(A, parts, d_in, T, G, xdt):
    say(f"search output parts={parts} d_in={d_in} T={T} G={G} {xdt}")
    Ws = [WL.make_weight(500 + 7 * i + T, r, d_in) for i, r in enumerate(parts)]
    X = WL.make_activations(600 + T, T, d_in, xdt)
    xm = O.act_stats(X)
    res = A.search_scales([dev_f16(p) for p in Ws], dev_f32(xm), group_size=G, score="output", X=dev_x(X))
    errs, k, _ = O.search_scales(Ws, xm, G, 20, "output", X=X)
    g_err = host(res.err).astype(np.float64)
    np.testing.assert_allclose(g_err, errs, rtol=1e-3)
    assert argmin_ok(int(host(res.best_idx)[0]), errs, k)


@pytest.mark.parametrize("parts,d_in,T,G", [([64], 256, 150, 128), ([136], 384, 70, 64),
                                            ([24, 0, 40], 256, 60, 128), ([272], 128, 385, 64)])
def test_clip_search(A, parts, d_in, T, G):
    d_out = sum(parts)
    say(f"clip search parts={parts} d_in={d_in} T={T} G={G}")
    Ws = [WL.make_weight(700 + d_out + 3 * i, r, d_in) for i, r in enumerate(parts)]
    W = np.concatenate(Ws, axis=0)
    X = WL.make_activations(800 + d_out, T, d_in, "bf16")
    xm = O.act_stats(X)
    res = A.search_scales([dev_f16(p) for p in Ws], dev_f32(xm), group_size=G, score="output", X=dev_x(X),
                          n_clip=20, want_clip_err=True)
    errs, k, _ = O.search_scales([W], xm, G, 20, "output", X=X)
    g_k = int(host(res.best_idx)[0])
    assert argmin_ok(g_k, errs, k)
    s = O.candidate_scales(xm, 20)[g_k]          # the clip search runs on the chosen row
    assert ulp_dist(host(res.best_s), s) <= 2
    E, c = O.clip_search(W, s, X, G, 20, 0.5)
    g_E = host(res.clip_err).astype(np.float64)
    np.testing.assert_allclose(g_E, E, rtol=1e-3)
    g_c = host(res.clip)
    ratios = O.clip_ratios(20, 0.5)
    for o in range(d_out):
        gj = int(np.nonzero(ratios == g_c[o])[0][0])
        assert argmin_ok(gj, E[o], O.first_argmin(E[o]), rel=1e-4), o
    # the oracle's scale and clip choice pack bit-exactly
    _pack_compare(A, W, G, s, c)


def test_deterministic(A):
    say("determinism")
    W = WL.make_weight(1, 512, 1024)
    X = WL.make_activations(2, 100, 1024, "bf16")
    xm = dev_f32(O.act_stats(X))
    a = A.search_scales([dev_f16(W)], xm)
    b = A.search_scales([dev_f16(W)], xm)
    assert np.array_equal(host(a.err), host(b.err))
    c = A.search_scales([dev_f16(W)], xm, score="output", X=dev_x(X))
    d = A.search_scales([dev_f16(W)], xm, score="output", X=dev_x(X))
    assert np.array_equal(host(c.err), host(d.err))


def test_search_output_full_size_row_sample(A):
    """Fused QKV at its calibration size (16384 tokens x 4096 inputs): the first
    64 rows of each of q, k, v form the scored group (the oracle evaluates
    every candidate exactly on them)."""
    import workloads as WL
    wl = WL.WORKLOADS["qkv_6144x4096_output"]
    say("search output qkv full size, 3 x 64 rows")
    parts, X = WL.host_group_inputs(wl, 0, 0, rows_limit=64)
    xm = O.act_stats(X)
    res = A.search_scales([dev_f16(p) for p in parts], dev_f32(xm), group_size=128, score="output", X=dev_x(X))
    errs, k, _ = O.search_scales(parts, xm, 128, 20, "output", X=X)
    np.testing.assert_allclose(host(res.err).astype(np.float64), errs, rtol=1e-3)
    assert argmin_ok(int(host(res.best_idx)[0]), errs, k)
    np.testing.assert_allclose(host(A.act_stats(dev_x(X))), xm, rtol=1e-6)
