"""W4A16 product on the packed layout against the oracle ("AWQ architecture, in
depth", "Kernels: why W4A16 is fast at decode").

Packed inputs come from the oracle's pack or from random codes (never from the
HIP path).  Tolerance, from the arithmetic, with B = sum_i |x_i| (u_i + z) scale:
* decode GEMV (fewer than 9 tokens, or X not 16-byte aligned): products u * x
  are exact in fp32; a wave adds 32 of them and the 32 activations in fp32,
  folds the zero point and the scale (3 roundings), then 8 waves and n_slices
  row slices are added in fp32: within 2^-24 (32 + 8 + 8 + n_slices) B;
* few tokens (2 to 16, X 16-byte aligned rows): the matrix cores add the G
  exact products (u - z) x (or 16 (u - z) x) of a group in fp32, one fma
  applies the scale per group, a wave adds its groups, the block adds its 4
  waves in LDS (3 roundings), and at most d_in / (4 G) input ranges are added
  by the reduction: within 2^-24 (G + 5 + d_in / G + d_in / (4 G)) B;
* prefill GEMM (17 tokens or more): the matrix cores add G exact products
  (u - z) x of a group in fp32, one fma applies the scale, d_in / G groups are
  added: within 2^-24 (G + 2 + d_in / G) B.  Split over K into S ranges of
  at least two 128-input units, a range adds at most d_in / G / S + 1 groups
  and S range results are added after it, which stays within the same count.
An fp16 output adds one rounding (at most one fp16 ulp, taken at the larger
magnitude)."""
import numpy as np
import pytest

from oracle import awq_oracle as O
import workloads as WL
from tests._util import dev_f16, host, say

pytestmark = pytest.mark.gpu

F32, F64 = np.float32, np.float64


@pytest.fixture(scope="module")
def A():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import post_weight_quantization_awq_amd as A
    A.lib()
    return A


def _random_packed(seed, d_out, d_in, G, zeros=True):
    rng = np.random.default_rng(seed)
    qw = rng.integers(0, 2 ** 32, (d_in, d_out // 8), dtype=np.uint64).astype(np.uint32)
    sc = (rng.uniform(0.002, 0.03, (d_in // G, d_out))).astype(np.float16)
    qz = rng.integers(0, 2 ** 32, (d_in // G, d_out // 8), dtype=np.uint64).astype(np.uint32) if zeros else None
    return qw, sc, qz


def _dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).cuda()


def _bound(X, qw, sc, qz, d_out, G, n_slices, kind="gemv"):
    u = O.unpack_codes(qw, d_out).astype(F64)                         # [d_out, d_in]
    z = (O.unpack_codes(qz, d_out).astype(F64) if qz is not None
         else np.full((d_out, qw.shape[0] // G), 7.0))
    zz = np.repeat(z, G, axis=1)
    ss = np.repeat(sc.astype(F64).T, G, axis=1)
    B = np.abs(O.decode_activations(X)) @ ((u + zz) * ss).T
    d_in = qw.shape[0]
    count = {"gemv": 32 + 8 + 8 + n_slices, "gemm": G + 2 + d_in // G,
             "few": G + 5 + d_in // G + d_in // (4 * G)}[kind]
    return 2.0 ** -24 * count * B


def _check(A, X, qw, sc, qz, d_out, G, out_dtype="f16", ld_x=None, ld_y=None):
    """With X rows 16-byte aligned the kernel is the few-token matrix-core path at
    2 to 64 tokens (d_out a multiple of 16), else the GEMM from 17 tokens; else
    (and at one token) the GEMV."""
    import torch
    M, d_in = X.shape
    Xp = X if ld_x is None else np.pad(X, ((0, 0), (0, ld_x - d_in)))
    Xd = dev_f16(Xp)[:, :d_in]
    tdt = torch.float16 if out_dtype == "f16" else torch.float32
    out = None
    if ld_y is not None:
        out = torch.full((M, ld_y), 7.0, dtype=tdt, device="cuda")[:, :d_out]
    plan = A.W4A16Plan(Xd, _dev_i32(qw), dev_f16(sc), None if qz is None else _dev_i32(qz), d_out, G, tdt, out=out)
    Y = host(plan.run()).astype(F64)
    ref = O.w4a16_matmul(X, qw, sc, qz, d_out, G)
    ldx = d_in if ld_x is None else ld_x
    aligned = ldx % 8 == 0
    few = aligned and 2 <= M <= 64 and (d_out // 8) % 2 == 0   # the few-token path reads word pairs
    kind = "few" if few else ("gemm" if aligned and M >= 17 else "gemv")
    tol = _bound(X, qw, sc, qz, d_out, G, (d_in + 255) // 256, kind)
    if out_dtype == "f16":
        tol = tol + np.spacing(np.abs(ref).astype(np.float16) * np.float16(1.002)).astype(F64)
    err = np.abs(Y - ref)
    assert np.all(err <= tol), (float((err - tol).max()), float(err.max()))
    if ld_y is not None:   # the padding columns are untouched
        assert np.all(host(plan.out.as_strided((M, ld_y), (ld_y, 1)))[:, d_out:] == 7.0)
    return Y


@pytest.mark.parametrize("name,d_out,d_in,G,zeros", [
    ("q_proj_4096x4096", 4096, 4096, 128, False),
    ("gate_up_24576x4096", 24576, 4096, 128, True),
    ("down_4096x12288", 4096, 12288, 128, True),
    ("k_proj_1024x4096_g64", 1024, 4096, 64, True),
])
def test_w4a16_decode_full_size(A, name, d_out, d_in, G, zeros):
    say(f"w4a16 {name} M=1")
    qw, sc, qz = _random_packed(d_out + d_in + G, d_out, d_in, G, zeros)
    X = (np.random.default_rng(d_in).standard_normal((1, d_in))).astype(np.float16)
    _check(A, X, qw, sc, qz, d_out, G)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 9, 12, 16, 17, 31, 33, 48, 64])
@pytest.mark.parametrize("d_out,d_in,G,out_dtype", [
    (1032, 384, 64, "f16"),    # odd word count: the GEMV below 17 tokens
    (520, 96, 32, "f32"),      # odd word count
    (1040, 384, 64, "f16"),    # 4 strips of 32 words + 2; one input range, its last wave past d_in
    (560, 672, 32, "f32"),     # 2 ranges, the second 160 rows (one wave of 4 steps, one of 1)
    (2064, 1088, 64, "f16"),   # 3 ranges, the last 64 rows
    (16, 256, 128, "f32"),     # one strip of 2 words
    (32, 32, 32, "f32"),       # one 32-row step (three past d_in in each wave's chunk), 4 words
])
def test_w4a16_tokens_and_ragged_shapes(A, M, d_out, d_in, G, out_dtype):
    say(f"w4a16 M={M} d_out={d_out} d_in={d_in} G={G} {out_dtype}")
    qw, sc, qz = _random_packed(7 * M + d_out, d_out, d_in, G, True)
    X = (np.random.default_rng(M + d_in).standard_normal((M, d_in)) * 3).astype(np.float16)
    _check(A, X, qw, sc, qz, d_out, G, out_dtype)


@pytest.mark.parametrize("M", [2, 8, 16, 40, 64])
@pytest.mark.parametrize("name,d_out,d_in,G,zeros,out_dtype", [
    ("qkv_6144x4096", 6144, 4096, 128, True, "f16"),
    ("gate_up_24576x4096", 24576, 4096, 128, False, "f32"),
    ("down_4096x12288_g64", 4096, 12288, 64, True, "f16"),
])
def test_w4a16_few_tokens_full_size(A, M, name, d_out, d_in, G, zeros, out_dtype):
    """2 to 64 tokens at Qwen3-8B linear sizes: the few-token matrix-core path
    (one or several 16-token tiles), its inputs split into ranges whose
    results the reduction adds."""
    say(f"w4a16 few tokens {name} M={M}")
    qw, sc, qz = _random_packed(3 * M + d_out + d_in, d_out, d_in, G, zeros)
    X = (np.random.default_rng(5 * M + d_in).standard_normal((M, d_in))).astype(np.float16)
    _check(A, X, qw, sc, qz, d_out, G, out_dtype)


def test_w4a16_strides(A):
    say("w4a16 strided X and Y")
    qw, sc, qz = _random_packed(11, 272, 256, 64, True)
    X = (np.random.default_rng(12).standard_normal((3, 256))).astype(np.float16)
    _check(A, X, qw, sc, qz, 272, 64, "f16", ld_x=264, ld_y=280)   # few-token path, padded rows
    _check(A, X, qw, sc, qz, 272, 64, "f32", ld_x=300, ld_y=276)   # rows not 16-byte aligned: GEMV


@pytest.mark.parametrize("asym", [False, True])
def test_w4a16_on_oracle_packed_weights(A, asym):
    """A quantized linear: the folded input x / s times the packed W * s
    reproduces x times the fake-quantized weights within the fp16 roundings."""
    say(f"w4a16 oracle-packed asym={asym}")
    W = WL.make_weight(90 + asym, 512, 1024)
    s = (np.exp(np.random.default_rng(91).standard_normal(1024) * 0.4)).astype(F32)
    if asym:
        qw, sc, qz, *_ = O.quantize_pack_asym(W, s, 128)
    else:
        qw, sc, qz, *_ = O.quantize_pack(W, s, 128)
    X = WL.make_activations(92, 4, 1024, "bf16")
    Xs = (O.decode_activations(X) / s.astype(F64)).astype(np.float16)
    Y = _check(A, Xs, qw, sc, qz, 512, 128, "f32")
    fq = O.fake_quant_asym(W, s, 128) if asym else O.fake_quant(W, s, 128)
    ref = O.decode_activations(X) @ fq.astype(F64).T
    # each term differs by the fp16 roundings of x / s and of the stored step
    # (2^-11 relative each) and the fp32 roundings of the fake quantization
    B2 = np.abs(O.decode_activations(X)) @ np.abs(fq.astype(F64)).T
    assert np.all(np.abs(Y - ref) <= (2.0 ** -10 + 2.0 ** -20) * B2)


def test_w4a16_deterministic(A):
    say("w4a16 determinism")
    import torch
    qw, sc, qz = _random_packed(13, 4096, 4096, 128, True)
    X = dev_f16((np.random.default_rng(14).standard_normal((2, 4096))).astype(np.float16))
    a = A.w4a16_matmul(X, _dev_i32(qw), dev_f16(sc), _dev_i32(qz), 4096, 128, torch.float32)
    b = A.w4a16_matmul(X, _dev_i32(qw), dev_f16(sc), _dev_i32(qz), 4096, 128, torch.float32)
    assert torch.equal(a, b)


@pytest.mark.parametrize("M", [9, 32, 100, 128, 129, 257, 1024])   # 128 | 129: the token tile grows to 256
@pytest.mark.parametrize("d_out,d_in,G,out_dtype,zeros", [(1032, 384, 64, "f16", True), (520, 256, 32, "f32", False),
                                                          (4096, 4096, 128, "f16", True)])
def test_w4a16_prefill_gemm(A, M, d_out, d_in, G, out_dtype, zeros):
    """Prefill sizes on the matrix cores: ragged token and output tiles, every group size."""
    say(f"w4a16 gemm M={M} d_out={d_out} d_in={d_in} G={G} {out_dtype}")
    qw, sc, qz = _random_packed(31 * M + d_out, d_out, d_in, G, zeros)
    X = (np.random.default_rng(M + 7 * d_in).standard_normal((M, d_in)) * 2).astype(np.float16)
    _check(A, X, qw, sc, qz, d_out, G, out_dtype)


@pytest.mark.parametrize("M,d_out,d_in,G,out_dtype,ld_y", [(64, 1032, 2112, 64, "f16", 1040),
                                                           (40, 520, 1056, 32, "f32", 520),
                                                           (300, 264, 4096, 128, "f32", 272)])
def test_w4a16_prefill_split_k(A, M, d_out, d_in, G, out_dtype, ld_y):
    """Small tile grids split K over several blocks (6, 3 and 8 splits here, the last
    ones shorter) and add the split partials in order."""
    say(f"w4a16 gemm split-K M={M} d_out={d_out} d_in={d_in} G={G} {out_dtype} ld_y={ld_y}")
    qw, sc, qz = _random_packed(53 * M + d_in, d_out, d_in, G, True)
    X = (np.random.default_rng(M + d_out).standard_normal((M, d_in))).astype(np.float16)
    _check(A, X, qw, sc, qz, d_out, G, out_dtype, ld_y=ld_y)


def test_w4a16_prefill_strides_and_fallback(A):
    say("w4a16 gemm strides; unaligned X falls back to the GEMV")
    qw, sc, qz = _random_packed(41, 264, 256, 64, True)
    X = (np.random.default_rng(42).standard_normal((70, 256))).astype(np.float16)
    _check(A, X, qw, sc, qz, 264, 64, "f32", ld_x=264, ld_y=300)     # GEMM, padded rows
    _check(A, X, qw, sc, qz, 264, 64, "f16", ld_x=259, ld_y=264)     # rows not 16-byte aligned: GEMV


def test_w4a16_prefill_on_oracle_packed_weights(A):
    say("w4a16 gemm oracle-packed asym")
    W = WL.make_weight(95, 384, 512)
    s = (np.exp(np.random.default_rng(96).standard_normal(512) * 0.4)).astype(F32)
    qw, sc, qz, *_ = O.quantize_pack_asym(W, s, 128)
    X = WL.make_activations(97, 300, 512, "bf16")
    Xs = (O.decode_activations(X) / s.astype(F64)).astype(np.float16)
    Y = _check(A, Xs, qw, sc, qz, 384, 128, "f32")
    fq = O.fake_quant_asym(W, s, 128)
    ref = O.decode_activations(X) @ fq.astype(F64).T
    B2 = np.abs(O.decode_activations(X)) @ np.abs(fq.astype(F64)).T
    assert np.all(np.abs(Y - ref) <= (2.0 ** -10 + 2.0 ** -20) * B2)
