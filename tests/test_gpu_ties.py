"""GPU parity on the method's tie cases.

* Exact half-way quotients v / step = k + 1/2 ("From-Scratch AWQ INT4
  Quantization on Qwen3-8B", "Group-wise symmetric INT4": codes are rounded;
  the rounding is half to even).  Built with power-of-two steps and
  power-of-two scales, so every product and quotient is exact and the tie is
  real: the pack kernel, the asymmetric zero point and the output-score
  operand (codes formed on the device) must all resolve it to the even
  neighbour, bit for bit with the oracle.
* Equal candidate errors ("AWQ architecture, in depth", "The scale search as
  code": the incumbent is replaced only on a strictly smaller error, so the
  first minimum wins).  A constant x_mean makes every candidate row of the
  scale table exactly 1 (x^a / sqrt(x^a x^a) = 1), so all candidates are the
  same quantizer: their errors must be bit-equal and the chosen index 0.
"""
import numpy as np
import pytest

from oracle import awq_oracle as O
import workloads as WL
from tests._util import argmin_ok, dev_f16, dev_f32, dev_x, host, say

pytestmark = pytest.mark.gpu

F32 = np.float32
HALVES = np.array([0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5], dtype=np.float64)


@pytest.fixture(scope="module")
def A():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import post_weight_quantization_awq_amd as A
    A.lib()
    return A


def sym_tie_weights(d_out, d_in, G, seed, with_s):
    """W (fp16) and s (fp32 powers of two or None) such that v = w s is exact and,
    in every group, max |v| = 7 * 2^e (step exactly 2^e) and every other element
    is (k + 1/2) 2^e or k 2^e with a random sign: most quotients are exact ties."""
    rng = np.random.default_rng(seed)
    s = (2.0 ** rng.integers(-2, 3, d_in)).astype(F32) if with_s else np.ones(d_in, dtype=F32)
    t = rng.choice(np.concatenate([HALVES, HALVES, np.arange(0.0, 7.0)]), (d_out, d_in))
    t *= rng.choice([-1.0, 1.0], (d_out, d_in))
    for g in range(d_in // G):                      # one element of every group at +-7
        cols = g * G + rng.integers(0, G, d_out)
        t[np.arange(d_out), cols] = 7.0 * rng.choice([-1.0, 1.0], d_out)
    e = rng.integers(-7, -2, (d_out, d_in // G)).astype(np.float64)
    v = t * np.repeat(2.0 ** e, G, axis=1)
    W = (v / s[None, :].astype(np.float64)).astype(np.float16)
    assert np.array_equal(W.astype(np.float64) * s.astype(np.float64), v)   # exact by construction
    return W, (s if with_s else None)


def n_ties(W, s, G):
    q, step, v = O.group_quantize(W, s, G)
    r = v.reshape(v.shape[0], -1, G) / step[:, :, None]
    return int(np.sum(np.abs(r - np.floor(r)) == 0.5))


@pytest.mark.parametrize("G", [128, 64, 32])
@pytest.mark.parametrize("with_s", [False, True])
def test_pack_half_way_ties(A, G, with_s):
    d_out, d_in = 48, 4 * G
    say(f"pack ties G={G} s={with_s}")
    W, s = sym_tie_weights(d_out, d_in, G, 11 + G + with_s, with_s)
    assert n_ties(W, s, G) > d_out * d_in // 3
    qw, sc, qz = A.quantize_pack(dev_f16(W), G, None if s is None else dev_f32(s))
    rqw, rsc, rqz, rq, rstep = O.quantize_pack(W, s, G)
    assert np.array_equal(host(qw), rqw)
    assert np.array_equal(host(sc).view(np.uint16), rsc.view(np.uint16))
    assert np.array_equal(host(qz), rqz)
    # the page's rounding at the ties themselves: half to the even neighbour
    u = O.unpack_codes(host(qw), d_out).astype(np.int64) - 7
    v = W.astype(np.float64) * (np.ones(d_in) if s is None else s.astype(np.float64))[None, :]
    r = v / np.repeat(rstep.astype(np.float64), G, axis=1)
    tie = np.abs(r - np.floor(r)) == 0.5
    assert np.all(u[tie] % 2 == 0)
    assert np.all(np.abs(u[tie] - r[tie]) == 0.5)


def asym_tie_weights(d_out, d_in, G, seed):
    """Groups whose range is [-(k + 1/2) 2^e, (14.5 - k) 2^e]: step exactly 2^e,
    and -lo / step = k + 1/2, an exact tie for the zero point; the other elements
    sit on half-way points or grid points inside the range."""
    rng = np.random.default_rng(seed)
    W = np.zeros((d_out, d_in), dtype=np.float64)
    for o in range(d_out):
        for g in range(d_in // G):
            k = int(rng.integers(0, 15))
            e = float(2.0 ** int(rng.integers(-8, -2)))
            lo, hi = -(k + 0.5), 14.5 - k
            vals = rng.integers(int(np.ceil(lo)), int(np.floor(hi)) + 1, G).astype(np.float64)
            vals += rng.choice([0.0, 0.5], G)
            vals = np.clip(vals, lo, hi)
            pos = rng.permutation(G)
            vals[pos[0]], vals[pos[1]] = lo, hi
            W[o, g * G:(g + 1) * G] = vals * e
    Wh = W.astype(np.float16)
    assert np.array_equal(Wh.astype(np.float64), W)
    return Wh


@pytest.mark.parametrize("G", [128, 32])
def test_pack_asym_zero_point_ties(A, G):
    d_out, d_in = 40, 2 * G
    say(f"asym pack zero-point ties G={G}")
    W = asym_tie_weights(d_out, d_in, G, 5 + G)
    qw, sc, qz = A.quantize_pack(dev_f16(W), G, None, asym=True)
    rqw, rsc, rqz, ru, rz, rstep = O.quantize_pack_asym(W, None, G)
    assert np.array_equal(host(qw), rqw)
    assert np.array_equal(host(sc).view(np.uint16), rsc.view(np.uint16))
    assert np.array_equal(host(qz), rqz)
    # every zero point came from an exact tie -lo / step = k + 1/2 and is even
    z = O.unpack_codes(host(qz), d_out)
    assert np.all(z % 2 == 0)
    # the top of a range with k odd rounds past 15 and is clamped
    assert np.any(O.unpack_codes(host(qw), d_out) == 15)


@pytest.mark.parametrize("asym", [False, True])
def test_output_score_operand_ties(A, asym):
    """Candidate 0 (s = 1) and the unclipped clip ratio see the exact ties: the
    device forms its operand W_hat - W from codes decided on the device, so a
    tie resolved the other way changes that candidate's error (the sign of the
    element's error flips) far beyond the 1e-3 bar."""
    G, d_in, T = 64, 256, 96
    say(f"output score ties asym={asym}")
    if asym:
        W = asym_tie_weights(64, d_in, G, 77)
    else:
        W, _ = sym_tie_weights(64, d_in, G, 78, False)
    X = WL.make_activations(79, T, d_in, "bf16")
    xm = O.act_stats(X)
    res = A.search_scales([dev_f16(W)], dev_f32(xm), group_size=G, score="output", X=dev_x(X), n_clip=20,
                          want_clip_err=True, asym=asym)
    errs, k, s = O.search_scales([W], xm, G, 20, "output", X=X, asym=asym)
    np.testing.assert_allclose(host(res.err).astype(np.float64), errs, rtol=1e-3)
    g_k = int(host(res.best_idx)[0])
    assert argmin_ok(g_k, errs, k)
    S = O.candidate_scales(xm, 20)
    E, _ = O.clip_search(W, S[g_k], X, G, 20, 0.5, asym=asym)
    np.testing.assert_allclose(host(res.clip_err).astype(np.float64), E, rtol=1e-3)


@pytest.mark.parametrize("score", ["weight", "output"])
@pytest.mark.parametrize("asym", [False, True])
def test_equal_candidate_errors_keep_the_first(A, score, asym):
    G, d_in, T = 128, 512, 80
    say(f"equal candidates score={score} asym={asym}")
    W = WL.make_weight(4242, 200, d_in)
    X = WL.make_activations(4343, T, d_in, "bf16")
    xm = np.full(d_in, 0.37, dtype=F32)
    kw = dict(score=score, X=dev_x(X)) if score == "output" else {}
    res = A.search_scales([dev_f16(W)], dev_f32(xm), group_size=G, asym=asym, **kw)
    S = host(A.candidate_scales(dev_f32(xm), 20))
    assert np.all(S == 1.0)
    g_err = host(res.err)
    assert np.all(g_err == g_err[0]), g_err
    assert int(host(res.best_idx)[0]) == 0
    assert np.all(host(res.best_s) == 1.0)
    errs, k, _ = O.search_scales([W], xm, G, 20, score, X=X if score == "output" else None, asym=asym)
    assert k == 0 and np.all(errs == errs[0])
    np.testing.assert_allclose(g_err[0], errs[0], rtol=1e-3)
