"""Rounding model of the output score's second-moment form, on the host.

For output row o, sum_t (X dW^T)[t, o]^2 = dW_o (X^T X) dW_o^T (the square
expanded), which is what lets the device score candidates against H = X^T X
instead of X ("AWQ architecture, in depth", The scale search as code: the
candidate's output error against the full-precision output).  This test
applies, in numpy, every rounding the device form adds -- X to fp16 times a
power of two, H accumulated in fp32, normalised to unit diagonal and rounded
to fp16 with the blocks right of each 384-wide diagonal block doubled, dW
columns times sqrt(H_ii) rounded to fp16 times a power of two, only the blocks
on and right of the diagonal summed -- and checks the 20 errors against the
oracle's plain definition at the output score's bars (1e-3 relative, the same
first minimum unless the oracle's errors tie within 1e-4).  It exercises no
device code: it pins the reading that the form is exact up to those roundings.
"""
import numpy as np

from oracle import awq_oracle as O
import workloads as WL

BLK = 384


def _pow2_scale(x: float) -> float:
    """2^e with x * 2^e in [2^14, 2^15)."""
    if not x > 0:
        return 1.0
    return 2.0 ** (15 - int(np.frexp(x)[1]))


def _device_form_errors(W, X, S, G):
    T, d_in = X.shape
    Xf = O.decode_activations(X).astype(np.float64)
    xs = _pow2_scale(np.abs(Xf).max())
    X16 = (Xf * xs).astype(np.float16).astype(np.float32)
    H = X16.T @ X16                                         # fp32 accumulation
    c = np.sqrt(np.diag(H)).astype(np.float32)
    r = np.where(c > 0, np.float32(1) / np.where(c > 0, c, 1), 0).astype(np.float32)
    blk = np.arange(d_in) // BLK
    weight = np.where(blk[None, :] > blk[:, None], 2.0, 1.0)   # right of the diagonal block: doubled
    keep = blk[None, :] >= blk[:, None]                          # on and right of it
    Hpp = ((H * r[:, None] * r[None, :]).astype(np.float16).astype(np.float64) * weight) * keep
    out = []
    for k in range(S.shape[0]):
        dW = (O.fake_quant(W, S[k], G).astype(np.float32) - W.astype(np.float32)) * c[None, :]
        ds = _pow2_scale(float(np.abs(dW).max()))
        dWp = (dW * ds).astype(np.float16).astype(np.float64)
        q = np.einsum("oi,ij,oj->", dWp, Hpp, dWp)
        out.append(q / (xs * ds) ** 2 / (T * W.shape[0]))
    return np.array(out)


def test_second_moment_form_roundings_match_oracle():
    d_out, d_in, T, G = 160, 768, 1024, 128          # two 384-wide blocks of H
    W = WL.make_weight(31, d_out, d_in)
    X = WL.make_activations(32, T, d_in, "bf16")
    xm = O.act_stats(X)
    errs, k, _ = O.search_scales([W], xm, G, 20, "output", X=X)
    got = _device_form_errors(W, X, O.candidate_scales(xm, 20), G)
    np.testing.assert_allclose(got, errs, rtol=1e-3)
    gk = int(np.argmin(got))
    assert gk == k or errs[gk] <= errs[k] * (1 + 1e-4)


def test_second_moment_identity_exact():
    """Without roundings the form is the plain definition to fp64 accuracy,
    triangular block sum included (a planted transposition or a missing factor
    of two breaks it)."""
    rng = np.random.default_rng(5)
    T, d_in, d_out = 50, 800, 7
    X = rng.standard_normal((T, d_in))
    dW = rng.standard_normal((d_out, d_in))
    H = X.T @ X
    blk = np.arange(d_in) // BLK
    tri = np.where(blk[None, :] > blk[:, None], 2.0, 1.0) * (blk[None, :] >= blk[:, None])
    rows = np.einsum("oi,ij,oj->o", dW, H * tri, dW)
    np.testing.assert_allclose(rows, ((X @ dW.T) ** 2).sum(axis=0), rtol=1e-10)


def test_second_moment_form_roundings_correlated_channels():
    """Activations whose channels are strongly correlated (a rank-4 mix plus 1%
    noise: H far from diagonal, off-diagonal entries as large as the diagonal
    ones): the fp16 rounding of H'' still leaves the 20 errors -- sums over all
    rows -- within the bar (single rows are not: the clip search, which
    decides per row, stays in the direct form by default)."""
    d_out, d_in, T, G = 160, 768, 1024, 128
    W = WL.make_weight(41, d_out, d_in)
    X = WL.make_correlated_activations(42, T, d_in, rank=4, noise=0.01)
    xm = O.act_stats(X)
    errs, k, _ = O.search_scales([W], xm, G, 20, "output", X=X)
    got = _device_form_errors(W, X, O.candidate_scales(xm, 20), G)
    np.testing.assert_allclose(got, errs, rtol=1e-3)
    gk = int(np.argmin(got))
    assert gk == k or errs[gk] <= errs[k] * (1 + 1e-4)
