"""Parity at the workloads' full sizes, in the launch shapes the benchmark
times.  Where the oracle cannot evaluate every output at that size it checks
sampled outputs (per-row clip errors, one row block) and the rest is checked
through properties that hold at any size (errors are sums over rows; the
chosen candidate is the first minimum of the reported errors)."""
import numpy as np
import pytest

from oracle import awq_oracle as O
import workloads as WL
from _util import say, dev_f16, dev_f32, dev_x, host, ulp_dist, argmin_ok

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    import post_weight_quantization_awq_amd as A
    A.lib()
    return A


def _sample_rows(part_rows, seed, n_inner=2):
    """First and last row of every part plus a few seeded interior rows."""
    rng = np.random.default_rng(seed)
    rows, base = [], 0
    for r in part_rows:
        rows += [base, base + r - 1] + list(base + rng.integers(1, r - 1, n_inner))
        base += r
    return np.array(sorted(set(int(x) for x in rows)))


def _output_clip_full(A, wl_name, gi, G, T_limit=None):
    wl = WL.WORKLOADS[wl_name]
    grp = wl.groups[gi]
    say(f"full size output+clip {wl_name} group {grp.name}: generating inputs")
    parts, X = WL.host_group_inputs(wl, 0, gi, T_limit=T_limit)
    xm = O.act_stats(X)
    say(f"  GPU search: rows {sum(p.shape[0] for p in parts)}, d_in {grp.d_in}, T {X.shape[0]}")
    res = A.search_scales([dev_f16(p) for p in parts], dev_f32(xm), group_size=G, score="output", X=dev_x(X),
                          n_clip=20, want_clip_err=True)
    g_err = host(res.err).astype(np.float64)
    k = int(host(res.best_idx)[0])
    # alpha search at full size: finite non-negative errors, first minimum taken,
    # never worse than plain RTN (candidate 0), s* is the oracle's candidate row k
    assert np.all(np.isfinite(g_err)) and np.all(g_err >= 0)
    assert k == O.first_argmin(g_err) and g_err[k] <= g_err[0]
    S = O.candidate_scales(xm, 20)
    assert ulp_dist(host(res.best_s), S[k]) <= 2
    # per-row clip errors of sampled rows against the oracle (given the oracle's s_k)
    W = np.concatenate(parts, axis=0)
    rows = _sample_rows([p.shape[0] for p in parts], 17 + gi)
    say(f"  oracle clip search on {len(rows)} sampled rows")
    E, c = O.clip_search(W[rows], S[k], X, G, 20, 0.5)
    g_E = host(res.clip_err).astype(np.float64)[rows]
    np.testing.assert_allclose(g_E, E, rtol=2e-3)
    g_c = host(res.clip)[rows]
    ratios = O.clip_ratios(20, 0.5)
    for i in range(len(rows)):
        gj = int(np.nonzero(ratios == g_c[i])[0][0])
        assert argmin_ok(gj, E[i], O.first_argmin(E[i]), rel=2e-3), rows[i]
    # the chosen codes of the sampled rows' 8-row words pack bit-exactly
    blocks = sorted(set(int(r) // 8 for r in rows))
    sel = np.concatenate([np.arange(8 * b, 8 * b + 8) for b in blocks])
    _, cs = O.clip_search(W[sel], S[k], X, G, 20, 0.5)
    qw, sc, qz = A.quantize_pack(dev_f16(W[sel]), G, dev_f32(S[k]), dev_f32(cs))
    rqw, rsc, rqz, _, _ = O.quantize_pack(W[sel], S[k], G, cs)
    assert np.array_equal(host(qw), rqw)
    assert np.array_equal(host(sc).view(np.uint16), rsc.view(np.uint16))


def test_qkv_output_full_size_rows(A):
    """Fused QKV, 6144 x 4096, 16384 tokens: the alpha-search GEMM launches
    [16384 x 4096] x [4096 x 122880] as in the benchmark."""
    _output_clip_full(A, "qkv_6144x4096_output", 0, 128)


def test_mlp_gate_up_output_clip_full_size_rows(A):
    """MLP gate/up, 2 x 12288 x 4096, 16384 tokens, with the clip search: the dW
    of the 20 candidates (4 GB) is built and multiplied in two chunks."""
    _output_clip_full(A, "mlp_output_clip", 0, 128)


def test_mlp_down_output_clip_rows(A):
    """MLP down_proj, 4096 x 12288 (the K = 12288 GEMM), on the first 512
    tokens of its synthetic input (the host oracle builds that input with two
    fp32 matrix products)."""
    _output_clip_full(A, "mlp_output_clip", 1, 128, T_limit=512)


@pytest.mark.parametrize("rows,d_in,G,n_blk", [
    ([12288, 12288], 4096, 128, 8),    # gate/up of one sweep block
    ([4096], 12288, 64, 4),            # down_proj of one sweep block, G = 64
])
def test_sweep_weight_search_row_blocks(A, rows, d_in, G, n_blk):
    """Weight score at sweep shapes.  The error is a sum over rows, so the
    full launch must equal the sum of launches over row blocks (the same
    candidate scales), and the oracle checks the first block exactly."""
    say(f"sweep-shape weight search rows={rows} d_in={d_in} G={G}")
    parts = [WL.make_weight(9100 + 31 * i + d_in, r, d_in) for i, r in enumerate(rows)]
    X = WL.make_activations(9200 + d_in, 2048, d_in, "bf16")
    xm = O.act_stats(X)
    full = A.search_scales([dev_f16(p) for p in parts], dev_f32(xm), group_size=G)
    g_full = host(full.err).astype(np.float64)
    W = np.concatenate(parts, axis=0)
    nb = W.shape[0] // n_blk
    blocks = []
    for b in range(n_blk):
        r = A.search_scales([dev_f16(W[b * nb:(b + 1) * nb])], dev_f32(xm), group_size=G)
        blocks.append(host(r.err).astype(np.float64))
    np.testing.assert_allclose(g_full, np.sum(blocks, axis=0), rtol=1e-5)
    assert int(host(full.best_idx)[0]) == O.first_argmin(g_full)
    say("  oracle on the first row block")
    errs, k, _ = O.search_scales([W[:nb]], xm, G, 20)
    np.testing.assert_allclose(blocks[0], errs, rtol=1e-3)
