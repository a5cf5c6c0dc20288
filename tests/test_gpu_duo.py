"""Duo scaling on the GPU against the oracle ("AWQ architecture, in depth",
"The scale search as code", duo_scaling=True): the row-normalised weight
channel mean, the duo candidate table, and weight- and output-score searches
over it."""
import numpy as np
import pytest

from oracle import awq_oracle as O
import workloads as WL
from tests._util import argmin_ok, dev_f16, dev_f32, dev_x, host, say, ulp_dist

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import post_weight_quantization_awq_amd as A
    A.lib()
    return A


def _parts(rows, d_in, seed, zero_rows=()):
    Ws = [WL.make_weight(seed + 17 * i, r, d_in) for i, r in enumerate(rows)]
    W = np.concatenate(Ws, axis=0) if Ws else None
    for z in zero_rows:                       # all-zero rows: their quotients would be 0/0
        base = 0
        for w in Ws:
            if z < base + w.shape[0]:
                w[z - base] = 0
                break
            base += w.shape[0]
    return Ws


@pytest.mark.parametrize("rows,d_in,zero_rows", [
    ([300], 512, ()),
    ([96, 40, 64], 256, (5, 100)),
    ([130, 0, 8], 384, (0, 137)),
    ([4096], 4096, (17,)),
    ([1], 128, ()),
])
def test_weight_channel_mean(A, rows, d_in, zero_rows):
    say(f"weight channel mean rows={rows} d_in={d_in}")
    Ws = _parts(rows, d_in, 900 + d_in, zero_rows)
    g = host(A.weight_channel_mean([dev_f16(w) for w in Ws]))
    assert ulp_dist(g, O.weight_channel_mean(Ws)) <= 1


@pytest.mark.parametrize("d_in,n_grid", [(512, 20), (4096, 20), (12288, 20), (1000, 64), (200, 2)])
def test_candidate_scales_duo(A, d_in, n_grid):
    say(f"duo candidates d_in={d_in} n_grid={n_grid}")
    X = WL.make_activations(950 + d_in, 64, d_in, "bf16")
    xm = O.act_stats(X)
    wm = np.random.default_rng(d_in).uniform(0.02, 0.8, d_in).astype(np.float32)
    wm[::97] = 0.0                             # w_mean = 0 where a column is zero
    S = host(A.candidate_scales_duo(dev_f32(xm), dev_f32(wm), n_grid))
    assert ulp_dist(S, O.candidate_scales(xm, n_grid, w_mean=wm)) <= 2


@pytest.mark.parametrize("rows,d_in,T,G", [([256], 512, 64, 128), ([96, 40, 64], 256, 50, 64), ([200], 384, 33, 32),
                                            ([4096], 4096, 4096, 128)])     # q_proj at full size
def test_search_weight_duo(A, rows, d_in, T, G):
    say(f"duo weight search rows={rows} d_in={d_in} G={G}")
    Ws = _parts(rows, d_in, 960 + d_in, (3,))
    X = WL.make_activations(970 + d_in, T, d_in, "bf16")
    xm = O.act_stats(X)
    res = A.search_scales([dev_f16(w) for w in Ws], dev_f32(xm), group_size=G, duo=True)
    errs, k, _ = O.search_scales(Ws, xm, G, 20, duo=True)
    g_err = host(res.err).astype(np.float64)
    np.testing.assert_allclose(g_err, errs, rtol=1e-3)
    gk = int(host(res.best_idx)[0])
    assert argmin_ok(gk, errs, k)
    S = O.candidate_scales(xm, 20, w_mean=O.weight_channel_mean(Ws))
    assert ulp_dist(host(res.best_s), S[gk]) <= 2


@pytest.mark.parametrize("rows,d_in,T,G", [([64], 256, 300, 128), ([96, 40, 64], 256, 129, 64)])
def test_search_output_duo(A, rows, d_in, T, G):
    say(f"duo output search rows={rows} d_in={d_in} T={T} G={G}")
    Ws = _parts(rows, d_in, 980 + T, ())
    X = WL.make_activations(990 + T, T, d_in, "bf16")
    xm = O.act_stats(X)
    res = A.search_scales([dev_f16(w) for w in Ws], dev_f32(xm), group_size=G, score="output", X=dev_x(X), duo=True)
    errs, k, _ = O.search_scales(Ws, xm, G, 20, "output", X=X, duo=True)
    np.testing.assert_allclose(host(res.err).astype(np.float64), errs, rtol=1e-3)
    assert argmin_ok(int(host(res.best_idx)[0]), errs, k)
