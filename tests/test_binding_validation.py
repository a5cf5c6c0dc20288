"""The Python binding rejects bad tensors before anything reaches the library:
wrong dtype, shape or layout, and host tensors (whose pointers a kernel would
dereference on the device).  No GPU is needed: every case below raises
ValueError in the binding, before any launch."""
import os

import pytest
import torch


@pytest.fixture(scope="module")
def A():
    from post_weight_quantization_awq_amd import LIB_PATH
    if not os.path.exists(LIB_PATH):
        from post_weight_quantization_awq_amd import build
        build.build()
    import post_weight_quantization_awq_amd as A
    A.lib()
    return A


def raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


D_OUT, D_IN, G = 64, 256, 128


def pack_out(d_out=D_OUT, d_in=D_IN, g=G):
    return (torch.zeros((d_in, d_out // 8), dtype=torch.int32), torch.zeros((d_in // g, d_out), dtype=torch.float16),
            torch.zeros((d_in // g, d_out // 8), dtype=torch.int32))


def test_pack_rejects_bad_tensors(A):
    W = torch.zeros((D_OUT, D_IN), dtype=torch.float16)
    raises(lambda: A.PackPlan(W.float(), G), "W must have dtype")
    raises(lambda: A.PackPlan(W[:, ::2], G), "contiguous")
    raises(lambda: A.PackPlan(W[:60], G), "d_out % 8")
    raises(lambda: A.PackPlan(W, 96), "group_size")
    raises(lambda: A.PackPlan(W, G, s=torch.ones(D_IN - 1)), r"s must have shape \[256\]")
    raises(lambda: A.PackPlan(W, G, s=torch.ones(D_IN, dtype=torch.float64)), "s must have dtype")
    raises(lambda: A.PackPlan(W, G, clip=torch.ones(D_OUT + 8)), r"clip must have shape \[64\]")
    qw, sc, qz = pack_out()
    raises(lambda: A.PackPlan(W, G, out=(qw[:-1], sc, qz)), r"qweight must have shape \[256, 8\]")
    raises(lambda: A.PackPlan(W, G, out=(qw, sc.float(), qz)), "scales must have dtype")
    raises(lambda: A.PackPlan(W, G, out=(qw, sc, qz[:, :4])), r"qzeros must have shape \[2, 8\]")
    raises(lambda: A.PackPlan(W, G, out=(qw, sc, None), asym=True), "qzeros is required")
    # right shapes on the host: rejected as host memory
    raises(lambda: A.PackPlan(W, G, out=(qw, sc, qz)), "W must be a device tensor")


def test_unpack_rejects_bad_tensors(A):
    qw, sc, qz = pack_out()
    raises(lambda: A.unpack_dequant(qw, sc, qz, D_OUT + 8, G), r"qweight must have shape \[\*, 9\]")
    raises(lambda: A.unpack_dequant(qw, sc[:1], qz, D_OUT, G), r"scales must have shape \[2, 64\]")
    raises(lambda: A.unpack_dequant(qw, sc, qz.view(torch.float32), D_OUT, G), "qzeros must have dtype")
    raises(lambda: A.unpack_dequant(qw, sc, qz, D_OUT, G, s=torch.ones(D_IN // 2)), r"s must have shape")
    raises(lambda: A.unpack_dequant(qw, sc, qz, D_OUT, 96), "group_size")
    raises(lambda: A.unpack_dequant(qw, sc, qz, D_OUT, G), "qweight must be a device tensor")


def test_w4a16_rejects_bad_tensors(A):
    qw, sc, qz = pack_out()
    X = torch.zeros((3, D_IN), dtype=torch.float16)
    raises(lambda: A.W4A16Plan(X.float(), qw, sc, qz, D_OUT, G), "X must have dtype")
    raises(lambda: A.W4A16Plan(X.t(), qw, sc, qz, D_OUT, G), "unit column stride")
    raises(lambda: A.W4A16Plan(X, qw.t(), sc, qz, D_OUT, G), r"qweight must have shape \[256, 8\]")
    raises(lambda: A.W4A16Plan(X, qw, sc[:, :32], qz, D_OUT, G), r"scales must have shape \[2, 64\]")
    raises(lambda: A.W4A16Plan(X, qw, sc, qz[:1], D_OUT, G), r"qzeros must have shape \[2, 8\]")
    raises(lambda: A.W4A16Plan(X, qw, sc, qz, D_OUT, G, out=torch.zeros((2, D_OUT))), r"out must have shape \[3, 64\]")
    raises(lambda: A.W4A16Plan(X, qw, sc, qz, D_OUT, G, out=torch.zeros((D_OUT, 3)).t()), "unit column stride")
    raises(lambda: A.W4A16Plan(X, qw, sc, qz, D_OUT, G, out=torch.zeros((3, D_OUT), dtype=torch.bfloat16)),
           "out must have dtype")
    raises(lambda: A.W4A16Plan(X, qw, sc, qz, D_OUT, G), "X must be a device tensor")


def test_search_and_stats_reject_bad_tensors(A):
    W = torch.zeros((D_OUT, D_IN), dtype=torch.float16)
    xm = torch.ones(D_IN)
    raises(lambda: A.SearchPlan([W], xm[:-1]), r"x_mean must have shape \[256\]")
    raises(lambda: A.SearchPlan([W], xm.double()), "x_mean must have dtype")
    raises(lambda: A.SearchPlan([W], xm, score="output", X=torch.zeros((4, D_IN - 8), dtype=torch.bfloat16)),
           r"X must have shape \[\*, 256\]")
    bad_out = A.SearchResult(torch.zeros(19), torch.zeros(1, dtype=torch.int32), torch.zeros(D_IN), None, None)
    raises(lambda: A.SearchPlan([W], xm, out=bad_out), r"out.err must have shape \[20\]")
    raises(lambda: A.SearchPlan([W], xm), "must be a device tensor")
    raises(lambda: A.ActStatsPlan(torch.zeros((4, D_IN))), "X must have dtype")
    raises(lambda: A.ActStatsPlan(torch.zeros((4, D_IN), dtype=torch.bfloat16), x_mean=torch.zeros(D_IN + 1)),
           r"x_mean must have shape")
    raises(lambda: A.ActStatsPlan(torch.zeros((4, D_IN), dtype=torch.bfloat16)), "X must be a device tensor")
