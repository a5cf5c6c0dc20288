"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/awq.h declares, and rejects bad arguments before launching anything.

Device pointers here are fake (never dereferenced): every call below fails
validation on the host, or has an empty size, so no kernel is enqueued.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq.h")


@pytest.fixture(scope="module")
def A():
    from post_weight_quantization_awq_amd import LIB_PATH
    if not os.path.exists(LIB_PATH):
        from post_weight_quantization_awq_amd import build
        build.build()
    import post_weight_quantization_awq_amd as A
    A.lib()
    return A


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(awq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ["awq_act_stats", "awq_search_scales", "awq_quantize_pack", "awq_unpack_dequant",
              "awq_search_workspace", "awq_last_error", "awq_abi_version", "awq_candidate_scales",
              "awq_act_stats_workspace", "awq_candidate_scales_workspace", "awq_set_timing_events"]:
        assert n in names


def test_every_declared_symbol_is_exported(A):
    names = declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for n in names:
        assert n in exported, n
        getattr(A.lib(), n)
    assert set(A.EXPORTED) == set(names)


def test_abi_version(A):
    assert A.lib().awq_abi_version() == 1


FAKE = 1 << 20          # 16- and 256-byte aligned, never dereferenced
FAKE_MIS = FAKE + 2     # misaligned


def st_pack(A, W=FAKE, d_out=64, d_in=256, G=128, s=None, clip=None, qw=FAKE, sc=FAKE, qz=None):
    return A.lib().awq_quantize_pack(W, d_out, d_in, G, s, clip, qw, sc, qz, None)


def test_pack_validation(A):
    assert st_pack(A, G=96) == A.AWQ_EINVAL
    assert st_pack(A, d_out=60) == A.AWQ_ESHAPE
    assert "d_out 60 not a multiple of 8" in A.lib().awq_last_error().decode()
    assert st_pack(A, d_in=200) == A.AWQ_ESHAPE
    assert "multiple of group_size 128" in A.lib().awq_last_error().decode()
    assert st_pack(A, W=None) == A.AWQ_EINVAL
    assert st_pack(A, W=FAKE_MIS) == A.AWQ_EALIGN
    assert st_pack(A, s=FAKE_MIS) == A.AWQ_EALIGN
    assert st_pack(A, d_out=-8) == A.AWQ_EINVAL
    assert "negative size" in A.lib().awq_last_error().decode()
    # empty inputs: nothing to do, no launch, NULL pointers allowed
    assert st_pack(A, W=None, d_out=0, qw=None, sc=None) == A.AWQ_OK
    assert st_pack(A, W=None, d_in=0, qw=None, sc=None) == A.AWQ_OK
    assert A.lib().awq_last_error().decode() == ""


def test_pack_asym_validation(A):
    L = A.lib()
    pk = lambda qz=FAKE, G=128, d_out=64, W=FAKE: L.awq_quantize_pack_asym(W, d_out, 256, G, None, None, FAKE, FAKE,
                                                                          qz, None)
    assert pk(qz=None) == A.AWQ_EINVAL          # zero points are data: qzeros required
    assert "qzeros" in L.awq_last_error().decode()
    assert pk(G=96) == A.AWQ_EINVAL
    assert pk(d_out=60) == A.AWQ_ESHAPE
    assert pk(W=FAKE_MIS) == A.AWQ_EALIGN
    assert pk(qz=FAKE + 1) == A.AWQ_EALIGN
    assert pk(qz=None, d_out=0, W=None) == A.AWQ_OK


def test_unpack_validation(A):
    L = A.lib()
    assert L.awq_unpack_dequant(FAKE, FAKE, None, 64, 256, 128, None, FAKE, 7, None) == A.AWQ_EDTYPE
    assert L.awq_unpack_dequant(FAKE, FAKE, None, 63, 256, 128, None, FAKE, A.AWQ_F32, None) == A.AWQ_ESHAPE
    assert L.awq_unpack_dequant(None, FAKE, None, 64, 256, 128, None, FAKE, A.AWQ_F32, None) == A.AWQ_EINVAL
    assert L.awq_unpack_dequant(None, None, None, 0, 256, 128, None, None, A.AWQ_F32, None) == A.AWQ_OK


def test_act_stats_validation(A):
    L = A.lib()
    n = ctypes.c_size_t()
    assert L.awq_act_stats_workspace(4096, 4096, ctypes.byref(n)) == 0 and n.value > 0
    need = n.value
    assert L.awq_act_stats(FAKE, 9, 4096, 4096, 4096, 1.0, 0, FAKE, FAKE, need, None) == A.AWQ_EDTYPE
    assert L.awq_act_stats(FAKE, A.AWQ_BF16, 4096, 4096, 4000, 1.0, 0, FAKE, FAKE, need, None) == A.AWQ_ESHAPE
    assert L.awq_act_stats(FAKE, A.AWQ_BF16, 4096, 4096, 4096, 1.0, 0, None, FAKE, need, None) == A.AWQ_EINVAL
    assert L.awq_act_stats(None, A.AWQ_BF16, 4096, 4096, 4096, 1.0, 0, FAKE, FAKE, need, None) == A.AWQ_EINVAL
    assert L.awq_act_stats(FAKE, A.AWQ_BF16, 4096, 4096, 4096, 1.0, 0, FAKE, FAKE, need - 8, None) == A.AWQ_EWORKSPACE
    assert L.awq_act_stats(FAKE, A.AWQ_BF16, 4096, 4096, 4096, float("inf"), 0, FAKE, FAKE, need, None) == A.AWQ_EINVAL
    assert L.awq_act_stats(FAKE, A.AWQ_BF16, -1, 4096, 4096, 1.0, 0, FAKE, FAKE, need, None) == A.AWQ_EINVAL
    # T = 0 needs no workspace
    assert L.awq_act_stats_workspace(0, 4096, ctypes.byref(n)) == 0 and n.value == 0


def _group(A, ptrs, rows):
    wp = (ctypes.c_void_p * len(ptrs))(*ptrs)
    rw = (ctypes.c_int64 * len(rows))(*rows)
    g = A.WGroup(len(ptrs), ctypes.cast(wp, ctypes.POINTER(ctypes.c_void_p)),
                 ctypes.cast(rw, ctypes.POINTER(ctypes.c_int64)))
    g._keep = (wp, rw)
    return g


def st_search(A, cfg, grp, d_in=256, X=None, T=0, ld=0, clip=None, ws=FAKE, ws_bytes=1 << 40, xdt=1,
              x_mean=FAKE):
    return A.lib().awq_search_scales(ctypes.byref(cfg), ctypes.byref(grp), d_in, x_mean, X, xdt, T, ld,
                                     FAKE, FAKE, FAKE, clip, None, ws, ws_bytes, None)


def test_search_validation(A):
    grp = _group(A, [FAKE, FAKE], [64, 32])
    good = A._cfg(128, 20, "weight", 0, 0.5, 1e-4)
    bad = [A._cfg(96, 20, "weight", 0, 0.5, 1e-4), A._cfg(128, 0, "weight", 0, 0.5, 1e-4),
           A._cfg(128, 65, "weight", 0, 0.5, 1e-4), A._cfg(128, 20, 5, 0, 0.5, 1e-4),
           A._cfg(128, 20, "weight", 20, 0.5, 1e-4), A._cfg(128, 20, "output", 1, 0.5, 1e-4),
           A._cfg(128, 20, "output", 20, 0.0, 1e-4), A._cfg(128, 20, "weight", 0, 0.5, 0.0)]
    for c in bad:
        assert st_search(A, c, grp, X=FAKE, T=16, ld=256, clip=FAKE) == A.AWQ_EINVAL
    c = A._cfg(128, 20, "weight", 0, 0.5, 1e-4)
    c.flags = 16                                   # no such flag
    assert st_search(A, c, grp) == A.AWQ_EINVAL
    c.flags = A.AWQ_FLAG_OUT_DIRECT | A.AWQ_FLAG_OUT_GRAM
    assert st_search(A, c, grp) == A.AWQ_EINVAL
    assert "exclude" in A.lib().awq_last_error().decode()
    assert st_search(A, good, grp, d_in=200) == A.AWQ_ESHAPE
    assert st_search(A, good, grp, d_in=64) == A.AWQ_ESHAPE
    assert st_search(A, good, _group(A, [FAKE_MIS], [64])) == A.AWQ_EALIGN
    assert st_search(A, good, _group(A, [None], [64])) == A.AWQ_EINVAL
    assert st_search(A, good, _group(A, [FAKE], [0])) == A.AWQ_EINVAL
    assert st_search(A, good, _group(A, [FAKE] * 9, [8] * 9)) == A.AWQ_EINVAL
    assert st_search(A, good, grp, x_mean=None) == A.AWQ_EINVAL
    assert st_search(A, good, grp, ws_bytes=100) == A.AWQ_EWORKSPACE
    assert st_search(A, good, grp, ws=FAKE + 16) == A.AWQ_EALIGN
    out = A._cfg(128, 20, "output", 0, 0.5, 1e-4)
    assert st_search(A, out, grp, X=None, T=16, ld=256) == A.AWQ_EINVAL
    assert st_search(A, out, grp, X=FAKE, T=0, ld=256) == A.AWQ_EINVAL
    assert st_search(A, out, grp, X=FAKE, T=16, ld=100) == A.AWQ_ESHAPE
    assert st_search(A, out, grp, X=FAKE, T=16, ld=260) == A.AWQ_EALIGN
    assert st_search(A, out, grp, X=FAKE_MIS, T=16, ld=256) == A.AWQ_EALIGN
    assert st_search(A, out, grp, X=FAKE, T=16, ld=256, xdt=2) == A.AWQ_EDTYPE
    clipc = A._cfg(128, 20, "output", 20, 0.5, 1e-4)
    assert st_search(A, clipc, grp, X=FAKE, T=16, ld=256, clip=None) == A.AWQ_EINVAL
    # the second-moment form addresses H with 32-bit offsets: forced at
    # d_in^2 >= 2^31 it is refused before anything is enqueued, and the
    # library's own choice falls back to the direct form there
    assert A.search_output_form(96, 49152, 1 << 20) == "direct"
    gram = A._cfg(128, 20, "output", 0, 0.5, 1e-4, out_form="gram")
    assert st_search(A, gram, grp, d_in=49152, X=FAKE, T=16, ld=49152) == A.AWQ_ESHAPE
    assert "second-moment" in A.lib().awq_last_error().decode()
    assert A.lib().awq_last_error().decode() != ""


def test_candidate_validation(A):
    L = A.lib()
    n = ctypes.c_size_t()
    # the table needs no scratch: zero bytes, ws may be NULL
    assert L.awq_candidate_scales_workspace(4096, 20, ctypes.byref(n)) == 0 and n.value == 0
    assert L.awq_candidate_scales_workspace(4096, 65, ctypes.byref(n)) == A.AWQ_EINVAL
    assert L.awq_candidate_scales(FAKE, 4096, 0, 1e-4, FAKE, FAKE, n.value, None) == A.AWQ_EINVAL
    assert L.awq_candidate_scales(FAKE, 4096, 20, 0.0, FAKE, FAKE, n.value, None) == A.AWQ_EINVAL
    assert L.awq_candidate_scales(None, 4096, 20, 1e-4, FAKE, FAKE, n.value, None) == A.AWQ_EINVAL
    assert L.awq_set_timing_events(FAKE, None) == A.AWQ_EINVAL
    assert L.awq_set_timing_events(None, None) == A.AWQ_OK


def test_workspace_sizes(A):
    wmode = A.search_workspace_bytes(4096, 4096)
    assert wmode < (1 << 21)                      # tables + per-block partials only
    omode = A.search_workspace_bytes(6144, 4096, 16384, score="output")
    assert omode >= 20 * 6144 * 4096 * 2          # dW of every candidate (bf16)
    big = A.search_workspace_bytes(24576, 4096, 16384, score="output", n_clip=20)
    assert big < (3 << 30)                        # dW built in chunks of <= 2 GiB
    with pytest.raises(A.AwqError):
        A.search_workspace_bytes(4096, 4000)
    # output score forms: the second-moment form holds X^T (as the direct form
    # holds X), H in fp32 and fp16, and the same dW chunk
    direct = A.search_workspace_bytes(6144, 4096, 16384, score="output", out_form="direct")
    gram = A.search_workspace_bytes(6144, 4096, 16384, score="output", out_form="gram")
    assert gram > direct + 4096 * 4096 * 4
    assert A.search_workspace_bytes(6144, 4096, 16384, score="output") == gram   # the default choice here
    assert A.search_workspace_bytes(6144, 4096, 64, score="output") == \
        A.search_workspace_bytes(6144, 4096, 64, score="output", out_form="direct")
    with pytest.raises(ValueError):
        A.search_workspace_bytes(6144, 4096, 64, score="output", out_form="hessian")


def test_output_form_choice(A):
    """The output score's form: the second-moment form where the calibration set
    has several times more tokens than inputs, the direct form where it has few;
    the flags force either; weight score and bad shapes are rejected."""
    assert A.search_output_form(6144, 4096, 16384) == "gram"            # fused QKV, 16384 tokens
    assert A.search_output_form(24576, 4096, 16384, n_clip=20) == "gram"  # MLP gate/up with the clip search
    assert A.search_output_form(4096, 12288, 16384, n_clip=20) == "gram"  # down_proj: triangular H products
    assert A.search_output_form(4096, 12288, 512, n_clip=20) == "direct"
    assert A.search_output_form(6144, 4096, 2048) == "direct"             # T near d_in
    assert A.search_output_form(6144, 4096, 512) == "direct"
    assert A.search_output_form(256, 512, 64) == "direct"
    assert A.search_output_form(6144, 4096, 16384, out_form="direct") == "direct"
    assert A.search_output_form(256, 512, 64, out_form="gram") == "gram"
    # the clip search (hi + lo parts of H in the second-moment form)
    assert A.search_output_forms(24576, 4096, 16384, n_clip=20) == ("gram", "gram")
    assert A.search_output_forms(6144, 4096, 16384) == ("gram", None)
    assert A.search_output_forms(6144, 4096, 2048, n_clip=20) == ("direct", "direct")
    assert A.search_output_forms(6144, 4096, 16384, n_clip=20, out_form="direct") == ("direct", "direct")
    assert A.search_output_forms(256, 512, 64, n_clip=20, out_form="gram") == ("gram", "gram")
    L = A.lib()
    f = ctypes.c_int32()
    w = A._cfg(128, 20, "weight", 0, 0.5, 1e-4)
    assert L.awq_search_output_form(ctypes.byref(w), 256, 512, 64, ctypes.byref(f)) == A.AWQ_EINVAL
    o = A._cfg(128, 20, "output", 0, 0.5, 1e-4)
    assert L.awq_search_output_form(ctypes.byref(o), 256, 500, 64, ctypes.byref(f)) == A.AWQ_ESHAPE
    assert L.awq_search_output_form(ctypes.byref(o), 256, 512, 0, ctypes.byref(f)) == A.AWQ_EINVAL
    assert L.awq_search_output_form(ctypes.byref(o), 256, 512, 64, None) == A.AWQ_EINVAL


def test_norm_group_fold_validation(A):
    L = A.lib()
    ptrs = lambda *p: ctypes.cast((ctypes.c_void_p * len(p))(*p), ctypes.POINTER(ctypes.c_void_p))
    s3 = ptrs(FAKE, FAKE, FAKE)
    f = lambda s=s3, n=3, d=4096, norm=FAKE, dt=A.AWQ_F16, out=FAKE, ssh=FAKE: \
        L.awq_norm_group_fold(s, n, d, norm, dt, out, ssh, None)
    assert f(s=None) == A.AWQ_EINVAL
    assert f(n=0) == A.AWQ_EINVAL and f(n=9) == A.AWQ_EINVAL
    assert f(s=ptrs(FAKE, None, FAKE)) == A.AWQ_EINVAL
    assert f(d=-1) == A.AWQ_EINVAL
    assert f(dt=7) == A.AWQ_EDTYPE
    assert f(out=None) == A.AWQ_EINVAL            # norm without norm_out
    assert f(norm=None) == A.AWQ_EINVAL           # norm_out without norm
    assert f(ssh=None) == A.AWQ_EINVAL
    assert f(norm=FAKE + 1) == A.AWQ_EALIGN       # fp16 norm at an odd address
    assert f(dt=A.AWQ_F32, out=FAKE + 2) == A.AWQ_EALIGN
    assert f(ssh=FAKE + 2) == A.AWQ_EALIGN
    assert f(d=0, norm=None, out=None, ssh=None) == A.AWQ_OK
    assert L.awq_last_error().decode() == ""


def test_duo_entry_validation(A):
    L = A.lib()
    n = ctypes.c_size_t()
    assert L.awq_weight_channel_mean_workspace(0, 256, ctypes.byref(n)) == A.AWQ_EINVAL
    assert L.awq_weight_channel_mean_workspace(64, 256, ctypes.byref(n)) == A.AWQ_OK and n.value > 0
    need = n.value
    ptrs = (ctypes.c_void_p * 1)(FAKE)
    rows = (ctypes.c_int64 * 1)(64)
    grp = A.WGroup(1, ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), ctypes.cast(rows, ctypes.POINTER(ctypes.c_int64)))
    wcm = lambda d_in=256, out=FAKE, ws=FAKE, nb=need: L.awq_weight_channel_mean(ctypes.byref(grp), d_in, out, ws, nb, None)
    assert wcm(d_in=100) == A.AWQ_ESHAPE
    assert wcm(out=None) == A.AWQ_EINVAL
    assert wcm(nb=need - 1) == A.AWQ_EWORKSPACE
    assert wcm(ws=FAKE + 16) == A.AWQ_EALIGN
    assert L.awq_weight_channel_mean(None, 256, FAKE, FAKE, need, None) == A.AWQ_EINVAL
    assert L.awq_candidate_scales_duo_workspace(256, 65, ctypes.byref(n)) == A.AWQ_EINVAL
    assert L.awq_candidate_scales_duo_workspace(256, 20, ctypes.byref(n)) == A.AWQ_OK and n.value > 0
    need = n.value
    cd = lambda x=FAKE, w=FAKE, s_min=1e-4, nb=need: L.awq_candidate_scales_duo(x, w, 256, 20, s_min, FAKE, FAKE, nb, None)
    assert cd(w=None) == A.AWQ_EINVAL
    assert cd(s_min=0.0) == A.AWQ_EINVAL
    assert cd(nb=0) == A.AWQ_EWORKSPACE
    # the duo flag enlarges the search workspace by the weight statistic and the fp64 table
    plain = A.search_workspace_bytes(64, 256, 1)
    assert A.search_workspace_bytes(64, 256, 1, duo=True) > plain


def test_w4a16_validation(A):
    L = A.lib()
    n = ctypes.c_size_t()
    assert L.awq_w4a16_workspace(1, 4096, 4096, ctypes.byref(n)) == A.AWQ_OK and n.value > 0
    need = n.value                      # fp32 partials of one token per input slice and output
    assert need % (4096 * 4) == 0
    assert L.awq_w4a16_workspace(3, 4096, 4096, ctypes.byref(n)) == A.AWQ_OK and n.value == 4 * need
    assert L.awq_w4a16_workspace(-1, 8, 128, ctypes.byref(n)) == A.AWQ_EINVAL
    # prefill GEMM: 256 tokens x 4096 outputs is 32 tiles of 256 x 128, split 8 ways over K
    # (fp32 partials [8][256][4096]); 2048 tokens give 256 tiles and run unsplit
    assert L.awq_w4a16_workspace(256, 4096, 4096, ctypes.byref(n)) == A.AWQ_OK and n.value == 8 * 256 * 4096 * 4
    assert L.awq_w4a16_workspace(2048, 4096, 4096, ctypes.byref(n)) == A.AWQ_OK and n.value == 4 * need
    # at most 8 splits, each at least two 128-input units: 32 tokens x 1024 outputs x 512 inputs -> 2
    assert L.awq_w4a16_workspace(32, 1024, 512, ctypes.byref(n)) == A.AWQ_OK and n.value == 2 * 32 * 1024 * 4

    def mm(X=FAKE, M=1, ld_x=4096, qw=FAKE, sc=FAKE, qz=None, d_out=4096, d_in=4096, G=128, Y=FAKE, ld_y=4096,
           ydt=A.AWQ_F16, ws=FAKE, nb=need):
        return L.awq_w4a16_matmul(X, M, ld_x, qw, sc, qz, d_out, d_in, G, Y, ld_y, ydt, ws, nb, None)

    assert mm(G=96) == A.AWQ_EINVAL
    assert mm(d_out=4092) == A.AWQ_ESHAPE
    assert mm(d_in=4000) == A.AWQ_ESHAPE
    assert mm(ld_x=4095) == A.AWQ_ESHAPE
    assert mm(ld_y=4094) == A.AWQ_ESHAPE
    assert mm(ydt=A.AWQ_BF16) == A.AWQ_EDTYPE
    assert mm(X=None) == A.AWQ_EINVAL
    assert mm(sc=FAKE + 8) == A.AWQ_EALIGN
    assert mm(Y=FAKE + 4) == A.AWQ_EALIGN
    assert mm(Y=FAKE + 8, ydt=A.AWQ_F32) == A.AWQ_EALIGN
    assert mm(nb=need - 1) == A.AWQ_EWORKSPACE
    assert mm(ws=FAKE + 16) == A.AWQ_EALIGN
    assert mm(M=0, X=None, Y=None) == A.AWQ_OK
