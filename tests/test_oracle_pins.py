"""Pins for the CPU oracle: values the pages print, closed forms derived from
their inputs, invariants the mathematics fixes, and brute force on tiny inputs.

Each test names what would break if the oracle held a plausible mistake (a
dropped term, a wrong sign, index or operand order).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import awq_oracle as O
import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32
F64 = np.float64


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# page 4's worked example ("Weight-Only Quantization: GPTQ and AWQ", 4. Tiny example)
# ---------------------------------------------------------------------------
class TestWorkedExample:
    g = load("worked_example.json")

    def arrays(self):
        w = np.array([self.g["w"]], dtype=F32)
        x = np.array(self.g["x"], dtype=F32)
        s = np.array(self.g["scale"], dtype=F32)
        return w, x, s

    def test_exact_output(self):
        w, x, _ = self.arrays()
        assert round(float(w[0].astype(np.float64) @ x.astype(np.float64)), 3) == self.g["printed"]["exact"]

    def test_naive_rtn_matches_print(self):
        w, x, _ = self.arrays()
        q, step, _ = O.group_quantize(w, None, 4)
        assert q[0].tolist() == self.g["derived_from_page_inputs"]["naive_codes"]
        wh = O.fake_quant(w, None, 4)[0]
        assert [round(float(v), 3) for v in wh] == self.g["printed"]["naive_dequant"]
        assert round(float(wh.astype(np.float64) @ x.astype(np.float64)), 3) == self.g["printed"]["naive_out"]

    def test_awq_scaled_matches_print(self):
        w, x, s = self.arrays()
        q, step, _ = O.group_quantize(w, s, 4)
        assert q[0].tolist() == self.g["derived_from_page_inputs"]["awq_codes"]
        wh = O.fake_quant(w, s, 4)[0]
        assert [round(float(v), 3) + 0.0 for v in wh] == self.g["printed"]["awq_dequant"]
        assert round(float(wh.astype(np.float64) @ x.astype(np.float64)), 3) == self.g["printed"]["awq_out"]

    def test_weight_error_closed_forms(self):
        w, x, s = self.arrays()
        d = self.g["derived_from_page_inputs"]
        naive = O.weight_error(w, np.ones(4, F32), x, 4)
        awq = O.weight_error(w, s, x, 4)
        assert naive == pytest.approx(d["weight_err_naive"][0] / d["weight_err_naive"][1], rel=1e-6)
        assert awq == pytest.approx(d["weight_err_awq"][0] / d["weight_err_awq"][1], rel=1e-5)

    def test_output_error_closed_forms(self):
        w, x, s = self.arrays()
        d = self.g["derived_from_page_inputs"]
        X = x[None, :].astype(np.float32)
        naive = O.output_error(w, np.ones(4, F32), X, 4)
        awq = O.output_error(w, s, X, 4)
        assert naive == pytest.approx(d["output_err_naive"][0] / d["output_err_naive"][1], rel=1e-6)
        assert awq == pytest.approx(d["output_err_awq"][0] / d["output_err_awq"][1], rel=1e-4)

    def test_embedded_in_search(self):
        """x_mean = [16,1,1,1] makes alpha = 0.5 give s = [2, .5, .5, .5] = [4,1,1,1]/2.

        A power-of-two factor on s leaves codes and w_hat unchanged, so the page's
        AWQ codes appear as candidate 10 and the page's naive codes as candidate 0.
        Weight-mode errors (x weighted by [16,1,1,1]): 2314/4900 and 66/4900.
        """
        w, _, _ = self.arrays()
        xm = np.array([16, 1, 1, 1], dtype=F32)
        S = O.candidate_scales(xm, 20)
        assert S[10].tolist() == [2.0, 0.5, 0.5, 0.5]
        assert O.group_quantize(w, S[10], 4)[0][0].tolist() == self.g["derived_from_page_inputs"]["awq_codes"]
        assert O.group_quantize(w, S[0], 4)[0][0].tolist() == self.g["derived_from_page_inputs"]["naive_codes"]
        errs, kb, sb = O.search_scales([w], xm, 4, 20)
        assert errs[0] == pytest.approx(2314 / 4900, rel=1e-6)
        assert errs[10] == pytest.approx(66 / 4900, rel=1e-5)
        assert errs[kb] <= errs[0]


# ---------------------------------------------------------------------------
# candidates ([cassindra] the scale search as code, non-duo branch)
# ---------------------------------------------------------------------------
class TestCandidates:
    def test_alpha_zero_is_ones(self):
        xm = np.array([0.0, 1e-9, 3.0, 250.0], dtype=F32)
        S = O.candidate_scales(xm, 20)
        assert np.array_equal(S[0], np.ones(4, F32))

    def test_closed_form_two_level(self):
        # x = [16, 1, ...]: t = [16^a, 1, ...], norm = 4^a -> s = [4^a, 4^-a, ...]
        xm = np.array([16, 1, 1, 1, 1, 1, 1, 1], dtype=F32)
        for k, a in enumerate(O.grid_alphas(20)):
            s = O.candidate_scales(xm, 20)[k]
            assert s[0] == pytest.approx(4.0 ** a, rel=1e-7)
            assert np.allclose(s[1:], 4.0 ** (-a), rtol=1e-7)

    def test_grid_is_k_over_n(self):
        assert O.grid_alphas(20)[0] == 0.0 and O.grid_alphas(20)[19] == 0.95
        assert O.grid_alphas(4) == [0.0, 0.25, 0.5, 0.75]

    def test_normalised_max_times_min_is_one(self):
        xm = WL.make_magnitudes(5, 512)
        S = O.candidate_scales(xm, 20)
        for k in range(20):
            assert float(S[k].max()) * float(S[k].min()) == pytest.approx(1.0, rel=1e-6)

    def test_clamp_before_normalisation(self):
        # a zero channel: 0^a = 0 -> clamped to 1e-4 (not 0), for a > 0
        xm = np.array([0.0, 1.0, 4.0, 4.0], dtype=F32)
        s = O.candidate_scale(xm, 0.5)
        t = np.array([1e-4, 1.0, 2.0, 2.0])
        assert np.allclose(s, (t / math.sqrt(2.0 * 1e-4)).astype(F32), rtol=1e-7)

    def test_scale_invariance_of_s(self):
        # s depends on x only up to a positive factor (the normalisation cancels c^a)
        xm = WL.make_magnitudes(9, 256) + 1.0
        S1 = O.candidate_scales(xm, 20)
        S2 = O.candidate_scales((xm * F32(8.0)).astype(F32), 20)
        assert np.allclose(S1, S2, rtol=2e-7, atol=0)


# ---------------------------------------------------------------------------
# quantizer ([konic] Group-wise symmetric INT4)
# ---------------------------------------------------------------------------
def nearest_code_exact(v: float, step: float) -> int:
    """argmin over the 15 codes of |v - q step| in exact rational arithmetic, ties to even."""
    fv, fs = Fraction(v), Fraction(step)
    best = None
    for q in range(-7, 8):
        d = abs(fv - q * fs)
        if best is None or d < best[0] or (d == best[0] and q % 2 == 0):
            best = (d, q)
    return best[1]


class TestQuantizer:
    def test_codes_are_nearest_grid_point(self):
        g = np.random.default_rng(1)
        W = (g.standard_normal((16, 64)) * 0.02).astype(np.float16)
        s = (np.exp(g.standard_normal(64) * 0.7)).astype(F32)
        q, step, v = O.group_quantize(W, s, 16)
        n_mismatch = 0
        for o in range(16):
            for i in range(64):
                st = float(step[o, i // 16])
                e = nearest_code_exact(float(v[o, i]), st)
                if e != int(q[o, i]):
                    # only where the exact quotient sits within an fp32 ulp of a half-integer
                    exact = Fraction(float(v[o, i])) / Fraction(st)
                    frac = exact - math.floor(exact)
                    assert abs(float(frac) - 0.5) < 1e-6
                    n_mismatch += 1
        assert n_mismatch <= 2

    def test_exact_ties_round_to_even(self):
        # a group whose max is 7 has step 7 / 7 = 1 exactly, so these fp16
        # values sit exactly on half-integers: round half to even (not away
        # from zero, not toward zero, not up)
        W = np.array([[7.0, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -6.5]], dtype=np.float16)
        q, step, _ = O.group_quantize(W, None, 8)
        assert step[0, 0] == 1.0
        assert q[0].tolist() == [7, 2, 4, -2, 0, 0, 2, -6]

    def test_code_range_and_zero_group(self):
        W = np.zeros((8, 32), dtype=np.float16)
        W[1, 5] = 0.5
        q, step, _ = O.group_quantize(W, None, 16)
        assert step[0, 0] == 0 and step[1, 1] == 0
        assert np.all(q[0] == 0)
        assert q[1, 5] == 7 and np.abs(q).max() <= 7
        assert np.all(O.fake_quant(W, None, 16)[0] == 0)

    def test_per_element_error_bound(self):
        # |v - q step| <= step/2 (up to rounding) unclipped ([repro] Q5: the rounding
        # error stays the same in the scaled domain; in W's domain it falls by 1/s)
        g = np.random.default_rng(2)
        W = (g.standard_normal((64, 256)) * 0.02).astype(np.float16)
        s = (np.exp(g.standard_normal(256))).astype(F32)
        q, step, v = O.group_quantize(W, s, 128)
        st = np.repeat(step, 128, axis=1).astype(np.float64)
        err = np.abs(v.astype(np.float64) - q * st)
        assert np.all(err <= st * 0.5 * (1 + 1e-6))
        wh = O.fake_quant(W, s, 128).astype(np.float64)
        err_w = np.abs(W.astype(np.float64) - wh)
        assert np.all(err_w <= st * 0.5 / s[None, :] * (1 + 1e-5) + 1e-12)

    def test_power_of_two_scaling_of_w(self):
        g = np.random.default_rng(3)
        W = (g.standard_normal((16, 256)) * 0.02).astype(F32)
        s = (np.exp(g.standard_normal(256))).astype(F32)
        xm = np.abs(g.standard_normal(256)).astype(F32)
        q1, st1, _ = O.group_quantize(W, s, 64)
        q2, st2, _ = O.group_quantize((W * 8).astype(F32), s, 64)
        assert np.array_equal(q1, q2) and np.array_equal(st2, st1 * 8)
        e1 = O.weight_error(W, s, xm, 64)
        e2 = O.weight_error((W * 8).astype(F32), s, xm, 64)
        assert e2 == pytest.approx(64 * e1, rel=1e-12)

    def test_unit_scale_equals_rtn(self):
        W = WL.make_weight(4, 32, 256)
        a = O.group_quantize(W, None, 128)
        b = O.group_quantize(W, np.ones(256, F32), 128)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])

    def test_clip_one_equals_unclipped_and_clip_clamps(self):
        W = WL.make_weight(5, 16, 128)
        a = O.group_quantize(W, None, 64)
        b = O.group_quantize(W, None, 64, clip=np.ones(16, F32))
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        c = O.group_quantize(W, None, 64, clip=np.full(16, 0.5, F32))
        assert np.abs(c[0]).max() == 7 and (np.abs(c[0]) == 7).sum() > (np.abs(a[0]) == 7).sum()


# ---------------------------------------------------------------------------
# errors and search
# ---------------------------------------------------------------------------
class TestErrorsAndSearch:
    def test_full_size_output_fixture(self):
        # the stored full-size oracle errors (GPU parity at calibration size):
        # 20 finite errors per group, the first minimum stored, never worse than
        # plain RTN (alpha = 0, candidate 0)
        for c in load("output_score_full_size.json")["cases"]:
            e = np.array(c["errors"])
            assert e.shape == (20,) and np.all(np.isfinite(e)) and np.all(e > 0)
            assert c["best_idx"] == O.first_argmin(e) and e[c["best_idx"]] <= e[0]
            assert c["tokens"] == 16384 and c["group_size"] == 128
        for c in load("weight_score_full_size.json")["cases"]:
            e = np.array(c["errors"])
            assert e.shape == (20,) and np.all(np.isfinite(e)) and np.all(e > 0)
            assert c["best_idx"] == O.first_argmin(e) and e[c["best_idx"]] <= e[0]
        ws = {(tuple(c["rows"]), c["d_in"], c["group_size"]): c["best_idx"]
              for c in load("weight_score_full_size.json")["cases"] if not c.get("duo") and not c.get("asym")}
        for c in load("pack_full_size.json")["cases"]:
            # the packs use the weight-score fixture's chosen candidate; three sha256 digests each
            assert ws[(tuple(c["rows"]), c["d_in"], c["group_size"])] == c["best_idx"]
            assert all(len(c[k]) == 64 and int(c[k], 16) >= 0 for k in ("qweight", "scales", "qzeros"))

    def test_act_stats_closed_form(self):
        X = np.array([[1.0, -2.0, 0.0], [-3.0, 2.0, 0.5]], dtype=np.float16)
        assert O.act_stats(X).tolist() == [2.0, 2.0, 0.25]
        Xb = WL.f32_to_bf16_bits(np.array([[-1.5, 4.0], [0.5, -4.0], [1.0, 1.0]], dtype=F32))
        assert O.act_stats(Xb).tolist() == pytest.approx([1.0, 3.0])

    def test_output_error_direct_difference(self):
        # X W_hat^T - X W^T evaluated as two separate products equals the difference form
        g = np.random.default_rng(6)
        W = (g.standard_normal((24, 64)) * 0.02).astype(np.float16)
        X = WL.make_activations(7, 9, 64, "bf16")
        s = O.candidate_scale(O.act_stats(X), 0.45)
        Xd = O.decode_activations(X)
        wh = O.fake_quant(W, s, 32).astype(np.float64)
        Y = Xd @ wh.T - Xd @ W.astype(np.float64).T
        ref = float((Y * Y).mean())
        assert O.output_error(W, s, X, 32) == pytest.approx(ref, rel=1e-9)

    def test_diagonal_x_links_the_two_modes(self):
        # X = diag(m): x_mean = m / T and E_out = (T / d_out) E_w; same argmin
        d_in, d_out = 64, 16
        m = WL.make_magnitudes(11, d_in)
        X = np.diag(m).astype(np.float32)
        W = WL.make_weight(12, d_out, d_in)
        xm = O.act_stats(X)
        assert np.allclose(xm, m / d_in, rtol=1e-7)
        ew, kw, _ = O.search_scales([W], xm, 32, 20, "weight")
        eo, ko, _ = O.search_scales([W], xm, 32, 20, "output", X=X)
        assert np.allclose(eo, ew * d_in / d_out, rtol=1e-5)
        assert kw == ko

    def test_activation_scaling_invariance(self):
        W = WL.make_weight(13, 32, 256)
        xm = WL.make_magnitudes(14, 256)
        e1, k1, s1 = O.search_scales([W], xm, 128, 20)
        e2, k2, s2 = O.search_scales([W], (xm * F32(4)).astype(F32), 128, 20)
        assert k1 == k2
        assert np.allclose(e2, 16 * e1, rtol=1e-5)

    def test_never_worse_than_rtn(self):
        for seed in range(3):
            W = WL.make_weight(20 + seed, 64, 256)
            X = WL.make_activations(30 + seed, 32, 256)
            xm = O.act_stats(X)
            errs, kb, _ = O.search_scales([W], xm, 128, 20)
            assert errs[kb] <= errs[0]
            assert errs[kb] == errs.min()
            erro, ko, _ = O.search_scales([W], xm, 128, 20, "output", X=X)
            assert erro[ko] <= erro[0]

    def test_outliers_pull_alpha_up(self):
        # with outlier channels the chosen alpha is > 0 and the error falls well below RTN
        W = WL.make_weight(2001, 256, 512)
        X = WL.make_activations(2002, 64, 512, "f16")
        errs, kb, _ = O.search_scales([W], O.act_stats(X), 128, 20)
        assert kb > 0 and errs[kb] < 0.8 * errs[0]

    def test_first_argmin_keeps_first_tie(self):
        assert O.first_argmin([3.0, 1.0, 1.0, 2.0]) == 1
        assert O.first_argmin([1.0, 1.0]) == 0

    def test_group_rows_concatenate(self):
        W1 = WL.make_weight(40, 16, 128)
        W2 = WL.make_weight(41, 8, 128)
        xm = WL.make_magnitudes(42, 128)
        e_parts, _, _ = O.search_scales([W1, W2], xm, 64, 20)
        e_cat, _, _ = O.search_scales([np.concatenate([W1, W2])], xm, 64, 20)
        S = O.candidate_scales(xm, 20)
        e_sum = [O.weight_error(W1, S[k], xm, 64) + O.weight_error(W2, S[k], xm, 64) for k in range(20)]
        assert np.array_equal(e_parts, e_cat) and np.allclose(e_parts, e_sum, rtol=1e-12)

    def test_brute_force_tiny_search(self):
        """8x16 W, G=8, T=5: every candidate's error from exact nearest-code
        quantization (rational arithmetic on the fp32 operands) matches."""
        W = WL.make_weight(50, 8, 16)
        X = WL.make_activations(51, 5, 16, "bf16")
        xm = O.act_stats(X)
        errs, kb, _ = O.search_scales([W], xm, 8, 20)
        S = O.candidate_scales(xm, 20)
        for k in range(20):
            tot = 0.0
            for o in range(8):
                for g0 in range(0, 16, 8):
                    v = [float(F32(float(W[o, i])) * S[k][i]) for i in range(g0, g0 + 8)]
                    a = max(abs(t) for t in v)
                    st = float(F32(a) / F32(7))
                    for j, i in enumerate(range(g0, g0 + 8)):
                        q = nearest_code_exact(v[j], st)
                        wh = float(F32(F32(q) * F32(st)) / S[k][i])
                        tot += ((float(W[o, i]) - wh) * float(xm[i])) ** 2
            assert errs[k] == pytest.approx(tot, rel=1e-12)
        assert kb == int(np.argmin(errs))


# ---------------------------------------------------------------------------
# clip search ([cassindra] pipeline step 5)
# ---------------------------------------------------------------------------
class TestClip:
    def test_ratios(self):
        r = O.clip_ratios(20, 0.5)
        assert r[0] == 1.0 and r[-1] == 0.5 and len(r) == 20
        assert np.all(np.diff(r) < 0)

    def test_hand_example_picks_point_seven(self):
        # row [1, .1, .1, .1], channel 0 unused by X: the best step is 0.1, i.e. ratio 0.7
        W = np.tile(np.array([[1.0, 0.1, 0.1, 0.1]], dtype=F32), (8, 1))
        X = np.diag([0.0, 1.0, 1.0, 1.0]).astype(F32)
        E, c = O.clip_search(W, np.ones(4, F32), X, 4, n_clip=6, clip_lo=0.5)
        assert np.all(c == F32(0.7))
        assert np.all(E[:, 3] < 1e-12) and np.all(E[:, 0] > 5e-3)

    def test_ratio_one_is_unclipped(self):
        W = WL.make_weight(60, 16, 64)
        X = WL.make_activations(61, 7, 64)
        s = O.candidate_scale(O.act_stats(X), 0.3)
        E, _ = O.clip_search(W, s, X, 32, n_clip=4)
        assert np.array_equal(E[:, 0], O.output_error_rows(W, s, X, 32))


# ---------------------------------------------------------------------------
# packing ([konic] AutoAWQ / HF-AWQ GEMM on-disk format; exporter step 4)
# ---------------------------------------------------------------------------
class TestPack:
    g = load("pack_order.json")

    def test_order_golden_word(self):
        u = np.tile((np.arange(16) % 8).astype(np.uint8)[:, None], (1, 4))
        words = O.pack_codes(u)
        assert words.shape == (4, 2)
        assert np.all(words == np.uint32(int(self.g["word_when_code_equals_row_mod_8"], 16)))

    def test_orientation_golden(self):
        u = np.tile(np.minimum(np.arange(16), 14).astype(np.uint8)[None, :], (8, 1))
        words = O.pack_codes(u)          # [d_in=16, d_out/8=1]
        for i in range(16):
            assert int(words[i, 0]) == int(f"{min(i, 14):x}" * 8, 16)

    def test_pack_shapes_zero_point_and_roundtrip(self):
        W = WL.make_weight(70, 64, 256)
        s = (np.exp(np.random.default_rng(0).standard_normal(256) * 0.3)).astype(F32)
        qw, sc, qz, q, step = O.quantize_pack(W, s, 128)
        assert qw.shape == (256, 8) and sc.shape == (2, 64) and qz.shape == (2, 8)
        assert sc.dtype == np.float16
        assert np.all(qz == np.uint32(int(self.g["qzeros_word"], 16)))
        u = O.unpack_codes(qw, 64)
        assert u.max() <= 14 and np.array_equal(u.astype(np.int16) - 7, q.astype(np.int16))
        # (u - zero) * scale reproduces q * fp16(step) exactly
        deq = O.unpack_dequant(qw, sc, qz, 64, 128)
        ref = (q.astype(F32) * np.repeat(step.astype(np.float16).astype(F32), 128, axis=1)).astype(F32)
        assert np.array_equal(deq, ref)
        assert np.array_equal(O.unpack_dequant(qw, sc, None, 64, 128), deq)

    def test_fp16_rne_golden(self):
        for hx, bits in load("fp16_rne.json")["cases"]:
            v = np.array([float.fromhex(hx)], dtype=F32)
            with np.errstate(over="ignore"):
                got = int(O.f32_to_f16(v).view(np.uint16)[0])
            assert got == int(bits, 16), hx

    def test_size_accounting(self):
        # Qwen3-8B linears: 13.9 GB in fp16 -> 3.5 GB of INT4 codes (4.0x);
        # 4 + 16/128 + 4/128 = 4.16 bits per weight with scales and zeros
        n = WL.qwen3_8b_linear_params()
        assert n == 36 * 192_937_984 == 6_945_767_424
        assert round(2 * n / 1e9, 1) == 13.9
        assert round(n / 2 / 1e9, 1) == 3.5
        assert round((2 * n) / (n / 2), 1) == 4.0
        bits = 4 + 16 / 128 + 4 / 128
        assert round(bits, 2) == 4.16


def ulps32(a, b) -> int:
    """Distance in fp32 units in the last place (same-sign finite values)."""
    ia = np.asarray(a, dtype=F32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, dtype=F32).view(np.int32).astype(np.int64)
    return int(np.max(np.abs(ia - ib)))


class TestNormGroupExport:
    """[konic] exporter steps 1-3: one shared scale per norm group (geometric
    mean of the member linears' scales) folded into the norm, the members
    re-quantized with it, o_proj / down_proj at RTN."""

    def test_geometric_mean_closed_forms(self):
        a = lambda *v: np.array(v, dtype=F32)
        assert np.array_equal(O.shared_scale([a(2.0, 0.5, 3.0), a(8.0, 2.0, 3.0)]), a(4.0, 1.0, 3.0))
        assert np.array_equal(O.shared_scale([a(1.0), a(4.0), a(16.0)]), a(4.0))
        assert np.array_equal(O.shared_scale([a(3.0), a(12.0), a(48.0)]), a(12.0))   # 1728 = 12^3
        assert np.array_equal(O.shared_scale([a(2.0), a(32.0)]), a(8.0))
        s = np.exp(np.random.default_rng(5).uniform(-5, 5, 300)).astype(F32)
        assert np.array_equal(O.shared_scale([s]), s)                              # one member
        assert np.array_equal(O.shared_scale([s, s, s]), s)                        # equal members

    def test_matches_root_of_product(self):
        rng = np.random.default_rng(6)
        for M in range(2, 9):
            S = np.exp(rng.uniform(-4, 4, (M, 64))).astype(F32)
            got = O.shared_scale(list(S))
            ref = np.array([math.prod(float(v) for v in S[:, i]) ** (1.0 / M) for i in range(64)])
            assert ulps32(got, ref.astype(F32)) <= 1, M

    def test_scaling_and_order(self):
        rng = np.random.default_rng(7)
        S = [np.exp(rng.uniform(-3, 3, 128)).astype(F32) for _ in range(3)]
        base = O.shared_scale(S)
        for c in (2.0 ** 7, 2.0 ** -9):
            assert np.array_equal(O.shared_scale([(x * F32(c)).astype(F32) for x in S]), (base * F32(c)).astype(F32))
        assert ulps32(O.shared_scale(S[::-1]), base) == 0
        # a member and its reciprocal cancel (exactly for powers of two)
        assert np.array_equal(O.shared_scale([np.full(4, 8.0, F32), np.full(4, 0.125, F32)]), np.ones(4, F32))

    def test_fold_closed_forms(self):
        s = np.array([2.0, 3.0, 1.0, 0.25], dtype=F32)
        assert np.array_equal(O.fold_norm(np.array([6.0, 1.0, -5.5, 1.5], F32), s),
                              np.array([3.0, F32(1.0) / F32(3.0), -5.5, 6.0], F32))
        h = O.fold_norm(np.array([1.0, 6.0], np.float16), np.array([3.0, 2.0], F32))
        assert h.dtype == np.float16 and [hex(v) for v in h.view(np.uint16)] == ["0x3555", "0x4200"]
        b = O.fold_norm(np.array([0x3F80, 0x4040], np.uint16), np.array([4.0, 1.0], F32))   # bf16 1.0, 3.0
        assert b.dtype == np.uint16 and [hex(v) for v in b] == ["0x3e80", "0x4040"]

    def test_bf16_rounding_against_library(self):
        import torch
        ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20, 1.5], F32)
        assert [hex(v) for v in O.f32_to_bf16_bits(ties)] == ["0x3f80", "0x3f82", "0xbf80", "0x3f81", "0x3fc0"]
        x = (np.random.default_rng(8).standard_normal(4096) * np.exp(np.random.default_rng(9).uniform(-20, 20, 4096)))
        x = x.astype(F32)
        lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(O.f32_to_bf16_bits(x), lib)

    def test_fold_identity_and_inverse(self):
        rng = np.random.default_rng(10)
        n32 = rng.uniform(0.2, 3.0, 500).astype(F32)
        for n in (n32, n32.astype(np.float16), O.f32_to_bf16_bits(n32)):
            assert np.array_equal(O.fold_norm(n, np.ones(500, F32)), n)
        s = np.exp(rng.uniform(-2, 2, 500)).astype(F32)
        back = (O.fold_norm(n32, s) * s).astype(F32)
        assert np.max(np.abs(back / n32 - 1)) < 2.5e-7

    def test_folding_reproduces_weight_dequantization(self):
        """Norm-folding (store Q(W s), divide the activation by s in the norm)
        and weight-dequantization (Q(W s)/s) give the same product up to the
        fp32 rounding of the folded norm ([konic] the two application
        strategies are the same mathematics)."""
        rng = np.random.default_rng(11)
        W = WL.make_weight(90, 64, 256)
        s = np.exp(rng.uniform(-1, 1, 256)).astype(F32)
        norm = rng.uniform(0.5, 2.0, 256).astype(F32)
        x = rng.standard_normal((5, 256)).astype(F32)
        s_sh, folded, packs = O.export_norm_group([W], [s], norm, 128)
        qw, sc, qz, _, _ = packs[0]
        deq = O.unpack_dequant(qw, sc, qz, 64, 128).astype(F64)                   # Q(W s), no 1/s
        y_fold = (x.astype(F64) * folded.astype(F64)) @ deq.T
        y_wd = (x.astype(F64) * norm.astype(F64)) @ (deq / s_sh.astype(F64)).T
        np.testing.assert_allclose(y_fold, y_wd, rtol=1e-5, atol=1e-6 * np.abs(y_wd).max())
        # o_proj / down_proj: RTN, the same as a unit scale
        r = O.export_rtn(W, 128)
        u = O.quantize_pack(W, np.ones(256, F32), 128)
        assert all(np.array_equal(a, b) for a, b in zip(r, u))


class TestDuoScaling:
    """[cassindra] The scale search as code, duo_scaling=True."""

    def test_weight_mean_closed_forms(self):
        f16 = lambda a: np.array(a, dtype=np.float16)
        assert np.array_equal(O.weight_channel_mean([f16(np.full((5, 8), -0.25))]), np.ones(8, F32))
        W = np.zeros((4, 6), np.float16)
        for o in range(4):
            W[o, o] = 0.5 * (o + 1)                   # one nonzero per row
        wm = O.weight_channel_mean([W])
        assert np.array_equal(wm, np.array([0.25, 0.25, 0.25, 0.25, 0, 0], F32))
        # an all-zero row counts in the mean with 0; row [1, -2] gives [0.5, 1]
        assert np.array_equal(O.weight_channel_mean([f16([[0, 0]]), f16([[1, -2]])]), np.array([0.25, 0.5], F32))

    def test_weight_mean_invariances(self):
        W = WL.make_weight(31, 40, 256)
        wm = O.weight_channel_mean([W])
        assert np.all(wm > 0) and np.all(wm <= 1)
        Ws = W.copy()
        Ws[::3] = (Ws[::3].astype(F32) * 4).astype(np.float16)      # power-of-two row scaling
        assert np.array_equal(O.weight_channel_mean([Ws]), wm)
        assert ulps32(O.weight_channel_mean([W[::-1]]), wm) <= 1        # row order
        assert np.array_equal(O.weight_channel_mean([W[:10], W[10:]]), wm)   # parts concatenate

    def test_candidates_closed_forms(self):
        x = np.full(16, 3.0, F32)
        for k in range(20):
            assert np.array_equal(O.candidate_scale_duo(x, np.full(16, 0.4, F32), k / 20), np.ones(16, F32))
        # w_mean = 1: the denominator is the constant 1 + 1e-4, which the
        # normalisation removes: the plain candidates (away from the clamp)
        xm = np.exp(np.random.default_rng(12).normal(0, 1, 300)).astype(F32)
        for a in (0.0, 0.35, 0.95):
            assert ulps32(O.candidate_scale_duo(xm, np.ones(300, F32), a), O.candidate_scale(xm, a)) <= 1

    def test_candidates_normalised_and_elementwise(self):
        rng = np.random.default_rng(13)
        xm = np.exp(rng.normal(0, 1, 64)).astype(F32)
        wm = rng.uniform(0.05, 0.6, 64).astype(F32)
        for a in (0.0, 0.25, 0.6):
            s = O.candidate_scale_duo(xm, wm, a)
            t = [max((float(xv) ** a if a else 1.0) / (float(wv) ** (1 - a) + 1e-4), 1e-4) for xv, wv in zip(xm, wm)]
            norm = math.sqrt(max(t) * min(t))
            assert ulps32(s, np.array([v / norm for v in t]).astype(F32)) <= 1
            assert abs(float(s.astype(F64).max()) * float(s.astype(F64).min()) - 1.0) < 1e-6
        # alpha = 0 is not RTN under duo scaling: s is proportional to 1 / (w_mean + 1e-4)
        s0 = O.candidate_scale_duo(xm, wm, 0.0).astype(F64)
        r = s0 * (wm.astype(F64) + 1e-4)
        assert np.allclose(r, r[0], rtol=1e-6)


# ---------------------------------------------------------------------------
# asymmetric INT4 ("AWQ architecture, in depth": the worked example in "Why it
# works" -- values up to 0.5 give a step of about 1/15 and a worst rounding
# error of about 0.033 -- and "Quantization, storage and packing": one 16-bit
# scale and one 4-bit zero point per group and output channel, about 4.16
# bits per weight)
# ---------------------------------------------------------------------------
class TestAsymmetricInt4:
    def test_worked_example_step_and_error(self):
        rng = np.random.default_rng(11)
        w = rng.uniform(-0.5, 0.5, 128).astype(F32)
        w[3], w[77] = -0.5, 0.5
        w[5] = 0.2                               # the channel scaled by 2 stays inside the range
        W = w[None, :]
        u, z, step, _ = O.group_quantize_asym(W, None, 128)
        assert step[0, 0] == F32(1.0) / F32(15)  # range 1 over 15 steps
        assert round(float(step[0, 0]), 3) == 0.067
        err = np.abs(O.fake_quant_asym(W, None, 128) - W)
        half = float(step[0, 0]) / 2
        assert err.max() <= half * (1 + 2 ** -20) and round(half, 3) == 0.033
        # activation 20 on that channel: 20 x 0.033 = 0.67 per output at worst;
        # scaling the weight by 2 (and the activation by 1/2) halves it
        assert round(20 * half, 2) == 0.67
        s = np.ones(128, F32)
        s[5] = 2.0
        u2, z2, step2, _ = O.group_quantize_asym(W, s, 128)
        assert step2[0, 0] == step[0, 0] and z2[0, 0] == z[0, 0]
        e5 = abs(float(O.fake_quant_asym(W, s, 128)[0, 5]) - 0.2)
        assert e5 <= half / 2 * (1 + 2 ** -20) and round(20 * half / 2, 2) == 0.33

    def test_grid_values_reconstruct_exactly(self):
        rng = np.random.default_rng(12)
        d = 2.0 ** -7
        for zz in range(16):
            k = np.concatenate([np.arange(16), rng.integers(0, 16, 16)])
            rng.shuffle(k)
            vals = ((k - zz) * d).astype(F32)[None, :]
            u, z, step, _ = O.group_quantize_asym(vals, None, 32)
            assert step[0, 0] == F32(d) and int(z[0, 0]) == zz
            assert np.array_equal(u[0].astype(np.int64), k)
            assert np.array_equal(O.fake_quant_asym(vals, None, 32), vals)

    def test_codes_are_nearest_level(self):
        rng = np.random.default_rng(13)
        W = (rng.standard_normal((24, 64)) * 0.05).astype(np.float16)
        W[3] = np.abs(W[3])                      # one-signed rows
        W[4] = -np.abs(W[4])
        W[5, :32] += np.float16(0.08)            # off-centre group
        s = np.exp(rng.standard_normal(64) * 0.4).astype(F32)
        u, z, step, v = O.group_quantize_asym(W, s, 32)
        for o in range(W.shape[0]):
            for g in range(2):
                st = float(step[o, g])
                vg = v[o, 32 * g:32 * (g + 1)].astype(F64)
                lo, hi = min(0.0, vg.min()), max(0.0, vg.max())
                assert abs(-lo / st - int(z[o, g])) <= 0.5 + 1e-6
                levels = (np.arange(16) - int(z[o, g])) * st
                dist = np.abs(vg[:, None] - levels[None, :])
                chosen = dist[np.arange(32), u[o, 32 * g:32 * (g + 1)].astype(np.int64)]
                assert np.all(chosen <= dist.min(axis=1) + 1e-6 * st)
                # the integer zero point shifts the grid by at most half a step
                assert levels[0] <= lo + (0.5 + 1e-6) * st and levels[15] >= hi - (0.5 + 1e-6) * st

    def test_one_signed_and_degenerate_groups(self):
        rng = np.random.default_rng(14)
        pos = rng.uniform(0.01, 0.3, 32).astype(F32)
        W = np.stack([pos, -pos, np.zeros(32, F32), np.full(32, 0.3, F32)])
        u, z, step, _ = O.group_quantize_asym(W, None, 32)
        assert int(z[0, 0]) == 0 and u[0].max() == 15 and u[0][np.argmax(pos)] == 15
        assert int(z[1, 0]) == 15 and u[1].min() == 0 and u[1][np.argmax(pos)] == 0
        assert step[2, 0] == 0 and int(z[2, 0]) == 0 and not u[2].any()
        assert int(z[3, 0]) == 0 and np.all(u[3] == 15)
        w_hat = O.fake_quant_asym(W, None, 32)
        assert not w_hat[2].any()
        assert np.all(w_hat[3] == F32(15) * (F32(0.3) / F32(15)))
        assert ulps32(w_hat[3], W[3]) <= 1

    def test_pack_zero_points_and_roundtrip(self):
        W = WL.make_weight(71, 64, 256)
        s = (np.exp(np.random.default_rng(1).standard_normal(256) * 0.3)).astype(F32)
        qw, sc, qz, u, z, step = O.quantize_pack_asym(W, s, 128)
        assert qw.shape == (256, 8) and sc.shape == (2, 64) and qz.shape == (2, 8)
        assert np.array_equal(O.unpack_codes(qw, 64), u)
        assert np.array_equal(O.unpack_codes(qz, 64), z)
        # qzeros use the qweight nibble order: zero point = row mod 8 gives the golden word
        zz = np.tile((np.arange(16) % 8).astype(np.uint8)[:, None], (1, 2))
        assert np.all(O.pack_codes(zz) == np.uint32(int(load("pack_order.json")["word_when_code_equals_row_mod_8"], 16)))
        deq = O.unpack_dequant(qw, sc, qz, 64, 128)
        ref = ((u.astype(np.int16) - np.repeat(z.astype(np.int16), 128, axis=1)).astype(F32)
               * np.repeat(step.astype(np.float16).astype(F32), 128, axis=1)).astype(F32)
        assert np.array_equal(deq, ref)

    def test_storage_bits_from_packed_sizes(self):
        W = WL.make_weight(72, 64, 1024)
        qw, sc, qz, *_ = O.quantize_pack_asym(W, None, 128)
        bits = 8 * (qw.nbytes + sc.nbytes + qz.nbytes) / W.size
        assert bits == 4 + (16 + 4) / 128 and round(bits, 2) == 4.16

    def test_search_asym_alpha_zero_is_rtn(self):
        W = WL.make_weight(73, 48, 256)
        X = WL.make_activations(74, 40, 256, "bf16")
        xm = O.act_stats(X)
        errs, k, s = O.search_scales([W], xm, 128, 20, asym=True)
        w_rtn = O.fake_quant_asym(W, None, 128)
        d = (W.astype(F64) - w_rtn.astype(F64)) * xm.astype(F64)[None, :]
        assert errs[0] == np.sum(d * d)
        assert errs[k] <= errs[0] and k == O.first_argmin(errs)
        eo, ko, _ = O.search_scales([W], xm, 128, 20, "output", X=X, asym=True)
        Y = O.decode_activations(X) @ (w_rtn.astype(F64) - W.astype(F64)).T
        assert abs(eo[0] - np.mean(Y * Y)) <= 1e-12 * np.mean(Y * Y)

    def test_clip_asym(self):
        rng = np.random.default_rng(15)
        d = 2.0 ** -6
        k = rng.integers(0, 16, (4, 32))
        k[:, 0], k[:, 1] = 0, 15
        W = ((k - 6) * d).astype(F32)           # range [-6d, 9d], step d, z = 6
        u1, z1, st1, _ = O.group_quantize_asym(W, None, 32, np.ones(4, F32))
        u0, z0, st0, _ = O.group_quantize_asym(W, None, 32)
        assert np.array_equal(u1, u0) and np.array_equal(z1, z0) and np.array_equal(st1, st0)
        uh, zh, sth, _ = O.group_quantize_asym(W, None, 32, np.full(4, 0.5, F32))
        assert np.all(sth == F32(d / 2)) and np.all(zh == 6)
        # values beyond the shrunk range saturate at the end codes
        assert np.array_equal(uh, np.clip(2 * (k - 6) + 6, 0, 15))


# ---------------------------------------------------------------------------
# W4A16 product on the packed layout ("AWQ architecture, in depth", "Kernels:
# why W4A16 is fast at decode"; "Weight-Only Quantization: GPTQ and AWQ",
# "The kernels" and "4. Tiny example")
# ---------------------------------------------------------------------------
class TestW4A16:
    g = load("worked_example.json")

    def test_worked_example_through_the_packed_layout(self):
        """The page's outputs (naive 4.629, AWQ 5.057) from the packed codes: the
        runtime multiplies x / s (fp16) with the stored q * fp16(step), so each
        result carries the fp16 roundings of the step and of x / s (2^-11
        relative each) on top of the page's 3-decimal print."""
        w = np.tile(np.array(self.g["w"], dtype=np.float16), (8, 1))          # 8 rows, one group of 4
        x = np.array(self.g["x"], dtype=F64)
        s = np.array(self.g["scale"], dtype=F32)
        for sv, key in [(None, "naive_out"), (s, "awq_out")]:
            qw, sc, qz, q, step = O.quantize_pack(w, sv, 4)
            xs = (x if sv is None else x / sv).astype(np.float16)[None, :]   # 1/s folded into the input
            y = O.w4a16_matmul(xs, qw, sc, qz, 8, 4)
            assert y.shape == (1, 8) and np.all(y == y[0, 0])
            assert abs(y[0, 0] - self.g["printed"][key]) <= 5e-4 + 3 * 2 ** -11 * abs(y[0, 0])

    def test_one_hot_rows_read_back_the_weights(self):
        W = WL.make_weight(80, 16, 64)
        qw, sc, qz, *_ = O.quantize_pack_asym(W, None, 32)
        eye = np.eye(64, dtype=np.float16)
        Y = O.w4a16_matmul(eye, qw, sc, qz, 16, 32)                       # Y[i, o] = W_hat[o, i]
        W_hat = O.unpack_dequant(qw, sc, qz, 16, 32)
        assert np.array_equal(Y, W_hat.T.astype(F64))
        Y2 = O.w4a16_matmul(eye[:3] * np.float16(2), qw, sc, qz, 16, 32)
        assert np.array_equal(Y2, 2 * W_hat.T[:3].astype(F64))

    def test_scaled_domain_equals_weight_domain(self):
        """(x / s) . W_hat_s = x . (W_hat_s / s): the packed product with the
        folded input reproduces the search's fake-quantized weights."""
        rng = np.random.default_rng(81)
        s = np.exp2(rng.integers(-2, 3, 128)).astype(F32)     # powers of two: the fold is exact
        # every group's max |w s| is 7 * 2^-6, so its step 2^-6 is stored exactly in fp16
        V = rng.uniform(-0.99, 0.99, (24, 128)) * 7 * 2.0 ** -6
        V[:, 5], V[:, 70] = 7 * 2.0 ** -6, -7 * 2.0 ** -6
        W = (V / s).astype(np.float16)
        X = (rng.standard_normal((3, 128)) * 4).astype(np.float16)
        qw, sc, qz, q, step = O.quantize_pack(W, s, 64)
        assert np.all(step == F32(2.0 ** -6))
        Y = O.w4a16_matmul((X.astype(F32) / s).astype(np.float16), qw, sc, qz, 24, 64)
        ref = X.astype(F64) @ O.fake_quant(W, s, 64).astype(F64).T
        np.testing.assert_allclose(Y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())

    def test_bytes_and_decode_speedup_bound(self):
        # weights at 4 + (16 + 4) / 128 bits against 16: the bandwidth-bound
        # speedup at batch 1 approaches 3 to 4 times
        n, k = 4096, 4096
        b = O.w4a16_bytes(n, k, 128)
        assert 8 * b / (n * k) == 4 + 20 / 128
        assert 3.0 < 2 * n * k / b < 4.0
        W = WL.make_weight(83, 64, 256)
        qw, sc, qz, *_ = O.quantize_pack_asym(W, None, 128)
        assert qw.nbytes + sc.nbytes + qz.nbytes == O.w4a16_bytes(64, 256, 128)
