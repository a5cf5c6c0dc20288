"""The oracle's pins are strong enough: each plausible single mistake planted in
the oracle (a dropped term, a wrong sign, index, constant, rounding mode or
operand order) makes at least one pin in test_oracle_pins.py fail.

Mistakes are planted by monkeypatching the oracle module on the CPU; the pins
are then run in-process, stopping at the first one that fails.
"""
import inspect

import numpy as np
import pytest

from oracle import awq_oracle as O
import test_oracle_pins as PINS

F32, F64 = np.float32, np.float64


def _pins():
    out = []
    for _, cls in inspect.getmembers(PINS, inspect.isclass):
        if cls.__name__.startswith("Test") and cls.__module__ == PINS.__name__:
            for name, fn in inspect.getmembers(cls, inspect.isfunction):
                if name.startswith("test_"):
                    out.append((f"{cls.__name__}.{name}", cls, name))
    return out


def _first_failing_pin():
    for label, cls, name in _pins():
        try:
            getattr(cls(), name)()
        except Exception:      # an assertion, or the mutant breaking a shape or type
            return label
    return None


# ---------------------------------------------------------------------------
# mutants: name -> list of (attribute, replacement)
# ---------------------------------------------------------------------------
def _act_stats_signed(X):
    Xd = O.decode_activations(X)
    return (Xd.sum(axis=0) / Xd.shape[0]).astype(F32)


def _act_stats_max(X):
    return np.abs(O.decode_activations(X)).max(axis=0).astype(F32)


def _act_stats_sum(X):
    return np.abs(O.decode_activations(X)).sum(axis=0).astype(F32)


def _grid_incl_one(n):
    return [k / (n - 1) for k in range(n)]


def _cand(x_mean, alpha, s_min=O.S_MIN, norm="geo", clamp_after=False):
    x = x_mean.astype(F64)
    t = np.ones_like(x) if alpha == 0.0 else np.power(x, alpha)
    if not clamp_after:
        t = np.maximum(t, s_min)
    d = np.sqrt(t.max() * t.min()) if norm == "geo" else t.max()
    t = t / d
    if clamp_after:
        t = np.maximum(t, s_min)
    return t.astype(F32)


def _gq(W, s, G, clip=None, rnd=np.rint, lo=-7, hi=7, div=7.0, use_s=True):
    Wf = np.asarray(W).astype(F32)
    d_out, d_in = Wf.shape
    v = Wf if (s is None or not use_s) else (Wf * s.astype(F32)[None, :]).astype(F32)
    vg = v.reshape(d_out, d_in // G, G)
    amax = np.abs(vg).max(axis=2)
    if clip is not None:
        amax = (clip.astype(F32)[:, None] * amax).astype(F32)
    step = (amax / F32(div)).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (vg / step[:, :, None]).astype(F32)
    ratio = np.where(step[:, :, None] > 0, ratio, F32(0))
    q = np.clip(rnd(ratio), lo, hi).astype(np.int8)
    return q.reshape(d_out, d_in), step, v


def _round_half_away(r):
    return np.sign(r) * np.floor(np.abs(r) + 0.5)


def _dequant(q, step, s, G, mode):
    d_out, d_in = q.shape
    qs = (q.astype(F32).reshape(d_out, -1, G) * step[:, :, None]).astype(F32).reshape(d_out, d_in)
    if s is None or mode == "none":
        return qs
    return (qs * s.astype(F32)[None, :]).astype(F32)   # mode "mul"


def _werr(W, s, x_mean, G, mode):
    w_hat = O.fake_quant(W, s, G)
    d = np.asarray(W).astype(F64) - w_hat.astype(F64)
    if mode == "x":
        return float(np.sum(d * d * x_mean.astype(F64)[None, :]))
    return float(np.sum(np.abs(d * x_mean.astype(F64)[None, :])))   # "l1"


def _oerr_rows_sum_first(W, s, X, G, clip=None):
    Xd = O.decode_activations(X)
    D = O.fake_quant(W, s, G, clip).astype(F64) - np.asarray(W).astype(F64)
    Y = Xd @ D.T
    return np.sum(Y, axis=0) ** 2


def _argmin_last(errors):
    best_i, best_e = -1, float("inf")
    for i, e in enumerate(errors):
        if e <= best_e:
            best_i, best_e = i, e
    return best_i


def _clip_ratios_rev(n, lo=0.5):
    return np.array([lo + j * (1.0 - lo) / (n - 1) for j in range(n)], dtype=F64).astype(F32)


def _clip_ratios_excl(n, lo=0.5):
    return np.array([1.0 - j * (1.0 - lo) / n for j in range(n)], dtype=F64).astype(F32)


_pack_codes_original = O.pack_codes   # captured before any test patches the module


def _pack_along_d_in(u):
    """codes packed 8 per word along the input axis: [d_in/8, d_out] words"""
    return _pack_codes_original(u.T.copy()).T.copy()


def _f16_trunc(x):
    b = np.asarray(x, dtype=F32).view(np.uint32)
    sign = (b >> 16) & 0x8000
    a = np.abs(np.asarray(x, dtype=F32)).astype(F64)
    h = np.asarray(a.astype(np.float16), dtype=np.float16)            # RNE magnitude
    over = h.astype(F64) > a                                          # rounded up -> step down
    hb = h.view(np.uint16) - over.astype(np.uint16)
    return (hb | sign.astype(np.uint16)).view(np.float16)


def _shared_arith(s_members):
    S = np.stack([np.asarray(x, dtype=F32).astype(F64) for x in s_members])
    return S.mean(axis=0).astype(F32)


def _shared_f32(s_members):
    S = np.stack([np.asarray(x, dtype=F32) for x in s_members])
    return np.exp(np.mean(np.log(S), axis=0, dtype=F32)).astype(F32)


def _fold_multiply(norm_w, s_shared):
    q = (O.decode_norm(norm_w) * np.asarray(s_shared, dtype=F32)).astype(F32)
    if norm_w.dtype == np.float16:
        return q.astype(np.float16)
    if norm_w.dtype == np.uint16:
        return O.f32_to_bf16_bits(q)
    return q


def _bf16_truncate(x):
    return (np.asarray(x, dtype=F32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _wmean_unnormalised(W_parts):
    W = np.concatenate([O.decode_weight(w) for w in W_parts], axis=0)
    return np.abs(W).astype(F64).mean(axis=0).astype(F32)


def _wmean_colmax(W_parts):
    W = np.abs(np.concatenate([O.decode_weight(w) for w in W_parts], axis=0))
    cmax = W.max(axis=0)
    q = np.where(cmax > 0, W / np.where(cmax > 0, cmax, 1), 0).astype(F32)
    return q.astype(F64).mean(axis=0).astype(F32)


def _duo(x_mean, w_mean, alpha, s_min=O.S_MIN, swap=False, eps_outside=False):
    x, w = x_mean.astype(F64), w_mean.astype(F64)
    num = np.ones_like(x) if alpha == 0.0 else np.power(x, alpha)
    e = alpha if swap else 1.0 - alpha
    t = num / np.power(w, e) + O.DUO_EPS if eps_outside else num / (np.power(w, e) + O.DUO_EPS)
    t = np.maximum(t, s_min)
    return (t / np.sqrt(t.max() * t.min())).astype(F32)


def _gqa(W, s, G, clip=None, div=15.0, zround=np.rint, zsign=1.0, with_zero=True, umax=15):
    Wf = np.asarray(W).astype(F32)
    d_out, d_in = Wf.shape
    v = Wf if s is None else (Wf * s.astype(F32)[None, :]).astype(F32)
    vg = v.reshape(d_out, d_in // G, G)
    hi, lo = vg.max(axis=2), vg.min(axis=2)
    if with_zero:
        hi, lo = np.maximum(hi, F32(0)), np.minimum(lo, F32(0))
    if clip is not None:
        c = clip.astype(F32)[:, None]
        hi, lo = (c * hi).astype(F32), (c * lo).astype(F32)
    step = ((hi - lo).astype(F32) / F32(div)).astype(F32)
    live = step > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        zr = (F32(-zsign) * lo / step).astype(F32)
        ratio = (vg / step[:, :, None]).astype(F32)
    z = np.where(live, np.clip(zround(zr), 0, 15), 0).astype(np.int16)
    n = np.where(live[:, :, None], np.rint(ratio), 0).astype(np.int64)
    u = np.clip(n + z[:, :, None], 0, umax).astype(np.uint8)
    return u.reshape(d_out, d_in), z.astype(np.uint8), step, v


def _deq_asym_no_zero(u, z, step, s, G):
    d_out, d_in = u.shape
    r = (u.astype(F32).reshape(d_out, -1, G) * step[:, :, None]).astype(F32).reshape(d_out, d_in)
    return r if s is None else (r / s.astype(F32)[None, :]).astype(F32)


def _pack_asym_zeros_row_order(W, s, G, clip=None):
    u, z, step, _ = O.group_quantize_asym(W, s, G, clip)
    qz = np.zeros((z.shape[1], z.shape[0] // 8), dtype=np.uint32)
    for j in range(8):
        qz |= z[j::8, :].astype(np.uint32).T << np.uint32(4 * j)
    return O.pack_codes(u), O.f32_to_f16(step.T), qz, u, z, step



def _w4a16_no_zero(X, qweight, scales, qzeros, d_out, G):
    return O.w4a16_matmul(X, qweight, scales, None, d_out, G)


def _w4a16_first_group_scales(X, qweight, scales, qzeros, d_out, G):
    sc = np.repeat(np.asarray(scales)[:1], np.asarray(scales).shape[0], axis=0)
    return _ORIG_W4A16(X, qweight, sc, qzeros, d_out, G)


def _w4a16_fp16_accumulate(X, qweight, scales, qzeros, d_out, G):
    W_hat = O.unpack_dequant(qweight, scales, qzeros, d_out, G).astype(np.float16)
    return (np.asarray(X, dtype=np.float16) @ W_hat.T).astype(F64)


_ORIG_W4A16 = O.w4a16_matmul
MUTANTS = {
    "act_stats: signed mean": [("act_stats", _act_stats_signed)],
    "act_stats: max |x|": [("act_stats", _act_stats_max)],
    "act_stats: sum, not mean": [("act_stats", _act_stats_sum)],
    "grid: k / (n - 1)": [("grid_alphas", _grid_incl_one)],
    "scales: divide by max": [("candidate_scale", lambda x, a, s_min=O.S_MIN: _cand(x, a, s_min, norm="max"))],
    "scales: clamp after normalising": [("candidate_scale",
                                         lambda x, a, s_min=O.S_MIN: _cand(x, a, s_min, clamp_after=True))],
    "quant: round half away from zero": [("group_quantize", lambda W, s, G, clip=None: _gq(W, s, G, clip,
                                                                                          rnd=_round_half_away))],
    "quant: truncate": [("group_quantize", lambda W, s, G, clip=None: _gq(W, s, G, clip, rnd=np.trunc))],
    "quant: clamp to [-8, 7]": [("group_quantize", lambda W, s, G, clip=None: _gq(W, s, G, clip, lo=-8))],
    "quant: step = max / 8": [("group_quantize", lambda W, s, G, clip=None: _gq(W, s, G, clip, div=8.0))],
    "quant: step = max / 15": [("group_quantize", lambda W, s, G, clip=None: _gq(W, s, G, clip, div=15.0))],
    "quant: scale s ignored": [("group_quantize", lambda W, s, G, clip=None: _gq(W, s, G, clip, use_s=False))],
    "dequant: no division by s": [("dequantize", lambda q, st, s, G: _dequant(q, st, s, G, "none"))],
    "dequant: multiply by s": [("dequantize", lambda q, st, s, G: _dequant(q, st, s, G, "mul"))],
    "weight error: x not squared": [("weight_error", lambda W, s, x, G: _werr(W, s, x, G, "x"))],
    "weight error: L1": [("weight_error", lambda W, s, x, G: _werr(W, s, x, G, "l1"))],
    "output error: sum before squaring": [("output_error_rows", _oerr_rows_sum_first)],
    "selection: last minimum": [("first_argmin", _argmin_last)],
    "selection: maximum": [("first_argmin", lambda e: int(np.argmax(np.asarray(e))))],
    "clip ratios: from clip_lo up": [("clip_ratios", _clip_ratios_rev)],
    "clip ratios: clip_lo never reached": [("clip_ratios", _clip_ratios_excl)],
    "pack: order 0..7": [("PACK_ORDER", [0, 1, 2, 3, 4, 5, 6, 7])],
    "pack: inverse order": [("PACK_ORDER", [0, 4, 1, 5, 2, 6, 3, 7])],
    "pack: zero point 8": [("ZERO_POINT", 8)],
    "pack: fp16 scales truncated": [("f32_to_f16", _f16_trunc)],
    "pack: qweight along d_in": [("pack_codes", _pack_along_d_in)],
    "duo: w_mean not row-normalised": [("weight_channel_mean", _wmean_unnormalised)],
    "duo: w_mean normalised by column max": [("weight_channel_mean", _wmean_colmax)],
    "duo: exponents swapped": [("candidate_scale_duo", lambda x, w, a, s_min=O.S_MIN: _duo(x, w, a, s_min, swap=True))],
    "duo: 1e-4 added outside the quotient": [("candidate_scale_duo",
                                              lambda x, w, a, s_min=O.S_MIN: _duo(x, w, a, s_min, eps_outside=True))],
    "export: arithmetic mean of the scales": [("shared_scale", _shared_arith)],
    "export: first member's scale": [("shared_scale", lambda s_members: np.asarray(s_members[0], dtype=F32))],
    "export: logarithms in fp32": [("shared_scale", _shared_f32)],
    "export: norm multiplied by s": [("fold_norm", _fold_multiply)],
    "export: bf16 by truncation": [("f32_to_bf16_bits", _bf16_truncate)],
    "asym: step = range / 16": [("group_quantize_asym", lambda W, s, G, clip=None: _gqa(W, s, G, clip, div=16.0))],
    "asym: zero point rounded down": [("group_quantize_asym", lambda W, s, G, clip=None: _gqa(W, s, G, clip,
                                                                                          zround=np.floor))],
    "asym: zero point with the wrong sign": [("group_quantize_asym",
                                              lambda W, s, G, clip=None: _gqa(W, s, G, clip, zsign=-1.0))],
    "asym: range need not contain zero": [("group_quantize_asym",
                                           lambda W, s, G, clip=None: _gqa(W, s, G, clip, with_zero=False))],
    "asym: codes clamped to [0, 14]": [("group_quantize_asym", lambda W, s, G, clip=None: _gqa(W, s, G, clip, umax=14))],
    "asym: dequant ignores the zero point": [("dequantize_asym", _deq_asym_no_zero)],
    "asym: qzeros in row order": [("quantize_pack_asym", _pack_asym_zeros_row_order)],
    "w4a16: zero points ignored": [("w4a16_matmul", _w4a16_no_zero)],
    "w4a16: first group's scales everywhere": [("w4a16_matmul", _w4a16_first_group_scales)],
    "w4a16: fp16 accumulation": [("w4a16_matmul", _w4a16_fp16_accumulate)],
    "export: o/down with the shared scale": [("export_rtn", lambda W, G: O.quantize_pack(W, np.full(W.shape[1], 2.0, F32), G))],
}


def test_unmutated_oracle_passes_every_pin():
    assert _first_failing_pin() is None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    for attr, repl in MUTANTS[name]:
        monkeypatch.setattr(O, attr, repl)
    caught = _first_failing_pin()
    assert caught is not None, f"no pin fails with the mistake '{name}' planted in the oracle"
