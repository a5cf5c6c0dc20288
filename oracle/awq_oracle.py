"""CPU oracle for the AWQ per-layer hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and shares no code,
header, table or constant generator with it.

It is a plain, slow and obviously correct restatement of what the pages
compute, written with numpy so that each step can be read against the page it
comes from.  Sources are cited by page title and section:

* [konic]   "From-Scratch AWQ INT4 Quantization on Qwen3-8B" (konic.io):
            "AWQ scaling", "Group-wise symmetric INT4", "AutoAWQ / HF-AWQ GEMM
            on-disk format", exporter step 4 (signed grid -> unsigned, zero 7).
* [cassindra] "AWQ architecture, in depth" (aicassindra.com): "The pipeline
            end to end" (steps 3 and 5), "The scale search as code",
            "Quantization, storage and packing".
* [lm]      "Weight-Only Quantization: GPTQ and AWQ" (learning-materials):
            "4. Tiny example", "5. Technical explanation / AWQ",
            "6-9. Under the hood: the packed format".
* [repro]   "AWQ, Reproduced" (romaanj.github.io): "Q5 why scaling protects",
            "Q6 where to stop".

Precision.  The pages fix no precision.  Quantization arithmetic (scaling,
group max, step, division, rounding, dequantization) is IEEE fp32 with
round-to-nearest-even -- every numpy float32 ufunc below rounds once, and
nothing is fused -- so that the integer codes are decided in the same
precision the GPU decides them.  Candidate scales are evaluated in fp64 and
rounded once to fp32.  Every error sum is accumulated in fp64.

Readings where the pages are silent, garbled or disagree (each is listed with
its reason in the design notes of the repository):

* statistic: mean |x| over calibration tokens ([konic] names it x_max but
  writes |X|.mean(0); [cassindra] uses the mean);
* candidates: s = clamp(x_mean^alpha, 1e-4) / sqrt(max(s) * min(s)),
  alpha_k = k / n_grid for k = 0..n_grid-1 (the non-duo branch of the
  [cassindra] search); pow(x, 0) = 1 for every x, so alpha = 0 gives s = 1;
* rounding: round-half-to-even;
* weight-mode error: sum over all elements of ((w - w_hat) * x_mean)^2
  ([konic] ||(W - Q(W s)/s) diag(x)||^2, a sum, not a mean);
* output-mode error: mean over tokens x output rows of (X (W_hat - W)^T)^2
  ([cassindra] compares the group output with the full-precision output and
  takes the mean of the squared difference; the difference is evaluated
  exactly as X (W_hat - W)^T);
* all-zero group: step 0, codes 0, dequantized weights 0;
* ties between candidates: the first (smallest index) minimum wins (strict <);
* clip search: one ratio per output row, ratios 1.0 down to clip_lo in
  n_clip equal steps, step = RN(RN(c * max|v|) / 7), strict < so that ties keep
  the larger ratio;
* packing: qweight[i, m] holds, in nibble j (bits 4j..4j+3), the unsigned code
  of output row 8m + order[j], order = [0, 2, 4, 6, 1, 3, 5, 7];
  scales[g, o] = fp16(step), qzeros[g, m] = 0x77777777.

Duo scaling: w_mean is the mean over the group's rows of |w| / rowmax|w|
(quotients in fp32, sums in fp64, all-zero rows contributing 0), and
t = max(x^r / (w_mean^(1-r) + 1e-4), 1e-4) before the same normalisation.

Asymmetric INT4: per group and output row the range [lo, hi] = [min(0, min v),
max(0, max v)], step = RN(RN(hi - lo) / 15), zero point z = clamp(rint(RN(-lo /
step)), 0, 15), code u = clamp(rint(RN(v / step)) + z, 0, 15), reconstruction
(u - z) * step; an all-zero group has step 0, z = 0, u = 0.  A clip ratio c
shrinks both ends (RN(c lo), RN(c hi)).  qzeros hold z in the qweight nibble
order.

W4A16 product: Y = X W_hat^T in fp64 with W_hat the exact fp32 dequantization
(u - z) * fp16 scale of the packed layout (the stored, scaled domain: the
activations are the ones that already carry the folded 1/s).

Norm-group export: the shared scale is the per-channel geometric mean of the
member scales, evaluated as exp(mean(ln s)) in fp64 and rounded once to fp32;
the folded norm is the IEEE fp32 quotient rounded once to the norm's dtype.

Parity unpinned: the nibble-order reading and the qweight orientation against
a real INT4 runtime (no runtime or checkpoint is available to compare with),
and the clip-search semantics beyond "ratio 1.0 reproduces the unclipped
quantizer".
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

F32 = np.float32
F64 = np.float64

QMAX = 7                      # symmetric signed grid [-7, 7] ([konic] Group-wise symmetric INT4)
UMAX = 15                     # asymmetric unsigned grid [0, 15] ([cassindra] 4-bit zero point, step ~ range / 15)
ZERO_POINT = 7                # u = q + 7 ([konic] exporter step 4)
PACK_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)   # [konic] AutoAWQ / HF-AWQ GEMM on-disk format
S_MIN = 1e-4                  # [cassindra] clamp(min=1e-4)


# ---------------------------------------------------------------------------
# input decoding (exact)
# ---------------------------------------------------------------------------
def decode_activations(X: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or float16 -> exact float64 values."""
    if X.dtype == np.uint16:
        return (X.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(F64)
    if X.dtype == np.float16:
        return X.astype(F64)
    if X.dtype in (np.float32, np.float64):
        return X.astype(F64)
    raise TypeError(X.dtype)


def decode_weight(W: np.ndarray) -> np.ndarray:
    """fp16 weight -> exact float32 values."""
    return np.asarray(W, dtype=np.float16).astype(F32)


# ---------------------------------------------------------------------------
# O1: activation statistic ([konic] AWQ scaling; [cassindra] search_scale's
#     first line: mean over tokens of |x| per input channel)
# ---------------------------------------------------------------------------
def act_stats(X: np.ndarray) -> np.ndarray:
    """x_mean[i] = (1/T) sum_t |X[t, i]|, summed in fp64, rounded once to fp32."""
    Xd = decode_activations(X)
    T = Xd.shape[0]
    total = np.zeros(Xd.shape[1], dtype=F64)
    for t in range(T):            # plain token-order sum
        total += np.abs(Xd[t])
    return (total / T).astype(F32)


# ---------------------------------------------------------------------------
# O2: candidate scales ([cassindra] The scale search as code, non-duo branch;
#     [lm] s = |X|^alpha with alpha in [0, 1])
# ---------------------------------------------------------------------------
def grid_alphas(n_grid: int) -> List[float]:
    """alpha_k = k / n_grid, k = 0 .. n_grid-1 (1.0 itself is not a grid point)."""
    return [k / n_grid for k in range(n_grid)]


def candidate_scale(x_mean: np.ndarray, alpha: float, s_min: float = S_MIN) -> np.ndarray:
    """s = max(x_mean^alpha, s_min) / sqrt(max(s) * min(s)) in fp64, rounded to fp32.

    pow(x, 0) is 1 for every x (including 0), so alpha = 0 gives s = 1 exactly.
    """
    x = x_mean.astype(F64)
    if alpha == 0.0:
        t = np.ones_like(x)
    else:
        t = np.power(x, alpha)
    t = np.maximum(t, s_min)
    norm = np.sqrt(t.max() * t.min())
    return (t / norm).astype(F32)


def candidate_scales(x_mean: np.ndarray, n_grid: int = 20, s_min: float = S_MIN,
                     w_mean: Optional[np.ndarray] = None) -> np.ndarray:
    """Rows s_k for alpha_k = k / n_grid; with w_mean given, the duo-scaling
    candidates (candidate_scale_duo)."""
    if w_mean is not None:
        return np.stack([candidate_scale_duo(x_mean, w_mean, a, s_min) for a in grid_alphas(n_grid)])
    return np.stack([candidate_scale(x_mean, a, s_min) for a in grid_alphas(n_grid)])


# ---------------------------------------------------------------------------
# O2b: duo scaling ([cassindra] The scale search as code, duo_scaling=True:
#      w_mean = (|W| / rowmax |W|).mean over rows, per input channel, of the
#      group's concatenated weights; s = x_mean^r / (w_mean^(1-r) + 1e-4),
#      then the same clamp and normalisation as the plain candidates)
# ---------------------------------------------------------------------------
DUO_EPS = 1e-4


def weight_channel_mean(W_parts: Sequence[np.ndarray]) -> np.ndarray:
    """w_mean[i] = (1/d_out) sum_o |W[o, i]| / max_j |W[o, j]| over the
    concatenated rows: each quotient in IEEE fp32, the sum over rows in fp64
    (row order), the mean rounded once to fp32.  A row whose entries are all
    zero contributes 0 (its quotients would be 0/0)."""
    W = np.concatenate([decode_weight(w) for w in W_parts], axis=0)       # exact fp32
    A = np.abs(W)
    rmax = A.max(axis=1)
    total = np.zeros(W.shape[1], dtype=F64)
    for o in range(W.shape[0]):
        if rmax[o] > 0:
            total += (A[o] / rmax[o]).astype(F32).astype(F64)
    return (total / W.shape[0]).astype(F32)


def candidate_scale_duo(x_mean: np.ndarray, w_mean: np.ndarray, alpha: float,
                        s_min: float = S_MIN) -> np.ndarray:
    """t = max(x^alpha / (w^(1-alpha) + 1e-4), s_min), s = t / sqrt(max t * min t),
    in fp64, rounded once to fp32.  pow(v, 0) = 1 for every v (R5)."""
    x, w = x_mean.astype(F64), w_mean.astype(F64)
    num = np.ones_like(x) if alpha == 0.0 else np.power(x, alpha)
    den = np.power(w, 1.0 - alpha) + DUO_EPS
    t = np.maximum(num / den, s_min)
    norm = np.sqrt(t.max() * t.min())
    return (t / norm).astype(F32)


# ---------------------------------------------------------------------------
# O3: group-wise symmetric INT4 fake quantization of W * s
#     ([konic] Group-wise symmetric INT4: step = max|group| / 7,
#      q = round(w / step).clamp(-7, 7); [konic] AWQ scaling: W' = W * s and
#      the reconstruction Q(W * s) / s; [lm] 4. Tiny example)
# ---------------------------------------------------------------------------
def group_quantize(W: np.ndarray, s: Optional[np.ndarray], group_size: int,
                   clip: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Quantize v = RN(w * s) group-wise along the input axis.

    W: [d_out, d_in] (fp16 or fp32 values), s: [d_in] fp32 or None (= 1),
    clip: [d_out] fp32 ratio per output row or None (= 1).
    Returns (q int8 [d_out, d_in], step fp32 [d_out, d_in/G], v fp32 [d_out, d_in]).
    """
    Wf = np.asarray(W).astype(F32)
    d_out, d_in = Wf.shape
    assert d_in % group_size == 0
    n_groups = d_in // group_size
    v = Wf if s is None else (Wf * s.astype(F32)[None, :]).astype(F32)
    vg = v.reshape(d_out, n_groups, group_size)
    amax = np.abs(vg).max(axis=2)                                   # [d_out, n_groups], exact
    if clip is not None:
        amax = (clip.astype(F32)[:, None] * amax).astype(F32)       # RN(c * a)
    step = (amax / F32(QMAX)).astype(F32)                           # RN(a / 7)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (vg / step[:, :, None]).astype(F32)                 # RN(v / step)
    ratio = np.where(step[:, :, None] > 0, ratio, F32(0))           # all-zero group -> 0
    q = np.clip(np.rint(ratio), -QMAX, QMAX).astype(np.int8)        # half-to-even, clamp
    return q.reshape(d_out, d_in), step, v


def dequantize(q: np.ndarray, step: np.ndarray, s: Optional[np.ndarray], group_size: int) -> np.ndarray:
    """w_hat = RN(RN(q * step) / s) in fp32 ([konic] Q(W s)/s)."""
    d_out, d_in = q.shape
    qs = (q.astype(F32).reshape(d_out, -1, group_size) * step[:, :, None]).astype(F32)
    qs = qs.reshape(d_out, d_in)
    if s is None:
        return qs
    return (qs / s.astype(F32)[None, :]).astype(F32)


def fake_quant(W: np.ndarray, s: Optional[np.ndarray], group_size: int,
               clip: Optional[np.ndarray] = None) -> np.ndarray:
    q, step, _ = group_quantize(W, s, group_size, clip)
    return dequantize(q, step, s, group_size)


# ---------------------------------------------------------------------------
# O3a: group-wise asymmetric INT4 ([cassindra] "Why it works" worked example:
#      values up to 0.5 in a group give a step of about 1/15 and a worst
#      rounding error of about half that; "Quantization, storage and packing":
#      one 16-bit scale and one 4-bit zero point per group and output channel,
#      4 + (16 + 4) / 128 bits per weight; "The recipe": W4A16_ASYM)
# ---------------------------------------------------------------------------
def group_quantize_asym(W: np.ndarray, s: Optional[np.ndarray], group_size: int,
                        clip: Optional[np.ndarray] = None):
    """Asymmetric quantization of v = RN(w * s) group-wise along the input axis.

    The range of a group is [lo, hi] = [min(0, min v), max(0, max v)] (zero
    inside, so it is representable and z is an integer code), optionally
    shrunk by the row's clip ratio c to [RN(c lo), RN(c hi)];
    step = RN(RN(hi - lo) / 15); z = clamp(rint(RN(-lo / step)), 0, 15);
    u = clamp(rint(RN(v / step)) + z, 0, 15).  An all-zero group has step 0,
    z = 0 and u = 0.
    Returns (u uint8 [d_out, d_in], z uint8 [d_out, d_in/G], step fp32 [d_out, d_in/G], v fp32).
    """
    Wf = np.asarray(W).astype(F32)
    d_out, d_in = Wf.shape
    assert d_in % group_size == 0
    n_groups = d_in // group_size
    v = Wf if s is None else (Wf * s.astype(F32)[None, :]).astype(F32)
    vg = v.reshape(d_out, n_groups, group_size)
    hi = np.maximum(vg.max(axis=2), F32(0))                          # exact
    lo = np.minimum(vg.min(axis=2), F32(0))
    if clip is not None:
        c = clip.astype(F32)[:, None]
        hi, lo = (c * hi).astype(F32), (c * lo).astype(F32)          # RN(c hi), RN(c lo)
    step = ((hi - lo).astype(F32) / F32(UMAX)).astype(F32)          # RN(RN(hi - lo) / 15)
    live = step > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        zr = (-lo / step).astype(F32)                                # RN(-lo / step)
        ratio = (vg / step[:, :, None]).astype(F32)                  # RN(v / step)
    z = np.where(live, np.clip(np.rint(zr), 0, UMAX), 0).astype(np.int16)
    n = np.where(live[:, :, None], np.rint(ratio), 0).astype(np.int64)
    u = np.clip(n + z[:, :, None], 0, UMAX).astype(np.uint8)
    return u.reshape(d_out, d_in), z.astype(np.uint8), step, v


def dequantize_asym(u: np.ndarray, z: np.ndarray, step: np.ndarray, s: Optional[np.ndarray],
                    group_size: int) -> np.ndarray:
    """w_hat = RN(RN((u - z) * step) / s) in fp32."""
    d_out, d_in = u.shape
    qs = u.astype(np.int16).reshape(d_out, -1, group_size) - z.astype(np.int16)[:, :, None]
    r = (qs.astype(F32) * step[:, :, None]).astype(F32).reshape(d_out, d_in)
    if s is None:
        return r
    return (r / s.astype(F32)[None, :]).astype(F32)


def fake_quant_asym(W: np.ndarray, s: Optional[np.ndarray], group_size: int,
                    clip: Optional[np.ndarray] = None) -> np.ndarray:
    u, z, step, _ = group_quantize_asym(W, s, group_size, clip)
    return dequantize_asym(u, z, step, s, group_size)


def _fq(W, s, group_size, clip=None, asym=False):
    return fake_quant_asym(W, s, group_size, clip) if asym else fake_quant(W, s, group_size, clip)


# ---------------------------------------------------------------------------
# O4w: activation-weighted reconstruction error ([konic] AWQ scaling:
#      || (W - Q(W s)/s) diag(x) ||^2)
# ---------------------------------------------------------------------------
def weight_error(W: np.ndarray, s: np.ndarray, x_mean: np.ndarray, group_size: int,
                 asym: bool = False) -> float:
    w_hat = _fq(W, s, group_size, None, asym)
    d = (np.asarray(W).astype(F64) - w_hat.astype(F64)) * x_mean.astype(F64)[None, :]
    return float(np.sum(d * d))


# ---------------------------------------------------------------------------
# O4o: group output error ([cassindra] err = mean((block_fn(x) - ref)^2) with
#      the linears' weights replaced by Q(w0 s)/s; [lm] 2. Why: the layer's
#      output error is X (W - W_hat))
# ---------------------------------------------------------------------------
def output_error_rows(W: np.ndarray, s: Optional[np.ndarray], X: np.ndarray, group_size: int,
                      clip: Optional[np.ndarray] = None, asym: bool = False) -> np.ndarray:
    """Per output row o: sum_t (sum_i X[t,i] (w_hat[o,i] - W[o,i]))^2, fp64."""
    Xd = decode_activations(X)
    w_hat = _fq(W, s, group_size, clip, asym)
    D = w_hat.astype(F64) - np.asarray(W).astype(F64)              # [d_out, d_in]
    Y = Xd @ D.T                                                    # [T, d_out]
    return np.sum(Y * Y, axis=0)


def output_error(W: np.ndarray, s: np.ndarray, X: np.ndarray, group_size: int, asym: bool = False) -> float:
    rows = output_error_rows(W, s, X, group_size, None, asym) if asym else output_error_rows(W, s, X, group_size)
    T = X.shape[0]
    return float(rows.sum() / (T * np.asarray(W).shape[0]))


# ---------------------------------------------------------------------------
# O5: grid search with first-minimum selection ([cassindra] loop over
#     i in range(n_grid), keep (err, s) when err < best; [konic] alpha = 0 is
#     plain RTN so the search is never worse than RTN)
# ---------------------------------------------------------------------------
def first_argmin(errors: Sequence[float]) -> int:
    best_i, best_e = -1, float("inf")
    for i, e in enumerate(errors):
        if e < best_e:
            best_i, best_e = i, e
    return best_i


def search_scales(W_parts: Sequence[np.ndarray], x_mean: np.ndarray, group_size: int,
                  n_grid: int = 20, score: str = "weight", X: Optional[np.ndarray] = None,
                  s_min: float = S_MIN, duo: bool = False, asym: bool = False):
    """Returns (errors [n_grid] fp64, best index, best s fp32 [d_in]).

    The linears of one input-sharing group are scored together, their rows
    concatenated ([cassindra] torch.cat of the group's weights); duo = True
    takes the duo-scaling candidates of those rows; asym = True scores the
    asymmetric quantizer (O3a).
    """
    W = np.concatenate([np.asarray(w) for w in W_parts], axis=0)
    S = candidate_scales(x_mean, n_grid, s_min, weight_channel_mean(W_parts) if duo else None)
    errs = []
    for k in range(n_grid):
        if score == "weight":
            errs.append(weight_error(W, S[k], x_mean, group_size, asym=True) if asym
                        else weight_error(W, S[k], x_mean, group_size))
        elif score == "output":
            errs.append(output_error(W, S[k], X, group_size, asym=True) if asym
                        else output_error(W, S[k], X, group_size))
        else:
            raise ValueError(score)
    k_best = first_argmin(errs)
    return np.array(errs, dtype=F64), k_best, S[k_best]


# ---------------------------------------------------------------------------
# O6: per-output-channel clip-ratio search ([cassindra] The pipeline end to end,
#     step 5: search a clipping range per output channel that shrinks the
#     quantization range; [repro] Q6: the paper also clips the weight range)
# ---------------------------------------------------------------------------
def clip_ratios(n_clip: int, clip_lo: float = 0.5) -> np.ndarray:
    """c_j = 1 - j (1 - clip_lo) / (n_clip - 1), j = 0..n_clip-1, fp64 -> fp32."""
    return np.array([1.0 - j * (1.0 - clip_lo) / (n_clip - 1) for j in range(n_clip)],
                    dtype=F64).astype(F32)


def clip_search(W: np.ndarray, s: np.ndarray, X: np.ndarray, group_size: int,
                n_clip: int = 20, clip_lo: float = 0.5, asym: bool = False):
    """Returns (E [d_out, n_clip] fp64, chosen ratio [d_out] fp32)."""
    Wa = np.asarray(W)
    ratios = clip_ratios(n_clip, clip_lo)
    E = np.zeros((Wa.shape[0], n_clip), dtype=F64)
    for j, c in enumerate(ratios):
        clip = np.full(Wa.shape[0], c, dtype=F32)
        E[:, j] = output_error_rows(Wa, s, X, group_size, clip, asym) if asym \
            else output_error_rows(Wa, s, X, group_size, clip)
    best = np.array([first_argmin(E[o]) for o in range(Wa.shape[0])])
    return E, ratios[best]


# ---------------------------------------------------------------------------
# O7: quantize + pack into the AutoAWQ GEMM layout ([konic] AutoAWQ / HF-AWQ
#     GEMM on-disk format and exporter step 4; [lm] 6-9 packed format:
#     scales [in/G, out] fp16, zeros [in/G, out/8] int32)
# ---------------------------------------------------------------------------
def f32_to_f16(x: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 round-to-nearest-even (numpy's cast; pinned by golden values)."""
    return np.asarray(x, dtype=F32).astype(np.float16)


def pack_codes(u: np.ndarray) -> np.ndarray:
    """u [d_out, d_in] unsigned codes (0..15) -> qweight [d_in, d_out/8] uint32.

    Word (i, m) holds the code of output row 8m + PACK_ORDER[j] in nibble j.
    """
    d_out, d_in = u.shape
    assert d_out % 8 == 0
    words = np.zeros((d_in, d_out // 8), dtype=np.uint32)
    for j, e in enumerate(PACK_ORDER):
        rows = u[e::8, :].astype(np.uint32)            # rows 8m + e for all m: [d_out/8, d_in]
        words |= rows.T << np.uint32(4 * j)
    return words


def unpack_codes(qweight: np.ndarray, d_out: int) -> np.ndarray:
    """Inverse of pack_codes: qweight [d_in, d_out/8] -> u [d_out, d_in]."""
    qw = np.asarray(qweight).view(np.uint32) if qweight.dtype == np.int32 else np.asarray(qweight, np.uint32)
    d_in = qw.shape[0]
    u = np.zeros((d_out, d_in), dtype=np.uint8)
    for j, e in enumerate(PACK_ORDER):
        u[e::8, :] = ((qw >> np.uint32(4 * j)) & np.uint32(0xF)).T
    return u


def quantize_pack(W: np.ndarray, s: Optional[np.ndarray], group_size: int,
                  clip: Optional[np.ndarray] = None):
    """Returns (qweight uint32 [d_in, d_out/8], scales fp16 [d_in/G, d_out],
    qzeros uint32 [d_in/G, d_out/8], q int8 [d_out, d_in], step fp32 [d_out, d_in/G])."""
    q, step, _ = group_quantize(W, s, group_size, clip)
    u = (q.astype(np.int16) + ZERO_POINT).astype(np.uint8)
    qweight = pack_codes(u)
    scales = f32_to_f16(step.T)                                      # [d_in/G, d_out]
    d_out = q.shape[0]
    zword = np.uint32(0)
    for j in range(8):
        zword |= np.uint32(ZERO_POINT) << np.uint32(4 * j)
    qzeros = np.full((step.shape[1], d_out // 8), zword, dtype=np.uint32)
    return qweight, scales, qzeros, q, step


def quantize_pack_asym(W: np.ndarray, s: Optional[np.ndarray], group_size: int,
                       clip: Optional[np.ndarray] = None):
    """Asymmetric codes (O3a) in the same layout: qweight nibbles hold u,
    scales fp16(step), and qzeros [d_in/G, d_out/8] hold z in the qweight
    nibble order (word (g, m), nibble j: row 8m + PACK_ORDER[j]).
    Returns (qweight, scales, qzeros, u [d_out, d_in], z [d_out, d_in/G], step)."""
    u, z, step, _ = group_quantize_asym(W, s, group_size, clip)
    qweight = pack_codes(u)
    scales = f32_to_f16(step.T)
    qzeros = pack_codes(z)                                           # [d_in/G, d_out/8]
    return qweight, scales, qzeros, u, z, step


# ---------------------------------------------------------------------------
# O8: unpack + dequantize ([konic] exporter step 4: (q - zero) * scale
#     reproduces q_signed * group_scale exactly)
# ---------------------------------------------------------------------------
def unpack_dequant(qweight: np.ndarray, scales: np.ndarray, qzeros: Optional[np.ndarray],
                   d_out: int, group_size: int, s: Optional[np.ndarray] = None) -> np.ndarray:
    u = unpack_codes(qweight, d_out).astype(F32)                    # [d_out, d_in]
    d_in = u.shape[1]
    if qzeros is None:
        z = np.full((d_out, d_in // group_size), ZERO_POINT, dtype=F32)
    else:
        z = unpack_codes(qzeros, d_out).astype(F32)                 # [d_out, d_in/G]
    sc = np.asarray(scales, dtype=np.float16).astype(F32)           # [d_in/G, d_out]
    zz = np.repeat(z, group_size, axis=1)                           # [d_out, d_in]
    ss = np.repeat(sc.T, group_size, axis=1)
    w = ((u - zz) * ss).astype(F32)
    if s is not None:
        w = (w / s.astype(F32)[None, :]).astype(F32)
    return w


# ---------------------------------------------------------------------------
# O10: W4A16 product on the packed layout ([cassindra] "Kernels: why W4A16 is
#      fast at decode": the packed 4-bit weights are dequantized with the
#      group's scale and zero point and multiplied with 16-bit activations;
#      decode is bound by reading the weights; [lm] "The kernels": W4A16 GEMM)
# ---------------------------------------------------------------------------
def w4a16_matmul(X: np.ndarray, qweight: np.ndarray, scales: np.ndarray, qzeros: Optional[np.ndarray],
                 d_out: int, group_size: int) -> np.ndarray:
    """Y [M, d_out] = X [M, d_in] W_hat^T, fp64, where W_hat [d_out, d_in] is
    unpack_dequant of the packed tensors (exact fp32 values); X is fp16 (or
    bf16 bits), decoded exactly."""
    W_hat = unpack_dequant(qweight, scales, qzeros, d_out, group_size)   # [d_out, d_in]
    return decode_activations(X) @ W_hat.astype(F64).T


def w4a16_bytes(d_out: int, d_in: int, group_size: int) -> int:
    """Bytes a W4A16 product reads for its weights: 4-bit codes, fp16 scales
    and 4-bit zero points per group and output channel."""
    return d_out * d_in // 2 + 2 * d_out * (d_in // group_size) + d_out * (d_in // group_size) // 2


# ---------------------------------------------------------------------------
# O9: norm-group export ([konic] "AutoAWQ / HF-AWQ GEMM on-disk format", the
#     exporter's steps 1-3: q/k/v share input_layernorm and gate/up share
#     post_attention_layernorm, so their per-linear scales become one shared
#     scale per norm group -- the geometric mean over the member linears --
#     folded into that norm as norm.weight /= s_shared; the norm-following
#     linears are re-quantized with the shared scale, and o_proj / down_proj,
#     which have no preceding norm, are exported as plain RTN, s = 1)
# ---------------------------------------------------------------------------
def shared_scale(s_members: Sequence[np.ndarray]) -> np.ndarray:
    """s_shared[i] = (prod_m s_m[i]) ** (1/M), evaluated as the exponential of
    the mean natural logarithm in fp64 and rounded once to fp32."""
    S = np.stack([np.asarray(s, dtype=F32).astype(F64) for s in s_members])   # [M, d_in]
    return np.exp(np.mean(np.log(S), axis=0)).astype(F32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest, ties to even: the
    two bf16 neighbours of x (mantissa truncated toward zero, and one unit
    further from zero) are compared with x in exact fp64 arithmetic."""
    x = np.asarray(x, dtype=F32)
    toward0 = x.view(np.uint32) >> np.uint32(16)
    away = toward0 + np.uint32(1)
    v0 = (toward0 << np.uint32(16)).view(F32).astype(F64)
    v1 = (away << np.uint32(16)).view(F32).astype(F64)
    xd = x.astype(F64)
    d0, d1 = np.abs(xd - v0), np.abs(v1 - xd)
    pick_away = (d1 < d0) | ((d1 == d0) & ((toward0 & np.uint32(1)) == 1))
    return np.where(pick_away, away, toward0).astype(np.uint16)


def decode_norm(norm_w: np.ndarray) -> np.ndarray:
    """fp16, bf16 (uint16 bit patterns) or fp32 norm weight -> exact fp32 values."""
    if norm_w.dtype == np.uint16:
        return (norm_w.astype(np.uint32) << np.uint32(16)).view(F32)
    if norm_w.dtype in (np.float16, np.float32):
        return norm_w.astype(F32)
    raise TypeError(norm_w.dtype)


def fold_norm(norm_w: np.ndarray, s_shared: np.ndarray) -> np.ndarray:
    """norm.weight /= s_shared: the IEEE fp32 quotient, rounded once to the
    norm's own dtype (the in-place division of an fp16 / bf16 tensor)."""
    q = (decode_norm(norm_w) / np.asarray(s_shared, dtype=F32)).astype(F32)
    if norm_w.dtype == np.float16:
        return q.astype(np.float16)
    if norm_w.dtype == np.uint16:
        return f32_to_bf16_bits(q)
    return q


def export_norm_group(W_members: Sequence[np.ndarray], s_members: Sequence[np.ndarray],
                      norm_w: np.ndarray, group_size: int):
    """Steps 1-2 for one norm group: (s_shared, folded norm, [quantize_pack of
    every member with s_shared])."""
    s_sh = shared_scale(s_members)
    return s_sh, fold_norm(norm_w, s_sh), [quantize_pack(W, s_sh, group_size) for W in W_members]


def export_rtn(W: np.ndarray, group_size: int):
    """Step 3: o_proj / down_proj at plain round-to-nearest (s = 1)."""
    return quantize_pack(W, None, group_size)
