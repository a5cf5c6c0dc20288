"""Seeded synthetic inputs for the AWQ per-layer hot path.

This module only draws random numbers and encodes them as fp16 / bf16 bit
patterns.  It holds none of the quantization method's arithmetic, so both the
CPU oracle and the GPU library can be fed from it without sharing any code.

Workloads are the Qwen3-8B-shaped linear groups that the scale search runs on:

* weights  W[d_out, d_in] ~ N(0, 0.02^2), stored fp16 (round-to-nearest-even);
* calibration activations X[t, i] = m_i * z_ti with z ~ N(0, 1) and per-input-
  channel magnitudes m_i = exp(N(0, 0.5^2)) (lognormal(0, 0.5)); a seeded
  random 1% of the channels (round(0.01 * d_in)) is multiplied by 50 to model
  the outlier channels whose weights AWQ protects;
* the down-projection input of an MLP is SiLU(X W_gate^T) * (X W_up^T),
  evaluated in fp32 from the fp16 weights and rounded to bf16;
* norm weights (the export's RMSNorm gains) g_i = 1 + 0.1 * N(0, 1), fp16.

bf16 tensors are carried as ``uint16`` arrays holding the bit pattern, since
numpy has no bf16 dtype.  Large device-resident workloads (the full-model sweep)
are drawn with torch's device generator instead; the statistics are the same,
the streams differ.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

WEIGHT_STD = 0.02
MAG_SIGMA = 0.5
OUTLIER_FRACTION = 0.01
OUTLIER_GAIN = 50.0


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round-to-nearest-even (inputs hold no NaN)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_weight(seed: int, d_out: int, d_in: int) -> np.ndarray:
    """W[d_out, d_in] fp16 ~ N(0, 0.02^2)."""
    z = rng(seed).standard_normal((d_out, d_in), dtype=np.float32)
    return (z * np.float32(WEIGHT_STD)).astype(np.float16)


def n_outliers(d_in: int) -> int:
    return int(round(OUTLIER_FRACTION * d_in))


def make_magnitudes(seed: int, d_in: int) -> np.ndarray:
    """Per-channel magnitudes m_i (float32): lognormal(0, 0.5), 1% of channels x50."""
    g = rng(seed)
    m = np.exp(MAG_SIGMA * g.standard_normal(d_in)).astype(np.float32)
    idx = g.permutation(d_in)[: n_outliers(d_in)]
    m[idx] *= np.float32(OUTLIER_GAIN)
    return m


def make_activations(seed: int, T: int, d_in: int, dtype: str = "bf16",
                     magnitudes: Optional[np.ndarray] = None) -> np.ndarray:
    """X[T, d_in]: bf16 bits (uint16) or float16, X[t,i] = m_i * z_ti."""
    m = make_magnitudes(seed + 7, d_in) if magnitudes is None else magnitudes
    z = rng(seed).standard_normal((T, d_in), dtype=np.float32)
    x = z * m[None, :]
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return x.astype(np.float16)
    raise ValueError(dtype)


def make_correlated_activations(seed: int, T: int, d_in: int, rank: int, noise: float,
                                dtype: str = "bf16") -> np.ndarray:
    """X[T, d_in] with strongly correlated channels: a rank-`rank` mix Z M
    (Z [T, rank] ~ N(0, 1), M [rank, d_in] ~ N(0, 1) times the per-channel
    magnitudes, outliers included) plus `noise` times independent N(0, 1);
    bf16 bits (uint16) or float16."""
    g = rng(seed)
    z = g.standard_normal((T, rank), dtype=np.float32)
    m = g.standard_normal((rank, d_in), dtype=np.float32) * make_magnitudes(seed + 7, d_in)[None, :]
    x = z @ m + np.float32(noise) * g.standard_normal((T, d_in), dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return x.astype(np.float16)
    raise ValueError(dtype)


def activations_to_f32(X: np.ndarray) -> np.ndarray:
    if X.dtype == np.uint16:
        return bf16_bits_to_f32(X)
    return X.astype(np.float32)


def make_down_input(X_bits: np.ndarray, W_gate: np.ndarray, W_up: np.ndarray) -> np.ndarray:
    """bf16 bits of SiLU(X W_gate^T) * (X W_up^T), computed in fp32 (host)."""
    X = activations_to_f32(X_bits)
    g = X @ W_gate.astype(np.float32).T
    u = X @ W_up.astype(np.float32).T
    h = (g / (np.float32(1.0) + np.exp(-g))) * u
    return f32_to_bf16_bits(h.astype(np.float32))


# --------------------------------------------------------------------------
# device-side generation (torch), used where host generation would take minutes
# --------------------------------------------------------------------------
def torch_weight(seed: int, d_out: int, d_in: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = torch.randn((d_out, d_in), generator=g, device=device, dtype=torch.float32)
    return (z * WEIGHT_STD).to(torch.float16)


NORM_STD = 0.1


def make_norm(seed: int, d: int) -> np.ndarray:
    """Norm weight [d] fp16 ~ 1 + N(0, 0.1^2)."""
    return (1.0 + rng(seed).standard_normal(d, dtype=np.float32) * np.float32(NORM_STD)).astype(np.float16)


def torch_norm(seed: int, d: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return (1.0 + torch.randn(d, generator=g, device=device, dtype=torch.float32) * NORM_STD).to(torch.float16)


def torch_activations(seed: int, T: int, d_in: int, device, dtype: str = "bf16"):
    import torch
    m = torch.from_numpy(make_magnitudes(seed + 7, d_in)).to(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty((T, d_in), device=device,
                      dtype=torch.bfloat16 if dtype == "bf16" else torch.float16)
    chunk = max(1, (1 << 26) // d_in)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        z = torch.randn((t1 - t0, d_in), generator=g, device=device, dtype=torch.float32)
        out[t0:t1] = (z * m[None, :]).to(out.dtype)
    return out


def torch_down_input(X, W_gate, W_up):
    """bf16 SiLU(X W_gate^T) * (X W_up^T), fp32 math on the device (setup only)."""
    import torch
    Xf = X.float()
    out = torch.empty((X.shape[0], W_gate.shape[0]), device=X.device, dtype=torch.bfloat16)
    chunk = 2048
    Wg = W_gate.float()
    Wu = W_up.float()
    for t0 in range(0, X.shape[0], chunk):
        xs = Xf[t0:t0 + chunk]
        g = xs @ Wg.t()
        u = xs @ Wu.t()
        out[t0:t0 + chunk] = (torch.nn.functional.silu(g) * u).to(torch.bfloat16)
    return out


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Group:
    """One input-sharing group of linears: parts [rows_p, d_in], one calibration X."""
    name: str
    parts: List[int]
    d_in: int
    T: int
    x_dtype: str = "bf16"
    x_from: Optional[str] = None  # "mlp_down": X is SiLU(gate) * up of another group

    @property
    def d_out(self) -> int:
        return sum(self.parts)


@dataclasses.dataclass
class Workload:
    name: str
    groups: List[Group]
    group_sizes: Sequence[int]
    n_grid: int = 20
    score: str = "weight"  # or "output"
    n_clip: int = 0
    clip_lo: float = 0.5
    blocks: int = 1
    seed_base: int = 0

    def seed(self, block: int, group: int, tensor_id: int) -> int:
        return self.seed_base + 10 * block + 100 * group + tensor_id

    @property
    def n_weights(self) -> int:
        return self.blocks * sum(g.d_out * g.d_in for g in self.groups)


QWEN3_8B_BLOCK = [
    Group("qkv", [4096, 1024, 1024], 4096, 65536),
    Group("o", [4096], 4096, 65536),
    Group("gate_up", [12288, 12288], 4096, 65536),
    Group("down", [4096], 12288, 65536),
]

WORKLOADS = {
    "single_linear_256x512": Workload(
        "single_linear_256x512", [Group("linear", [256], 512, 64, x_dtype="f16")], [128],
        seed_base=1000),
    "q_proj_4096x4096": Workload(
        "q_proj_4096x4096", [Group("q_proj", [4096], 4096, 4096)], [128], seed_base=2000),
    "qkv_6144x4096_output": Workload(
        "qkv_6144x4096_output", [Group("qkv", [4096, 1024, 1024], 4096, 16384)], [128],
        score="output", seed_base=3000),
    "mlp_output_clip": Workload(
        "mlp_output_clip",
        [Group("gate_up", [12288, 12288], 4096, 16384),
         Group("down", [4096], 12288, 16384, x_from="mlp_down")],
        [128], score="output", n_clip=20, seed_base=4000),
    "qwen3_8b_sweep": Workload(
        "qwen3_8b_sweep", QWEN3_8B_BLOCK, [128, 64], blocks=36, seed_base=5000),
    # export of the same blocks: per-linear searches of q/k/v and gate/up, the
    # two norm folds, packing with the shared scales, o/down at RTN
    "qwen3_8b_export": Workload(
        "qwen3_8b_export", QWEN3_8B_BLOCK, [128], blocks=36, seed_base=6000),
    # decode through the packed linears of the same blocks (fused QKV and
    # gate/up as a serving engine runs them): random codes, scales and zero
    # points of the packed layout, fp16 activations of a few tokens
    "qwen3_8b_decode_w4a16": Workload(
        "qwen3_8b_decode_w4a16", QWEN3_8B_BLOCK, [128], blocks=36, seed_base=7000),
}


def qwen3_8b_linear_params() -> int:
    """Sum of the linear weights of 36 Qwen3-8B-shaped blocks."""
    w = WORKLOADS["qwen3_8b_sweep"]
    return w.n_weights


def host_group_inputs(wl: Workload, block: int, gi: int, rows_limit: Optional[int] = None,
                      T_limit: Optional[int] = None):
    """Host arrays (parts list of fp16 W, X) for one group; optionally truncated."""
    grp = wl.groups[gi]
    parts = []
    for p, rows in enumerate(grp.parts):
        W = make_weight(wl.seed(block, gi, 1 + 1000 * p), rows, grp.d_in)
        parts.append(W)
    T = grp.T if T_limit is None else min(T_limit, grp.T)
    if grp.x_from == "mlp_down":
        src = wl.groups[gi - 1]
        Xsrc = make_activations(wl.seed(block, gi - 1, 2), T, src.d_in, src.x_dtype)
        Wg = make_weight(wl.seed(block, gi - 1, 1), src.parts[0], src.d_in)
        Wu = make_weight(wl.seed(block, gi - 1, 1 + 1000), src.parts[1], src.d_in)
        X = make_down_input(Xsrc, Wg, Wu)
    else:
        X = make_activations(wl.seed(block, gi, 2), T, grp.d_in, grp.x_dtype)
    if rows_limit is not None:
        parts = [w[:rows_limit] for w in parts]
    return parts, X


