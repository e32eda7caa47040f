"""Seeded synthetic inputs for the Walsh-Hadamard adapter (WHA) path.

This module is the ONLY code shared by the CPU oracle (``oracle/``) and the HIP
path (``quantization_aware_sparse_amd``). It holds none of the adapter's own
arithmetic: it draws weights and activations, applies the upstream quantizer
that produces the adapter's input (the quantization error), and rounds to the
activation dtype. Everything the adapter computes from there on lives on the
two sides separately.

Workloads follow the layer shapes of LLaMA/Mistral-class projections named in
the QWHA pages (papernotes.org notes, 实验关键数据 › 主实验: LLaMA-3.1-8B,
LLaMA-3.2-3B, Mistral-7B) at the adapter budget P(r=64) (same notes, 损失函数 /
训练策略), with Gaussian weights plus injected outliers standing in for the
heavy-tailed quantization error the notes describe (研究背景与动机 › 切入角度).
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "LayerSpec",
    "Layer",
    "CONFIGS",
    "config_specs",
    "make_layer",
    "make_activations",
    "make_calibration",
    "rtn_quantize",
    "rtn_codes",
    "pack_codes",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "round_to_bf16",
]


# --------------------------------------------------------------------------
# bf16 helpers (round-to-nearest-even on the fp32 bit pattern)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs are finite (NaN/Inf are never generated here)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16, returned as fp32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


# --------------------------------------------------------------------------
# Workload description
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """One synthetic quantized linear layer plus its activation batch."""

    name: str
    d_out: int
    d_in: int
    outlier_frac: float       # fraction of W0 entries turned into outliers
    outlier_mult: float       # outlier multiplier
    bits: int                 # RTN bit width
    group: int                # RTN group size along d_in
    p: int                    # adapter budget (number of nonzeros of F)
    T: int                    # tokens in the activation batch
    act: str                  # "f32" or "bf16"
    seed_key: int = 0         # distinguishes layers that share one seed


def _lora_budget(d_out: int, d_in: int, r: int = 64) -> int:
    # P(r=64): the parameter count of a rank-64 LoRA on this shape.
    return r * (d_out + d_in)


# The five workloads. c1 is the small case the oracle finishes in seconds;
# c2 is the 4096x4096 q_proj-shaped layer the throughput is quoted on.
CONFIGS: Dict[str, List[LayerSpec]] = {
    "c1": [LayerSpec("c1", 256, 256, 0.005, 20.0, 4, 64, 2048, 64, "f32")],
    "c2": [LayerSpec("c2", 4096, 4096, 0.001, 20.0, 4, 128,
                     _lora_budget(4096, 4096), 8192, "bf16")],
    "c3": [LayerSpec("c3", 14336, 4096, 0.001, 20.0, 3, 128,
                     _lora_budget(14336, 4096), 8192, "bf16")],
    "c4": [LayerSpec("c4", 8192, 8192, 0.001, 30.0, 2, 64, 1048576, 16384,
                     "bf16")],
    # GQA attention block at hidden 4096: q/o 4096x4096, k/v 1024x4096.
    # q, k, v consume the same x; o consumes its own x (the attention output).
    "c5": [
        LayerSpec("c5.q", 4096, 4096, 0.001, 20.0, 4, 128,
                  _lora_budget(4096, 4096), 32768, "bf16", seed_key=1),
        LayerSpec("c5.k", 1024, 4096, 0.001, 20.0, 4, 128,
                  _lora_budget(1024, 4096), 32768, "bf16", seed_key=2),
        LayerSpec("c5.v", 1024, 4096, 0.001, 20.0, 4, 128,
                  _lora_budget(1024, 4096), 32768, "bf16", seed_key=3),
        LayerSpec("c5.o", 4096, 4096, 0.001, 20.0, 4, 128,
                  _lora_budget(4096, 4096), 32768, "bf16", seed_key=4),
    ],
    # Not one of the five measured workloads: the down_proj shape of the same
    # models, whose input width 14336 = 7 * 2048 is not a power of two
    # (block-diagonal transform).
    "down": [LayerSpec("down", 4096, 14336, 0.001, 20.0, 4, 128,
                       _lora_budget(4096, 14336), 8192, "bf16", seed_key=6)],
}

# Which activation stream each c5 projection reads: q/k/v share one.
C5_X_STREAM = {"c5.q": 0, "c5.k": 0, "c5.v": 0, "c5.o": 1}


def config_specs(name: str) -> List[LayerSpec]:
    return CONFIGS[name]


# --------------------------------------------------------------------------
# Upstream quantizer (produces the adapter's input, the quantization error)
# --------------------------------------------------------------------------

def _rtn_parts(w0: np.ndarray, bits: int, group: int):
    d_out, d_in = w0.shape
    assert d_in % group == 0
    w = w0.astype(np.float32).reshape(d_out, d_in // group, group)
    mn = w.min(axis=2, keepdims=True)
    mx = w.max(axis=2, keepdims=True)
    qmax = np.float32(2 ** bits - 1)
    s = ((mx - mn) / qmax).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    half = np.float32(0.5)
    z = np.floor(-mn / safe + half).astype(np.float32)
    q = np.clip(np.floor(w / safe + half) + z, np.float32(0), qmax)
    return w, s, safe, z, q


def rtn_codes(w0: np.ndarray, bits: int, group: int):
    """The same quantizer in integer form: codes q (uint8 [d_out][d_in]) and
    per-group scale s and zero z (fp32 [d_out][d_in/group], z integer-valued)
    with W_Q = (q - z) * s in fp32, exactly what rtn_quantize returns.
    Groups of equal values (s = 0) are not representable and raise."""
    d_out, d_in = w0.shape
    w, s, safe, z, q = _rtn_parts(w0, bits, group)
    if not np.all(s > 0):
        raise ValueError("constant quantization group")
    return (q.reshape(d_out, d_in).astype(np.uint8), safe[..., 0].astype(np.float32),
            z[..., 0].astype(np.float32))


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Storage of b-bit codes: each uint32 word holds floor(32/b) codes of a
    row, code j in word j // cpw at bits (j % cpw) * b (least significant
    first); rows padded to whole words with zero codes."""
    d_out, d_in = q.shape
    cpw = 32 // bits
    nw = -(-d_in // cpw)
    words = np.zeros((d_out, nw), dtype=np.uint64)
    j = np.arange(d_in)
    sh = ((j % cpw) * bits).astype(np.uint64)
    for col in range(d_in):
        words[:, col // cpw] |= q[:, col].astype(np.uint64) << sh[col]
    return words.astype(np.uint32)


def rtn_quantize(w0: np.ndarray, bits: int, group: int) -> np.ndarray:
    """Asymmetric min/max round-to-nearest quantization along d_in, fp32.

    Per group of ``group`` consecutive input columns:
      s = (max - min) / (2^b - 1), z = floor(-min/s + 1/2),
      q = clip(floor(w/s + 1/2) + z, 0, 2^b - 1), W_Q = (q - z) * s.
    Rounding is half-up so the in-range error lies in [-s/2, s/2), the
    half-open interval the QWHA notes give (研究背景与动机 › 切入角度).
    Returns W_Q (fp32, same shape)."""
    d_out, d_in = w0.shape
    w, s, safe, z, q = _rtn_parts(w0, bits, group)
    wq = ((q - z) * safe).astype(np.float32)
    wq = np.where(s > 0, wq, w).astype(np.float32)
    return wq.reshape(d_out, d_in)


# --------------------------------------------------------------------------
# Generators
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Layer:
    spec: LayerSpec
    w0: np.ndarray     # fp32 [d_out][d_in]
    wq: np.ndarray     # fp32 [d_out][d_in]
    dwq: np.ndarray    # fp32 [d_out][d_in], W0 - W_Q


def _children(seed: int, key: int, n: int) -> List[np.random.SeedSequence]:
    return np.random.SeedSequence([int(seed), int(key)]).spawn(n)


def make_layer(spec: LayerSpec, seed: int = 0) -> Layer:
    """W0 ~ fp32(0.02 N(0,1)), outliers at seeded distinct positions scaled by
    ``outlier_mult``, RTN quantized; returns W0, W_Q and dW_Q = W0 - W_Q."""
    ss_w, ss_pos, _, _ = _children(seed, spec.seed_key, 4)
    rng_w = np.random.Generator(np.random.PCG64(ss_w))
    w0 = rng_w.standard_normal((spec.d_out, spec.d_in), dtype=np.float32)
    w0 *= np.float32(0.02)
    k = int(np.floor(spec.outlier_frac * spec.d_out * spec.d_in))
    if k > 0:
        rng_p = np.random.Generator(np.random.PCG64(ss_pos))
        pos = rng_p.choice(spec.d_out * spec.d_in, size=k, replace=False)
        flat = w0.reshape(-1)
        flat[pos] = flat[pos] * np.float32(spec.outlier_mult)
    wq = rtn_quantize(w0, spec.bits, spec.group)
    dwq = (w0 - wq).astype(np.float32)
    return Layer(spec, w0, wq, dwq)


def _draw(ss: np.random.SeedSequence, shape, act: str) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(ss))
    a = rng.standard_normal(shape, dtype=np.float32)
    if act == "bf16":
        return f32_to_bf16_bits(a)
    assert act == "f32"
    return a


def make_activations(spec: LayerSpec, seed: int = 0, T: Optional[int] = None,
                     x_stream: Optional[int] = None):
    """Activations x [T][d_in] and upstream gradient dy [T][d_out], N(0,1).

    bf16 layers return uint16 bit patterns (round-to-nearest-even), fp32
    layers return float32. ``x_stream`` lets several layers share one x
    (q/k/v of the attention block)."""
    T = spec.T if T is None else T
    _, _, ss_x, ss_dy = _children(seed, spec.seed_key, 4)
    if x_stream is not None:
        ss_x = np.random.SeedSequence([int(seed), 1000 + int(x_stream)])
    x = _draw(ss_x, (T, spec.d_in), spec.act)
    dy = _draw(ss_dy, (T, spec.d_out), spec.act)
    return x, dy


def make_calibration(d_in: int, N: int, seed: int = 0, act: str = "bf16",
                     outlier_channels: float = 0.005, outlier_mult: float = 10.0,
                     channel_spread: float = 0.5) -> np.ndarray:
    """Calibration activations X [N][d_in], the stand-in for the WikiText-2
    tokens the init is calibrated on: N(0,1) entries times a per-channel
    scale exp(channel_spread * N(0,1)), with a seeded `outlier_channels`
    fraction of channels (at least one) scaled by `outlier_mult` -- the
    channel-wise outliers of LLM activations. bf16 as uint16 bit patterns
    (round-to-nearest-even) or float32."""
    ss_s, ss_o, ss_x = np.random.SeedSequence([int(seed), 2000, int(d_in)]).spawn(3)
    scale = np.exp(channel_spread * np.random.default_rng(ss_s).standard_normal(d_in))
    n_out = max(1, int(round(outlier_channels * d_in)))
    idx = np.random.default_rng(ss_o).choice(d_in, size=min(n_out, d_in), replace=False)
    scale[idx] *= outlier_mult
    x = np.random.default_rng(ss_x).standard_normal((N, d_in)) * scale
    x = x.astype(np.float32)
    return f32_to_bf16_bits(x) if act == "bf16" else x


def act_to_f64(a: np.ndarray) -> np.ndarray:
    """Activation array (bf16 bits or fp32) -> exact float64 values."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)
