"""Seeded synthetic inputs for the SVDQuant linear layer.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark.  It holds NONE of the method's arithmetic (no smoothing, no SVD, no
quantizer, no matmul): only the random recipes that stand in for the activations
and weights of the FLUX.1 / PixArt-Sigma layers the pages evaluate on, which are
not available here.

Notation follows the SVDQuant technical review ("SVDQuant: How a Small
High-Precision Branch Makes 4-Bit Diffusion Practical", section 2.1):
X is b x m (b token rows, m input channels), W is m x n.

Conventions of every recipe (stated once so a reader can re-derive the inputs):
  * numpy ``default_rng(seed)`` (PCG64); draws happen in the order written below.
  * ``N(0, v)``: the second argument is the VARIANCE.
  * outlier channel count = round(fraction * m), picked with
    ``rng.choice(m, count, replace=False)``.
  * X is drawn in float64, rounded to float32 (round-to-nearest-even) and then to
    bfloat16 (round-to-nearest-even); the result is returned as raw bf16 bits
    (uint16) and as the float32 value of those bits.
  * W is drawn in float64 and rounded to float32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = ["LayerConfig", "CONFIGS", "make_inputs", "bf16_bits_of", "bf16_bits_to_f32"]


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    b: int
    m: int
    n: int
    rank: int            # SVD rank of the protected branch
    lora_rank: int       # 0 = no adapter
    x_recipe: str        # "gauss" | "laplace_tail" | "gelu"
    x_outlier_frac: float
    x_outlier_count: Optional[int]  # explicit count overrides the fraction
    x_outlier_gain: float
    w_outlier_rows: str  # "none" | "independent" | "same_as_x"
    w_outlier_count: int
    w_outlier_gain: float
    rows: Optional[int] = None   # keep only the first `rows` rows of X
    description: str = ""

    @property
    def total_rank(self) -> int:
        return self.rank + self.lora_rank


CONFIGS = {
    "tiny": LayerConfig(
        "tiny", 64, 256, 256, 16, 0, "gauss", 0.0, 4, 50.0, "independent", 4, 10.0,
        description="Tiny SVDQuant linear, b=64 m=256 n=256, rank 16"),
    "pixart_fc1": LayerConfig(
        "pixart_fc1", 4096, 1152, 4608, 32, 0, "laplace_tail", 0.01, None, 30.0, "none", 0, 1.0,
        description="PixArt-Sigma-shaped MLP fc1 (1024px latent, 4096 tokens), rank 32"),
    "flux_qkv": LayerConfig(
        "flux_qkv", 4608, 3072, 9216, 32, 0, "gauss", 0.005, None, 50.0, "same_as_x", 0, 8.0,
        description="FLUX-shaped fused QKV (4096 image + 512 text tokens), rank 32"),
    "flux_fc2": LayerConfig(
        "flux_fc2", 4608, 12288, 3072, 32, 0, "gelu", 0.005, None, 40.0, "none", 0, 1.0,
        description="FLUX-shaped MLP fc2 (K-heavy, post-GELU input), rank 32"),
    "flux_single_fc": LayerConfig(
        "flux_single_fc", 4608, 3072, 21504, 32, 16, "gauss", 0.005, None, 50.0, "same_as_x", 0, 8.0,
        description="FLUX-shaped single-block fused projection, rank 32 + LoRA 16 = 48"),
    "flux_single_out": LayerConfig(
        "flux_single_out", 4608, 15360, 3072, 32, 16, "gelu", 0.005, None, 40.0, "none", 0, 1.0,
        description="FLUX-shaped single-block output projection, rank 32 + LoRA 16 = 48"),
    "flux_single_fc_b256": LayerConfig(
        "flux_single_fc_b256", 4608, 3072, 21504, 32, 16, "gauss", 0.005, None, 50.0, "same_as_x", 0, 8.0,
        rows=256, description="first 256 rows of flux_single_fc (memory-bound variant)"),
    "flux_single_out_b256": LayerConfig(
        "flux_single_out_b256", 4608, 15360, 3072, 32, 16, "gelu", 0.005, None, 40.0, "none", 0, 1.0,
        rows=256, description="first 256 rows of flux_single_out (memory-bound variant)"),
}


def _f64_to_f32_rne(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def bf16_bits_of(a32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return raw uint16 bits.

    Input-recipe helper only (turns a float32 draw into a bf16 tensor); NaN is
    not produced by any recipe.
    """
    u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _gelu_erf(z: np.ndarray) -> np.ndarray:
    from scipy.special import erf
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def make_inputs(cfg: "LayerConfig | str", seed: int = 0, rows: Optional[int] = None,
                with_w: bool = True) -> dict:
    """Draw one layer's synthetic X (bf16), W (fp32) and, if configured, LoRA A, B.

    Returns a dict with keys: ``x_bits`` (uint16 [b][m]), ``x`` (float32 values of
    x_bits), ``w`` (float32 [m][n]) unless ``with_w`` is False, ``lora_a``
    (float32 [m][k]) / ``lora_b`` (float32 [k][n]) / ``lora_scale`` when the
    config carries an adapter, plus ``cfg`` and the outlier index sets.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    rng = np.random.default_rng(seed)
    b, m, n = cfg.b, cfg.m, cfg.n

    # --- activations -------------------------------------------------------
    z = rng.standard_normal((b, m))
    if cfg.x_recipe == "gelu":
        z = _gelu_erf(z)
    cnt = cfg.x_outlier_count if cfg.x_outlier_count is not None else int(round(cfg.x_outlier_frac * m))
    x_ch = np.sort(rng.choice(m, cnt, replace=False)) if cnt > 0 else np.zeros(0, dtype=np.int64)
    if cfg.x_recipe == "laplace_tail" and cnt > 0:
        # unit-variance Laplace(0, 1/sqrt(2)) replaces the chosen channels
        z[:, x_ch] = rng.laplace(0.0, 1.0 / math.sqrt(2.0), size=(b, cnt))
    if cnt > 0:
        z[:, x_ch] *= cfg.x_outlier_gain
    keep = rows if rows is not None else cfg.rows
    if keep is not None:
        z = z[:keep]
    x32 = _f64_to_f32_rne(z)
    x_bits = bf16_bits_of(x32)
    out = {"cfg": cfg, "x_bits": x_bits, "x": bf16_bits_to_f32(x_bits), "x_outlier_channels": x_ch}

    # --- weights -----------------------------------------------------------
    w = rng.standard_normal((m, n)) / math.sqrt(m) if with_w else None
    if cfg.w_outlier_rows == "independent":
        w_rows = np.sort(rng.choice(m, cfg.w_outlier_count, replace=False))
    elif cfg.w_outlier_rows == "same_as_x":
        w_rows = x_ch
    else:
        w_rows = np.zeros(0, dtype=np.int64)
    if with_w:
        if len(w_rows):
            w[w_rows, :] *= cfg.w_outlier_gain
        out["w"] = _f64_to_f32_rne(w)
        del w
    out["w_outlier_rows"] = w_rows

    # --- adapter -----------------------------------------------------------
    if cfg.lora_rank > 0:
        k = cfg.lora_rank
        out["lora_a"] = _f64_to_f32_rne(rng.standard_normal((m, k)) * math.sqrt(0.02))
        out["lora_b"] = _f64_to_f32_rne(rng.standard_normal((k, n)) * math.sqrt(0.02))
        out["lora_scale"] = 1.0
    return out


def random_bf16_bits(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    """Gaussian bf16 tensor (raw bits) for small ad-hoc parity cases."""
    return bf16_bits_of(_f64_to_f32_rne(rng.standard_normal(shape) * scale))
