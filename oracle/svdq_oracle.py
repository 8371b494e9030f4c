"""CPU oracle of the SVDQuant linear layer.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything under ``oracle/``.  The product
(the C-ABI library and its Python binding) never does, and this module imports
nothing from the product.

What it is: a plain, slow, readable restatement of the method in numpy, in
float64 except at the rounding points the method fixes in float32 / fp16 / bf16.
Sources, cited by section and equation:

  [Review]  "SVDQuant: How a Small High-Precision Branch Makes 4-Bit Diffusion
            Practical" (Zhou's technical review of arXiv:2411.05007v4):
            sec. 2.2 Eq.(1) quantizer; sec. 3.1 Eq.(3)-(4) smoothing;
            sec. 4.1 Eq.(5)-(6) error split and bound; sec. 4.2 Eq.(7)-(8)
            two-branch output; sec. 4.3 Eq.(9) residual bound; sec. 5 Eq.(10)
            and Algorithm 1 (protected-layer construction); sec. 6.1 Eq.(11)
            and Algorithm 2 (fused execution); sec. 6.2 Eq.(12); sec. 7 Eq.(13)
            LoRA; sec. 8 (INT4: group 64 on both operands, 16-bit scales).
  [Nunchaku article] "SVDQuant: 4-bit Quantization Enables Efficient Diffusion
            Model Inference on Consumer GPUs", section "Nunchaku": two 4-bit
            values per byte.

Readings taken where the pages are silent:
  R1  ties in round() go to even (IEEE default).
  R2  codes are emitted in [-7, 7]: the review's symmetric grid (sec. 2.2).
  R3  16-bit scale = fp16(fl32(amax / 7)), saturated at 65504.
  R4  a group whose fp16 scale is 0 (all-zero or underflowing group) gets code 0
      everywhere (sec. 2.2 sets the all-zero group aside without defining it).
  R5  lambda_k = 1 where the activation or weight statistic of channel k is 0
      (sec. 3.1 declines to pick a safeguard).
  R6  the smoothing scale multiplies W on the left, W~ = diag(lambda) W (sec. 3.1
      notes the paper's W diag(lambda) is dimensionally inconsistent).
  R7  X~ = X diag(lambda)^-1 is computed as x * fl32(1/lambda32) in float32 and
      materialised once as bf16; both branches use that bf16 X~ (Algorithm 2
      steps 1-3 read one 16-bit smoothed tile and feed it to both branches).
  R8  Sigma goes into L1 (Eq.10); the stored factors are bf16; the residual
      R = W~ - L1 L2 uses the STORED (rounded) factors, so W~ = L1 L2 + R holds
      exactly with respect to what runs.
  R9  the up-projection operand Z is rounded to bf16 before Z L2 (the branch is
      a bf16 matrix product).
  R10 the LoRA scale is absorbed into B (sec. 7 allows either factor).
  R11 quantization groups run along the input channels for both operands
      (sec. 8: group quantization on both operands, group 64).
  R16 the candidate-selection score of Algorithm 1 step 8 is the relative
      Frobenius error of the quantized layer's output against X W (float64) on
      the calibration rows.
  R19 the 8-bit setting (sec. 8: rank 16, dynamic per-token activation and
      per-channel weight quantization) uses the same symmetric round-to-nearest
      quantizer as INT4 with 127 in place of 7: codes in [-127, 127], 16-bit
      (fp16) scales fp16(fl32(amax / 127)) over a whole row of X~ (per token)
      or a whole column of R (per output channel).
  R20 the NVFP4 setting (sec. 8: group size 16 with FP8 scales; sec. 2.2 notes
      FP4's nonuniform grid): element codes are FP4 E2M1 (values 0, 0.5, 1,
      1.5, 2, 3, 4, 6; sign bit 3), block scales FP8 E4M3 (bias 7, largest
      finite 448, subnormal quantum 2^-9), one per 16 consecutive input
      channels of a row of X~ or of a column of R, and one power-of-two fp32
      scale t per tensor that places the block scales in E4M3's range:
      t = 2^ceil(log2(A / (6 * 448))) with A the tensor's largest magnitude
      (for X~, its calibration maximum; t = 1 without calibration).  Per block
      sb = E4M3_RNE_sat(fl32(amax / 6) / t) and S = sb * t; codes are
      E2M1_RNE_sat(fl32(v / S)) with ties to the even code and the sign of the
      quotient (so -0 is code 8); sb = 0 gives codes 0.  The product is
      Y = t_x t_w (X^ W^) + bf16(Z) L2 (+ bias), X^ and W^ the dequantized
      codes (exact), the rank-r branch as for INT4 (the 4-bit setting's rank
      32).
  R17 the optional factor update of step 6 refits rank-r SVD factors to
      W~ - Q(R) (Q(R) dequantized exactly); the residual of step 7 is then
      formed and quantized again; of equal scores the first candidate
      (migration strengths in the order given, then refinement steps) wins.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

GROUP = 64
QMAX = 7           # [Review] sec. 2.2: symmetric INT4 grid spans -7..7
FP16_MAX = 65504.0

# --------------------------------------------------------------------------
# Rounding primitives (the method's fixed rounding points).
# --------------------------------------------------------------------------


def f32(a) -> np.ndarray:
    """Round to IEEE float32, nearest-even."""
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_from_f32(a32) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32.

    bf16 keeps the top 16 bits of the float32 encoding; rounding adds
    0x7FFF + (bit 16) before truncating, the usual integer form of RNE.
    """
    u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return u.astype(np.uint32).view(np.float32)


def bf16_bits_from_f32(a32) -> np.ndarray:
    return (bf16_from_f32(a32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_from_f64(a) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even) in ONE rounding, as float32.

    bf16 has 8 significant bits and the float32 exponent range; the grid
    spacing for |x| in [2^e, 2^(e+1)) is 2^(e-7), never below 2^-133.
    """
    a = np.asarray(a, dtype=np.float64)
    out = np.zeros_like(a)
    nz = a != 0
    e = np.floor(np.log2(np.abs(a[nz])))
    # guard the log2 floor against off-by-one at exact powers of two
    av = np.abs(a[nz])
    e = np.where(2.0 ** e > av, e - 1, e)
    e = np.where(2.0 ** (e + 1) <= av, e + 1, e)
    q = 2.0 ** (np.maximum(e, -126.0) - 7.0)
    out[nz] = np.rint(a[nz] / q) * q     # a/q is exact (power-of-two scaling)
    big = np.abs(out) > 3.3895313892515355e38   # beyond the largest finite bf16
    out[big] = np.sign(out[big]) * np.inf
    return out.astype(np.float32)


def fp16_from_f32_sat(a32) -> np.ndarray:
    """float32 -> nearest fp16 (ties to even), saturated at +-65504 (reading R3).

    Returned as float32 holding the fp16 value.
    """
    a32 = np.asarray(a32, dtype=np.float32)
    with np.errstate(over="ignore"):
        h = a32.astype(np.float16)
    h = np.where(np.isinf(h) & np.isfinite(a32), np.sign(a32) * np.float16(FP16_MAX), h)
    return h.astype(np.float32)


# --------------------------------------------------------------------------
# Quantizer: [Review] sec. 2.2, Eq.(1)  s = max|Z| / 7,  Q(Z) = s * round(Z / s)
# --------------------------------------------------------------------------


def quantize_groups(v32: np.ndarray, group: int = GROUP):
    """Symmetric per-group INT4 round-to-nearest along the LAST axis.

    v32: float32 array [..., K] with K % group == 0.
    Returns (codes int8 [..., K] in [-7, 7], scales float32 [..., K/group]
    holding fp16 values).

    Steps per group (Eq.1 with readings R1-R4):
      amax = max|v| (exact);  s = fp16(fl32(amax / 7));
      q = clamp(round_half_even(fl32(v / s)), -7, 7);  q = 0 where s == 0.
    """
    v32 = np.asarray(v32, dtype=np.float32)
    K = v32.shape[-1]
    assert K % group == 0
    g = v32.reshape(v32.shape[:-1] + (K // group, group))
    amax = np.max(np.abs(g), axis=-1)                      # exact in float32
    s = fp16_from_f32_sat(np.float32(amax) / np.float32(QMAX))   # fl32 divide, then fp16
    s_b = s[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = np.where(s_b > 0, g / np.where(s_b > 0, s_b, np.float32(1)), np.float32(0))
    quot = quot.astype(np.float32)                         # fl32(v / s)
    q = np.clip(np.rint(quot), -QMAX, QMAX)                # rint: ties to even
    q = np.where(s_b > 0, q, 0).astype(np.int8)
    return q.reshape(v32.shape), s.astype(np.float32)


def dequantize_groups(codes: np.ndarray, scales: np.ndarray, group: int = GROUP) -> np.ndarray:
    """Q(v) = s * q, in float64 (exact: a 4-bit integer times an fp16 value)."""
    K = codes.shape[-1]
    c = codes.astype(np.float64).reshape(codes.shape[:-1] + (K // group, group))
    return (c * scales.astype(np.float64)[..., None]).reshape(codes.shape)


# --------------------------------------------------------------------------
# Calibration and smoothing: [Review] sec. 3.1, Eq.(3)-(4)
# --------------------------------------------------------------------------


def act_amax(x32: np.ndarray) -> np.ndarray:
    """Calibration statistic a_k = max_i |X_ik| (exact), float32 [m]."""
    return np.max(np.abs(np.asarray(x32, dtype=np.float32)), axis=0)


def smoothing_lambda(a: np.ndarray, w32: np.ndarray, alpha: float = 0.5):
    """lambda_k = a_k^alpha / w_k^(1-alpha), w_k = max_j |W_kj|  (Eq.4).

    Computed in float64; lambda_k = 1 where a_k or w_k is 0 (reading R5).
    Returns (lam64, lam32, inv32) with lam32 = fl32(lam64) and
    inv32 = fl32(1 / lam32) (the smoothing multiply of reading R7).
    """
    a = np.asarray(a, dtype=np.float64)
    wmax = np.max(np.abs(np.asarray(w32, dtype=np.float64)), axis=1)
    ok = (a > 0) & (wmax > 0)
    lam = np.ones_like(a)
    lam[ok] = np.power(a[ok], alpha) / np.power(wmax[ok], 1.0 - alpha)
    lam32 = lam.astype(np.float32)
    inv32 = (1.0 / lam32.astype(np.float64)).astype(np.float32)
    return lam, lam32, inv32


def smooth_weight(w32: np.ndarray, lam32: np.ndarray) -> np.ndarray:
    """W~ = diag(lambda) W in float64 (Eq.3, reading R6); products are exact."""
    return np.asarray(w32, dtype=np.float64) * lam32.astype(np.float64)[:, None]


def smooth_activation(x32: np.ndarray, inv32: Optional[np.ndarray]) -> np.ndarray:
    """X~ = bf16(fl32(x * inv32))  (Eq.3 with reading R7); None = no smoothing."""
    x32 = np.asarray(x32, dtype=np.float32)
    if inv32 is None:
        return bf16_from_f32(x32)
    return bf16_from_f32(x32 * np.asarray(inv32, dtype=np.float32)[None, :])


# --------------------------------------------------------------------------
# Low-rank decomposition: [Review] sec. 5, Eq.(10), Algorithm 1 steps 3-5
# --------------------------------------------------------------------------


def truncated_svd(wt: np.ndarray, rank: int, method: str = "lapack"):
    """L1 = U_r Sigma_r, L2 = V_r^T of the smoothed weight (Eq.10), float64.

    method "lapack": numpy's full SVD, the textbook routine (returns every
    singular value).  method "arpack": scipy's truncated SVD (ARPACK, tol 0)
    for large layers; returns only the top `rank` singular values.  Sign
    convention for reproducible dumps: the largest-magnitude entry of each U
    column is made positive (a sign flip of a singular pair leaves L1 L2
    unchanged).  Returns (L1 [m][r], L2 [r][n], sigma).
    """
    if method == "arpack" and 0 < rank < min(wt.shape) - 1:
        from scipy.sparse.linalg import svds
        U, S, Vt = svds(wt, k=rank, tol=0, random_state=0)
        order = np.argsort(S)[::-1]
        U, S, Vt = U[:, order], S[order], Vt[order]
    else:
        U, S, Vt = np.linalg.svd(wt, full_matrices=False)
    U = U[:, :rank].copy()
    Vt = Vt[:rank].copy()
    if rank:
        idx = np.argmax(np.abs(U), axis=0)
        sgn = np.sign(U[idx, np.arange(rank)])
        sgn[sgn == 0] = 1
        U *= sgn[None, :]
        Vt *= sgn[:, None]
    return U * S[None, :rank], Vt, S


def residual(wt: np.ndarray, l1b: np.ndarray, l2b: np.ndarray) -> np.ndarray:
    """R = W~ - L1 L2 with the stored bf16 factors, in float64 (reading R8)."""
    return np.asarray(wt, dtype=np.float64) - l1b.astype(np.float64) @ l2b.astype(np.float64)


def quantize_weight_residual(r32: np.ndarray, group: int = GROUP):
    """INT4 group quantization of the residual (Algorithm 1 step 5).

    r32: float32 [m][n].  Groups of 64 consecutive rows k per column j
    (reading R11).  Returns (codes int8 [m][n], scales float32 [m/64][n]).
    """
    codes_t, s_t = quantize_groups(np.ascontiguousarray(np.asarray(r32, np.float32).T), group)
    return np.ascontiguousarray(codes_t.T), np.ascontiguousarray(s_t.T)


def prepare_weights(w32: np.ndarray, a: Optional[np.ndarray], rank: int,
                    group: int = GROUP, alpha: float = 0.5, svd: str = "lapack") -> dict:
    """Offline preparation of one protected layer (Algorithm 1 steps 2-5, 9).

    w32: float32 [m][n]; a: float32 [m] calibration maxima, or None (no smoothing).
    Returns a dict with lam32, inv32, wt (float64 W~), l1 (float32 holding bf16,
    [m][r]), l2 ([r][n]), r32 (float32 residual), qw (int8 codes [m][n]),
    sw (fp16 values as float32 [m/64][n]), sigma.
    """
    w32 = np.asarray(w32, dtype=np.float32)
    m, n = w32.shape
    if a is None:
        lam32 = np.ones(m, np.float32)
        inv32 = None
    else:
        _, lam32, inv32 = smoothing_lambda(a, w32, alpha)
    wt = smooth_weight(w32, lam32)
    l1, l2, sigma = truncated_svd(wt, rank, svd)
    l1b = bf16_from_f64(l1)
    l2b = bf16_from_f64(l2)
    r64 = residual(wt, l1b, l2b)
    r32 = r64.astype(np.float32)
    qw, sw = quantize_weight_residual(r32, group)
    return {"lam32": lam32, "inv32": inv32, "wt": wt, "l1": l1b, "l2": l2b,
            "r64": r64, "r32": r32, "qw": qw, "sw": sw, "sigma": sigma,
            "rank": rank, "group": group, "alpha": alpha}


def dequantize_weight_residual(qw: np.ndarray, sw: np.ndarray, group: int = GROUP) -> np.ndarray:
    """Q(R) = s q in float64 (exact), from codes [m][n] and scales [m/64][n]."""
    return np.asarray(qw, np.float64) * np.repeat(np.asarray(sw, np.float64), group, axis=0)


def refit_factors(layer: dict, group: int = GROUP, svd: str = "lapack") -> dict:
    """Algorithm 1 steps 6-7: the factors are fitted again to what the quantized
    residual leaves out, L1 L2 <- SVD_r(W~ - Q(R)), and the residual is formed
    and quantized again from the new (bf16) factors."""
    rank = layer["rank"]
    if rank == 0:
        return dict(layer)
    target = layer["wt"] - dequantize_weight_residual(layer["qw"], layer["sw"], group)
    l1, l2, sigma = truncated_svd(target, rank, svd)
    l1b, l2b = bf16_from_f64(l1), bf16_from_f64(l2)
    r64 = residual(layer["wt"], l1b, l2b)
    r32 = r64.astype(np.float32)
    qw, sw = quantize_weight_residual(r32, group)
    return dict(layer, l1=l1b, l2=l2b, r64=r64, r32=r32, qw=qw, sw=sw, sigma=sigma)


def layer_output_error(x32: np.ndarray, w32: np.ndarray, layer: dict, group: int = GROUP) -> float:
    """Algorithm 1 step 8's criterion: ||Y(X) - X W||_F / ||X W||_F with Y the
    quantized layer (``linear``) on calibration rows X and X W in float64."""
    yref = np.asarray(x32, np.float64) @ np.asarray(w32, np.float64)
    y = linear(x32, layer, group=group)["y"]
    return float(np.linalg.norm(y - yref) / np.linalg.norm(yref))


def refine_weights(w32: np.ndarray, a: Optional[np.ndarray], x_cal32: np.ndarray, rank: int,
                   alphas=(0.5,), iters: int = 0, group: int = GROUP, svd: str = "lapack") -> dict:
    """Algorithm 1 steps 2-8: for each migration strength the layer is built
    (steps 2-5) and its factors refitted `iters` times (steps 6-7); every
    candidate is scored by ``layer_output_error`` on the calibration rows and
    the first one with the lowest error is kept (step 8).

    Returns the chosen layer dict with added keys alpha, iteration, rel_err and
    candidates (a list of (alpha, iteration, rel_err) in evaluation order)."""
    best, cands = None, []
    for alpha in alphas:
        lay = prepare_weights(w32, a, rank, group, float(np.float32(alpha)), svd)
        for it in range(iters + 1):
            err = layer_output_error(x_cal32, w32, lay, group)
            cands.append((float(np.float32(alpha)), it, err))
            if best is None or err < best[2]:
                best = (lay, it, err)
            if it == iters or rank == 0:
                break
            lay = refit_factors(lay, group, svd)
    out = dict(best[0], iteration=best[1], rel_err=best[2], candidates=cands)
    return out


def append_lora(l1b: np.ndarray, l2b: np.ndarray, lam32: Optional[np.ndarray],
                lora_a: np.ndarray, lora_b: np.ndarray, scale: float):
    """Widen the protected branch with an adapter W += scale * A B  (Eq.13).

    In smoothed coordinates the adapter becomes (D A) B (sec. 7), so
    L1' = [L1 | bf16(diag(lambda) A)], L2' = [L2 ; bf16(scale * B)] (reading
    R10); the quantized residual is untouched.
    """
    a64 = np.asarray(lora_a, dtype=np.float64)
    if lam32 is not None:
        a64 = a64 * np.asarray(lam32, dtype=np.float64)[:, None]
    b64 = float(scale) * np.asarray(lora_b, dtype=np.float64)
    return (np.concatenate([l1b, bf16_from_f64(a64)], axis=1),
            np.concatenate([l2b, bf16_from_f64(b64)], axis=0))


# --------------------------------------------------------------------------
# Runtime: [Review] sec. 4.2 Eq.(7) and sec. 6.1 Algorithm 2
# --------------------------------------------------------------------------


def quantize_activation(x32: np.ndarray, inv32: Optional[np.ndarray], group: int = GROUP):
    """Algorithm 2 steps 1 and 3: smooth, round to bf16, group-quantize per row.

    Returns (xt float32 [b][m] bf16 values, qx int8 [b][m], sx float32 [b][m/64]).
    """
    xt = smooth_activation(x32, inv32)
    qx, sx = quantize_groups(xt, group)
    return xt, qx, sx


def lowrank_down(xt: np.ndarray, l1b: np.ndarray) -> np.ndarray:
    """Algorithm 2 step 2: Z = X~ L1, accumulated in float64."""
    return np.asarray(xt, dtype=np.float64) @ np.asarray(l1b, dtype=np.float64)


def group_isums(qx: np.ndarray, qw: np.ndarray, group: int = GROUP) -> np.ndarray:
    """isum[i, j, g] = sum_{k in group g} qx[i, k] * qw[k, j], exact int64.

    Brute-force reference for small shapes (sum of integer products)."""
    b, m = qx.shape
    G = m // group
    out = np.zeros((b, qw.shape[1], G), dtype=np.int64)
    for g in range(G):
        ks = slice(g * group, (g + 1) * group)
        out[:, :, g] = qx[:, ks].astype(np.int64) @ qw[ks, :].astype(np.int64)
    return out


def gemm_main(qx, sx, qw, sw, group: int = GROUP) -> np.ndarray:
    """Low-bit main branch Q(X~) Q(R) = sum_g sx[i,g] sw[g,j] isum[i,j,g]  (Eq.7).

    Evaluated as one float64 product of the dequantized matrices; every
    dequantized entry is exact in float64.
    """
    xq = dequantize_groups(qx, sx, group)                          # [b][m]
    wq = dequantize_groups(np.ascontiguousarray(qw.T), np.ascontiguousarray(sw.T), group).T
    return xq @ wq


def lowrank_up(z64: np.ndarray, l2b: np.ndarray) -> np.ndarray:
    """Algorithm 2 step 6: bf16(Z) L2 in float64 (reading R9)."""
    return bf16_from_f64(z64).astype(np.float64) @ np.asarray(l2b, dtype=np.float64)


def linear(x32: np.ndarray, layer: dict, bias: Optional[np.ndarray] = None,
           group: int = GROUP) -> dict:
    """Whole fused layer, Algorithm 2 steps 1-8:  Y = Q(X~)Q(R) + bf16(X~ L1) L2 (+ bias).

    layer: dict with inv32 (or None), l1 [m][r], l2 [r][n], qw [m][n], sw [m/64][n].
    Returns dict(y=float64 [b][n], xt, qx, sx, z).
    """
    xt, qx, sx = quantize_activation(x32, layer.get("inv32"), group)
    y = gemm_main(qx, sx, layer["qw"], layer["sw"], group)
    r = layer["l1"].shape[1]
    z = lowrank_down(xt, layer["l1"]) if r else np.zeros((x32.shape[0], 0))
    if r:
        y = y + lowrank_up(z, layer["l2"])
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return {"y": y, "xt": xt, "qx": qx, "sx": sx, "z": z}


def linear_rows(x32_rows: np.ndarray, layer: dict, cols: Optional[np.ndarray] = None,
                bias: Optional[np.ndarray] = None, group: int = GROUP) -> np.ndarray:
    """Y for a subset of rows (and optionally columns), for sampled full-size checks.

    Rows are independent in every step (quantization groups run along a row),
    so this equals the corresponding slice of ``linear``."""
    qw, sw, l2 = layer["qw"], layer["sw"], layer["l2"]
    if cols is not None:
        qw, sw, l2 = qw[:, cols], sw[:, cols], l2[:, cols]
        bias = None if bias is None else np.asarray(bias)[cols]
    sub = dict(layer, qw=qw, sw=sw, l2=l2)
    return linear(x32_rows, sub, bias, group)["y"]


# --------------------------------------------------------------------------
# Analysis: [Review] sec. 4.1 Eq.(5)-(6), sec. 4.3 Eq.(9), sec. 6.1-6.2 Eq.(11)-(12)
# --------------------------------------------------------------------------


def prop41_bound(x, w, qx_deq, qw_deq) -> float:
    """Right-hand side of Eq.(6): ||X||F ||dW||F + ||dX||F (||W||F + ||dW||F)."""
    dW = np.linalg.norm(w - qw_deq)
    dX = np.linalg.norm(x - qx_deq)
    return float(np.linalg.norm(x) * dW + dX * (np.linalg.norm(w) + dW))


def eq9_group_bound(v: np.ndarray, qmax: int = QMAX) -> float:
    """Eq.(9) for one group of N values: sqrt(N) / (2 qmax) * max|v|."""
    v = np.asarray(v, dtype=np.float64)
    return math.sqrt(v.size) / (2 * qmax) * float(np.max(np.abs(v)))


def mac_ratio(m: int, n: int, r: int) -> float:
    """Eq.(11): low-rank MACs over dense MACs, r/m + r/n."""
    return r / m + r / n


def storage_ratio(m: int, n: int, r: int) -> float:
    """Eq.(12): (mn/2 + 2r(m+n)) bytes over 2mn BF16 bytes = 1/4 + r/m + r/n."""
    return (m * n / 2 + 2 * r * (m + n)) / (2 * m * n)


def lowrank_fix_of_quant_error(x32, w32, a, rank: int, alpha: float = 0.5,
                               group: int = GROUP) -> np.ndarray:
    """Negative control discussed in sec. 5: quantize W~ first, then protect a
    rank-r SVD of the rounding error E = W~ - Q(W~) in a bf16 branch.

    Returns Y_hat = Q(X~) Q(W~) + X~ L1e L2e in float64.
    """
    _, lam32, inv32 = smoothing_lambda(a, w32, alpha)
    wt = smooth_weight(w32, lam32)
    qw, sw = quantize_weight_residual(wt.astype(np.float32), group)
    wq = dequantize_groups(np.ascontiguousarray(qw.T), np.ascontiguousarray(sw.T), group).T
    l1, l2, _ = truncated_svd(wt - wq, rank)
    xt, qx, sx = quantize_activation(x32, inv32, group)
    return gemm_main(qx, sx, qw, sw, group) + lowrank_up(lowrank_down(xt, bf16_from_f64(l1)),
                                                         bf16_from_f64(l2))


def smoothed_w4a4_no_branch(x32, w32, a, alpha: float = 0.5, group: int = GROUP) -> np.ndarray:
    """Q(X~) Q(W~): smoothing alone, no protected branch (rank 0)."""
    _, lam32, inv32 = smoothing_lambda(a, w32, alpha)
    wt = smooth_weight(w32, lam32)
    qw, sw = quantize_weight_residual(wt.astype(np.float32), group)
    _, qx, sx = quantize_activation(x32, inv32, group)
    return gemm_main(qx, sx, qw, sw, group)


def naive_w4a4(x32, w32, group: int = GROUP) -> np.ndarray:
    """Q(X) Q(W): no smoothing, no branch."""
    qw, sw = quantize_weight_residual(np.asarray(w32, np.float32), group)
    _, qx, sx = quantize_activation(x32, None, group)
    return gemm_main(qx, sx, qw, sw, group)


# --------------------------------------------------------------------------
# The 8-bit setting ([Review] sec. 8; reading R19): W8A8 with the same
# smoothing and low-rank branch, per-token / per-channel INT8 quantization.
# --------------------------------------------------------------------------

QMAX8 = 127


def quantize_rows8(v32: np.ndarray):
    """Symmetric INT8 quantization of each row (last axis) of a float32 array:
    s = fp16(fl32(amax / 127)), q = clamp(round_half_even(fl32(v / s)), -127, 127),
    q = 0 where s == 0 (readings R1, R3, R4 with 127 for 7).
    Returns (codes int16 [..., K], scales float32 [...] holding fp16 values)."""
    v32 = np.asarray(v32, dtype=np.float32)
    amax = np.max(np.abs(v32), axis=-1)
    s = fp16_from_f32_sat(np.float32(amax) / np.float32(QMAX8))
    sb = s[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = np.where(sb > 0, v32 / np.where(sb > 0, sb, np.float32(1)), np.float32(0)).astype(np.float32)
    q = np.clip(np.rint(quot), -QMAX8, QMAX8)
    q = np.where(sb > 0, q, 0).astype(np.int16)
    return q, s.astype(np.float32)


def prepare_weights_w8a8(w32: np.ndarray, a: Optional[np.ndarray], rank: int = 16, alpha: float = 0.5,
                         svd: str = "lapack") -> dict:
    """The 8-bit protected layer: smoothing and the rank-r branch as in
    ``prepare_weights``, the residual quantized per output channel to INT8.
    Returns lam32, inv32, wt, l1, l2, r64, r32, qw (int16 codes [m][n]),
    sw (float32 fp16 values [n]), rank."""
    base = prepare_weights(w32, a, rank, GROUP, alpha, svd)
    codes_t, sw = quantize_rows8(np.ascontiguousarray(base["r32"].T))
    return dict(base, qw=np.ascontiguousarray(codes_t.T), sw=sw, bits=8)


def quantize_activation_w8a8(x32: np.ndarray, inv32: Optional[np.ndarray]):
    """Per-token INT8 quantization of the smoothed bf16 activations."""
    xt = smooth_activation(x32, inv32)
    qx, sx = quantize_rows8(xt)
    return xt, qx, sx


def linear_w8a8(x32: np.ndarray, layer: dict, bias: Optional[np.ndarray] = None) -> dict:
    """Y = sx sw (Q8(X~) Q8(R)) + bf16(X~ L1) L2 (+ bias), the integer product
    exact (int64) and everything else in float64."""
    xt, qx, sx = quantize_activation_w8a8(x32, layer.get("inv32"))
    isum = qx.astype(np.int64) @ layer["qw"].astype(np.int64)
    y = sx.astype(np.float64)[:, None] * isum.astype(np.float64) * layer["sw"].astype(np.float64)[None, :]
    r = layer["l1"].shape[1]
    z = lowrank_down(xt, layer["l1"]) if r else np.zeros((x32.shape[0], 0))
    if r:
        y = y + lowrank_up(z, layer["l2"])
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return {"y": y, "xt": xt, "qx": qx, "sx": sx, "z": z, "isum": isum}


# --------------------------------------------------------------------------
# The NVFP4 setting ([Review] sec. 8 and sec. 2.2; reading R20): FP4 E2M1
# codes in blocks of 16 with FP8 E4M3 block scales and a power-of-two tensor
# scale.
# --------------------------------------------------------------------------

FP4_BLOCK = 16
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E4M3_MAX = 448.0
FP4_RANGE = 6.0 * E4M3_MAX   # the largest magnitude a block can represent at t = 1


def e4m3_round(x) -> np.ndarray:
    """Nearest FP8 E4M3 value of x >= 0 (float64 result): quantum 2^(e-3) in
    the binade [2^e, 2^(e+1)) for e >= -6 and 2^-9 below (subnormals), ties to
    even, saturated at 448."""
    x = np.asarray(x, dtype=np.float64)
    _, ex = np.frexp(np.where(x > 0, x, 1.0))          # x = m 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, -6)
    quantum = np.ldexp(1.0, e - 3)
    return np.minimum(np.rint(x / quantum) * quantum, E4M3_MAX)


def e4m3_bits(v) -> np.ndarray:
    """FP8 E4M3 bit patterns (uint8) of non-negative E4M3 values."""
    v = np.asarray(v, dtype=np.float64)
    _, ex = np.frexp(np.where(v > 0, v, 1.0))
    e = ex - 1
    normal = (v >= 2.0 ** -6)
    mant_n = np.rint((v / np.ldexp(1.0, e) - 1.0) * 8.0)
    mant_s = np.rint(v / 2.0 ** -9)
    bits = np.where(normal, ((e + 7) << 3) + mant_n, mant_s)
    return bits.astype(np.uint8)


def e4m3_from_bits(bits) -> np.ndarray:
    """Value of FP8 E4M3 bit patterns (sign ignored; 0x7F/0xFF are NaN and not produced)."""
    b = np.asarray(bits, dtype=np.int64) & 0x7F
    e, m = b >> 3, b & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))


def e2m1_codes(y32) -> np.ndarray:
    """FP4 E2M1 codes (uint8, sign in bit 3) of float32 quotients: the nearest
    grid value, ties to the even code, magnitudes beyond 6 saturated; the sign
    bit is the quotient's (so -0 and small negatives give code 8)."""
    y = np.asarray(y32, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    d = np.abs(a[..., None] - E2M1_VALUES)
    i = np.argmin(d, axis=-1)                            # lowest index among equal distances
    nxt = np.minimum(i + 1, 7)
    tie_up = (i % 2 == 1) & (np.take_along_axis(d, nxt[..., None], -1)[..., 0] ==
                             np.take_along_axis(d, i[..., None], -1)[..., 0])
    i = np.where(tie_up, nxt, i)
    return (i + np.where(np.signbit(y), 8, 0)).astype(np.uint8)


def e2m1_values(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c & 8, -1.0, 1.0) * E2M1_VALUES[c & 7]


def pow2_ceil(x: float) -> float:
    """2^ceil(log2 x) for x > 0 (exact), 1.0 for x <= 0."""
    if not x > 0:
        return 1.0
    m, e = math.frexp(x)
    return x if m == 0.5 else math.ldexp(1.0, e)


def fp4_tensor_scale(amax: float) -> float:
    """Power-of-two tensor scale t = 2^ceil(log2(amax / (6 * 448))) (reading R20)."""
    return pow2_ceil(float(amax) / FP4_RANGE)


def quantize_fp4_blocks(v32: np.ndarray, t: float):
    """Blocks of 16 along the last axis of a float32 array.  Returns (codes
    uint8 [..., K], block scales sb float64 [..., K/16] holding E4M3 values)."""
    v32 = np.asarray(v32, dtype=np.float32)
    K = v32.shape[-1]
    blocks = v32.reshape(v32.shape[:-1] + (K // FP4_BLOCK, FP4_BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    u = (amax / np.float32(6.0)).astype(np.float32)     # fl32(amax / 6)
    sb = e4m3_round(u.astype(np.float64) / t)             # t is a power of two: exact
    S = (sb * t).astype(np.float32)                       # exact
    Sb = S[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(Sb > 0, blocks / np.where(Sb > 0, Sb, np.float32(1)), np.float32(0)).astype(np.float32)
    codes = np.where(Sb > 0, e2m1_codes(y), 0).astype(np.uint8)
    return codes.reshape(v32.shape), sb


def dequantize_fp4_blocks(codes: np.ndarray, sb: np.ndarray) -> np.ndarray:
    """code value x block scale (float64, exact; the tensor scale is separate)."""
    return e2m1_values(codes) * np.repeat(np.asarray(sb, np.float64), FP4_BLOCK, axis=-1)


def prepare_weights_fp4(w32: np.ndarray, a: Optional[np.ndarray], rank: int = 32, alpha: float = 0.5,
                        svd: str = "lapack") -> dict:
    """The NVFP4 protected layer: smoothing and the rank-r branch as in
    ``prepare_weights``, R quantized per output column in blocks of 16 input
    channels.  Returns the keys of ``prepare_weights`` plus qw (codes [m][n]),
    sbw (E4M3 block scales [m/16][n]), t_w, t_x."""
    base = prepare_weights(w32, a, rank, GROUP, alpha, svd)
    r32 = base["r32"]
    t_w = fp4_tensor_scale(np.max(np.abs(r32)))
    codes_t, sb_t = quantize_fp4_blocks(np.ascontiguousarray(r32.T), t_w)
    if a is None:
        t_x = 1.0
    else:
        # calibration maximum of |X~| per channel: bf16(fl32(a_k * inv_k)) (reading R7)
        xt_max = bf16_from_f32(np.asarray(a, np.float32) * base["inv32"]).astype(np.float64)
        t_x = fp4_tensor_scale(np.max(xt_max))
    return dict(base, qw=np.ascontiguousarray(codes_t.T), sbw=np.ascontiguousarray(sb_t.T), t_w=t_w, t_x=t_x,
                fmt="nvfp4")


def quantize_activation_fp4(x32: np.ndarray, inv32: Optional[np.ndarray], t_x: float):
    xt = smooth_activation(x32, inv32)
    qx, sbx = quantize_fp4_blocks(xt, t_x)
    return xt, qx, sbx


def linear_fp4(x32: np.ndarray, layer: dict, bias: Optional[np.ndarray] = None) -> dict:
    """Y = t_x t_w (X^ W^) + bf16(X~ L1) L2 (+ bias) in float64 (reading R20)."""
    xt, qx, sbx = quantize_activation_fp4(x32, layer.get("inv32"), layer["t_x"])
    xhat = dequantize_fp4_blocks(qx, sbx)
    what = dequantize_fp4_blocks(layer["qw"].T, layer["sbw"].T).T
    y = (layer["t_x"] * layer["t_w"]) * (xhat @ what)
    r = layer["l1"].shape[1]
    z = lowrank_down(xt, layer["l1"]) if r else np.zeros((x32.shape[0], 0))
    if r:
        y = y + lowrank_up(z, layer["l2"])
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return {"y": y, "xt": xt, "qx": qx, "sbx": sbx, "z": z}
