"""Test-side layout conversions between the oracle's logical matrices and the
C-ABI's packed buffers.  Pure data movement (bit packing, transposes, dtype
bit casts); no arithmetic of the method lives here.
"""
import numpy as np

GROUP = 64


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """int8 codes [R][K] -> group-major packed records uint8 [K/64][R][32].

    Byte t of a record holds code 2t in the low nibble and code 2t+1 in the high
    nibble (two's complement nibbles)."""
    R, K = codes.shape
    G = K // GROUP
    c = (codes.astype(np.int16) & 0xF).astype(np.uint8).reshape(R, G, 32, 2)
    packed = c[..., 0] | (c[..., 1] << 4)
    return np.ascontiguousarray(packed.transpose(1, 0, 2))


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """group-major records uint8 [G][R][32] -> int8 codes [R][G*64]."""
    packed = np.asarray(packed, dtype=np.uint8)
    G, R, _ = packed.shape
    lo = (packed & 0xF).astype(np.int8)
    hi = (packed >> 4).astype(np.int8)
    lo = np.where(lo > 7, lo - 16, lo)
    hi = np.where(hi > 7, hi - 16, hi)
    codes = np.stack([lo, hi], axis=-1).reshape(G, R, GROUP)
    return np.ascontiguousarray(codes.transpose(1, 0, 2).reshape(R, G * GROUP)).astype(np.int8)


def f32_to_fp16_bits(v: np.ndarray) -> np.ndarray:
    """float32 values that ARE fp16 values -> their fp16 bit patterns."""
    h = np.asarray(v, np.float32).astype(np.float16)
    assert np.array_equal(h.astype(np.float32), np.asarray(v, np.float32)), "not fp16 values"
    return h.view(np.uint16)


def fp16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float32)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float32 values that ARE bf16 values -> bf16 bit patterns."""
    u = np.ascontiguousarray(v, np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "not bf16 values"
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def oracle_layer_to_host_abi(lay: dict) -> dict:
    """Oracle-prepared layer (logical matrices) -> host arrays in the ABI layouts."""
    m, n = lay["qw"].shape
    r = lay["l1"].shape[1]
    inv = lay.get("inv32")
    return {
        "m": m, "n": n, "rank": r,
        "qw": pack_codes(np.ascontiguousarray(lay["qw"].T)),
        "wscale": f32_to_fp16_bits(lay["sw"]),
        "l1": np.ascontiguousarray(f32_to_bf16_bits(lay["l1"]).T),
        "l2": np.ascontiguousarray(f32_to_bf16_bits(lay["l2"]).T),
        "smooth_inv": np.ones(m, np.float32) if inv is None else np.asarray(inv, np.float32),
        "lambda": lay.get("lam32", np.ones(m, np.float32)),
    }


def host_abi_to_oracle_layer(host: dict) -> dict:
    """Host arrays in the ABI layouts (as the library's preparation returns
    them) -> the oracle's logical layer dict (codes [m][n], scales [m/64][n],
    L1 [m][r], L2 [r][n] as float32 holding bf16 values, inv32)."""
    return {
        "qw": np.ascontiguousarray(unpack_codes(host["qw"]).T),
        "sw": fp16_bits_to_f32(host["wscale"]),
        "l1": np.ascontiguousarray(bf16_bits_to_f32(host["l1"]).T),
        "l2": np.ascontiguousarray(bf16_bits_to_f32(host["l2"]).T),
        "inv32": np.asarray(host["smooth_inv"], np.float32),
        "lam32": np.asarray(host["lambda"], np.float32),
    }


# ---- the 8-bit setting: one code per byte, 64-byte group-major records ----------

def pack_codes8(codes: np.ndarray) -> np.ndarray:
    """integer codes [R][K] in [-127, 127] -> int8 records [K/64][R][64]."""
    R, K = codes.shape
    c = np.asarray(codes).astype(np.int8).reshape(R, K // GROUP, GROUP)
    return np.ascontiguousarray(c.transpose(1, 0, 2))


def unpack_codes8(recs: np.ndarray) -> np.ndarray:
    """int8 records [G][R][64] -> codes int16 [R][G*64]."""
    recs = np.asarray(recs, dtype=np.int8)
    G, R, _ = recs.shape
    return np.ascontiguousarray(recs.transpose(1, 0, 2).reshape(R, G * GROUP)).astype(np.int16)


def oracle_w8a8_to_host_abi(lay: dict) -> dict:
    """Oracle-prepared 8-bit layer -> host arrays in the ABI layouts."""
    m, n = lay["qw"].shape
    inv = lay.get("inv32")
    return {
        "m": m, "n": n, "rank": lay["l1"].shape[1],
        "qw": pack_codes8(np.ascontiguousarray(lay["qw"].T)),
        "wscale": f32_to_fp16_bits(lay["sw"]),
        "l1": np.ascontiguousarray(f32_to_bf16_bits(lay["l1"]).T),
        "l2": np.ascontiguousarray(f32_to_bf16_bits(lay["l2"]).T),
        "smooth_inv": np.ones(m, np.float32) if inv is None else np.asarray(inv, np.float32),
    }


# ---- the NVFP4 setting: E2M1 codes two per byte, E4M3 block-scale bytes -------

def pack_fp4_codes(codes: np.ndarray) -> np.ndarray:
    """4-bit code patterns [R][K] (uint8, sign in bit 3) -> records uint8 [K/64][R][32]."""
    R, K = codes.shape
    c = (np.asarray(codes).astype(np.uint8) & 0xF).reshape(R, K // GROUP, 32, 2)
    return np.ascontiguousarray((c[..., 0] | (c[..., 1] << 4)).transpose(1, 0, 2))


def unpack_fp4_codes(recs: np.ndarray) -> np.ndarray:
    """records uint8 [G][R][32] -> 4-bit code patterns uint8 [R][G*64]."""
    recs = np.asarray(recs, dtype=np.uint8)
    G, R, _ = recs.shape
    codes = np.stack([recs & 0xF, recs >> 4], axis=-1).reshape(G, R, GROUP)
    return np.ascontiguousarray(codes.transpose(1, 0, 2).reshape(R, G * GROUP))


def pack_fp4_scales(scale_bits: np.ndarray) -> np.ndarray:
    """E4M3 bytes [R][K/16] -> [K/64][R][4]."""
    R, B = scale_bits.shape
    return np.ascontiguousarray(np.asarray(scale_bits, np.uint8).reshape(R, B // 4, 4).transpose(1, 0, 2))


def unpack_fp4_scales(recs: np.ndarray) -> np.ndarray:
    """[G][R][4] bytes -> [R][G*4]."""
    recs = np.asarray(recs, dtype=np.uint8)
    G, R, _ = recs.shape
    return np.ascontiguousarray(recs.transpose(1, 0, 2).reshape(R, G * 4))


def oracle_fp4_to_host_abi(lay: dict, e4m3_bits) -> dict:
    """Oracle-prepared NVFP4 layer -> host arrays in the ABI layouts (e4m3_bits:
    the E4M3 value -> byte map, passed in so this module stays arithmetic-free)."""
    m, n = lay["qw"].shape
    inv = lay.get("inv32")
    return {
        "m": m, "n": n, "rank": lay["l1"].shape[1], "t_x": lay["t_x"], "t_w": lay["t_w"],
        "qw": pack_fp4_codes(np.ascontiguousarray(lay["qw"].T)),
        "wscale": pack_fp4_scales(e4m3_bits(np.ascontiguousarray(lay["sbw"].T))),
        "l1": np.ascontiguousarray(f32_to_bf16_bits(lay["l1"]).T),
        "l2": np.ascontiguousarray(f32_to_bf16_bits(lay["l2"]).T),
        "smooth_inv": np.ones(m, np.float32) if inv is None else np.asarray(inv, np.float32),
    }
