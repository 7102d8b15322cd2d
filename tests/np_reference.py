"""An independent float64 numpy evaluation of the routed-expert layer.

Used only to pin the C++ oracle (and never the HIP path directly).  It is
written from the format and layer definitions rather than from the oracle:
E2M1 values come from the element's bit fields, the weight matrices are
decoded whole with numpy, the products are numpy matmuls in float64 and the
top-k is a stable argsort.
"""
import numpy as np


def e2m1_from_bits(code: int) -> float:
    """OCP MX v1.0 FP4 E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa
    bit; exponent field 0 encodes subnormals 0 and 0.5."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -mag if s else mag


E2M1_F64 = np.array([e2m1_from_bits(c) for c in range(16)], dtype=np.float64)


def decode_mxfp4(q: np.ndarray, s: np.ndarray, N: int, K: int) -> np.ndarray:
    """q: N*K/2 bytes (element 2m in the low nibble of byte m), s: N*K/32 E8M0
    bytes -> float64 [N, K]."""
    q = q.reshape(N, K // 2)
    codes = np.empty((N, K), dtype=np.uint8)
    codes[:, 0::2] = q & 0xF
    codes[:, 1::2] = q >> 4
    scale = np.ldexp(1.0, s.reshape(N, K // 32).astype(np.int64) - 127)
    return E2M1_F64[codes] * np.repeat(scale, 32, axis=1)


def bf16_bits_to_f64(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def expert_matrices(slab: np.ndarray, H: int, I: int):
    qb, sb = I * H // 2, I * H // 32
    parts = []
    o = 0
    for N, K in ((I, H), (I, H), (H, I)):
        q = slab[o:o + qb]
        o += qb
        s = slab[o:o + sb]
        o += sb
        parts.append(decode_mxfp4(q, s, N, K))
    return parts  # Wg [I,H], Wu [I,H], Wd [H,I]


def layer_f64(x_bits: np.ndarray, logits: np.ndarray, k: int, slabs: np.ndarray, H: int, I: int):
    """Returns (ids, weights, out) with out in float64."""
    T, E = logits.shape
    x = bf16_bits_to_f64(x_bits)
    mats = [expert_matrices(slabs[e], H, I) for e in range(E)]
    ids = np.zeros((T, k), np.int64)
    w = np.zeros((T, k), np.float64)
    out = np.zeros((T, H), np.float64)
    for t in range(T):
        order = np.argsort(-logits[t].astype(np.float64), kind="stable")[:k]
        ids[t] = order
        sel = logits[t, order].astype(np.float64)
        ex = np.exp(sel - sel.max())
        w[t] = ex / ex.sum()
        for j, e in enumerate(order):
            Wg, Wu, Wd = mats[e]
            g = Wg @ x[t]
            u = Wu @ x[t]
            h = g / (1.0 + np.exp(-g)) * u
            out[t] += w[t, j] * (Wd @ h)
    return ids, w, out
