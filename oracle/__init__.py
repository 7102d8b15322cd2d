"""ctypes wrapper of the CPU oracle (moe_oracle.cpp).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's
CPU-baseline leg use it; the product path never imports it.  Inputs and
outputs are numpy arrays in host memory.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_SANITIZE=1 loads the AddressSanitizer + UBSan build (liboracle_san.so;
# the process must preload clang's ASan runtime, tests/run_sanitized.py does)
SANITIZE = os.environ.get("MOE_SANITIZE") == "1"
LIB_PATH = os.path.join(_HERE, "liboracle_san.so" if SANITIZE else "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32


class OracleWeights(ctypes.Structure):
    _fields_ = [("gate_q", _P), ("gate_s", _P), ("up_q", _P), ("up_s", _P), ("down_q", _P), ("down_s", _P),
                ("expert_stride", ctypes.c_int64), ("num_experts", _I32), ("hidden", _I32), ("inter", _I32)]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """g++ build of moe_oracle.cpp; sanitize=True builds liboracle_san.so with
    clang's AddressSanitizer and UBSan instead (same flags otherwise)."""
    path = os.path.join(_HERE, "liboracle_san.so" if sanitize else "liboracle.so")
    cxx = ["/opt/rocm/llvm/bin/clang++", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-g", "-shared-libsan"] if sanitize else ["g++"]
    cmd = cxx + ["-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra", "-shared",
                 "-fPIC", "-pthread", os.path.join(_HERE, "moe_oracle.cpp"), "-o", path + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(path + ".tmp", path)
    return path


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        W = ctypes.POINTER(OracleWeights)
        L.oracle_e2m1_value.restype = ctypes.c_float
        L.oracle_e2m1_value.argtypes = [ctypes.c_int]
        L.oracle_dequant.restype = ctypes.c_float
        L.oracle_dequant.argtypes = [_P, _P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
        L.oracle_route_topk.argtypes = [_P, _I32, _I32, _I32, _P, _P]
        L.oracle_group_rows.argtypes = [_P, _I32, _I32, _I32, _P, _P, _P, _P]
        L.oracle_gateup.argtypes = [_P, _I32, _I32, W, _P, _P, _P, _P, _I32]
        L.oracle_down.argtypes = [_P, W, _P, _P, _P, _I32]
        L.oracle_combine.argtypes = [_P, _P, _P, _I32, _I32, _I32, _P]
        L.oracle_rms_rescale_bf16.argtypes = [_P, _I32, _I32, ctypes.c_float, _P]
        L.oracle_token_layer.argtypes = [_P, _P, _P, _I32, W, _P]
        L.oracle_token_layer_f64.argtypes = [_P, _P, _P, _I32, W, _P]
        L.oracle_dense_token.argtypes = [_P, _P, _I32, _I32, W, _P]
        L.oracle_router_logits.argtypes = [_P, _I32, _I32, _P, _I32, _P, _I32]
        for f in ("oracle_route_topk", "oracle_group_rows", "oracle_gateup", "oracle_down", "oracle_combine",
                  "oracle_rms_rescale_bf16", "oracle_token_layer", "oracle_token_layer_f64",
                  "oracle_dense_token", "oracle_router_logits"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


class Pool:
    """One layer's expert pool as a host uint8 array [E, slab] in the slab
    layout gate_q | gate_s | up_q | up_s | down_q | down_s."""

    def __init__(self, slabs: np.ndarray, H: int, I: int):
        assert slabs.dtype == np.uint8 and slabs.ndim == 2 and slabs.flags.c_contiguous
        qb, sb = I * H // 2, I * H // 32
        assert slabs.shape[1] == 3 * (qb + sb)
        self.slabs, self.H, self.I, self.E = slabs, H, I, slabs.shape[0]
        base = slabs.ctypes.data
        offs = [0, qb, qb + sb, 2 * qb + sb, 2 * qb + 2 * sb, 3 * qb + 2 * sb]
        self.w = OracleWeights(*[base + o for o in offs], slabs.shape[1], self.E, H, I)

    def ref(self):
        return ctypes.byref(self.w)


def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(code)


def route_topk(logits: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float32)
    rc = lib().oracle_route_topk(logits.ctypes.data, T, E, k, ids.ctypes.data, w.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_route_topk rejected its input (code {rc})")
    return ids, w


def group_rows(ids: np.ndarray, E: int) -> Dict[str, np.ndarray]:
    ids = _c(ids, np.int32)
    T, k = ids.shape
    R = T * k
    offsets = np.zeros(E + 1, np.int32)
    sorted_rows = np.zeros(R, np.int32)
    row_pos = np.zeros(R, np.int32)
    active = np.zeros(E + 1, np.int32)
    rc = lib().oracle_group_rows(ids.ctypes.data, T, k, E, offsets.ctypes.data, sorted_rows.ctypes.data,
                                 row_pos.ctypes.data, active.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_group_rows: expert id out of range")
    return {"expert_offsets": offsets, "sorted_rows": sorted_rows, "row_pos": row_pos, "active": active}


def gateup(x: np.ndarray, k: int, pool: Pool, grp: Dict[str, np.ndarray], nthreads: int = 8) -> np.ndarray:
    x = _c(x, np.uint16)
    T = x.shape[0]
    R = T * k
    h = np.zeros((R, pool.I), np.float32)
    lib().oracle_gateup(x.ctypes.data, T, k, pool.ref(), grp["expert_offsets"].ctypes.data,
                        grp["sorted_rows"].ctypes.data, grp["active"].ctypes.data, h.ctypes.data, nthreads)
    return h


def down(h: np.ndarray, pool: Pool, grp: Dict[str, np.ndarray], nthreads: int = 8) -> np.ndarray:
    h = _c(h, np.float32)
    y = np.zeros((h.shape[0], pool.H), np.float32)
    lib().oracle_down(h.ctypes.data, pool.ref(), grp["expert_offsets"].ctypes.data, grp["active"].ctypes.data,
                      y.ctypes.data, nthreads)
    return y


def combine(y_rows: np.ndarray, w: np.ndarray, row_pos: np.ndarray, T: int, k: int, H: int) -> np.ndarray:
    y_rows, w, row_pos = _c(y_rows, np.float32), _c(w, np.float32), _c(row_pos, np.int32)
    out = np.zeros((T, H), np.float32)
    lib().oracle_combine(y_rows.ctypes.data, w.ctypes.data, row_pos.ctypes.data, T, k, H, out.ctypes.data)
    return out


def rms_rescale_bf16(y: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    y = _c(y, np.float32)
    T, H = y.shape
    x = np.zeros((T, H), np.uint16)
    lib().oracle_rms_rescale_bf16(y.ctypes.data, T, H, eps, x.ctypes.data)
    return x


def router_logits(x: np.ndarray, w_router: np.ndarray, nthreads: int = 8) -> np.ndarray:
    """logits[T][E] = x[T][H] (bf16 bits) . w_router[E][H]^T (fp32), fp32 sums in
    ascending H (the router projection before the path)."""
    x, wr = _c(x, np.uint16), _c(w_router, np.float32)
    T, H = x.shape
    E = wr.shape[0]
    assert wr.shape[1] == H
    out = np.zeros((T, E), np.float32)
    lib().oracle_router_logits(x.ctypes.data, T, H, wr.ctypes.data, E, out.ctypes.data, nthreads)
    return out


def layer(x: np.ndarray, logits: np.ndarray, k: int, pool: Pool, nthreads: int = 8) -> Dict[str, np.ndarray]:
    """All steps of one layer through the grouped path."""
    ids, w = route_topk(logits, k)
    grp = group_rows(ids, logits.shape[1])
    h = gateup(x, k, pool, grp, nthreads)
    y_rows = down(h, pool, grp, nthreads)
    out = combine(y_rows, w, grp["row_pos"], x.shape[0], k, pool.H)
    return dict(ids=ids, w=w, h=h, y_rows=y_rows, out=out, **grp)


def token_layer(x_t: np.ndarray, ids_t: np.ndarray, w_t: np.ndarray, pool: Pool) -> np.ndarray:
    x_t, ids_t, w_t = _c(x_t, np.uint16), _c(ids_t, np.int32), _c(w_t, np.float32)
    out = np.zeros(pool.H, np.float32)
    lib().oracle_token_layer(x_t.ctypes.data, ids_t.ctypes.data, w_t.ctypes.data, ids_t.size, pool.ref(),
                             out.ctypes.data)
    return out


def token_layer_f64(x_t: np.ndarray, ids_t: np.ndarray, w_t: np.ndarray, pool: Pool) -> np.ndarray:
    x_t, ids_t, w_t = _c(x_t, np.uint16), _c(ids_t, np.int32), _c(w_t, np.float32)
    out = np.zeros(pool.H, np.float64)
    lib().oracle_token_layer_f64(x_t.ctypes.data, ids_t.ctypes.data, w_t.ctypes.data, ids_t.size, pool.ref(),
                                 out.ctypes.data)
    return out


def dense_token(x_t: np.ndarray, logits_t: np.ndarray, k: int, pool: Pool) -> np.ndarray:
    x_t, logits_t = _c(x_t, np.uint16), _c(logits_t, np.float32)
    out = np.zeros(pool.H, np.float32)
    lib().oracle_dense_token(x_t.ctypes.data, logits_t.ctypes.data, logits_t.size, k, pool.ref(), out.ctypes.data)
    return out


def token_layers_parallel(x: np.ndarray, ids: np.ndarray, w: np.ndarray, pool: Pool, tokens,
                          nthreads: int = 8) -> np.ndarray:
    """oracle_token_layer for a list of tokens on a thread pool (ctypes drops
    the GIL during the call)."""
    from concurrent.futures import ThreadPoolExecutor

    tokens = list(tokens)
    with ThreadPoolExecutor(max_workers=max(1, nthreads)) as ex:
        outs = list(ex.map(lambda t: token_layer(x[t], ids[t], w[t], pool), tokens))
    return np.stack(outs) if outs else np.zeros((0, pool.H), np.float32)
