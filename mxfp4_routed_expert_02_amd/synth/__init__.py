"""Seeded synthetic inputs for the routed-expert MXFP4 layer.

This module draws inputs only: expert weight slabs (uniform E2M1 nibbles,
E8M0 scale bytes with exponent uniform over {-6..-3}), bf16 N(0,1)
activations and fp32 router logits with the per-workload bias.  It holds none
of the layer's arithmetic, and both the HIP path and the CPU oracle receive
exactly the bytes it returns.  The generator itself (counter-mode SplitMix64,
Box-Muller) lives in moe_synth.c next to this file.

Workloads follow the pages' shapes: the Kimi K3 routed-expert layer with
896 experts per layer (82,432 experts over 92 layers), top-16 routing
(page "hn.213312.xyz/article/49090233", section on how it works), hidden 7168
and intermediate 1536.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_SANITIZE=1 loads the AddressSanitizer + UBSan build of the host generator
SANITIZE = os.environ.get("MOE_SANITIZE") == "1"
LIB_PATH = os.path.join(_HERE, "libmoe_synth_san.so" if SANITIZE else "libmoe_synth.so")
GPU_LIB_PATH = os.path.join(_HERE, "libmoe_synth_gpu.so")  # device twin of the slab generator

# array ids of the tag field (weights use 1..6 inside moe_synth.c)
ARR_X = 16
ARR_LOGITS = 17
ARR_BIAS = 18
ARR_TIES = 19
ARR_ROUTER = 20

_lib = None
_gpu_lib = None


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile moe_synth.c into libmoe_synth.so with gcc (host code) and
    synth_gpu.hip into libmoe_synth_gpu.so with hipcc (gfx950).
    sanitize=True builds only the host generator, with clang's
    AddressSanitizer and UBSan, into libmoe_synth_san.so."""
    import subprocess

    path = os.path.join(_HERE, "libmoe_synth_san.so" if sanitize else "libmoe_synth.so")
    cc = ["/opt/rocm/llvm/bin/clang", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", "-g", "-shared-libsan"] if sanitize else ["gcc"]
    cmd = cc + ["-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                os.path.join(_HERE, "moe_synth.c"), "-o", path + ".tmp", "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(path + ".tmp", path)
    if sanitize:
        return path
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fvisibility=hidden",
           os.path.join(_HERE, "synth_gpu.hip"), "-o", GPU_LIB_PATH + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(GPU_LIB_PATH + ".tmp", GPU_LIB_PATH)
    return LIB_PATH


def gpu_lib():
    global _gpu_lib
    if _gpu_lib is None:
        if not os.path.exists(GPU_LIB_PATH):
            raise RuntimeError(f"{GPU_LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(GPU_LIB_PATH)
        L.synth_expert_slabs_gpu.restype = ctypes.c_int
        L.synth_expert_slabs_gpu.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                             ctypes.c_uint64, ctypes.c_void_p]
        L.synth_stream_read.restype = ctypes.c_int
        L.synth_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p]
        _gpu_lib = L
    return _gpu_lib


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        u64, i32 = ctypes.c_uint64, ctypes.c_int
        L.synth_tag.restype = u64
        L.synth_tag.argtypes = [u64, u64, u64, u64]
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u64]
        L.synth_draw.restype = u64
        L.synth_draw.argtypes = [u64, u64]
        L.synth_bytes.argtypes = [u64, u64, u64, ctypes.c_void_p]
        L.synth_small_bytes.argtypes = [u64, u64, u64, ctypes.c_uint8, ctypes.c_uint8, ctypes.c_void_p]
        L.synth_normal_f32.argtypes = [u64, u64, u64, ctypes.c_float, ctypes.c_void_p]
        L.synth_normal_bf16.argtypes = [u64, u64, u64, ctypes.c_void_p]
        L.synth_slab_bytes.restype = u64
        L.synth_slab_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64]
        L.synth_expert_slabs.restype = i32
        L.synth_expert_slabs.argtypes = [u64, i32, i32, i32, i32, i32, i32, ctypes.c_void_p, u64, i32]
        _lib = L
    return _lib


def key(seed: int, array: int, sub: int = 0, layer: int = 0, expert: int = 0) -> int:
    L = lib()
    return L.synth_key(seed, L.synth_tag(array, sub, layer, expert))


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload of the routed-expert layer.

    E experts per layer pool, H hidden, I intermediate, k experts per token,
    T tokens, `layers` stacked layers.  `logits` names the router-logit
    recipe; `pool` names the weight pool (workloads with equal pool id, H, I
    share expert bytes); `sub` separates activation/logit streams.
    """

    name: str
    E: int
    H: int
    I: int
    k: int
    T: int
    layers: int = 1
    logits: str = "normal"
    pool: int = 0
    sub: int = 0

    @property
    def R(self) -> int:
        return self.T * self.k


# pool 0: the realistic 896-expert layer (H 7168, I 1536) shared by the
# single-layer workloads; pool 1: tiny; pool 3: the 92-layer stack.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", E=8, H=256, I=128, k=2, T=4, pool=1, sub=1),
    "decode896": Workload("decode896", E=896, H=7168, I=1536, k=16, T=1, pool=0, sub=2),
    "stack92": Workload("stack92", E=96, H=7168, I=1536, k=16, T=1, layers=92, pool=3, sub=3),
    "verify8": Workload("verify8", E=896, H=7168, I=1536, k=16, T=8, logits="shared_bias", pool=0, sub=4),
    "prefill512": Workload("prefill512", E=896, H=7168, I=1536, k=16, T=512, logits="zipf", pool=0, sub=5),
    # long prompt: hot experts reach thousands of rows (the grouped GEMM's MFMA-bound regime)
    "prefill4096": Workload("prefill4096", E=896, H=7168, I=1536, k=16, T=4096, logits="zipf", pool=0, sub=7),
    # auxiliary dense case: every token routes to the same 16 experts (512 rows each)
    "prefill_dense": Workload("prefill_dense", E=896, H=7168, I=1536, k=16, T=512, logits="dense16", pool=0,
                              sub=6),
    # one GPU's share of decode896 when every expert's I = 1536 is split 8 ways
    # (gate/up rows and the matching down columns): the same layer at I = 192
    "decode896_tp8": Workload("decode896_tp8", E=896, H=7168, I=192, k=16, T=1, pool=8, sub=8),
}


def router_weights(seed: int, wl: Workload, layer: int = 0) -> np.ndarray:
    """Router projection weights w_r[E][H] fp32 ~ N(0, 1/H), so that for
    activations N(0, 1) the logits are about N(0, 1) like the logit recipes."""
    return normal_f32(key(seed, ARR_ROUTER, wl.pool, layer), wl.E * wl.H,
                      stddev=float(1.0 / np.sqrt(wl.H))).reshape(wl.E, wl.H)


def slab_bytes(H: int, I: int) -> int:
    return 3 * (I * H // 2 + I * H // 32)


def slab_offsets(H: int, I: int) -> Dict[str, int]:
    """Byte offsets of the six arrays inside one expert slab."""
    qb, sb = I * H // 2, I * H // 32
    return {"gate_q": 0, "gate_s": qb, "up_q": qb + sb, "up_s": 2 * qb + sb,
            "down_q": 2 * qb + 2 * sb, "down_s": 3 * qb + 2 * sb}


def expert_slabs(seed: int, pool: int, layer: int, e0: int, n: int, H: int, I: int,
                 nthreads: int = 8, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Slabs of experts e0..e0+n-1 as a uint8 array [n, slab_bytes]."""
    sb = slab_bytes(H, I)
    if out is None:
        out = np.empty((n, sb), dtype=np.uint8)
    assert out.dtype == np.uint8 and out.flags.c_contiguous and out.size >= n * sb
    rc = lib().synth_expert_slabs(seed, pool, layer, e0, n, H, I, out.ctypes.data, sb, nthreads)
    if rc != 0:
        raise RuntimeError("synth_expert_slabs failed")
    return out


def fill_slabs_ptr(seed: int, pool: int, layer: int, e0: int, n: int, H: int, I: int, ptr: int,
                   stride: int, nthreads: int = 8) -> None:
    """Fills n slabs at a raw host pointer (e.g. a pinned staging tensor)."""
    if lib().synth_expert_slabs(seed, pool, layer, e0, n, H, I, ptr, stride, nthreads) != 0:
        raise RuntimeError("synth_expert_slabs failed")


def normal_f32(k: int, n: int, stddev: float = 1.0, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().synth_normal_f32(k, start, n, stddev, out.ctypes.data)
    return out


def activations_bf16(seed: int, wl: Workload, layer: int = 0, variant: int = 0) -> np.ndarray:
    """x[T][H] as raw bf16 bits (uint16), N(0,1) rounded to nearest even."""
    out = np.empty((wl.T, wl.H), dtype=np.uint16)
    k = key(seed, ARR_X, wl.sub, layer, variant)
    lib().synth_normal_bf16(k, 0, wl.T * wl.H, out.ctypes.data)
    return out


def router_logits(seed: int, wl: Workload, layer: int = 0, variant: int = 0) -> np.ndarray:
    """logits[T][E] fp32 for the workload's recipe.

    normal       N(0,1)
    shared_bias  N(0,1) + b_e, b_e = 0.5 * N(0,1) drawn once per expert and
                 shared by all tokens of the batch (neighbouring draft tokens
                 overlap in expert choice)
    zipf         N(0,1) - 1.1 * ln(e + 1): expert popularity ~ Zipf(1.1) over
                 ids (rank = id + 1); bias added in fp32
    dense16      N(0,1) + 64 for experts 0..15: every token routes to the
                 same 16 experts
    ties         integers drawn uniformly from {0, 1, 2, 3} (tie stress)
    """
    T, E = wl.T, wl.E
    v = variant
    if wl.logits == "ties":
        raw = np.empty(T * E, dtype=np.uint8)
        lib().synth_bytes(key(seed, ARR_TIES, wl.sub, layer, v), 0, T * E, raw.ctypes.data)
        return (raw & 3).astype(np.float32).reshape(T, E)
    base = normal_f32(key(seed, ARR_LOGITS, wl.sub, layer, v), T * E).reshape(T, E)
    if wl.logits == "normal":
        return base
    if wl.logits == "shared_bias":
        b = normal_f32(key(seed, ARR_BIAS, wl.sub, layer, v), E, stddev=0.5)
        return (base + b[None, :]).astype(np.float32)
    if wl.logits == "zipf":
        b = (-1.1 * np.log(np.arange(E, dtype=np.float64) + 1.0)).astype(np.float32)
        return (base + b[None, :]).astype(np.float32)
    if wl.logits == "dense16":
        b = np.zeros(E, dtype=np.float32)
        b[:16] = 64.0
        return (base + b[None, :]).astype(np.float32)
    raise ValueError(f"unknown logits recipe {wl.logits}")


def device_pool_slabs(seed: int, pool: int, layer: int, E: int, H: int, I: int, device, out=None,
                      first: int = 0):
    """Experts first..first+E-1 of (pool, layer) generated on the device: a
    uint8 tensor [E, slab] holding the same bytes as expert_slabs() /
    upload_pool()."""
    import torch

    sb = slab_bytes(H, I)
    dst = torch.empty((E, sb), dtype=torch.uint8, device=device) if out is None else out
    assert dst.dtype == torch.uint8 and dst.is_contiguous() and dst.numel() >= E * sb
    stream = torch.cuda.current_stream(dst.device).cuda_stream
    for e0 in range(0, E, 65535):
        n = min(65535, E - e0)
        rc = gpu_lib().synth_expert_slabs_gpu(seed, pool, layer, first + e0, n, H, I, dst[e0].data_ptr(), sb,
                                              stream)
        if rc != 0:
            raise RuntimeError(f"synth_expert_slabs_gpu failed ({rc})")
    return dst


def upload_pool(seed: int, pool: int, layer: int, E: int, H: int, I: int, device, nthreads: int = 16,
                chunk_experts: int = 8):
    """Generates experts 0..E-1 of (pool, layer) on the host in pinned staging
    buffers and copies them to a device uint8 tensor [E, slab]."""
    import torch

    sb = slab_bytes(H, I)
    dst = torch.empty((E, sb), dtype=torch.uint8, device=device)
    n = max(1, min(chunk_experts, E))
    stage = [torch.empty((n, sb), dtype=torch.uint8, pin_memory=True) for _ in range(2)]
    done = [None, None]
    stream = torch.cuda.current_stream(device)
    for i, e0 in enumerate(range(0, E, n)):
        b = i & 1
        if done[b] is not None:
            done[b].synchronize()
        cnt = min(n, E - e0)
        fill_slabs_ptr(seed, pool, layer, e0, cnt, H, I, stage[b].data_ptr(), sb, nthreads)
        dst[e0:e0 + cnt].copy_(stage[b][:cnt], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record(stream)
        done[b] = ev
    torch.cuda.synchronize(device)
    return dst
