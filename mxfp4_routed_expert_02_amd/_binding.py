"""ctypes binding of libmoe_mxfp4.so (argument marshalling only)."""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_SANITIZE=1 loads the build with host-side AddressSanitizer + UBSan
LIB_PATH = os.path.join(_PKG, "lib", "libmoe_mxfp4_san.so" if os.environ.get("MOE_SANITIZE") == "1"
                        else "libmoe_mxfp4.so")

MAX_EXPERTS = 4096
MAX_TOPK = 32
MAX_DIM = 16384

_P = ctypes.c_void_p
_I32 = ctypes.c_int32

_STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED_DEVICE",
           3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_HIP", 5: "MOE_ERR_SCRATCH_TOO_SMALL"}
NOALLOC_SCRATCH_BYTES = 1 << 20  # MOE_NOALLOC_SCRATCH_BYTES


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {status_string(status)}")


class MoeWeights(ctypes.Structure):
    """Mirror of moe_mxfp4_weights (host struct holding device pointers)."""

    _fields_ = [("gate_q", _P), ("gate_s", _P), ("up_q", _P), ("up_s", _P), ("down_q", _P), ("down_s", _P),
                ("expert_stride", ctypes.c_int64), ("num_experts", _I32), ("hidden", _I32), ("inter", _I32)]


_lib = None


def lib():
    """The loaded library; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library {LIB_PATH} is not built: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        W = ctypes.POINTER(MoeWeights)
        L.moe_route_topk.argtypes = [_P, _I32, _I32, _I32, _P, _P, _P]
        L.moe_group_rows.argtypes = [_P, _I32, _I32, _I32, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_expert_ffn_mxfp4.argtypes = [_P, _I32, _I32, W, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_combine.argtypes = [_P, _P, _P, _I32, _I32, _I32, _P, _P]
        L.moe_rms_rescale_bf16.argtypes = [_P, _I32, _I32, ctypes.c_float, _P, _P]
        L.moe_router_logits.argtypes = [_P, _I32, _I32, _P, _I32, _P, _P]
        L.moe_route_group_one.argtypes = [_P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P]
        L.moe_combine_rms_bf16.argtypes = [_P, _P, _P, _I32, _I32, _I32, ctypes.c_float, _P, _P, _P]
        L.moe_expert_ffn_combine_mxfp4.argtypes = [_P, _I32, _I32, W, _P, _P, _P, _P, _P, _P, _P, _P,
                                                   ctypes.c_size_t, _P]
        L.moe_decode_layer_mxfp4.argtypes = [_P, _P, _I32, W, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                             _P]
        L.moe_decode_layer_rms_mxfp4.argtypes = [_P, _P, ctypes.c_float, _P, _I32, W, _P, _P, _P, _P, _P, _P, _P,
                                                 _P, _P, ctypes.c_size_t, _P]
        L.moe_decode_layer_mxfp4_noalloc.argtypes = [_P, _P, _I32, W, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        L.moe_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32, _I32]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        for f in ("moe_route_topk", "moe_group_rows", "moe_expert_ffn_mxfp4", "moe_combine",
                  "moe_rms_rescale_bf16", "moe_router_logits", "moe_route_group_one", "moe_combine_rms_bf16",
                  "moe_expert_ffn_combine_mxfp4", "moe_decode_layer_mxfp4", "moe_decode_layer_rms_mxfp4",
                  "moe_decode_layer_mxfp4_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    try:
        return lib().moe_status_string(status).decode()
    except RuntimeError:
        return _STATUS.get(status, f"status {status}")


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MoeError(fn, status)


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def workspace_bytes(T: int, k: int, E: int, H: int, I: int) -> int:
    return int(lib().moe_workspace_bytes(T, k, E, H, I))


@dataclasses.dataclass
class Grouping:
    expert_offsets: torch.Tensor  # [E+1] int32
    sorted_rows: torch.Tensor  # [R] int32
    row_pos: torch.Tensor  # [R] int32
    active: torch.Tensor  # [E+1] int32


class ExpertPool:
    """One layer's resident expert pool: a device uint8 tensor [E, slab] in
    the slab layout gate_q | gate_s | up_q | up_s | down_q | down_s."""

    def __init__(self, slabs: torch.Tensor, H: int, I: int):
        if slabs.dim() != 2 or slabs.dtype != torch.uint8 or slabs.device.type != "cuda":
            raise ValueError("slabs must be a device uint8 tensor [E, slab]")
        qb, sb = I * H // 2, I * H // 32
        if slabs.shape[1] != 3 * (qb + sb):
            raise ValueError("slab width does not match H, I")
        self.slabs, self.H, self.I, self.E = slabs, H, I, slabs.shape[0]
        base = slabs.data_ptr()
        stride = slabs.stride(0)
        offs = [0, qb, qb + sb, 2 * qb + sb, 2 * qb + 2 * sb, 3 * qb + 2 * sb]
        self.weights = MoeWeights(*[base + o for o in offs], stride, self.E, H, I)

    @property
    def device(self) -> torch.device:
        return self.slabs.device


def route_topk(logits: torch.Tensor, k: int, ids: Optional[torch.Tensor] = None,
               weights: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check("moe_route_topk", lib().moe_route_topk(
        _dev(logits, torch.float32, "logits"), T, E, k, _dev(ids, torch.int32, "ids"),
        _dev(weights, torch.float32, "weights"), _stream(logits.device)))
    return ids, weights


def group_rows(ids: torch.Tensor, E: int, workspace: torch.Tensor, out: Optional[Grouping] = None) -> Grouping:
    T, k = ids.shape
    R = T * k
    dev = ids.device
    if out is None:
        out = Grouping(torch.empty(E + 1, dtype=torch.int32, device=dev), torch.empty(R, dtype=torch.int32, device=dev),
                       torch.empty(R, dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev))
    _check("moe_group_rows", lib().moe_group_rows(
        _dev(ids, torch.int32, "ids"), T, k, E, _dev(out.expert_offsets, torch.int32, "expert_offsets"),
        _dev(out.sorted_rows, torch.int32, "sorted_rows"), _dev(out.row_pos, torch.int32, "row_pos"),
        _dev(out.active, torch.int32, "active"), _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream(dev)))
    return out


def expert_ffn_mxfp4(x: torch.Tensor, k: int, pool: ExpertPool, grp: Grouping, workspace: torch.Tensor,
                     y_rows: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x: [T, H] bf16 (or its raw int16 bits); returns y_rows [T*k, H] fp32 in sorted order."""
    T, H = x.shape
    xb = x.view(torch.int16) if x.dtype == torch.bfloat16 else x
    if y_rows is None:
        y_rows = torch.empty((T * k, H), dtype=torch.float32, device=x.device)
    _check("moe_expert_ffn_mxfp4", lib().moe_expert_ffn_mxfp4(
        _dev(xb, torch.int16, "x"), T, k, ctypes.byref(pool.weights),
        _dev(grp.expert_offsets, torch.int32, "expert_offsets"), _dev(grp.sorted_rows, torch.int32, "sorted_rows"),
        _dev(grp.active, torch.int32, "active"), _dev(y_rows, torch.float32, "y_rows"),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(x.device)))
    return y_rows


def expert_ffn_combine_mxfp4(x: torch.Tensor, k: int, pool: ExpertPool, grp: Grouping, weights: torch.Tensor,
                             workspace: torch.Tensor, y_rows: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """expert_ffn_mxfp4 then combine in one call: y_rows [T*k, H] and out [T, H] fp32 written; returns out."""
    T, H = x.shape
    xb = x.view(torch.int16) if x.dtype == torch.bfloat16 else x
    _check("moe_expert_ffn_combine_mxfp4", lib().moe_expert_ffn_combine_mxfp4(
        _dev(xb, torch.int16, "x"), T, k, ctypes.byref(pool.weights),
        _dev(grp.expert_offsets, torch.int32, "expert_offsets"), _dev(grp.sorted_rows, torch.int32, "sorted_rows"),
        _dev(grp.active, torch.int32, "active"), _dev(weights, torch.float32, "weights"),
        _dev(grp.row_pos, torch.int32, "row_pos"), _dev(y_rows, torch.float32, "y_rows"),
        _dev(out, torch.float32, "out"), _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream(x.device)))
    return out


def decode_layer_mxfp4(logits: torch.Tensor, x: torch.Tensor, k: int, pool: ExpertPool, ids: torch.Tensor,
                       weights: torch.Tensor, grp: Grouping, workspace: torch.Tensor, y_rows: torch.Tensor,
                       out: torch.Tensor) -> torch.Tensor:
    """One token through the layer: logits [1, E] fp32, x [1, H] bf16 -> ids, weights, grp, y_rows and
    out [1, H] fp32 written; returns out."""
    if logits.shape[0] != 1 or x.shape[0] != 1:
        raise ValueError("decode_layer_mxfp4 takes one token")
    xb = x.view(torch.int16) if x.dtype == torch.bfloat16 else x
    _check("moe_decode_layer_mxfp4", lib().moe_decode_layer_mxfp4(
        _dev(logits, torch.float32, "logits"), _dev(xb, torch.int16, "x"), k, ctypes.byref(pool.weights),
        _dev(ids, torch.int32, "ids"), _dev(weights, torch.float32, "weights"),
        _dev(grp.expert_offsets, torch.int32, "expert_offsets"), _dev(grp.sorted_rows, torch.int32, "sorted_rows"),
        _dev(grp.row_pos, torch.int32, "row_pos"), _dev(grp.active, torch.int32, "active"),
        _dev(y_rows, torch.float32, "y_rows"), _dev(out, torch.float32, "out"),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(x.device)))
    return out


def decode_layer_mxfp4_noalloc(logits: torch.Tensor, x: torch.Tensor, k: int, pool: ExpertPool, ids: torch.Tensor,
                               weights: torch.Tensor, grp: Grouping, y_rows: torch.Tensor,
                               out: torch.Tensor) -> torch.Tensor:
    """decode_layer_mxfp4 without a workspace: the library's static device scratch serves instead (nothing is
    allocated; calls that may overlap on one GPU race)."""
    if logits.shape[0] != 1 or x.shape[0] != 1:
        raise ValueError("decode_layer_mxfp4_noalloc takes one token")
    xb = x.view(torch.int16) if x.dtype == torch.bfloat16 else x
    _check("moe_decode_layer_mxfp4_noalloc", lib().moe_decode_layer_mxfp4_noalloc(
        _dev(logits, torch.float32, "logits"), _dev(xb, torch.int16, "x"), k, ctypes.byref(pool.weights),
        _dev(ids, torch.int32, "ids"), _dev(weights, torch.float32, "weights"),
        _dev(grp.expert_offsets, torch.int32, "expert_offsets"), _dev(grp.sorted_rows, torch.int32, "sorted_rows"),
        _dev(grp.row_pos, torch.int32, "row_pos"), _dev(grp.active, torch.int32, "active"),
        _dev(y_rows, torch.float32, "y_rows"), _dev(out, torch.float32, "out"), _stream(x.device)))
    return out


def decode_layer_rms_mxfp4(logits: torch.Tensor, y_prev: torch.Tensor, eps: float, x_next: torch.Tensor, k: int,
                           pool: ExpertPool, ids: torch.Tensor, weights: torch.Tensor, grp: Grouping,
                           workspace: torch.Tensor, y_rows: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """The next stacked layer from the previous layer's output: y_prev [1, H] fp32 -> x_next [1, H] bf16 (its RMS
    rescale), then the layer as decode_layer_mxfp4 on x_next; returns out."""
    if logits.shape[0] != 1 or y_prev.shape[0] != 1:
        raise ValueError("decode_layer_rms_mxfp4 takes one token")
    _check("moe_decode_layer_rms_mxfp4", lib().moe_decode_layer_rms_mxfp4(
        _dev(logits, torch.float32, "logits"), _dev(y_prev, torch.float32, "y_prev"), eps,
        _dev(x_next.view(torch.int16), torch.int16, "x_next"), k, ctypes.byref(pool.weights),
        _dev(ids, torch.int32, "ids"), _dev(weights, torch.float32, "weights"),
        _dev(grp.expert_offsets, torch.int32, "expert_offsets"), _dev(grp.sorted_rows, torch.int32, "sorted_rows"),
        _dev(grp.row_pos, torch.int32, "row_pos"), _dev(grp.active, torch.int32, "active"),
        _dev(y_rows, torch.float32, "y_rows"), _dev(out, torch.float32, "out"),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(y_prev.device)))
    return out


def combine(y_rows: torch.Tensor, weights: torch.Tensor, row_pos: torch.Tensor,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    T, k = weights.shape
    H = y_rows.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=y_rows.device)
    _check("moe_combine", lib().moe_combine(
        _dev(y_rows, torch.float32, "y_rows"), _dev(weights, torch.float32, "weights"),
        _dev(row_pos, torch.int32, "row_pos"), T, k, H, _dev(out, torch.float32, "out"), _stream(y_rows.device)))
    return out


def rms_rescale_bf16(y: torch.Tensor, eps: float = 1e-6, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Returns bf16 x_next [T, H] as a bfloat16 tensor."""
    T, H = y.shape
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _check("moe_rms_rescale_bf16", lib().moe_rms_rescale_bf16(
        _dev(y, torch.float32, "y"), T, H, eps, _dev(out.view(torch.int16), torch.int16, "x_next"),
        _stream(y.device)))
    return out


def route_group_one(logits: torch.Tensor, k: int, ids: torch.Tensor, weights: torch.Tensor,
                    out: Grouping) -> Grouping:
    """route_topk then group_rows for one token, in one launch; logits [1, E]."""
    T, E = logits.shape
    if T != 1:
        raise ValueError("route_group_one takes one token")
    _check("moe_route_group_one", lib().moe_route_group_one(
        _dev(logits, torch.float32, "logits"), E, k, _dev(ids, torch.int32, "ids"),
        _dev(weights, torch.float32, "weights"), _dev(out.expert_offsets, torch.int32, "expert_offsets"),
        _dev(out.sorted_rows, torch.int32, "sorted_rows"), _dev(out.row_pos, torch.int32, "row_pos"),
        _dev(out.active, torch.int32, "active"), _stream(logits.device)))
    return out


def combine_rms_bf16(y_rows: torch.Tensor, weights: torch.Tensor, row_pos: torch.Tensor, out: torch.Tensor,
                     x_next: torch.Tensor, eps: float = 1e-6) -> torch.Tensor:
    """combine into out [T, H] fp32, then x_next [T, H] bf16 = its RMS rescale, in one launch."""
    T, k = weights.shape
    H = y_rows.shape[1]
    _check("moe_combine_rms_bf16", lib().moe_combine_rms_bf16(
        _dev(y_rows, torch.float32, "y_rows"), _dev(weights, torch.float32, "weights"),
        _dev(row_pos, torch.int32, "row_pos"), T, k, H, eps, _dev(out, torch.float32, "out"),
        _dev(x_next.view(torch.int16), torch.int16, "x_next"), _stream(y_rows.device)))
    return x_next


def router_logits(x: torch.Tensor, w_router: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """logits [T, E] fp32 = x [T, H] (bf16) . w_router [E, H] (fp32)^T."""
    T, H = x.shape
    E = w_router.shape[0]
    xb = x.view(torch.int16) if x.dtype == torch.bfloat16 else x
    if out is None:
        out = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _check("moe_router_logits", lib().moe_router_logits(
        _dev(xb, torch.int16, "x"), T, H, _dev(w_router, torch.float32, "w_router"), E,
        _dev(out, torch.float32, "logits"), _stream(x.device)))
    return out
