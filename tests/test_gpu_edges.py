"""Edge cases of the HIP path against the oracle and against exact values:

- the fp32 -> bf16 rounding of the RMS rescale (the separate kernel, the
  combine + rescale launch and the rescale prologue inside the one-token
  gate/up launch) bit for bit against torch's own float32 -> bfloat16 cast;
- the hand-computed single-expert examples (tests/golden/single_expert.json)
  on the one-token decode kernels, the small-shape GEMV and the grouped GEMM,
  exactly where the values are exact;
- weight scale bytes over the whole finite range 0..252 (including the
  subnormal 2^-127 of byte 0) on every kernel family, with activations
  scaled per token so that each regime's output is finite: the register
  GEMVs of a batch, the one-token decode kernels and the grouped GEMM,
  whose activation terms then cover h blocks from 2^-139 to 2^116.

Scale bytes 253 and 254 are outside the domain: the dequantized value
E2M1 * 2^(s-127) of a code of magnitude 2 or more overflows fp32 there, so
the plain definition itself is not finite.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from mxfp4_routed_expert_02_amd import ExpertPool, combine_rms_bf16, decode_layer_rms_mxfp4, rms_rescale_bf16
from mxfp4_routed_expert_02_amd import synth, workspace_bytes
from mxfp4_routed_expert_02_amd.layer import RoutedExpertLayer
from tests import bf16_patterns as bf16p
from tests.gpu_common import assert_close, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _torch_bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# ---------------------------------------------------------- bf16 rounding --
def test_rms_rescale_rounding_matches_torch():
    y, tt = bf16p.anchored_rows()
    want = _torch_bf16_bits(tt)
    yd = torch.from_numpy(y).to(DEV)
    for eps in (0.0, 1e-6):
        x = _bits(rms_rescale_bf16(yd, eps))
        assert np.all(x[:, 0] == 0x4100)
        bad = np.nonzero(x[:, 1:] != want)
        assert bad[0].size == 0, [(hex(tt.view(np.uint32)[r, c]), hex(x[r, 1 + c]), hex(want[r, c]))
                                  for r, c in zip(*bad)][:8]
    # the combine + rescale launch: one routed row per token with weight 1.0,
    # so its combine reproduces the row and the rescale sees the same y
    T, H = y.shape
    w = torch.ones((T, 1), dtype=torch.float32, device=DEV)
    row_pos = torch.arange(T, dtype=torch.int32, device=DEV)
    out = torch.empty((T, H), dtype=torch.float32, device=DEV)
    xn = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    combine_rms_bf16(yd, w, row_pos, out, xn, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(out, yd)
    x = _bits(xn)
    assert np.array_equal(x[:, 1:], want) and np.all(x[:, 0] == 0x4100)


def test_decode_rms_prologue_rounding_matches_torch():
    """The rescale inside the one-token gate/up launch (decode shape H 7168,
    I 1536): x_next bit for bit as torch rounds the exact rescaled row."""
    y, trow, anchor = bf16p.anchored_row_7168()
    wl = synth.Workload("rms_prologue", E=96, H=7168, I=1536, k=16, T=1, pool=44, sub=44)
    pool = ExpertPool(synth.device_pool_slabs(0, wl.pool, 0, wl.E, wl.H, wl.I, DEV), wl.H, wl.I)
    L = RoutedExpertLayer(wl.E, wl.H, wl.I, wl.k, 1, DEV)
    lg = torch.from_numpy(synth.router_logits(0, wl)).to(DEV)
    yd = torch.from_numpy(y.reshape(1, -1)).to(DEV)
    xn = torch.empty((1, wl.H), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((1, wl.H), dtype=torch.float32, device=DEV)
    for eps in (0.0, 1e-6):
        L.step_rms(yd, lg, pool, out, xn, eps)
        torch.cuda.synchronize()
        got = _bits(xn)[0]
        want = _torch_bf16_bits(trow)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, [(int(i), hex(trow.view(np.uint32)[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


# --------------------------------------------------------- golden experts --
def _uniform_slab(H, I, gate_byte, up_byte, down_byte, scale=127, up_scale=None, down_scale=None):
    qb, sb = I * H // 2, I * H // 32
    parts = [np.full(qb, gate_byte, np.uint8), np.full(sb, scale, np.uint8),
             np.full(qb, up_byte, np.uint8), np.full(sb, scale if up_scale is None else up_scale, np.uint8),
             np.full(qb, down_byte, np.uint8), np.full(sb, scale if down_scale is None else down_scale, np.uint8)]
    return np.concatenate(parts)[None, :].copy()


GOLDEN_SHAPES = [  # H, I, T: the small-shape GEMV, the one-token decode kernels, the grouped GEMM
    (32, 32, 1), (7168, 1536, 1), (512, 512, 24)]


@pytest.mark.parametrize("H,I,T", GOLDEN_SHAPES, ids=[f"H{h}_I{i}_T{t}" for h, i, t in GOLDEN_SHAPES])
def test_golden_single_expert(H, I, T):
    """x = 1.0 everywhere, one expert, k = 1.  With every weight 1.0 the
    layer gives g = u = H, h = H * H (SiLU(H) = H in fp32 for H >= 32) and
    out = I * H^2 exactly, at every shape; a +1 up scale and a -1 down scale
    keep out and double h; a zero gate gives exactly 0; a -1.0 gate gives
    the closed form -H^2 / (1 + e^H)."""
    spec = json.load(open(os.path.join(GOLDEN, "single_expert.json")))
    for case in spec["cases"]:
        slab = _uniform_slab(H, I, case["gate_byte"], case["up_byte"], case["down_byte"], case["scale"],
                             case.get("up_scale"), case.get("down_scale"))
        say(f"golden {case['name']} H={H} I={I} T={T}")
        pool = ExpertPool(torch.from_numpy(slab).to(DEV), H, I)
        L = RoutedExpertLayer(1, H, I, 1, T, DEV)
        x = torch.full((T, H), 1.0, dtype=torch.bfloat16, device=DEV)
        out = L(x, torch.zeros((T, 1), dtype=torch.float32, device=DEV), pool)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ref = oracle.layer(np.full((T, H), 0x3F80, np.uint16), np.zeros((T, 1), np.float32), 1,
                           oracle.Pool(slab, H, I), nthreads=8)["out"]
        if case["name"] in ("ones", "scale_up_down"):
            want = float(I) * float(H) * float(H)
            assert np.all(ref == np.float32(want)) and np.all(got == np.float32(want)), (got.min(), got.max())
        elif case["name"] == "zero_gate":
            assert np.all(got == 0.0) and np.all(ref == 0.0)
        else:  # negative gate: -H^2/(1+e^H) per h, times I
            h = -float(H) * float(H) / (1.0 + math.exp(min(H, 700)))
            want = I * h
            if abs(want) > 1e-30:
                np.testing.assert_allclose(got, want, rtol=1e-5)
                np.testing.assert_allclose(ref, want, rtol=1e-5)
            else:
                assert np.all(np.abs(got) <= 1e-30) and np.all(np.abs(ref) <= 1e-30)
        if H == 32 and case["exact"]:
            assert np.all(got == np.float32(case["out"]))


# ------------------------------------------------------ scale-byte regimes --
# (gate/up scale centre, half width, log2 of the token's activation scale,
#  down scale centre, half width): each regime keeps its output finite while
# its scale bytes cover one band; together they span 0..252
REGIMES = [(8, 8, 100, 119, 8), (40, 8, 80, 94, 8), (72, 8, 40, 110, 8), (104, 8, -38, 203, 8),
           (136, 8, -20, 102, 8), (168, 8, -60, 119, 8), (200, 8, -39, 8, 8), (232, 8, -100, 70, 8),
           (244, 8, -100, 42, 8), (104, 8, -43, 244, 8), (72, 8, -17, 224, 8), (72, 8, -20, 230, 8),
           (1, 1, 110, 127, 4), (200, 8, -30, 1, 1)]


def _regime_inputs(H, I, ntok, seed):
    rng = np.random.default_rng(seed)
    E = len(REGIMES)
    qb, sb = I * H // 2, I * H // 32
    slabs = np.zeros((E, 3 * (qb + sb)), np.uint8)
    for e, (cg, wg, _, cd, wd) in enumerate(REGIMES):
        parts = []
        for m in range(3):
            c, w = (cg, wg) if m < 2 else (cd, wd)
            parts.append(rng.integers(0, 256, qb, dtype=np.uint8))
            parts.append(np.clip(rng.integers(c - w, c + w + 1, sb), 0, 252).astype(np.uint8))
        slabs[e] = np.concatenate(parts)
    T = E * ntok
    xf = rng.standard_normal((T, H)).astype(np.float32)
    for e, (_, _, a, _, _) in enumerate(REGIMES):
        xf[e * ntok:(e + 1) * ntok] *= np.float32(2.0 ** a)
    x = _torch_bf16_bits(xf)
    logits = np.zeros((T, E), np.float32)
    logits[np.arange(T), np.arange(T) // ntok] = 10.0  # token t -> expert t // ntok, k = 1
    return slabs, x, logits


def _check_regimes(slabs, x, logits, H, I, ntok, got_out, got_y):
    ref = oracle.layer(x, logits, 1, oracle.Pool(slabs, H, I), nthreads=16)
    o = synth.slab_offsets(H, I)
    qb, sb = I * H // 2, I * H // 32
    scales = np.concatenate([slabs[:, o[n]:o[n] + sb].reshape(-1) for n in ("gate_s", "up_s", "down_s")])
    assert int(scales.min()) == 0 and int(scales.max()) == 252
    for e in range(len(REGIMES)):
        rows = slice(e * ntok, (e + 1) * ntok)  # k = 1 and tokens in expert order: sorted rows = tokens
        assert np.all(np.isfinite(ref["out"][rows]))
        assert_close(got_y[rows], ref["y_rows"][rows], f"regime {e} {REGIMES[e]} y_rows")
        assert_close(got_out[rows], ref["out"][rows], f"regime {e} out")


@pytest.mark.parametrize("H,I,ntok", [(512, 512, 24), (7168, 1536, 1)], ids=["gemm_H512_T336", "gemv_H7168_T14"])
def test_scale_byte_regimes_batch(H, I, ntok):
    """A batch over all regimes: 24 tokens per expert at H = I = 512 take the
    grouped GEMM; one token per expert at the decode shape (14 tokens) takes
    the register GEMVs."""
    slabs, x, logits = _regime_inputs(H, I, ntok, seed=5)
    say(f"scale regimes H={H} I={I}: {len(REGIMES)} experts x {ntok} tokens")
    pool = ExpertPool(torch.from_numpy(slabs).to(DEV), H, I)
    T = x.shape[0]
    L = RoutedExpertLayer(len(REGIMES), H, I, 1, T, DEV)
    xd = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    out = L(xd, torch.from_numpy(logits).to(DEV), pool)
    torch.cuda.synchronize()
    assert np.array_equal(L.grp.sorted_rows[:T].cpu().numpy(), np.arange(T))
    _check_regimes(slabs, x, logits, H, I, ntok, out.cpu().numpy(), L.y_rows[:T].cpu().numpy())


def test_scale_byte_regimes_decode():
    """Each regime's token alone through the one-token decode kernels (top-k
    inside the gate/up launch, down + combine in one launch)."""
    H, I = 7168, 1536
    slabs, x, logits = _regime_inputs(H, I, 1, seed=6)
    pool = ExpertPool(torch.from_numpy(slabs).to(DEV), H, I)
    E = len(REGIMES)
    L = RoutedExpertLayer(E, H, I, 1, 1, DEV)
    outs, ys = [], []
    for t in range(E):
        xd = torch.from_numpy(x[t:t + 1].view(np.int16)).to(DEV).view(torch.bfloat16)
        o = L(xd, torch.from_numpy(logits[t:t + 1]).to(DEV), pool)
        torch.cuda.synchronize()
        assert int(L.ids[0, 0].item()) == t
        outs.append(o.cpu().numpy()[0])
        ys.append(L.y_rows[0].cpu().numpy())
    _check_regimes(slabs, x, logits, H, I, 1, np.stack(outs), np.stack(ys))
