"""Helpers for the GPU tests: upload seeded inputs, run the C ABI, read results.

Nothing here computes any part of the layer; expected values come from the
oracle (``oracle/``) on the same seeded inputs.
"""

from __future__ import annotations

import numpy as np

import synth


def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def moe_mod():
    import mixture_experts_decode_gate_amd as moe
    moe.load()  # fails loudly when libmoe.so is missing
    return moe


def upload(weights: "synth.MoeLayerWeights"):
    from mixture_experts_decode_gate_amd.device import DeviceLayer
    moe = moe_mod()
    cfg = moe.MoeConfig.from_shape(weights.shape)
    return DeviceLayer(cfg, weights.router_w, weights.bias, weights.shared_gate_vec, weights.shared, weights.expert)


def x_dev(bits: np.ndarray):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).cuda()


def ws_for(cfg, fill: int = 0xFF):
    """A workspace of moe_workspace_bytes(cfg), filled with ``fill``: the
    library reads nothing it has not written in the same call."""
    torch = torch_cuda()
    moe = moe_mod()
    return torch.full((moe.moe_workspace_bytes(cfg),), fill, dtype=torch.uint8, device="cuda")


def ws_read(ws, offset: int, dtype, count: int) -> np.ndarray:
    nb = np.dtype(dtype).itemsize * count
    return ws[offset:offset + nb].cpu().numpy().view(dtype).copy()


def out_bits(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def run_forward(dl, x_bits: np.ndarray, ws=None):
    torch = torch_cuda()
    moe = moe_mod()
    x = x_dev(x_bits)
    out = torch.zeros_like(x)
    ws = ws_for(dl.cfg) if ws is None else ws
    moe.moe_forward(dl.cfg, dl.weights, x, out, ws)
    torch.cuda.synchronize()
    return out_bits(out), ws


def output_errors(gpu_bits: np.ndarray, ref_bits: np.ndarray):
    """Per-row relative L2 error and max-abs error relative to the row's max |ref|."""
    g, r = bits_to_f64(gpu_bits), bits_to_f64(ref_bits)
    rel_l2 = np.linalg.norm(g - r, axis=-1) / np.maximum(np.linalg.norm(r, axis=-1), 1e-30)
    rel_max = np.abs(g - r).max(axis=-1) / np.maximum(np.abs(r).max(axis=-1), 1e-30)
    return rel_l2, rel_max


# Output tolerance: relative L2 per row <= 1e-2 and max-abs <= 2e-2 of the
# row's largest |value|.  bf16 rounding of silu(g)*u between the projections
# and of the output each add about 2^-9/sqrt(3) relative rms error, so the
# expected relative L2 is near 2e-3.
REL_L2_TOL = 1e-2
REL_MAX_TOL = 2e-2
# Routing weights: relative 1e-6.
W_RTOL = 1e-6
