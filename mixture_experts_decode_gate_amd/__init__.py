"""Python binding of libmoe.so, the MI355X routed-MoE decode/verify layer.

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe.so.  The names match the C ABI in include/moe.h:

    moe_workspace_bytes(cfg)                         -> int
    moe_workspace_layout(cfg)                        -> MoeWsLayout
    moe_route(cfg, w, x, topk_ids, topk_w, ws)       router + top-k
    moe_union(topk_ids, union_ids, union_count, slot_to_union, row_mask, num_experts)
    moe_forward(cfg, w, x, out, ws)                  the whole layer
    moe_forward_static(cfg, w, x, out)               the whole layer, library-held workspace (no allocation)
    moe_forward_token_major(cfg, w, x, out, ws)      the layer without the union (one slot per pair)
    moe_forward_prefill(cfg, w, x, out, ws)          any number of rows, in sub-chunks of up to 16 rows
    moe_forward_timed(cfg, w, x, out, ws, events)    same, with per-stage events
    moe_read_probe(src, sink)                        streaming-read ceiling (measurement aid)
    moe_union_local(topk_ids, lo, hi, union_ids, union_count, slot_to_union, row_mask, num_experts)
    moe_forward_ep_partial(cfg, w, x, partial, lo, hi, ws)   one GPU's expert-parallel share
    moe_ep_combine(cfg, reduced, out, ws)            shared expert added after the reduce

Tensors are torch CUDA (HIP) tensors; torch only provides device memory and
the current stream.  There is no CPU fallback: loading fails loudly when the
library is missing.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
MOE_ROUTE_SOFTMAX, MOE_ROUTE_SIGMOID_BIAS = 0, 1
MOE_MAX_ROWS, MOE_MAX_IDS, MOE_MAX_EXPERTS, MOE_MAX_DIM, MOE_MAX_INTER = 16, 128, 1024, 8192, 4096
MOE_BLOCK_IDS, MOE_MAX_CHUNK_ROWS = 64, 36
MOE_STATIC_SCRATCH_BYTES = 8 << 20
# Expert activations and outputs in the workspace are stored by (row, expert)
# pair: pair r*k + j is row r's j-th routed expert, rows*k + r row r's shared expert.
MAX_PAIRS = MOE_MAX_IDS + MOE_MAX_ROWS

STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE",
                4: "MOE_ERR_DEVICE"}


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class MoeConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("moe_inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32), ("route_kind", ctypes.c_int32),
                ("norm_topk_prob", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_float)]

    @classmethod
    def from_shape(cls, s) -> "MoeConfig":
        """From any object with hidden, num_experts, top_k, moe_inter, shared_inter,
        route_kind, norm_topk_prob and routed_scaling_factor attributes."""
        return cls(int(s.hidden), int(s.num_experts), int(s.top_k), int(s.moe_inter), int(s.shared_inter),
                   int(s.route_kind), int(bool(s.norm_topk_prob)), float(s.routed_scaling_factor))


class MoeNvfp4(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("scale2", ctypes.c_float)]


class MoeExpertTable(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("scale2", ctypes.c_void_p)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("correction_bias", ctypes.c_void_p),
                ("gate", MoeExpertTable), ("up", MoeExpertTable), ("down", MoeExpertTable),
                ("shared_gate", MoeNvfp4), ("shared_up", MoeNvfp4), ("shared_down", MoeNvfp4),
                ("shared_expert_gate", ctypes.c_void_p), ("router_nvfp4", MoeNvfp4)]


class MoeWsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "logits", "score", "gamma", "topk_ids", "topk_w", "union_ids", "union_count", "slot_to_union",
        "row_mask", "slot_info", "segments", "act", "y", "total")]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so (built by ``python -m mixture_experts_decode_gate_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m mixture_experts_decode_gate_amd.build`")
    # torch's HIP runtime must be loaded first: libmoe.so then binds to that
    # same runtime (same soname) instead of bringing in a second copy.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, C = ctypes.POINTER, ctypes
    lib.moe_workspace_bytes.argtypes = [P(MoeConfig)]
    lib.moe_workspace_bytes.restype = C.c_size_t
    lib.moe_workspace_layout.argtypes = [P(MoeConfig), P(MoeWsLayout)]
    lib.moe_workspace_layout.restype = C.c_int
    lib.moe_route.argtypes = [P(MoeConfig), P(MoeWeights), C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                              C.c_void_p, C.c_size_t, C.c_void_p]
    lib.moe_route.restype = C.c_int
    lib.moe_union.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                              C.c_void_p, C.c_void_p]
    lib.moe_union.restype = C.c_int
    lib.moe_forward.argtypes = [P(MoeConfig), P(MoeWeights), C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                                C.c_size_t, C.c_void_p]
    lib.moe_forward.restype = C.c_int
    lib.moe_forward_static.argtypes = [P(MoeConfig), P(MoeWeights), C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p]
    lib.moe_forward_static.restype = C.c_int
    lib.moe_forward_prefill.argtypes = lib.moe_forward.argtypes
    lib.moe_forward_prefill.restype = C.c_int
    lib.moe_forward_token_major.argtypes = lib.moe_forward.argtypes
    lib.moe_forward_token_major.restype = C.c_int
    lib.moe_union_local.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                    C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
    lib.moe_union_local.restype = C.c_int
    lib.moe_forward_ep_partial.argtypes = [P(MoeConfig), P(MoeWeights), C.c_void_p, C.c_void_p, C.c_int32,
                                           C.c_int32, C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.moe_forward_ep_partial.restype = C.c_int
    lib.moe_ep_combine.argtypes = [P(MoeConfig), C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t,
                                   C.c_void_p]
    lib.moe_ep_combine.restype = C.c_int
    lib.moe_read_probe.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p]
    lib.moe_read_probe.restype = C.c_int
    lib.moe_read_probe_sink_words.argtypes = []
    lib.moe_read_probe_sink_words.restype = C.c_int32
    lib.moe_forward_timed.argtypes = [P(MoeConfig), P(MoeWeights), C.c_void_p, C.c_void_p, C.c_int32,
                                      C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p]
    lib.moe_forward_timed.restype = C.c_int
    lib.moe_num_stages.argtypes = []
    lib.moe_num_stages.restype = C.c_int32
    lib.moe_stage_name.argtypes = [C.c_int32]
    lib.moe_stage_name.restype = C.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = C.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, load().moe_last_error().decode())


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return int(getattr(stream, "cuda_stream", stream))


def moe_workspace_bytes(cfg: MoeConfig) -> int:
    return int(load().moe_workspace_bytes(ctypes.byref(cfg)))


def moe_workspace_layout(cfg: MoeConfig) -> MoeWsLayout:
    L = MoeWsLayout()
    _check(load().moe_workspace_layout(ctypes.byref(cfg), ctypes.byref(L)))
    return L


def moe_route(cfg: MoeConfig, w: MoeWeights, x, topk_ids, topk_w, ws, stream=None) -> None:
    """x [rows, h] bf16 -> topk_ids [rows, k] int32, topk_w [rows, k] float32 (device tensors)."""
    _check(load().moe_route(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), int(x.shape[0]), _ptr(topk_ids),
                            _ptr(topk_w), _ptr(ws), int(ws.numel() * ws.element_size()), _stream(stream)))


def moe_union(topk_ids, union_ids, union_count, slot_to_union, row_mask=None, num_experts: int = MOE_MAX_EXPERTS,
              stream=None) -> None:
    """topk_ids [rows, k] int32 -> union_ids [MOE_MAX_IDS], union_count [1], slot_to_union [rows*k],
    row_mask [MOE_MAX_IDS] (int32 / uint32 device tensors)."""
    rows, k = int(topk_ids.shape[0]), int(topk_ids.shape[1])
    _check(load().moe_union(_ptr(topk_ids), rows, k, int(num_experts), _ptr(union_ids), _ptr(union_count),
                            _ptr(slot_to_union), _ptr(row_mask), _stream(stream)))


def moe_forward(cfg: MoeConfig, w: MoeWeights, x, out, ws, stream=None) -> None:
    """x [rows, h] bf16 -> out [rows, h] bf16 (device tensors); ws a uint8 device tensor."""
    _check(load().moe_forward(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), _ptr(out), int(x.shape[0]), _ptr(ws),
                              int(ws.numel() * ws.element_size()), _stream(stream)))


def moe_forward_static(cfg: MoeConfig, w: MoeWeights, x, out, stream=None) -> None:
    """moe_forward with the library's own per-GPU workspace: allocates nothing."""
    _check(load().moe_forward_static(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), _ptr(out), int(x.shape[0]),
                                     _stream(stream)))


def moe_forward_prefill(cfg: MoeConfig, w: MoeWeights, x, out, ws, stream=None) -> None:
    """x [rows, h] bf16 (any rows >= 1) -> out [rows, h] bf16, in sub-chunks of the most rows one
    moe_forward takes for this config (up to MOE_MAX_ROWS)."""
    _check(load().moe_forward_prefill(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), _ptr(out), int(x.shape[0]),
                                      _ptr(ws), int(ws.numel() * ws.element_size()), _stream(stream)))


def moe_forward_token_major(cfg: MoeConfig, w: MoeWeights, x, out, ws, stream=None) -> None:
    """moe_forward with one slot per (row, selected expert) instead of the union."""
    _check(load().moe_forward_token_major(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), _ptr(out), int(x.shape[0]),
                                          _ptr(ws), int(ws.numel() * ws.element_size()), _stream(stream)))


def moe_union_local(topk_ids, lo: int, hi: int, union_ids, union_count, slot_to_union, row_mask=None,
                    num_experts: int = MOE_MAX_EXPERTS, stream=None) -> None:
    """moe_union over the ids in [lo, hi) only; other slots map to -1."""
    rows, k = int(topk_ids.shape[0]), int(topk_ids.shape[1])
    _check(load().moe_union_local(_ptr(topk_ids), rows, k, int(num_experts), int(lo), int(hi), _ptr(union_ids),
                                  _ptr(union_count), _ptr(slot_to_union), _ptr(row_mask), _stream(stream)))


def moe_forward_ep_partial(cfg: MoeConfig, w: MoeWeights, x, partial, lo: int, hi: int, ws, stream=None) -> None:
    """x [rows, h] bf16 -> partial [rows, h] float32: the routed sum over experts in [lo, hi)."""
    _check(load().moe_forward_ep_partial(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), _ptr(partial),
                                         int(x.shape[0]), int(lo), int(hi), _ptr(ws),
                                         int(ws.numel() * ws.element_size()), _stream(stream)))


def moe_ep_combine(cfg: MoeConfig, reduced, out, ws, stream=None) -> None:
    """reduced [rows, h] float32 -> out [rows, h] bf16 = reduced + gate * shared expert."""
    _check(load().moe_ep_combine(ctypes.byref(cfg), _ptr(reduced), _ptr(out), int(reduced.shape[0]), _ptr(ws),
                                 int(ws.numel() * ws.element_size()), _stream(stream)))


def moe_forward_timed(cfg: MoeConfig, w: MoeWeights, x, out, ws, events: Sequence, stream=None) -> None:
    """moe_forward whose stage i kernel records events[2i] at its start and events[2i+1] at its end.
    ``events`` holds hipEvent_t handles (ints, objects with a ``handle`` attribute, or None)."""
    n = 2 * moe_num_stages()
    ev = list(events) + [None] * n
    arr = (ctypes.c_void_p * n)(*[(0 if e is None else int(getattr(e, "handle", e))) for e in ev[:n]])
    _check(load().moe_forward_timed(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), _ptr(out), int(x.shape[0]),
                                    _ptr(ws), int(ws.numel() * ws.element_size()), _stream(stream), arr))


def moe_read_probe(src, sink, stream=None) -> None:
    """Read every byte of the device tensor ``src`` once (streaming-read ceiling);
    ``sink`` holds at least moe_read_probe_sink_words() uint32 words."""
    _check(load().moe_read_probe(_ptr(src), int(src.numel() * src.element_size()), _ptr(sink), _stream(stream)))


def moe_read_probe_sink_words() -> int:
    return int(load().moe_read_probe_sink_words())


def moe_num_stages() -> int:
    return int(load().moe_num_stages())


def moe_stage_names():
    lib = load()
    return [lib.moe_stage_name(i).decode() for i in range(lib.moe_num_stages())]
