"""Seeded synthetic inputs for the routed-MoE decode/verify layer.

This module only draws random numbers and packs them into the storage formats
the layer consumes (bf16 activations, fp32 router and shared-gate vectors,
NVFP4 expert weights).  It holds none of the layer's arithmetic: no decode,
no dot product, no routing.  Both the CPU oracle (``oracle/``) and the GPU
path (``mixture_experts_decode_gate_amd``) receive exactly these arrays.

Workloads follow the five synthetic configurations of the layer (tiny parity
case, 64/128/256-expert decode and verify shapes).  The pages the layer is
built from ("Function forward_moe" rustdoc and the two ``metrale_model_layers``
MoE source listings) describe no dataset: the routing trace and probe set they
measure on are not available, so these seeded inputs stand in for them, with
row correlation standing in for token-to-token correlation of a verify step.

Every tensor has its own numpy PCG64 substream keyed by
``(seed, kind, index, projection)`` so any single expert regenerates alone.
"""

from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# Substream kinds.
KIND_ROUTER = 0
KIND_BIAS = 1
KIND_SHARED_GATE_VEC = 2
KIND_EXPERT = 3
KIND_SHARED_EXPERT = 4
KIND_ACTIVATION = 5

PROJ_GATE, PROJ_UP, PROJ_DOWN = 0, 1, 2
PROJ_NAMES = ("gate", "up", "down")

ROUTE_SOFTMAX = 0
ROUTE_SIGMOID_BIAS = 1


@dataclasses.dataclass(frozen=True)
class MoeShape:
    """One layer shape plus its routing mode and activation recipe."""

    name: str
    hidden: int
    num_experts: int
    top_k: int
    moe_inter: int
    shared_inter: int
    rows: int
    route_kind: int
    norm_topk_prob: bool
    routed_scaling_factor: float
    # "normal": independent N(0,1) rows.  "correlated": row 0 = x0 and
    # rows r >= 1 = a*x0 + sqrt(1-a^2)*z_r.
    x_kind: str = "normal"
    row_corr: float = 0.0
    scale_sigma: float = 0.05  # E4M3 block scale = |N(0,1)| * scale_sigma
    seed: int = 0

    def with_rows(self, rows: int) -> "MoeShape":
        return dataclasses.replace(self, rows=rows, name=f"{self.name}_r{rows}")

    def expert_bytes(self, inter: Optional[int] = None) -> int:
        """Bytes of one NVFP4 expert (gate, up, down): codes + scales + scale2."""
        i = self.moe_inter if inter is None else inter
        per = i * self.hidden // 2 + i * self.hidden // 16 + 4
        return 3 * per


# Row correlation for the 256-expert K=4 verify shape: tuned (see
# tests/golden/tune_c3_row_corr.py) so that the mean expert union over steps 0..999 is close
# to the 23.35 experts the "Function forward_moe" rustdoc reports at K=4 in its
# "amortize PARTIALLY" note.
C3_ROW_CORR = 0.58  # mean union 23.39 over steps 0..999

CONFIGS: Dict[str, MoeShape] = {
    "c0_tiny": MoeShape("c0_tiny", 256, 16, 4, 128, 128, 1, ROUTE_SOFTMAX, True, 1.0),
    "c1_e64_decode": MoeShape("c1_e64_decode", 2048, 64, 8, 768, 768, 1, ROUTE_SOFTMAX, True, 1.0),
    "c2_e128_verify2": MoeShape(
        "c2_e128_verify2", 4096, 128, 8, 1536, 1536, 2, ROUTE_SIGMOID_BIAS, True, 2.5,
        x_kind="correlated", row_corr=0.8),
    "c3_e256_verify4": MoeShape(
        "c3_e256_verify4", 6144, 256, 8, 2048, 2048, 4, ROUTE_SIGMOID_BIAS, True, 2.5,
        x_kind="correlated", row_corr=C3_ROW_CORR),
    "c4_e256_prefill8": MoeShape(
        "c4_e256_prefill8", 6144, 256, 8, 2048, 2048, 8, ROUTE_SIGMOID_BIAS, True, 2.5,
        x_kind="normal"),
}
CONFIG_ORDER = list(CONFIGS)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


# ---------------------------------------------------------------- encoders
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def f32_to_e4m3fn_bytes(x: np.ndarray) -> np.ndarray:
    """Encode non-negative finite float32 to OCP E4M3FN bytes, RNE, saturating.

    Normal range (>= 2^-6): round the 23-bit mantissa to 3 bits (RNE) and
    rebias the exponent from 127 to 7.  Below 2^-6: the value is m * 2^-9 with
    m = rint(x * 512) (ties to even), which also yields byte 8 (= 2^-6) on
    carry.  Values above 448 saturate to 0x7E.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if np.any(x < 0) or not np.all(np.isfinite(x)):
        raise ValueError("encoder expects non-negative finite scales")
    out = np.empty(x.shape, dtype=np.uint8)
    small = x < np.float32(2.0 ** -6)
    m = np.rint(x[small].astype(np.float64) * 512.0).astype(np.uint8)
    out[small] = m
    big = ~small
    u = x[big].view(np.uint32).astype(np.int64)
    u = u + 0x7FFFF + ((u >> 20) & 1)
    e = (u >> 23) - 127 + 7
    mant = (u >> 20) & 7
    code = (e << 3) | mant
    code = np.where((e > 15) | (code > 0x7E), 0x7E, code)
    out[big] = code.astype(np.uint8)
    return out


# ---------------------------------------------------------------- tensors
@dataclasses.dataclass
class Nvfp4Tensor:
    """One untransposed NVFP4 matrix [n, k]: K-contiguous rows.

    packed : uint8 [n, k/2]   two E2M1 codes per byte, low nibble = even column
    scales : uint8 [n, k/16]  one E4M3FN scale per 16 consecutive columns
    scale2 : float            per-tensor fp32 scale
    """

    n: int
    k: int
    packed: np.ndarray
    scales: np.ndarray
    scale2: float = 1.0


def nvfp4_random(shape: MoeShape, n: int, k: int, *key: int) -> Nvfp4Tensor:
    rng = _rng(shape.seed, *key)
    packed = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    s = np.abs(rng.standard_normal((n, k // 16), dtype=np.float32)) * np.float32(shape.scale_sigma)
    return Nvfp4Tensor(n, k, packed, f32_to_e4m3fn_bytes(s), 1.0)


def expert_tensor(shape: MoeShape, expert: int, proj: int) -> Nvfp4Tensor:
    """Routed expert ``expert``'s projection: gate/up [I, h], down [h, I]."""
    n, k = (shape.moe_inter, shape.hidden) if proj != PROJ_DOWN else (shape.hidden, shape.moe_inter)
    return nvfp4_random(shape, n, k, KIND_EXPERT, expert, proj)


def shared_tensor(shape: MoeShape, proj: int) -> Nvfp4Tensor:
    n, k = (shape.shared_inter, shape.hidden) if proj != PROJ_DOWN else (shape.hidden, shape.shared_inter)
    return nvfp4_random(shape, n, k, KIND_SHARED_EXPERT, 0, proj)


def router_weight(shape: MoeShape) -> np.ndarray:
    """fp32 [E, h] ~ N(0, 1/h)."""
    rng = _rng(shape.seed, KIND_ROUTER, 0, 0)
    w = rng.standard_normal((shape.num_experts, shape.hidden)) / math.sqrt(shape.hidden)
    return w.astype(np.float32)


# Mean of e2m1(c)^2 over the 16 codes: (0 + .25 + 1 + 2.25 + 4 + 9 + 16 + 36) / 8.
_E2M1_MEAN_SQ = 8.5625


def router_nvfp4(shape: MoeShape) -> Nvfp4Tensor:
    """NVFP4 [E, h] router: codes and block scales drawn as for the experts, and
    a per-tensor scale2 that brings the weights' variance to about 1/h, as the
    fp32 router's N(0, 1/h): Var(w) = mean(e2m1^2) * E[scale^2] * scale2^2
    with E[scale^2] = scale_sigma^2."""
    t = nvfp4_random(shape, shape.num_experts, shape.hidden, KIND_ROUTER, 0, 1)
    t.scale2 = float(np.float32(1.0 / math.sqrt(_E2M1_MEAN_SQ * shape.scale_sigma ** 2 * shape.hidden)))
    return t


def correction_bias(shape: MoeShape) -> Optional[np.ndarray]:
    """fp32 [E] ~ U(-0.1, 0.1) for sigmoid routing, else None."""
    if shape.route_kind != ROUTE_SIGMOID_BIAS:
        return None
    rng = _rng(shape.seed, KIND_BIAS, 0, 0)
    return rng.uniform(-0.1, 0.1, size=shape.num_experts).astype(np.float32)


def shared_gate_vector(shape: MoeShape) -> np.ndarray:
    """fp32 [h] ~ N(0, 1/h): the shared-expert gate vector."""
    rng = _rng(shape.seed, KIND_SHARED_GATE_VEC, 0, 0)
    return (rng.standard_normal(shape.hidden) / math.sqrt(shape.hidden)).astype(np.float32)


def activations(shape: MoeShape, step: int = 0, rows: Optional[int] = None) -> np.ndarray:
    """bf16 bits uint16 [rows, h] for step ``step``.

    Rows are drawn in float64, rounded to float32 and then to bf16.  With
    ``x_kind == "correlated"``, row 0 is x0 and row r >= 1 mixes x0 with an
    independent draw so consecutive verify rows share part of their routing.
    The first ``rows`` rows of a step never depend on ``rows``.
    """
    rows = shape.rows if rows is None else rows
    rng = _rng(1, KIND_ACTIVATION, step, 0)
    base = rng.standard_normal((max(rows, 1), shape.hidden))
    if shape.x_kind == "correlated":
        a = shape.row_corr
        b = math.sqrt(max(0.0, 1.0 - a * a))
        x = base.copy()
        x[1:] = a * base[0:1] + b * base[1:]
    elif shape.x_kind == "normal":
        x = base
    else:
        raise ValueError(shape.x_kind)
    return f32_to_bf16_bits(x[:rows].astype(np.float32))


# ---------------------------------------------------------------- a layer
@dataclasses.dataclass
class MoeLayerWeights:
    shape: MoeShape
    router_w: object  # fp32 [E, h] array, or an Nvfp4Tensor [E, h]
    bias: Optional[np.ndarray]
    shared_gate_vec: np.ndarray
    shared: Tuple[Nvfp4Tensor, Nvfp4Tensor, Nvfp4Tensor]
    _experts: Dict[Tuple[int, int], Nvfp4Tensor] = dataclasses.field(default_factory=dict)
    lazy: bool = True

    def expert(self, e: int, proj: int) -> Nvfp4Tensor:
        key = (e, proj)
        t = self._experts.get(key)
        if t is None:
            t = expert_tensor(self.shape, e, proj)
            if not self.lazy:
                self._experts[key] = t
        return t

    def materialise(self, threads: int = 8) -> None:
        """Generate every routed expert now (parallel over experts)."""
        self.lazy = False
        keys = [(e, p) for e in range(self.shape.num_experts) for p in range(3)
                if (e, p) not in self._experts]
        with ThreadPoolExecutor(max(1, threads)) as ex:
            for key, t in zip(keys, ex.map(lambda kp: expert_tensor(self.shape, *kp), keys)):
                self._experts[key] = t


def layer_weights(shape: MoeShape, materialise: bool = False, threads: int = 8,
                  router: str = "fp32") -> MoeLayerWeights:
    """``router`` "fp32" (dense [E, h]) or "nvfp4" (an Nvfp4Tensor [E, h] in router_w)."""
    if router not in ("fp32", "nvfp4"):
        raise ValueError(router)
    w = MoeLayerWeights(
        shape=shape,
        router_w=router_weight(shape) if router == "fp32" else router_nvfp4(shape),
        bias=correction_bias(shape),
        shared_gate_vec=shared_gate_vector(shape),
        shared=tuple(shared_tensor(shape, p) for p in range(3)),
    )
    if materialise:
        w.materialise(threads)
    return w

