"""GPU parity on seeded random layer shapes (every entry point of the layer).

Each case draws h, E, top_k, rows, I and Is (multiples of 32, partial
2048-column chunks included), the routing kind, norm_topk_prob,
routed_scaling_factor, a gated or ungated shared expert and an fp32 or NVFP4
router, then checks moe_forward against the oracle (ids, weights, the union,
per-row output tolerance), moe_forward_token_major byte for byte against
moe_forward, and a random expert-parallel split against the oracle.  The
seed is fixed; cases are never redrawn.
"""

import numpy as np
import pytest

import synth

from test_gpu_forward import check_against_oracle, check_ep_shares, check_token_major
from gpu_common import upload

pytestmark = pytest.mark.gpu


def random_case(i):
    rng = np.random.default_rng([2026, i])
    k = int(rng.integers(1, 9))
    E = int(rng.integers(k, 97))
    rows = int(rng.integers(1, min(8, 64 // k) + 1))
    h = 32 * int(rng.integers(2, 81))        # 64 .. 2560
    inter = 32 * int(rng.integers(1, 21))    # 32 .. 640
    shared = 32 * int(rng.integers(1, 21))
    kind = int(rng.integers(0, 2))
    norm = bool(rng.integers(0, 2))
    rsf = float(np.float32(rng.uniform(0.5, 3.0))) if kind == synth.ROUTE_SIGMOID_BIAS else 1.0
    shape = synth.MoeShape(f"rand{i}", h, E, k, inter, shared, rows, kind, norm, rsf, seed=100 + i)
    router = "nvfp4" if rng.integers(0, 2) else "fp32"
    gated = bool(rng.integers(0, 3))          # one case in three ungated
    cut = sorted(int(c) for c in rng.integers(0, E + 1, size=2))
    return shape, router, gated, [(0, cut[0]), (cut[0], cut[1]), (cut[1], E)]


@pytest.mark.parametrize("i", range(12))
def test_random_shape(i):
    shape, router, gated, ranges = random_case(i)
    weights = synth.layer_weights(shape, router=router)
    if not gated:
        weights.shared_gate_vec = None
    dl = upload(weights)
    x = synth.activations(shape, i)
    print(shape, router, "gated" if gated else "ungated", ranges)
    check_against_oracle(weights, dl, x)
    check_token_major(dl, x)
    check_ep_shares(weights, dl, x, ranges)


def random_case_wide(i):
    """More than 8 rows (up to 16, top_k * rows up to 128; hidden up to 4096
    so every row of x fits the gate/up sweep's LDS)."""
    rng = np.random.default_rng([2027, i])
    k = int(rng.integers(1, 13))
    E = int(rng.integers(k, 300))
    rows = int(rng.integers(9, min(16, 128 // k) + 1)) if 128 // k >= 9 else int(rng.integers(1, 128 // k + 1))
    h = 32 * int(rng.integers(2, 129))       # 64 .. 4096
    inter = 32 * int(rng.integers(1, 21))
    shared = 32 * int(rng.integers(1, 21))
    kind = int(rng.integers(0, 2))
    norm = bool(rng.integers(0, 2))
    rsf = float(np.float32(rng.uniform(0.5, 3.0))) if kind == synth.ROUTE_SIGMOID_BIAS else 1.0
    shape = synth.MoeShape(f"wide{i}", h, E, k, inter, shared, rows, kind, norm, rsf, seed=200 + i)
    cut = sorted(int(c) for c in rng.integers(0, E + 1, size=2))
    return shape, [(0, cut[0]), (cut[0], cut[1]), (cut[1], E)]


@pytest.mark.parametrize("i", range(6))
def test_random_shape_more_rows(i):
    shape, ranges = random_case_wide(i)
    weights = synth.layer_weights(shape)
    dl = upload(weights)
    x = synth.activations(shape, i)
    print(shape, ranges)
    check_against_oracle(weights, dl, x)
    check_token_major(dl, x)
    check_ep_shares(weights, dl, x, ranges)
