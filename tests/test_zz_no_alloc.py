"""moe_forward_static (library-held workspace, no allocation) against moe_forward."""
import numpy as np
import pytest

import synth
from gpu_common import moe_mod, out_bits, run_forward, torch_cuda, upload, x_dev

pytestmark = pytest.mark.gpu


def static_forward(dl, x_bits):
    torch = torch_cuda()
    moe = moe_mod()
    x = x_dev(x_bits)
    out = torch.full_like(x, -1)
    moe.moe_forward_static(dl.cfg, dl.weights, x, out)
    torch.cuda.synchronize()
    return out_bits(out)


@pytest.mark.parametrize("name", ["c2_e128_verify2", "c0_tiny"])
def test_static_workspace_matches_forward(name):
    # Two calls in a row on the one static workspace, the second with fewer
    # rows: each equals moe_forward with a workspace of its own, byte for byte.
    shape = synth.CONFIGS[name]
    big = shape.with_rows(8) if shape.top_k * 8 <= 64 else shape
    weights = synth.layer_weights(big)
    dl = upload(weights)
    x8 = synth.activations(big, 7, rows=big.rows)
    for x in (x8, x8[:1]):
        want, _ = run_forward(dl, x)
        assert np.array_equal(static_forward(dl, x), want), x.shape


def test_static_workspace_256_experts_then_smaller():
    shape = synth.CONFIGS["c3_e256_verify4"]
    weights = synth.layer_weights(shape)
    dl = upload(weights)
    x = synth.activations(shape, 3)
    for rows in (4, 2):
        want, _ = run_forward(dl, x[:rows])
        assert np.array_equal(static_forward(dl, x[:rows]), want), rows


def test_static_workspace_serves_every_accepted_config():
    # The largest workspace any configuration the ABI accepts can need (every
    # dimension at its cap) fits the static array, so moe_forward_static
    # refuses no valid layer; a call with a NULL weights pointer is refused
    # with an argument error before any device work.
    moe = moe_mod()
    torch = torch_cuda()
    big = moe.MoeConfig(moe.MOE_MAX_DIM, moe.MOE_MAX_EXPERTS, moe.MOE_MAX_IDS, moe.MOE_MAX_INTER, moe.MOE_MAX_INTER,
                        moe.MOE_ROUTE_SIGMOID_BIAS, 1, 2.5)
    assert 0 < moe.moe_workspace_bytes(big) <= moe.MOE_STATIC_SCRATCH_BYTES
    x = torch.zeros((1, moe.MOE_MAX_DIM), dtype=torch.int16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_static(big, moe.MoeWeights(), x, torch.zeros_like(x))
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
