"""GPU parity of routing (moe_route) and the expert union (moe_union) against the oracle.

Top-k ids must match bit for bit (ties to the lower id), routing weights to
1e-6 relative, logits to the fp32 value of the float64 sum; union ids, their
order, U, slot_to_union and the row masks must match exactly.
"""

import dataclasses

import numpy as np
import pytest

import synth
from oracle import route as RT
from oracle.union import expert_union

from gpu_common import W_RTOL, moe_mod, torch_cuda, ws_for, ws_read, x_dev

pytestmark = pytest.mark.gpu


class RouteWeights:
    """Only the router-side tensors moe_route reads."""

    def __init__(self, shape, router_w=None, bias=None, gate_vec=None, router="fp32"):
        torch = torch_cuda()
        moe = moe_mod()
        self.shape = shape
        self.cfg = moe.MoeConfig.from_shape(shape)
        if router_w is None:
            router_w = synth.router_weight(shape) if router == "fp32" else synth.router_nvfp4(shape)
        self.router_w_np = router_w
        self.bias_np = synth.correction_bias(shape) if bias is None else bias
        self.gate_vec_np = synth.shared_gate_vector(shape) if gate_vec is None else gate_vec
        self.bias = None if self.bias_np is None else torch.from_numpy(self.bias_np).cuda()
        self.gate_vec = torch.from_numpy(self.gate_vec_np).cuda()
        w = moe.MoeWeights()
        if hasattr(router_w, "packed"):  # NVFP4 router
            self.router_w = (torch.from_numpy(router_w.packed).cuda(), torch.from_numpy(router_w.scales).cuda())
            w.router_nvfp4 = moe.MoeNvfp4(self.router_w[0].data_ptr(), self.router_w[1].data_ptr(),
                                          float(router_w.scale2))
        else:
            self.router_w = torch.from_numpy(router_w).cuda()
            w.router_w = self.router_w.data_ptr()
        w.correction_bias = 0 if self.bias is None else self.bias.data_ptr()
        w.shared_expert_gate = self.gate_vec.data_ptr()
        self.weights = w

    def run(self, x_bits, ws=None):
        torch = torch_cuda()
        moe = moe_mod()
        R, k = x_bits.shape[0], self.shape.top_k
        ids = torch.full((R, k), -1, dtype=torch.int32, device="cuda")
        wts = torch.zeros((R, k), dtype=torch.float32, device="cuda")
        ws = ws_for(self.cfg) if ws is None else ws
        moe.moe_route(self.cfg, self.weights, x_dev(x_bits), ids, wts, ws)
        torch.cuda.synchronize()
        L = moe.moe_workspace_layout(self.cfg)
        E = self.shape.num_experts
        logits = ws_read(ws, L.logits, np.float32, R * E).reshape(R, E)
        gamma = ws_read(ws, L.gamma, np.float32, R)
        return ids.cpu().numpy(), wts.cpu().numpy(), logits, gamma


def check_route(rw, x_bits, ws=None):
    s = rw.shape
    ids, wts, logits, gamma = rw.run(x_bits, ws)
    L_ref, ids_ref, w_ref = RT.route(x_bits, rw.router_w_np, rw.bias_np, s.route_kind, s.top_k, s.norm_topk_prob,
                                     s.routed_scaling_factor)
    gamma_ref = RT.shared_gate(x_bits, rw.gate_vec_np)
    # logits: the fp32 rounding of a float64 sum on both sides
    ulp = np.spacing(np.abs(L_ref).astype(np.float32))
    assert np.all(np.abs(logits.astype(np.float64) - L_ref.astype(np.float64)) <= ulp), "logit off by > 1 ulp"
    assert np.count_nonzero(logits != L_ref) <= max(1, L_ref.size // 1000)
    assert np.array_equal(ids, ids_ref), (ids, ids_ref)
    np.testing.assert_allclose(wts, w_ref, rtol=W_RTOL, atol=0)
    np.testing.assert_allclose(gamma, gamma_ref, rtol=1e-6, atol=0)
    return ids


@pytest.mark.parametrize("name", synth.CONFIG_ORDER)
def test_route_configs(name):
    shape = synth.CONFIGS[name]
    rw = RouteWeights(shape)
    for step in range(4):
        check_route(rw, synth.activations(shape, step))


@pytest.mark.parametrize("rows", [1, 3, 8])
def test_route_rows_256_experts(rows):
    shape = synth.CONFIGS["c4_e256_prefill8"]
    rw = RouteWeights(shape)
    check_route(rw, synth.activations(shape, 11, rows=rows))


@pytest.mark.parametrize("name,max_rows", [("c4_e256_prefill8", 16), ("c2_e128_verify2", 16)])
def test_route_rows_match_one_row_calls(name, max_rows):
    # A row's logits, gate, ids and weights do not depend on the other rows
    # of the call: the router sums each row in one fixed order for any row
    # count, so R rows give the bytes of R one-row calls, up to MOE_MAX_ROWS
    # (routing alone takes 16 rows at any hidden size).
    shape = synth.CONFIGS[name]
    rw = RouteWeights(shape)
    x = synth.activations(shape, 13, rows=max_rows)
    singles = [rw.run(x[r:r + 1]) for r in range(max_rows)]
    for R in sorted({2, 3, 5, 8, max_rows}):
        got = rw.run(x[:R])
        for r in range(R):
            for a, b in zip(got, singles[r]):
                assert np.array_equal(a[r], b[0]), f"rows={R} row={r}"
    check_route(rw, x)


def test_route_largest_shape():
    # MOE_MAX_DIM columns (16 router chunks, one per wave) and MOE_MAX_EXPERTS experts
    shape = synth.MoeShape("max", 8192, 1024, 8, 64, 64, 8, synth.ROUTE_SIGMOID_BIAS, True, 2.5)
    rw = RouteWeights(shape)
    check_route(rw, synth.activations(shape, 3))


def test_route_one_workspace_many_calls():
    # Calls with different row counts share one workspace back to back.
    shape = synth.CONFIGS["c3_e256_verify4"]
    rw = RouteWeights(shape)
    ws = ws_for(rw.cfg)
    for step, rows in enumerate([4, 1, 8, 2, 8, 1]):
        check_route(rw, synth.activations(shape, 20 + step, rows=rows), ws)


@pytest.mark.parametrize("fill", [0x00, 0xFF, "random"])
def test_route_any_workspace_contents(fill):
    # The workspace needs no initialisation: moe_route reads only what it
    # wrote earlier in the same call, whatever the bytes held before.
    torch = torch_cuda()
    shape = synth.CONFIGS["c2_e128_verify2"]
    rw = RouteWeights(shape)
    ws = ws_for(rw.cfg, 0 if fill == "random" else fill)
    if fill == "random":
        g = torch.Generator(device="cuda").manual_seed(5)
        ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.int32, device="cuda", generator=g).to(torch.uint8))
    for step in range(3):
        check_route(rw, synth.activations(shape, 30 + step), ws)


def test_route_exact_ties_pick_lower_id():
    # Duplicate router rows give bit-identical logits on both sides.
    shape = dataclasses.replace(synth.CONFIGS["c1_e64_decode"], name="ties")
    w = synth.router_weight(shape).copy()
    w[40] = w[3]
    w[17] = w[3]
    w[9] = w[60]
    x = synth.activations(shape, 0)
    # make expert 3's row the largest logit by aligning it with x
    xf = (x.astype(np.uint32) << 16).view(np.float32)[0]
    w[3] = (xf / np.linalg.norm(xf)).astype(np.float32)
    w[40] = w[3]
    w[17] = w[3]
    rw = RouteWeights(shape, router_w=w)
    ids = check_route(rw, x)
    assert ids[0, :3].tolist() == [3, 17, 40]


@pytest.mark.parametrize("kind,norm", [(synth.ROUTE_SOFTMAX, False), (synth.ROUTE_SIGMOID_BIAS, False),
                                       (synth.ROUTE_SOFTMAX, True)])
def test_route_all_experts_and_norm_variants(kind, norm):
    shape = synth.MoeShape("allk", 512, 8, 8, 64, 64, 8, kind, norm, 1.75)
    rw = RouteWeights(shape)
    check_route(rw, synth.activations(shape, 2))


@pytest.mark.parametrize("E,k,rows", [(128, 65, 1), (200, 100, 1), (128, 128, 1), (256, 64, 2)])
def test_route_more_than_64_selected(E, k, rows):
    # top_k past one wave's lanes: the selected ids are held in two registers
    # (lanes j and j - 64) until the last round; k = E selects every expert.
    shape = synth.MoeShape(f"k{k}_e{E}", 512, E, k, 64, 64, rows, synth.ROUTE_SOFTMAX, True, 1.0)
    rw = RouteWeights(shape)
    check_route(rw, synth.activations(shape, 4))


def test_route_zero_router_closed_form():
    shape = synth.MoeShape("zero", 256, 32, 4, 64, 64, 2, synth.ROUTE_SIGMOID_BIAS, True, 2.5)
    rw = RouteWeights(shape, router_w=np.zeros((32, 256), np.float32))
    ids, wts, logits, _ = rw.run(synth.activations(shape, 0))
    keys = (np.float32(0.5) + rw.bias_np).astype(np.float64)
    ref = np.argsort(-keys, kind="stable")[:4]
    assert np.all(logits == 0)
    assert ids.tolist() == [ref.tolist()] * 2
    assert np.all(wts == np.float32(2.5 / 4))


# ---------------------------------------------------------------- union
def run_union(ids_np, E):
    torch = torch_cuda()
    moe = moe_mod()
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, np.int32)).cuda()
    uid = torch.full((moe.MOE_MAX_IDS,), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    s2u = torch.full((ids_np.size,), -7, dtype=torch.int32, device="cuda")
    rmask = torch.zeros((moe.MOE_MAX_IDS,), dtype=torch.int32, device="cuda")
    moe.moe_union(ids, uid, cnt, s2u, rmask, num_experts=E)
    torch.cuda.synchronize()
    U = int(cnt.item())
    return uid.cpu().numpy()[:U], U, s2u.cpu().numpy(), rmask.cpu().numpy().view(np.uint32)[:U], uid.cpu().numpy()


def check_union(ids_np, E):
    u, U, s2u, m, raw = run_union(ids_np, E)
    u_ref, U_ref, s2u_ref, m_ref = expert_union(ids_np)
    assert U == U_ref
    assert np.array_equal(u, u_ref)
    assert np.array_equal(s2u, s2u_ref)
    assert np.array_equal(m, m_ref)
    assert np.all(raw[U:] == -7)  # entries past U untouched


def test_union_random():
    rng = np.random.default_rng(7)
    for trial in range(200):
        E = int(rng.integers(8, 1025))
        k = int(rng.integers(1, 9))
        R = int(rng.integers(1, min(8, 64 // k) + 1))
        ids = np.stack([rng.choice(min(E, int(rng.integers(k, 3 * k + 1))), size=k, replace=False)
                        for _ in range(R)]).astype(np.int32)
        check_union(ids, E)


def test_union_random_two_tiles():
    # More than 64 ids (rows up to 16, top_k * rows up to 128): the scan runs
    # over two 64-slot tiles; first occurrences in the second tile continue the
    # union positions of the first, and a slot in the second tile may repeat
    # an id first seen in the first.
    rng = np.random.default_rng(8)
    for trial in range(200):
        E = int(rng.integers(16, 1025))
        k = int(rng.integers(1, 17))
        R = int(rng.integers(1, min(16, 128 // k) + 1))
        pool = min(E, int(rng.integers(k, 4 * k + 1)))
        ids = np.stack([rng.choice(pool, size=k, replace=False) for _ in range(R)]).astype(np.int32)
        check_union(ids, E)


def test_union_extremes():
    check_union(np.tile(np.arange(8, dtype=np.int32), (8, 1)), 256)        # U = k
    check_union(np.arange(64, dtype=np.int32).reshape(8, 8)[:, ::-1], 256)  # U = 64
    check_union(np.array([[255, 0, 128, 7]], np.int32), 256)              # one row
    check_union(np.array([[5], [5], [5]], np.int32), 16)                  # k = 1
    check_union(np.arange(64, dtype=np.int32)[::-1].reshape(1, 64), 64)   # k = 64, one row
    check_union(np.arange(128, dtype=np.int32).reshape(16, 8), 256)       # U = 128
    check_union(np.tile(np.arange(8, dtype=np.int32), (16, 1)), 256)       # 128 ids, U = 8
    check_union(np.arange(128, dtype=np.int32)[::-1].reshape(2, 64), 128)  # k = 64, two rows
    check_union(np.arange(100, dtype=np.int32)[::-1].reshape(1, 100), 128)  # k = 100: one row's slots span both tiles
    check_union(np.arange(128, dtype=np.int32).reshape(1, 128), 128)        # k = 128, one row
    # the second tile's first slot repeats the first tile's last id
    ids = np.arange(72, dtype=np.int32).reshape(9, 8)
    ids[8, 0] = 63
    check_union(ids, 256)


# ---------------------------------------------------------------- NVFP4 router
@pytest.mark.parametrize("name", synth.CONFIG_ORDER)
def test_route_nvfp4_router(name):
    shape = synth.CONFIGS[name]
    rw = RouteWeights(shape, router="nvfp4")
    for step in range(2):
        check_route(rw, synth.activations(shape, step))


def test_route_nvfp4_router_ragged():
    # h with a partial 512-column router chunk; k = E; 64 ids
    shape = synth.MoeShape("r", 2080, 12, 12, 96, 96, 5, synth.ROUTE_SIGMOID_BIAS, True, 2.5)
    check_route(RouteWeights(shape, router="nvfp4"), synth.activations(shape, 3))
    shape = synth.MoeShape("r2", 4160, 96, 8, 96, 96, 8, synth.ROUTE_SOFTMAX, False, 1.0)
    check_route(RouteWeights(shape, router="nvfp4"), synth.activations(shape, 4))


# ---------------------------------------------------------------- streaming-read probe (measurement aid)
@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 24) + 160])
def test_read_probe_reads_every_word(nbytes):
    # The blocks' fold words XOR to the XOR of every 32-bit word of the buffer:
    # each word was read exactly once (a word read twice or skipped would
    # change the fold for random contents).
    torch = torch_cuda()
    moe = moe_mod()
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(moe.moe_read_probe_sink_words(), dtype=torch.int32, device="cuda")
    moe.moe_read_probe(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
