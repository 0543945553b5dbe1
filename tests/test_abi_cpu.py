"""C ABI of libmoe.so on the CPU: exports and argument refusals (no GPU calls).

Every refusal below happens before any HIP call, so these tests run in a
container without a GPU.  Device pointers are fake, aligned addresses that
the library never dereferences on these paths.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

moe = pytest.importorskip("mixture_experts_decode_gate_amd")
if not os.path.exists(moe.LIB_PATH):
    pytest.skip("libmoe.so not built", allow_module_level=True)

lib = moe.load()

BASE = 0x7F0000000000  # fake device addresses, 256-byte aligned


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = header_functions()
    assert {"moe_route", "moe_union", "moe_forward", "moe_workspace_bytes", "moe_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def cfg_c4(**kw):
    c = moe.MoeConfig(6144, 256, 8, 2048, 2048, moe.MOE_ROUTE_SIGMOID_BIAS, 1, 2.5)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def fake_weights(sigmoid=True):
    w = moe.MoeWeights()
    w.router_w = BASE + 0x1000
    w.correction_bias = (BASE + 0x2000) if sigmoid else 0
    for i, name in enumerate(("gate", "up", "down")):
        setattr(w, name, moe.MoeExpertTable(BASE + 0x10000 * (i + 1), BASE + 0x10000 * (i + 1) + 0x4000,
                                            BASE + 0x10000 * (i + 1) + 0x8000))
    for i, name in enumerate(("shared_gate", "shared_up", "shared_down")):
        setattr(w, name, moe.MoeNvfp4(BASE + 0x100000 * (i + 1), BASE + 0x100000 * (i + 1) + 0x40000, 1.0))
    w.shared_expert_gate = BASE + 0x3000
    return w


WS = BASE + 0x10000000
X = BASE + 0x20000000
OUT = BASE + 0x30000000


def forward(cfg, w, x=X, out=OUT, rows=4, ws=WS, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.moe_workspace_bytes(ctypes.byref(cfg)) or 1
    return lib.moe_forward(ctypes.byref(cfg), ctypes.byref(w) if w is not None else None, x, out, rows, ws,
                           ws_bytes, None)


def test_workspace_layout_is_ordered_and_aligned():
    cfg = cfg_c4()
    L = moe.moe_workspace_layout(cfg)
    names = [f[0] for f in moe.MoeWsLayout._fields_]
    offs = [getattr(L, n) for n in names]
    assert offs == sorted(offs) and len(set(offs)) == len(offs)
    assert all(o % 256 == 0 for o in offs)
    assert L.total == moe.moe_workspace_bytes(cfg)
    # act holds 128 + 16 (row, expert) pairs x max(I, Is) bf16; y 144 pairs x h fp32
    assert L.y - L.act >= 144 * 2048 * 2
    assert L.total - L.y >= 144 * 6144 * 4
    assert L.total < 5 << 20
    assert lib.moe_workspace_bytes(ctypes.byref(cfg_c4(hidden=100))) == 0


@pytest.mark.parametrize("field,value", [
    ("hidden", 0), ("hidden", 100), ("hidden", 16384), ("moe_inter", 48), ("moe_inter", 8192), ("shared_inter", 0),
    ("num_experts", 0), ("num_experts", 2048), ("top_k", 0), ("top_k", 257), ("route_kind", 7),
    ("norm_topk_prob", 2), ("routed_scaling_factor", float("nan")),
])
def test_bad_config_refused(field, value):
    cfg = cfg_c4(**{field: value})
    assert forward(cfg, fake_weights(), ws_bytes=1 << 30) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_last_error().decode()


@pytest.mark.parametrize("rows", [0, 17, -1])
def test_bad_rows_refused(rows):
    assert forward(cfg_c4(), fake_weights(), rows=rows) == moe.MOE_ERR_INVALID_ARG


def test_too_many_ids_refused():
    # top_k * rows > 128: more ids than the union's two 64-slot tiles
    assert forward(cfg_c4(top_k=16), fake_weights(), rows=9) == moe.MOE_ERR_INVALID_ARG
    assert "128" in lib.moe_last_error().decode()


def test_rows_beyond_staged_x_refused():
    # rows * ceil(hidden / 2048) > 36: x for every row does not fit the gate/up
    # sweep's LDS; 12 rows fit at hidden 6144 (3 chunks), 16 at hidden 4096
    assert forward(cfg_c4(), fake_weights(), rows=13) == moe.MOE_ERR_UNSUPPORTED
    assert "moe_forward_prefill" in lib.moe_last_error().decode()
    assert forward(cfg_c4(hidden=8192), fake_weights(), rows=10) == moe.MOE_ERR_UNSUPPORTED


def test_pointer_refusals():
    cfg = cfg_c4()
    assert forward(cfg, None) == moe.MOE_ERR_INVALID_ARG
    assert forward(cfg, fake_weights(), x=0) == moe.MOE_ERR_INVALID_ARG
    assert forward(cfg, fake_weights(), out=0) == moe.MOE_ERR_INVALID_ARG
    assert forward(cfg, fake_weights(), x=X + 8) == moe.MOE_ERR_INVALID_ARG        # misaligned
    assert forward(cfg, fake_weights(), out=X + 64) == moe.MOE_ERR_INVALID_ARG     # overlaps x
    assert forward(cfg, fake_weights(), ws=WS + 16) == moe.MOE_ERR_INVALID_ARG     # ws alignment
    assert forward(cfg, fake_weights(), x=WS + 1024) == moe.MOE_ERR_INVALID_ARG    # x inside ws
    w = fake_weights()
    w.router_w = BASE + 0x1004
    assert forward(cfg, w) == moe.MOE_ERR_INVALID_ARG
    w = fake_weights()
    w.up = moe.MoeExpertTable(0, 0, 0)
    assert forward(cfg, w) == moe.MOE_ERR_INVALID_ARG


def test_bias_must_match_route_kind():
    assert forward(cfg_c4(), fake_weights(sigmoid=False)) == moe.MOE_ERR_INVALID_ARG
    assert forward(cfg_c4(route_kind=moe.MOE_ROUTE_SOFTMAX), fake_weights(sigmoid=True)) == moe.MOE_ERR_INVALID_ARG


def test_unsupported_layers():
    w = fake_weights()
    w.shared_up = moe.MoeNvfp4(0, 0, 1.0)          # no shared expert
    assert forward(cfg_c4(), w) == moe.MOE_ERR_UNSUPPORTED
    w = fake_weights()
    w.shared_expert_gate = BASE + 0x3008           # misaligned gate vector
    assert forward(cfg_c4(), w) == moe.MOE_ERR_INVALID_ARG


def test_small_workspace_refused():
    cfg = cfg_c4()
    need = lib.moe_workspace_bytes(ctypes.byref(cfg))
    assert forward(cfg, fake_weights(), ws_bytes=need - 1) == moe.MOE_ERR_WORKSPACE


def test_union_refusals():
    u = lambda rows, k, E, ids=X, uid=OUT, cnt=OUT + 512, s2u=OUT + 1024, rm=OUT + 2048: lib.moe_union(
        ids, rows, k, E, uid, cnt, s2u, rm, None)
    assert u(0, 8, 256) == moe.MOE_ERR_INVALID_ARG
    assert u(17, 1, 256) == moe.MOE_ERR_INVALID_ARG
    assert u(16, 9, 256) == moe.MOE_ERR_INVALID_ARG     # 144 ids
    assert u(2, 8, 4) == moe.MOE_ERR_INVALID_ARG        # top_k > num_experts
    assert u(1, 8, 256, ids=0) == moe.MOE_ERR_INVALID_ARG
    assert u(1, 8, 256, s2u=OUT + 64) == moe.MOE_ERR_INVALID_ARG  # overlaps union_ids


def test_route_refusals():
    cfg = cfg_c4()
    need = lib.moe_workspace_bytes(ctypes.byref(cfg))
    r = lambda ids, wts, rows=2: lib.moe_route(ctypes.byref(cfg), ctypes.byref(fake_weights()), X, rows, ids,
                                               wts, WS, need, None)
    assert r(0, OUT) == moe.MOE_ERR_INVALID_ARG
    assert r(OUT, OUT + 16) == moe.MOE_ERR_INVALID_ARG   # ids and weights overlap
    assert r(OUT, OUT + 4096, rows=17) == moe.MOE_ERR_INVALID_ARG
    big = cfg_c4(top_k=16)
    assert lib.moe_route(ctypes.byref(big), ctypes.byref(fake_weights()), X, 9, OUT, OUT + 4096, WS,
                         lib.moe_workspace_bytes(ctypes.byref(big)), None) == moe.MOE_ERR_INVALID_ARG
    assert "128" in lib.moe_last_error().decode()  # top_k * rows past the union's ids


def test_stage_names():
    n = lib.moe_num_stages()
    assert n >= 1
    assert [lib.moe_stage_name(i) is not None for i in range(n)] == [True] * n
    assert lib.moe_stage_name(n) is None and lib.moe_stage_name(-1) is None


def test_token_major_refuses_like_forward():
    """moe_forward_token_major validates exactly as moe_forward does."""
    def both(cfg, w, **kw):
        a = forward(cfg, w, **kw)
        ws_bytes = kw.pop("ws_bytes", None)
        if ws_bytes is None:
            ws_bytes = lib.moe_workspace_bytes(ctypes.byref(cfg)) or 1
        b = lib.moe_forward_token_major(ctypes.byref(cfg), ctypes.byref(w) if w is not None else None,
                                        kw.get("x", X), kw.get("out", OUT), kw.get("rows", 4), kw.get("ws", WS),
                                        ws_bytes, None)
        return a, b

    cases = [
        (cfg_c4(hidden=100), fake_weights(), {}),
        (cfg_c4(), fake_weights(), {"rows": 17}),
        (cfg_c4(top_k=16), fake_weights(), {"rows": 9}),
        (cfg_c4(), None, {}),
        (cfg_c4(), fake_weights(), {"out": X + 64}),
        (cfg_c4(), fake_weights(sigmoid=False), {}),
    ]
    for cfg, w, kw in cases:
        a, b = both(cfg, w, **kw)
        assert a == b == moe.MOE_ERR_INVALID_ARG, (kw, a, b)
    cfg = cfg_c4()
    need = lib.moe_workspace_bytes(ctypes.byref(cfg))
    assert both(cfg, fake_weights(), ws_bytes=need - 1) == (moe.MOE_ERR_WORKSPACE, moe.MOE_ERR_WORKSPACE)


def test_ep_refusals():
    cfg = cfg_c4()
    need = lib.moe_workspace_bytes(ctypes.byref(cfg))
    P = BASE + 0x40000000

    def ep(lo, hi, partial=P, rows=4, x=X):
        return lib.moe_forward_ep_partial(ctypes.byref(cfg), ctypes.byref(fake_weights()), x, partial, rows, lo, hi,
                                          WS, need, None)
    for lo, hi in [(-1, 8), (9, 8), (0, 257), (0, -1)]:
        assert ep(lo, hi) == moe.MOE_ERR_INVALID_ARG, (lo, hi)
    assert ep(0, 32, partial=0) == moe.MOE_ERR_INVALID_ARG
    assert ep(0, 32, partial=P + 4) == moe.MOE_ERR_INVALID_ARG         # misaligned
    assert ep(0, 32, partial=X + 256) == moe.MOE_ERR_INVALID_ARG       # overlaps x
    assert ep(0, 32, partial=WS + 4096) == moe.MOE_ERR_INVALID_ARG     # inside the workspace
    assert ep(0, 32, rows=17) == moe.MOE_ERR_INVALID_ARG

    def comb(red, out, rows=4, ws_bytes=need):
        return lib.moe_ep_combine(ctypes.byref(cfg), red, out, rows, WS, ws_bytes, None)
    assert comb(0, OUT) == moe.MOE_ERR_INVALID_ARG
    assert comb(P, 0) == moe.MOE_ERR_INVALID_ARG
    assert comb(P, P + 1024) == moe.MOE_ERR_INVALID_ARG                # out overlaps reduced
    assert comb(P, OUT, rows=0) == moe.MOE_ERR_INVALID_ARG
    assert comb(P, OUT, ws_bytes=need - 1) == moe.MOE_ERR_WORKSPACE

    u = lambda lo, hi, E=256: lib.moe_union_local(X, 2, 8, E, lo, hi, OUT, OUT + 512, OUT + 1024, OUT + 2048, None)
    for lo, hi in [(-1, 4), (5, 4), (0, 300)]:
        assert u(lo, hi) == moe.MOE_ERR_INVALID_ARG, (lo, hi)
    assert lib.moe_union_local(X, 17, 8, 256, 0, 8, OUT, OUT + 512, OUT + 1024, OUT + 2048, None) == \
        moe.MOE_ERR_INVALID_ARG


def test_router_refusals():
    cfg = cfg_c4()
    w = fake_weights()
    w.router_nvfp4 = moe.MoeNvfp4(BASE + 0x500000, BASE + 0x540000, 1.0)   # both routers set
    assert forward(cfg, w) == moe.MOE_ERR_INVALID_ARG
    w = fake_weights()
    w.router_w = 0                                                       # no router at all
    assert forward(cfg, w) == moe.MOE_ERR_INVALID_ARG
    w.router_nvfp4 = moe.MoeNvfp4(BASE + 0x500008, BASE + 0x540000, 1.0)  # misaligned codes
    assert forward(cfg, w) == moe.MOE_ERR_INVALID_ARG
    w.router_nvfp4 = moe.MoeNvfp4(BASE + 0x500000, BASE + 0x540000, float("nan"))
    assert forward(cfg, w) == moe.MOE_ERR_INVALID_ARG


def test_read_probe_refusals():
    sink = OUT
    assert lib.moe_read_probe(0, 4096, sink, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_read_probe(X + 8, 4096, sink, None) == moe.MOE_ERR_INVALID_ARG     # misaligned
    assert lib.moe_read_probe(X, 0, sink, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_read_probe(X, 4100, sink, None) == moe.MOE_ERR_INVALID_ARG        # not a multiple of 16
    assert lib.moe_read_probe(X, 4096, 0, None) == moe.MOE_ERR_INVALID_ARG


def test_prefill_refusals():
    cfg = cfg_c4()
    need = lib.moe_workspace_bytes(ctypes.byref(cfg))
    pf = lambda rows, x=X, out=OUT, w=None, ws_bytes=need: lib.moe_forward_prefill(
        ctypes.byref(cfg), ctypes.byref(w or fake_weights()), x, out, rows, WS, ws_bytes, None)
    assert pf(0) == moe.MOE_ERR_INVALID_ARG
    assert pf(-3) == moe.MOE_ERR_INVALID_ARG
    assert pf(40, out=X + 6144 * 2 * 20) == moe.MOE_ERR_INVALID_ARG   # out overlaps x
    assert pf(40, x=WS + 4096) == moe.MOE_ERR_INVALID_ARG             # x inside the workspace
    assert pf(40, ws_bytes=need - 1) == moe.MOE_ERR_WORKSPACE
    w = fake_weights()
    w.router_w = BASE + 0x1004
    assert pf(40, w=w) == moe.MOE_ERR_INVALID_ARG


def test_static_forward_refusals():
    """moe_forward_static refuses bad arguments as moe_forward does, before any HIP call."""
    cfg = cfg_c4()
    st = lambda rows=4, x=X, out=OUT, w=None, c=cfg: lib.moe_forward_static(
        ctypes.byref(c), ctypes.byref(w or fake_weights()), x, out, rows, None)
    assert st(rows=0) == moe.MOE_ERR_INVALID_ARG
    assert st(rows=17) == moe.MOE_ERR_INVALID_ARG
    assert st(x=0) == moe.MOE_ERR_INVALID_ARG
    assert st(out=0) == moe.MOE_ERR_INVALID_ARG
    assert st(x=X + 2) == moe.MOE_ERR_INVALID_ARG                # misaligned
    assert st(out=X + 6144 * 2) == moe.MOE_ERR_INVALID_ARG       # out overlaps x
    assert st(c=cfg_c4(hidden=100)) == moe.MOE_ERR_INVALID_ARG
    w = fake_weights()
    w.router_w = BASE + 0x1004
    assert st(w=w) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_forward_static(ctypes.byref(cfg), None, X, OUT, 4, None) == moe.MOE_ERR_INVALID_ARG
    # the workspace of every configuration the caps allow fits the static array
    big = moe.MoeConfig(moe.MOE_MAX_DIM, moe.MOE_MAX_EXPERTS, moe.MOE_MAX_IDS, moe.MOE_MAX_INTER, moe.MOE_MAX_INTER,
                        moe.MOE_ROUTE_SIGMOID_BIAS, 1, 2.5)
    assert 0 < lib.moe_workspace_bytes(ctypes.byref(big)) <= moe.MOE_STATIC_SCRATCH_BYTES
