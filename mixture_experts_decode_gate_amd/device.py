"""Layer weights resident in HBM, with the device pointer tables moe_weights needs.

Each projection of the routed experts is one contiguous device tensor
[E, n, k/2] (codes) and [E, n, k/16] (scales); the tables hold per-expert
device addresses into them, the way forward_token_major.rs hands its kernels
``packed_ptrs``, ``scale_ptrs`` and ``scale2_vals``.  Host arrays are uploaded
expert by expert; nothing here computes any part of the layer.
"""

from __future__ import annotations

from typing import Callable, Optional, Sequence

import numpy as np

from . import MoeConfig, MoeExpertTable, MoeNvfp4, MoeWeights


def _torch():
    import torch
    return torch


class DeviceLayer:
    """router_w [E, h] fp32 or an NVFP4 object [E, h], bias [E] fp32 or None, shared_gate_vec [h] fp32 or None (ungated),
    shared = (gate, up, down) NVFP4 objects (n, k, packed, scales, scale2),
    expert(e, p) -> NVFP4 object of routed expert e, projection p (0 gate, 1 up, 2 down)."""

    def __init__(self, cfg: MoeConfig, router_w: np.ndarray, bias: Optional[np.ndarray],
                 shared_gate_vec: Optional[np.ndarray], shared: Sequence, expert: Callable[[int, int], object],
                 device: str = "cuda"):
        torch = _torch()
        self.cfg = cfg
        self.device = device
        E, h, I = cfg.num_experts, cfg.hidden, cfg.moe_inter
        dev = torch.device(device)
        if hasattr(router_w, "packed"):  # NVFP4 router [E, h]
            self.router_w = None
            self.router_nvfp4 = (torch.from_numpy(np.ascontiguousarray(router_w.packed)).to(dev),
                                 torch.from_numpy(np.ascontiguousarray(router_w.scales)).to(dev),
                                 float(router_w.scale2))
        else:
            self.router_w = torch.from_numpy(np.ascontiguousarray(router_w, np.float32)).to(dev)
            self.router_nvfp4 = None
        self.bias = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias, np.float32)).to(dev)
        self.shared_gate_vec = None if shared_gate_vec is None else torch.from_numpy(
            np.ascontiguousarray(shared_gate_vec, np.float32)).to(dev)
        self.shared = []
        for t in shared:
            self.shared.append((torch.from_numpy(np.ascontiguousarray(t.packed)).to(dev),
                                torch.from_numpy(np.ascontiguousarray(t.scales)).to(dev), float(t.scale2)))
        dims = [(I, h), (I, h), (h, I)]
        self.packed, self.scales, self.scale2 = [], [], []
        for p, (n, k) in enumerate(dims):
            pk = torch.empty((E, n, k // 2), dtype=torch.uint8, device=dev)
            sc = torch.empty((E, n, k // 16), dtype=torch.uint8, device=dev)
            s2 = np.zeros(E, np.float32)
            for e in range(E):
                t = expert(e, p)
                pk[e].copy_(torch.from_numpy(np.ascontiguousarray(t.packed).reshape(n, k // 2)))
                sc[e].copy_(torch.from_numpy(np.ascontiguousarray(t.scales).reshape(n, k // 16)))
                s2[e] = t.scale2
            self.packed.append(pk)
            self.scales.append(sc)
            self.scale2.append(torch.from_numpy(s2).to(dev))
        self._build_tables()

    def _build_tables(self) -> None:
        torch = _torch()
        E = self.cfg.num_experts
        self.tables = []
        for p in range(3):
            pk, sc = self.packed[p], self.scales[p]
            pk_ptrs = pk.data_ptr() + np.arange(E, dtype=np.int64) * pk[0].numel()
            sc_ptrs = sc.data_ptr() + np.arange(E, dtype=np.int64) * sc[0].numel()
            self.tables.append((torch.from_numpy(pk_ptrs).to(pk.device), torch.from_numpy(sc_ptrs).to(pk.device)))
        self.weights = self._weights()

    def _weights(self) -> MoeWeights:
        w = MoeWeights()
        if self.router_w is not None:
            w.router_w = self.router_w.data_ptr()
        else:
            pk, sc, s2 = self.router_nvfp4
            w.router_w = 0
            w.router_nvfp4 = MoeNvfp4(pk.data_ptr(), sc.data_ptr(), s2)
        w.correction_bias = 0 if self.bias is None else self.bias.data_ptr()
        for name, p in (("gate", 0), ("up", 1), ("down", 2)):
            setattr(w, name, MoeExpertTable(self.tables[p][0].data_ptr(), self.tables[p][1].data_ptr(),
                                            self.scale2[p].data_ptr()))
        for name, (pk, sc, s2) in zip(("shared_gate", "shared_up", "shared_down"), self.shared):
            setattr(w, name, MoeNvfp4(pk.data_ptr(), sc.data_ptr(), s2))
        w.shared_expert_gate = 0 if self.shared_gate_vec is None else self.shared_gate_vec.data_ptr()
        return w

    def clone(self) -> "DeviceLayer":
        """A copy of every tensor at new device addresses (same values)."""
        new = object.__new__(DeviceLayer)
        new.cfg, new.device = self.cfg, self.device
        new.router_w = None if self.router_w is None else self.router_w.clone()
        new.router_nvfp4 = None if self.router_nvfp4 is None else (
            self.router_nvfp4[0].clone(), self.router_nvfp4[1].clone(), self.router_nvfp4[2])
        new.bias = None if self.bias is None else self.bias.clone()
        new.shared_gate_vec = None if self.shared_gate_vec is None else self.shared_gate_vec.clone()
        new.shared = [(pk.clone(), sc.clone(), s2) for pk, sc, s2 in self.shared]
        new.packed = [t.clone() for t in self.packed]
        new.scales = [t.clone() for t in self.scales]
        new.scale2 = [t.clone() for t in self.scale2]
        new._build_tables()
        return new

    def nbytes(self) -> int:
        n = (self.router_w.numel() * 4 if self.router_w is not None
             else self.router_nvfp4[0].numel() + self.router_nvfp4[1].numel())
        n += 0 if self.shared_gate_vec is None else self.shared_gate_vec.numel() * 4
        n += 0 if self.bias is None else self.bias.numel() * 4
        n += sum(pk.numel() + sc.numel() for pk, sc, _ in self.shared)
        n += sum(t.numel() for t in self.packed) + sum(t.numel() for t in self.scales)
        return int(n)
