"""Glue between the seeded inputs (torch tensors) and the fp64 oracle (NumPy)."""
from __future__ import annotations

import numpy as np
import torch

import oracle


def np_u16(t: torch.Tensor) -> np.ndarray:
    """bf16/fp16 tensor -> its bit patterns as uint16 (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def router_cfg(geom: dict) -> oracle.RouterConfig:
    # the library decides on the float32 value of the top-p parameter
    p = float(np.float32(geom.get("expert_top_p", 0.0)))
    return oracle.RouterConfig(geom["n_routed_experts"], geom["n_group"], geom["topk_group"],
                               geom["top_k"], geom["routed_scaling_factor"], top_p=p)


def _proj_np(p, wfmt):
    q = p.q.detach().cpu().numpy()
    if wfmt == "int4":
        s = np_u16(p.scale)
        g = None
    else:
        s = p.scale.detach().cpu().numpy()
        g = None if p.gscale is None else p.gscale.detach().cpu().numpy()
    return (q, s, g)


def expert_source(qe, wfmt) -> oracle.ExpertSource:
    """Copy all experts to the host (small layers)."""
    return oracle.ExpertSource(wfmt, _proj_np(qe.gate, wfmt), _proj_np(qe.up, wfmt),
                               _proj_np(qe.down, wfmt))


class LazyExperts:
    """Same interface as oracle.ExpertSource, but copies one expert at a time
    from (GPU) memory -- for full-size layers where only the experts that the
    sampled tokens chose are needed."""

    def __init__(self, qe, wfmt):
        self.qe, self.wfmt = qe, wfmt
        self._cache = {}

    def packed(self, e):
        """Host copies of expert e's packed bytes, (q, scale, gscale) per
        projection, each with a leading expert dimension of one."""
        out = []
        for proj in ("gate", "up", "down"):
            p = getattr(self.qe, proj)
            q = p.q[e:e + 1].detach().cpu().numpy()
            if self.wfmt == "int4":
                out.append((q, np_u16(p.scale[e:e + 1]), None))
            elif self.wfmt in oracle.ROW_FORMATS or self.wfmt in oracle.A8_FORMATS:
                out.append((q, p.scale[e:e + 1].detach().cpu().numpy(), None))
            else:
                out.append((q, p.scale[e:e + 1].detach().cpu().numpy(),
                            p.gscale[e:e + 1].detach().cpu().numpy()))
        return tuple(out)

    def weight(self, proj, e):
        key = (proj, e)
        if key not in self._cache:
            p = getattr(self.qe, proj)
            q = p.q[e].detach().cpu().numpy()
            if self.wfmt == "int4":
                w = oracle.dequant_int4(q, np_u16(p.scale[e]))
            elif self.wfmt in oracle.ROW_FORMATS or self.wfmt in oracle.A8_FORMATS:
                base = oracle.A8_FORMATS.get(self.wfmt, self.wfmt)
                w = oracle.ROW_FORMATS[base](q, p.scale[e].detach().cpu().numpy())
            else:
                w = oracle.dequant_nvfp4(q, p.scale[e].detach().cpu().numpy(),
                                         float(p.gscale[e].item()))
            if len(self._cache) > 64:
                self._cache.clear()
            self._cache[key] = w
        return self._cache[key]


def oracle_inputs(L, lazy=False):
    """Host copies of a synth.LayerInputs for the oracle."""
    x = np_u16(L.x)
    Wr = L.router_w.detach().cpu().numpy().astype(np.float64)
    b = L.bias.detach().cpu().numpy().astype(np.float64)
    mk = (lambda qe: LazyExperts(qe, L.wfmt)) if lazy else (lambda qe: expert_source(qe, L.wfmt))
    routed = mk(L.routed)
    shared = mk(L.shared) if L.shared is not None else None
    return x, Wr, b, router_cfg(L.geom), routed, shared


def row_rel_err(y, y_ref) -> np.ndarray:
    """Per token row: max_h |y - y_ref| / max_h |y_ref|."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    den = np.abs(y_ref).max(axis=1)
    den = np.where(den > 0, den, 1.0)
    return np.abs(y - y_ref).max(axis=1) / den
