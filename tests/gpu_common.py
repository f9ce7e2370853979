"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and check its results against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import quantized_moe_02_amd as q
from helpers import np_u16, oracle_inputs, row_rel_err

TOL = 2e-3          # max row-normalised relative error of outputs
TAU = 1e-9          # selections whose fp64 margin is below this may differ (checked for validity)


def proj_tuple(p):
    return (p.q, p.scale, p.gscale)


def qexp(qe):
    return q.qexperts(proj_tuple(qe.gate), proj_tuple(qe.up), proj_tuple(qe.down))


def run_layer(L, out_dtype=q.MOE_OUT_F32, x=None, T=None):
    """moe_layer on the GPU; returns (y, ids, tw) as torch tensors on the GPU."""
    cfg = q.make_config(L.geom, L.wfmt)
    x = L.x if x is None else x
    T = x.shape[0] if T is None else T
    H, k = L.geom["hidden"], L.geom["top_k"]
    ws = q.workspace(cfg, T)
    y = torch.empty(T, H, device="cuda",
                    dtype=torch.float32 if out_dtype == q.MOE_OUT_F32 else torch.bfloat16)
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    tw = torch.empty(T, k, dtype=torch.float32, device="cuda")
    q.moe_layer(cfg, T, x, L.router_w, L.bias, qexp(L.routed),
                qexp(L.shared) if L.shared is not None else None, y, out_dtype, ids, tw, ws)
    torch.cuda.synchronize()
    return y, ids, tw


def check_routing(L, ids_gpu, tw_gpu, x_np=None):
    """ids exact where the fp64 decision margin is >= TAU, valid otherwise;
    weights within TOL of the oracle's weights for the GPU's ids."""
    x, Wr, b, cfg, _, _ = oracle_inputs(L, lazy=True)
    if x_np is not None:
        x = x_np
    X = oracle.bf16_bits_to_f64(x)
    ids_ref, _, info = oracle.route(X, Wr, b, cfg)
    ids_g = ids_gpu.cpu().numpy().astype(np.int64)
    exact = info["margin"] >= TAU
    mism = np.nonzero(exact & np.any(ids_g != ids_ref, axis=1))[0]
    assert len(mism) == 0, f"routing differs at tokens {mism[:8]}: gpu {ids_g[mism[:2]]} ref {ids_ref[mism[:2]]}"
    for t in np.nonzero(~exact)[0]:
        assert oracle.valid_under_perturbation(ids_g[t], info["sb"][t], cfg, TAU), t
    w_ref = oracle.route_weights(info["s"], ids_g, cfg.routed_scaling_factor)
    rel = np.abs(tw_gpu.cpu().numpy() - w_ref) / np.abs(w_ref)
    assert rel.max() <= TOL, rel.max()
    return ids_g, int((~exact).sum())


def check_outputs(L, y_gpu, ids_g, token_idx=None, tol=TOL, x_np=None):
    """y within tol (row-normalised) of the oracle evaluated on the GPU's ids."""
    x, Wr, b, cfg, routed, shared = oracle_inputs(L, lazy=True)
    if x_np is not None:
        x = x_np
    idx = np.arange(x.shape[0]) if token_idx is None else np.asarray(token_idx)
    y_ref, _, _ = oracle.layer(x, Wr, b, cfg, routed, shared, ids=ids_g[idx], token_idx=idx)
    y = y_gpu.float().cpu().numpy()[idx]
    err = row_rel_err(y, y_ref)
    assert err.max() <= tol, f"max row error {err.max():.3e} at token {idx[err.argmax()]}"
    return err.max()
