"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and check its results against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import quantized_moe_02_amd as q
from helpers import np_u16, oracle_inputs, row_rel_err

TOL = 2e-3          # max row-normalised relative error of outputs
W_TOL = 1e-6        # routing weights: decided in fp64 on both sides, rounded to fp32 by the GPU
TAU = 1e-9          # selections whose fp64 margin is below this may differ (checked for validity)


def proj_tuple(p):
    return (p.q, p.scale, p.gscale)


def qexp(qe):
    return q.qexperts(proj_tuple(qe.gate), proj_tuple(qe.up), proj_tuple(qe.down))


def run_layer(L, out_dtype=q.MOE_OUT_F32, x=None, T=None, options=0, ws=None):
    """moe_layer on the GPU; returns (y, ids, tw) as torch tensors on the GPU."""
    cfg = q.make_config(L.geom, L.wfmt, options)
    x = L.x if x is None else x
    T = x.shape[0] if T is None else T
    H, k = L.geom["hidden"], L.geom["top_k"]
    ws = q.workspace(cfg, T) if ws is None else ws
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
    if 0.0 < cfg.top_p < 1.0:
        plain = oracle.RouterConfig(cfg.n_experts, cfg.n_group, cfg.topk_group, cfg.top_k,
                                    cfg.routed_scaling_factor)
        chosen, _, _ = oracle.route(X, Wr, b, plain)
        for t in np.nonzero(~exact)[0]:
            assert oracle.valid_top_p(ids_g[t], info["s"][t], chosen[t], cfg.top_p, TAU), t
    else:
        for t in np.nonzero(~exact)[0]:
            assert oracle.valid_under_perturbation(ids_g[t], info["sb"][t], cfg, TAU), t
    w_ref = oracle.route_weights(info["s"], ids_g, cfg.routed_scaling_factor)
    tw = tw_gpu.cpu().numpy()
    kept = ids_g >= 0
    assert np.all(tw[~kept] == 0.0)
    rel = np.abs(tw[kept] - w_ref[kept]) / np.abs(w_ref[kept])
    assert rel.max() <= W_TOL, rel.max()
    return ids_g, int((~exact).sum())


def check_outputs(L, y_gpu, ids_g, token_idx=None, tol=TOL, x_np=None, ffn_map=None, srcs=None):
    """y within tol (row-normalised) of the oracle evaluated on the GPU's ids.
    ffn_map: where the oracle's expert FFNs run (see FFNCache); srcs: the
    (routed, shared) expert sources that ffn_map was filled from."""
    x, Wr, b, cfg, routed, shared = oracle_inputs(L, lazy=True)
    if srcs is not None:
        routed, shared = srcs
    if x_np is not None:
        x = x_np
    idx = np.arange(x.shape[0]) if token_idx is None else np.asarray(token_idx)
    y_ref, _, _ = oracle.layer(x, Wr, b, cfg, routed, shared, ids=ids_g[idx], token_idx=idx,
                               ffn_map=ffn_map)
    y = y_gpu.float().cpu().numpy()[idx]
    err = row_rel_err(y, y_ref)
    assert err.max() <= tol, f"max row error {err.max():.3e} at token {idx[err.argmax()]}"
    return err.max()


class FFNCache:
    """The oracle's expert FFN rows, computed in worker processes
    (oracle_pool) and kept per (source, expert, activation row), so that
    several checks over one layer dequantise each expert once.  Called with a
    list of (source, expert, X rows) jobs, as oracle.layer's ffn_map."""

    def __init__(self):
        self.rows = {}

    @staticmethod
    def _key(src, e, xrow):
        return (id(src), int(e), xrow.tobytes())

    def fill(self, jobs):
        import oracle_pool
        todo = []
        for src, e, X in jobs:
            need = [r for r in range(X.shape[0]) if self._key(src, e, X[r]) not in self.rows]
            if need:
                todo.append((src, e, X[need]))
        for (src, e, X), F in zip(todo, oracle_pool.expert_ffns(todo)):
            for r in range(X.shape[0]):
                self.rows[self._key(src, e, X[r])] = F[r]

    def __call__(self, jobs):
        self.fill(jobs)
        return [np.stack([self.rows[self._key(src, e, X[r])] for r in range(X.shape[0])])
                for src, e, X in jobs]


def cover_tokens(ids_g, limit=64, always=()):
    """A few tokens whose picks together touch every selected expert (greedy
    set cover), plus `always`."""
    chosen = [int(t) for t in always]
    covered = set(ids_g[chosen].ravel().tolist()) if chosen else set()
    need = set(ids_g.ravel().tolist())
    sets = [set(r) for r in ids_g.tolist()]
    while covered != need and len(chosen) < limit:
        t = max(range(len(sets)), key=lambda i: len(sets[i] - covered))
        chosen.append(t)
        covered |= sets[t]
    return np.array(sorted(set(chosen)))


def expert_slots_to_check(offsets, n_full=8, seed=0):
    """Sorted slots to compare for a routed expert-FFN output: every slot of
    n_full experts (the most and least loaded, ones whose last work unit is
    shortest and longest, random others) and the first, a middle and the last
    slot of every other active expert.  Returns {expert: slot array}."""
    offsets = np.asarray(offsets)
    counts = np.diff(offsets)
    active = np.nonzero(counts)[0]
    rng = np.random.default_rng(seed)
    full = []
    by = lambda key: sorted(active, key=key)
    for cand in (by(lambda e: -counts[e])[0], by(lambda e: counts[e])[0],
                 by(lambda e: (counts[e] - 1) % 128)[0], by(lambda e: -((counts[e] - 1) % 128))[0],
                 by(lambda e: (counts[e] - 1) % 32)[0]):
        if cand not in full:
            full.append(int(cand))
    rest = [int(e) for e in active if e not in full]
    rng.shuffle(rest)
    full += rest[: max(0, n_full - len(full))]
    out = {}
    for e in active:
        lo, hi = offsets[e], offsets[e + 1]
        if int(e) in full:
            out[int(e)] = np.arange(lo, hi)
        else:
            out[int(e)] = np.unique([lo, (lo + hi - 1) // 2, hi - 1])
    return out


def entry_point_chain(L, T=None, x=None, pool=False):
    """moe_route -> moe_permute -> moe_expert_ffn_q4 (routed, then dense on the
    shared expert) -> moe_combine, each result against the oracle: ids exact,
    permutation exact, expert outputs per sorted slot within TOL, combine
    within 1e-6 of its own fp64 sum."""
    g = L.geom
    x = L.x if x is None else x
    T = x.shape[0] if T is None else T
    H, E, k = g["hidden"], g["n_routed_experts"], g["top_k"]
    P = T * k
    cfg = q.make_config(g, L.wfmt)
    ws = q.workspace(cfg, T)
    dev = dict(device="cuda")
    ids = torch.empty(T, k, dtype=torch.int32, **dev)
    tw = torch.empty(T, k, dtype=torch.float32, **dev)
    q.moe_route(cfg, T, x, L.router_w, L.bias, ids, tw, ws)
    torch.cuda.synchronize()
    x_np = np_u16(x)
    ids_g, _ = check_routing(L, ids, tw, x_np=x_np)

    offs = torch.empty(E + 1, dtype=torch.int32, **dev)
    st = torch.empty(P, dtype=torch.int32, **dev)
    inv = torch.empty(P, dtype=torch.int32, **dev)
    act = torch.empty(E, dtype=torch.int32, **dev)
    na = torch.empty(1, dtype=torch.int32, **dev)
    q.moe_permute(cfg, T, ids, offs, st, inv, act, na, ws)
    torch.cuda.synchronize()
    r_off, r_st, r_inv, r_act = oracle.permute(ids_g, E)
    assert np.array_equal(offs.cpu().numpy(), r_off)
    assert np.array_equal(st.cpu().numpy()[: len(r_st)], r_st)
    assert np.array_equal(inv.cpu().numpy(), r_inv)
    assert int(na.item()) == len(r_act)
    assert np.array_equal(act.cpu().numpy()[: len(r_act)], r_act)

    _, _, _, _, routed, shared = oracle_inputs(L, lazy=True)
    X = oracle.bf16_bits_to_f64(x_np)
    out = torch.empty(P, H, dtype=torch.float32, **dev)
    q.moe_expert_ffn_q4(cfg, T, x, qexp(L.routed), offs, st, act, na, out, ws)
    torch.cuda.synchronize()
    jobs = [(routed, int(e), X[r_st[r_off[e]:r_off[e + 1]]]) for e in r_act]
    jobs.append((shared, 0, X))
    refs = FFNCache()(jobs) if pool else [oracle.expert_ffn(*j) for j in jobs]
    Pk = int(r_off[-1])   # kept picks (all P unless the adaptive top-p dropped some)
    ref = np.zeros((Pk, H))
    for e, F in zip(r_act, refs):
        ref[r_off[e]:r_off[e + 1]] = F
    err = row_rel_err(out.cpu().numpy()[:Pk], ref)
    assert err.max() <= TOL, (err.max(), int(err.argmax()))

    outs = torch.empty(T, H, dtype=torch.float32, **dev)
    q.moe_expert_ffn_q4(cfg, T, x, qexp(L.shared), None, None, None, None, outs, ws)
    torch.cuda.synchronize()
    assert row_rel_err(outs.cpu().numpy(), refs[-1]).max() <= TOL

    y = torch.empty(T, H, dtype=torch.float32, **dev)
    q.moe_combine(cfg, T, out, inv, tw, outs, y)
    y16 = torch.empty(T, H, dtype=torch.bfloat16, **dev)
    q.moe_combine(cfg, T, out, inv, tw, outs, y16, q.MOE_OUT_BF16)
    torch.cuda.synchronize()
    o64, s64 = out.double().cpu().numpy(), outs.double().cpu().numpy()
    w64 = tw.double().cpu().numpy()
    inv2 = r_inv.reshape(T, k)
    yref = s64 + np.einsum("tk,tkh->th", np.where(inv2 >= 0, w64, 0.0), o64[np.maximum(inv2, 0)])
    assert row_rel_err(y.cpu().numpy(), yref).max() <= 1e-6
    assert torch.equal(y.to(torch.bfloat16), y16)
    return err.max()
