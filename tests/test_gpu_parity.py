"""Parity of the HIP path (through the C ABI) against the fp64 oracle.

Indices and permutations must match exactly (selections whose fp64 margin is
below 1e-9 must instead be valid under that perturbation); outputs must be
within 2e-3 of the oracle, row-normalised.  Small layers are compared on every
token; the full GLM-5.2-shaped workloads route and permute every token and
compare sampled tokens' outputs (the oracle dequantises each needed expert,
about a second each)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_moe_02_amd as q
import synth
from gpu_common import TOL, check_outputs, check_routing, qexp, run_layer
from helpers import oracle_inputs, row_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


_CACHE = {}


def layer(name, tokens=None):
    key = (name, tokens)
    if key not in _CACHE:
        _CACHE.clear()
        torch.cuda.empty_cache()
        _CACHE[key] = synth.make_layer(name, "cuda", tokens=tokens)
    return _CACHE[key]


# ---------------------------------------------------------------------------
# tiny layer: every token, every entry point
# ---------------------------------------------------------------------------

def test_tiny_layer():
    L = layer("tiny")
    y, ids, tw = run_layer(L)
    ids_g, _ = check_routing(L, ids, tw)
    check_outputs(L, y, ids_g)


@pytest.mark.parametrize("T", [8, 1, 3])
def test_tiny_bf16_output_is_rne_of_fp32(T):
    """bf16 output is the round-to-nearest-even of the fp32 output, on the
    large-batch path (8 tokens) and the small-batch down kernels (1 and 3)."""
    L = layer("tiny")
    x = L.x[:T].contiguous()
    y32, _, _ = run_layer(L, q.MOE_OUT_F32, x=x)
    y16, _, _ = run_layer(L, q.MOE_OUT_BF16, x=x)
    assert torch.equal(y32.to(torch.bfloat16), y16)


def test_tiny_entry_points():
    L = layer("tiny")
    g = L.geom
    T, H, E, k = L.T, g["hidden"], g["n_routed_experts"], g["top_k"]
    P = T * k
    cfg = q.make_config(g, L.wfmt)
    ws = q.workspace(cfg, T)
    dev = dict(device="cuda")
    ids = torch.empty(T, k, dtype=torch.int32, **dev)
    tw = torch.empty(T, k, dtype=torch.float32, **dev)
    q.moe_route(cfg, T, L.x, L.router_w, L.bias, ids, tw, ws)
    torch.cuda.synchronize()
    ids_g, _ = check_routing(L, ids, tw)

    offs = torch.empty(E + 1, dtype=torch.int32, **dev)
    st = torch.empty(P, dtype=torch.int32, **dev)
    inv = torch.empty(P, dtype=torch.int32, **dev)
    act = torch.empty(E, dtype=torch.int32, **dev)
    na = torch.empty(1, dtype=torch.int32, **dev)
    q.moe_permute(cfg, T, ids, offs, st, inv, act, na, ws)
    torch.cuda.synchronize()
    r_off, r_st, r_inv, r_act = oracle.permute(ids_g, E)
    assert np.array_equal(offs.cpu().numpy(), r_off)
    assert np.array_equal(st.cpu().numpy(), r_st)
    assert np.array_equal(inv.cpu().numpy(), r_inv)
    assert int(na.item()) == len(r_act)
    assert np.array_equal(act.cpu().numpy()[: len(r_act)], r_act)

    x_np, Wr, b, rcfg, routed, shared = oracle_inputs(L)
    X = oracle.bf16_bits_to_f64(x_np)
    out = torch.empty(P, H, dtype=torch.float32, **dev)
    q.moe_expert_ffn_q4(cfg, T, L.x, qexp(L.routed), offs, st, act, na, out, ws)
    torch.cuda.synchronize()
    ref = np.zeros((P, H))
    for e in range(E):
        lo, hi = r_off[e], r_off[e + 1]
        if hi > lo:
            W = [routed.weight(p, e) for p in ("gate", "up", "down")]
            ref[lo:hi] = oracle.swiglu_ffn(X[r_st[lo:hi]], *W)
    assert row_rel_err(out.cpu().numpy(), ref).max() <= TOL

    outs = torch.empty(T, H, dtype=torch.float32, **dev)
    q.moe_expert_ffn_q4(cfg, T, L.x, qexp(L.shared), None, None, None, None, outs, ws)
    torch.cuda.synchronize()
    refs = oracle.swiglu_ffn(X, *[shared.weight(p, 0) for p in ("gate", "up", "down")])
    assert row_rel_err(outs.cpu().numpy(), refs).max() <= TOL

    y = torch.empty(T, H, dtype=torch.float32, **dev)
    q.moe_combine(cfg, T, out, inv, tw, outs, y)
    torch.cuda.synchronize()
    o64, s64 = out.double().cpu().numpy(), outs.double().cpu().numpy()
    w64 = tw.double().cpu().numpy()
    yref = s64 + np.einsum("tk,tkh->th", w64, o64[r_inv.reshape(T, k)])
    assert row_rel_err(y.cpu().numpy(), yref).max() <= 1e-6


@pytest.mark.parametrize("T,k,E,dist", [
    (1, 1, 16, "uniform"),
    (3, 4, 16, "uniform"),
    (64, 8, 256, "hot"),
    (1024, 8, 256, "uniform"),     # 8192 picks: the one-workgroup permutation
    (1025, 8, 256, "uniform"),     # 8200 picks: the three-launch permutation
    (2048, 4, 16, "one"),
])
def test_permute_paths(T, k, E, dist):
    """moe_permute equals the oracle's stable argsort on seeded ids, on both
    sides of the one-workgroup bound, with a hot expert and with every pick on
    one expert."""
    g = synth.small_geom(n_routed_experts=E, top_k=k, n_group=4, topk_group=4)
    cfg = q.make_config(g, "int4")
    rng = np.random.default_rng(7000 + T)
    if dist == "uniform":
        ids_np = rng.integers(0, E, size=(T, k))
    elif dist == "hot":
        ids_np = np.where(rng.random((T, k)) < 0.7, 5, rng.integers(0, E, size=(T, k)))
    else:
        ids_np = np.zeros((T, k), dtype=np.int64)
    dev = dict(device="cuda")
    ids = torch.from_numpy(ids_np.astype(np.int32)).to("cuda")
    P = T * k
    offs = torch.empty(E + 1, dtype=torch.int32, **dev)
    st = torch.empty(P, dtype=torch.int32, **dev)
    inv = torch.empty(P, dtype=torch.int32, **dev)
    act = torch.empty(E, dtype=torch.int32, **dev)
    na = torch.empty(1, dtype=torch.int32, **dev)
    q.moe_permute(cfg, T, ids, offs, st, inv, act, na, q.workspace(cfg, T))
    torch.cuda.synchronize()
    r_off, r_st, r_inv, r_act = oracle.permute(ids_np, E)
    assert np.array_equal(offs.cpu().numpy(), r_off)
    assert np.array_equal(st.cpu().numpy(), r_st)
    assert np.array_equal(inv.cpu().numpy(), r_inv)
    assert int(na.item()) == len(r_act)
    assert np.array_equal(act.cpu().numpy()[: len(r_act)], r_act)


def test_empty_input_is_noop():
    L = layer("tiny")
    cfg = q.make_config(L.geom, L.wfmt)
    y = torch.full((1, L.geom["hidden"]), 7.0, device="cuda")
    q.moe_layer(cfg, 0, L.x, L.router_w, L.bias, qexp(L.routed), qexp(L.shared), y)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


def test_determinism():
    L = layer("tiny")
    a = run_layer(L)
    b = run_layer(L)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


EDGE = {
    "T1":        (dict(), 1, "int4", "normal0.1"),
    "ragged37":  (dict(), 37, "int4", "normal0.1"),
    "one_group": (dict(n_group=1, topk_group=1), 19, "int4", "normal0.1"),
    "group_of_one": (dict(n_group=16, topk_group=4), 11, "int4", "normal0.1"),
    "k1":        (dict(top_k=1), 9, "int4", "normal0.1"),
    "k16":       (dict(n_routed_experts=64, n_group=4, topk_group=4, top_k=16), 21, "int4", "normal0.1"),
    # one token with more picks than the single-token down kernel holds
    "T1_k16":    (dict(n_routed_experts=64, n_group=4, topk_group=4, top_k=16), 1, "int4", "normal0.1"),
    "T1_k16_nvfp4": (dict(n_routed_experts=64, n_group=4, topk_group=4, top_k=16), 1, "nvfp4", "zipf"),
    "no_shared": (dict(n_shared_experts=0), 12, "int4", "normal0.1"),
    "min_dims":  (dict(hidden=32, moe_inter=32, shared_inter=32), 7, "int4", "normal0.1"),
    "E256":      (dict(n_routed_experts=256, n_group=8, topk_group=4, top_k=8, hidden=256,
                       moe_inter=64, shared_inter=64), 33, "int4", "zipf"),
    "ragged_groups": (dict(hidden=2080, moe_inter=96, shared_inter=160), 5, "int4", "normal0.1"),
    "nvfp4":     (dict(), 8, "nvfp4", "normal0.1"),
    "nvfp4_ragged": (dict(hidden=96, moe_inter=160, shared_inter=64), 13, "nvfp4", "zipf"),
    "nvfp4_T1":  (dict(), 1, "nvfp4", "normal0.1"),
    "nvfp4_T3":  (dict(hidden=96, moe_inter=160, shared_inter=64), 3, "nvfp4", "zipf"),
    "T1_uneven_shared": (dict(moe_inter=64, shared_inter=96), 1, "int4", "normal0.1"),
    # the GEMM's work units: one expert takes every token, so it gets one full
    # thin unit (32 tokens); with few would-be fat units every expert is cut
    # into thin units: a full and a one-token unit (33), two full (64), five
    # (160; the shared expert likewise); with many (about 160 tokens for each
    # of 16 experts) a full and a short fat unit each
    "hot_thin32": (dict(top_k=2), 32, "int4", "hot1"),
    "hot_cut33": (dict(top_k=2), 33, "int4", "hot1"),
    "hot_cut64": (dict(top_k=2), 64, "int4", "hot1"),
    "hot_cut160": (dict(top_k=2), 160, "int4", "hot1"),
    "fat_units": (dict(), 640, "int4", "normal0.1"),
    # 2..4 tokens: the small-batch down kernel that stages h in LDS (several
    # tokens per expert, no shared expert, one group per row, full 64-group
    # rows), and shapes that fall back to the per-block kernel (65 slots,
    # shared inter != routed inter)
    "T2": (dict(), 2, "int4", "normal0.1"),
    "T4": (dict(), 4, "int4", "normal0.1"),
    "T4_hot": (dict(top_k=2), 4, "int4", "hot1"),
    "T4_no_shared": (dict(n_shared_experts=0), 4, "int4", "normal0.1"),
    "T4_min_dims": (dict(hidden=32, moe_inter=32, shared_inter=32), 4, "int4", "normal0.1"),
    "T4_inter2048": (dict(hidden=512, moe_inter=2048, shared_inter=2048), 4, "int4", "zipf"),
    "T4_k16": (dict(n_routed_experts=64, n_group=4, topk_group=4, top_k=16), 4, "int4", "normal0.1"),
    "T3_uneven_shared": (dict(moe_inter=64, shared_inter=96), 3, "int4", "normal0.1"),
    "nvfp4_T4": (dict(), 4, "nvfp4", "zipf"),
    # K a multiple of 512: thin units read their scales through LDS
    "lds_scales": (dict(hidden=512, moe_inter=512, shared_inter=512), 9, "int4", "normal0.1"),
    "lds_scales_nvfp4": (dict(hidden=1024, moe_inter=512, shared_inter=512), 11, "nvfp4", "zipf"),
}


@pytest.mark.parametrize("case", sorted(EDGE))
def test_edge_geometries(case):
    over, T, wfmt, bias = EDGE[case]
    geom = synth.small_geom(**over)
    L = synth.make_custom(geom, T, wfmt, bias, seed=100 + sorted(EDGE).index(case), device="cuda")
    y, ids, tw = run_layer(L)
    ids_g, _ = check_routing(L, ids, tw)
    check_outputs(L, y, ids_g)


# ---------------------------------------------------------------------------
# full GLM-5.2-shaped workloads
# ---------------------------------------------------------------------------

def _full(name, sample):
    L = layer(name)
    y, ids, tw = run_layer(L)
    ids_g, near = check_routing(L, ids, tw)
    T = L.T
    idx = np.unique(np.linspace(0, T - 1, min(sample, T)).astype(int))
    err = check_outputs(L, y, ids_g, token_idx=idx)
    print(f"{name}: T={T} near-ties={near} sampled={len(idx)} max_row_err={err:.2e}", flush=True)


def test_full_decode():
    _full("decode", 1)


def test_decode_poisoned_workspace_reused():
    """Two different single tokens through one workspace whose bytes are all
    0xFF before the first call: every workspace value a call reads is written
    by that call first -- in particular the experts' SwiGLU outputs, which
    are published between workgroups inside one launch before the down
    projection reads them (a read before the write would see the NaN fill or
    the previous token's values)."""
    from helpers import np_u16
    L = layer("decode")
    g = L.geom
    H, k = g["hidden"], g["top_k"]
    cfg = q.make_config(g, L.wfmt)
    ws = q.workspace(cfg, 1)
    ws.fill_(0xFF)
    for seed in (11, 12):
        x = synth.make_tokens("decode", 1, "cuda", seed=seed)
        y = torch.empty(1, H, device="cuda", dtype=torch.float32)
        ids = torch.empty(1, k, dtype=torch.int32, device="cuda")
        tw = torch.empty(1, k, dtype=torch.float32, device="cuda")
        q.moe_layer(cfg, 1, x, L.router_w, L.bias, qexp(L.routed), qexp(L.shared), y,
                    q.MOE_OUT_F32, ids, tw, ws)
        torch.cuda.synchronize()
        assert torch.isfinite(y).all()
        xn = np_u16(x)
        ids_g, _ = check_routing(L, ids, tw, x_np=xn)
        check_outputs(L, y, ids_g, x_np=xn)


@pytest.mark.parametrize("case", ["T1", "nvfp4_T1", "decode"])
def test_single_token_fused_matches_two_launches(case, monkeypatch):
    """One token runs gate/up and down in one launch with a grid barrier
    between them; QMOE_DECODE_FUSED=0 selects the two-launch kernels, which
    sum in the same order.  Both match the oracle, and each other bit for
    bit."""
    if case == "decode":
        L = layer("decode")
    else:
        over, T, wfmt, bias = EDGE[case]
        L = synth.make_custom(synth.small_geom(**over), T, wfmt, bias, seed=300, device="cuda")
    fused = run_layer(L)
    monkeypatch.setenv("QMOE_DECODE_FUSED", "0")
    split = run_layer(L)
    ids_g, _ = check_routing(L, split[1], split[2])
    check_outputs(L, split[0], ids_g)
    for u, v in zip(fused, split):
        assert torch.equal(u, v)


def test_fused_decode_gives_up_to_nan(monkeypatch):
    """The fused single-token kernel's barrier wait is bounded.  With the bound
    forced to zero polls from the host, no workgroup waits: every row of y is
    NaN (never a sum over an incomplete h), the routing outputs are still
    written, and the next call is exact again."""
    over, T, wfmt, bias = EDGE["T1"]
    L = synth.make_custom(synth.small_geom(**over), T, wfmt, bias, seed=301, device="cuda")
    monkeypatch.setenv("QMOE_BARRIER_SPINS", "0")
    y, ids, tw = run_layer(L)
    assert torch.isnan(y).all()
    check_routing(L, ids, tw)
    monkeypatch.delenv("QMOE_BARRIER_SPINS")
    y, ids, tw = run_layer(L)
    ids_g, _ = check_routing(L, ids, tw)
    check_outputs(L, y, ids_g)


def test_full_verify4():
    _full("verify4", 4)


def test_full_verify64():
    _full("verify64", 3)


def test_full_prefill4k():
    _full("prefill4k", 2)


def test_full_nvfp4_512():
    _full("nvfp4_512", 2)


def test_full_prefill16k_routing_and_permutation():
    """T = 16384: every token's routing and the permutation exactly; one
    sampled token's output."""
    L = layer("prefill16k")
    g = L.geom
    T, E, k = L.T, g["n_routed_experts"], g["top_k"]
    cfg = q.make_config(g, L.wfmt)
    ws = q.workspace(cfg, T)
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    tw = torch.empty(T, k, dtype=torch.float32, device="cuda")
    q.moe_route(cfg, T, L.x, L.router_w, L.bias, ids, tw, ws)
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    st = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    act = torch.empty(E, dtype=torch.int32, device="cuda")
    na = torch.empty(1, dtype=torch.int32, device="cuda")
    q.moe_permute(cfg, T, ids, offs, st, inv, act, na, ws)
    torch.cuda.synchronize()
    ids_g, near = check_routing(L, ids, tw)
    r_off, r_st, r_inv, r_act = oracle.permute(ids_g, E)
    assert np.array_equal(offs.cpu().numpy(), r_off)
    assert np.array_equal(st.cpu().numpy(), r_st)
    assert np.array_equal(inv.cpu().numpy(), r_inv)
    del ws
    y, ids2, _ = run_layer(L)
    assert torch.equal(ids2, ids)
    check_outputs(L, y, ids_g, token_idx=[T // 2])
