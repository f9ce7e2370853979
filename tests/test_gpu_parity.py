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
from gpu_common import (TOL, FFNCache, check_outputs, check_routing, cover_tokens,
                        entry_point_chain, expert_slots_to_check, qexp, run_layer)
from helpers import np_u16, oracle_inputs, row_rel_err

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
    entry_point_chain(layer("tiny"))


@pytest.mark.parametrize("wfmt", ["int4", "nvfp4"])
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_small_batch_entry_points(T, wfmt):
    """moe_expert_ffn_q4 at 1-4 tokens runs the GEMV kernels (routed and dense
    mode), then combine."""
    L = synth.make_custom(synth.small_geom(), T, wfmt, "normal0.1", seed=400 + T, device="cuda")
    entry_point_chain(L)


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
    # (160; the shared expert likewise).  With 16 to 63 fat units of 192
    # tokens they are cut at 128: 640 and 700 tokens over 16 experts (experts
    # of 33 to 571 tokens, several units each) and one expert with all 1200
    # tokens beside experts of 57 to 105.  With 64 or more, units of up to 192
    # tokens (ten and twelve column tiles, experts of up to 1536 tokens).
    "hot_thin32": (dict(top_k=2), 32, "int4", "hot1"),
    "hot_cut33": (dict(top_k=2), 33, "int4", "hot1"),
    "hot_cut64": (dict(top_k=2), 64, "int4", "hot1"),
    "hot_cut160": (dict(top_k=2), 160, "int4", "hot1"),
    "fat_units": (dict(), 640, "int4", "normal0.1"),
    "fat_units_hot": (dict(top_k=2), 1200, "int4", "hot1"),
    "fat_units_nvfp4": (dict(), 700, "nvfp4", "normal0.1"),
    "fat_wide": (dict(n_routed_experts=64, n_group=4, topk_group=4, top_k=8), 1152, "int4",
                 "normal0.1"),
    "fat_wide_nvfp4": (dict(n_routed_experts=64, n_group=4, topk_group=4, top_k=8), 1536, "nvfp4",
                       "zipf"),
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
    # the small-batch down kernel's rows per wave (2048 waves): two with some
    # waves holding one (hidden 2080), four with most holding three (6176),
    # four everywhere (8192)
    "T3_h2080": (dict(hidden=2080, moe_inter=96, shared_inter=96), 3, "int4", "normal0.1"),
    "T2_h6176_nvfp4": (dict(hidden=6176, moe_inter=64, shared_inter=64), 2, "nvfp4", "normal0.1"),
    "T4_h8192": (dict(hidden=8192, moe_inter=128, shared_inter=128), 4, "int4", "zipf"),
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

def _full(name):
    """Every token's routing exactly; at up to 64 tokens every token's output,
    else the outputs of a set of tokens that covers every selected expert."""
    L = layer(name)
    y, ids, tw = run_layer(L)
    ids_g, near = check_routing(L, ids, tw)
    T = L.T
    idx = np.arange(T) if T <= 64 else cover_tokens(ids_g, always=(0, T - 1))
    _, _, _, _, routed, shared = oracle_inputs(L, lazy=True)
    err = check_outputs(L, y, ids_g, token_idx=idx, ffn_map=FFNCache(), srcs=(routed, shared))
    print(f"{name}: T={T} near-ties={near} checked={len(idx)} max_row_err={err:.2e}", flush=True)


def test_full_decode():
    _full("decode")


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
def test_single_token_fused_matches_two_launches(case):
    """One token runs gate/up and down in one launch with a grid barrier
    between them; MOE_OPT_NO_GRID_WAIT selects the kernels without one, which
    sum in the same order.  Both match the oracle, and each other bit for
    bit."""
    if case == "decode":
        L = layer("decode")
    else:
        over, T, wfmt, bias = EDGE[case]
        L = synth.make_custom(synth.small_geom(**over), T, wfmt, bias, seed=300, device="cuda")
    fused = run_layer(L)
    split = run_layer(L, options=q.MOE_OPT_NO_GRID_WAIT)
    ids_g, _ = check_routing(L, split[1], split[2])
    check_outputs(L, split[0], ids_g)
    for u, v in zip(fused, split):
        assert torch.equal(u, v)


SMALL_MERGED = {
    "T2": (dict(), 2, "int4", "normal0.1"),
    "T3_no_shared": (dict(n_shared_experts=0), 3, "int4", "normal0.1"),
    "T4": (dict(), 4, "int4", "zipf"),
    "T4_top_p": (dict(expert_top_p=0.6, top_k=6, topk_group=4), 4, "int4", "normal0.1"),
    "nvfp4_T3": EDGE["nvfp4_T3"],       # shared inter below moe_inter
    "T2_wide_shared": (dict(moe_inter=64, shared_inter=96), 2, "int4", "normal0.1"),
}


@pytest.mark.parametrize("case", sorted(SMALL_MERGED))
def test_small_batch_merged_matches_two_launches(case):
    """2-4 tokens run the selection and gate/up in one launch, the gate/up
    workgroups waiting for the selecting one; MOE_OPT_NO_GRID_WAIT runs them as
    two launches.  Both match the oracle, and each other bit for bit."""
    over, T, wfmt, bias = SMALL_MERGED[case]
    L = synth.make_custom(synth.small_geom(**over), T, wfmt, bias, seed=310 + T, device="cuda")
    ws = q.workspace(q.make_config(L.geom, L.wfmt), T)
    merged = run_layer(L, ws=ws)
    assert q.moe_layer_flags(ws) == 0
    split = run_layer(L, options=q.MOE_OPT_NO_GRID_WAIT)
    ids_g, _ = check_routing(L, split[1], split[2])
    check_outputs(L, split[0], ids_g)
    for u, v in zip(merged, split):
        assert torch.equal(u, v)


def test_small_batch_gives_up_to_nan():
    """The gate/up workgroups' wait for the selection is bounded: with no poll
    allowed, every routed h row is NaN, so is y, the routing is written and
    the flag raised; the next call clears it and is exact."""
    over, T, wfmt, bias = SMALL_MERGED["T4"]
    L = synth.make_custom(synth.small_geom(**over), T, wfmt, bias, seed=320, device="cuda")
    ws = q.workspace(q.make_config(L.geom, L.wfmt), T)
    y, ids, tw = run_layer(L, options=q.MOE_OPT_GRID_WAIT_NONE, ws=ws)
    assert torch.isnan(y).all()
    check_routing(L, ids, tw)
    assert q.moe_layer_flags(ws) == q.MOE_FLAG_GRID_WAIT_TIMEOUT
    y, ids, tw = run_layer(L, ws=ws)
    assert q.moe_layer_flags(ws) == 0
    ids_g, _ = check_routing(L, ids, tw)
    check_outputs(L, y, ids_g)


def test_fused_decode_gives_up_to_nan():
    """The fused single-token kernel's barrier wait is bounded.  With no poll
    allowed (MOE_OPT_GRID_WAIT_NONE, set from the host), no workgroup waits:
    every row of y is NaN (never a sum over an incomplete h), the routing
    outputs are still written, and the workspace flag says so.  The next call
    on the same workspace clears the flag and is exact again."""
    over, T, wfmt, bias = EDGE["T1"]
    L = synth.make_custom(synth.small_geom(**over), T, wfmt, bias, seed=301, device="cuda")
    ws = q.workspace(q.make_config(L.geom, L.wfmt), T)
    y, ids, tw = run_layer(L, options=q.MOE_OPT_GRID_WAIT_NONE, ws=ws)
    assert torch.isnan(y).all()
    check_routing(L, ids, tw)
    assert q.moe_layer_flags(ws) == q.MOE_FLAG_GRID_WAIT_TIMEOUT
    y, ids, tw = run_layer(L, ws=ws)
    assert q.moe_layer_flags(ws) == 0
    ids_g, _ = check_routing(L, ids, tw)
    check_outputs(L, y, ids_g)
    # a large-batch call clears a raised flag too (the flags word is at offset
    # 0 of every workspace)
    L8 = layer("tiny")
    ws8 = q.workspace(q.make_config(L8.geom, L8.wfmt), L8.T)
    run_layer(L, options=q.MOE_OPT_GRID_WAIT_NONE, ws=ws8)
    assert q.moe_layer_flags(ws8) == q.MOE_FLAG_GRID_WAIT_TIMEOUT
    run_layer(L8, ws=ws8)
    assert q.moe_layer_flags(ws8) == 0


def test_full_verify4():
    _full("verify4")


def test_full_verify4_entry_points():
    """The GEMV kernels behind moe_expert_ffn_q4 at 4 tokens at full size."""
    entry_point_chain(layer("verify4"), pool=True)


def test_full_verify64():
    _full("verify64")


def _full_large(name):
    """A large batch at full size, through the entry points and the layer:
      * routing of every token exactly, and the permutation of the GPU's ids;
      * moe_expert_ffn_q4's routed output at every sorted slot of eight
        experts (the most and least loaded, ragged last work units) and at the
        first, a middle and the last slot of every other active expert;
      * its dense output (the shared expert) on 256 tokens, the last included;
      * moe_layer's output on tokens that together cover every selected
        expert.
    Each expert is dequantised once by the oracle (worker processes)."""
    L = layer(name)
    g = L.geom
    T, H, E, k = L.T, g["hidden"], g["n_routed_experts"], g["top_k"]
    P = T * k
    cfg = q.make_config(g, L.wfmt)
    y, ids, tw = run_layer(L)
    ids_g, near = check_routing(L, ids, tw)
    ws = q.workspace(cfg, T)
    dev = dict(device="cuda")
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
    out = torch.empty(P, H, dtype=torch.float32, **dev)
    q.moe_expert_ffn_q4(cfg, T, L.x, qexp(L.routed), offs, st, act, na, out, ws)
    outs = torch.empty(T, H, dtype=torch.float32, **dev)
    q.moe_expert_ffn_q4(cfg, T, L.x, qexp(L.shared), None, None, None, None, outs, ws)
    torch.cuda.synchronize()
    del ws

    slots = expert_slots_to_check(r_off, seed=T)
    cover = cover_tokens(ids_g, always=(0, T - 1))
    dense_rows = np.unique(np.append(np.linspace(0, T - 1, 255).astype(int), T - 1))
    x_np, _, _, _, routed, shared = oracle_inputs(L, lazy=True)
    X = oracle.bf16_bits_to_f64(x_np)
    # every expert's rows for all three checks in one job, so it is dequantised once
    cov_ids = ids_g[cover]
    jobs = []
    for e, sl in slots.items():
        toks = np.union1d(r_st[sl], cover[np.any(cov_ids == e, axis=1)])
        jobs.append((routed, e, X[toks]))
    jobs.append((shared, 0, X[np.union1d(dense_rows, cover)]))
    cache = FFNCache()
    cache.fill(jobs)

    all_sl = np.concatenate([slots[e] for e in sorted(slots)])
    got = out[torch.from_numpy(all_sl).to("cuda")].double().cpu().numpy()
    ref = np.concatenate(cache([(routed, e, X[r_st[slots[e]]]) for e in sorted(slots)]))
    err_o = row_rel_err(got, ref)
    assert err_o.max() <= TOL, f"expert output row error {err_o.max():.3e} at slot {all_sl[err_o.argmax()]}"
    err_s = row_rel_err(outs.cpu().numpy()[dense_rows], cache([(shared, 0, X[dense_rows])])[0])
    assert err_s.max() <= TOL, err_s.max()
    err_y = check_outputs(L, y, ids_g, token_idx=cover, ffn_map=cache, srcs=(routed, shared))
    print(f"{name}: T={T} near-ties={near} expert rows={len(all_sl)} ({len(slots)} experts) "
          f"max err {err_o.max():.2e}; shared rows {len(dense_rows)} {err_s.max():.2e}; "
          f"layer tokens {len(cover)} {err_y:.2e}", flush=True)


def test_full_nvfp4_512():
    _full_large("nvfp4_512")


def test_full_nvfp4_4_entry_points():
    """NVFP4 GEMV kernels at 4 tokens at full size (the NVFP4 layer's first
    four tokens)."""
    L = layer("nvfp4_512")
    entry_point_chain(L, x=L.x[:4].contiguous(), pool=True)


def test_full_prefill4k():
    _full_large("prefill4k")


def test_full_prefill16k():
    _full_large("prefill16k")


# ---------------------------------------------------------------------------
# raw packed bytes and exact router ties
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("wfmt", ["int4", "nvfp4"])
@pytest.mark.parametrize("T", [1, 3, 8, 40, 640])
def test_raw_weight_bytes(T, wfmt):
    """Uniformly random code bytes (int4 code 0, E2M1 -0 included) and random
    scales of either sign (finite E4M3 codes for NVFP4) through every path:
    one token (fused kernel), 3 tokens (small-batch kernels), 8 and 40 tokens
    (thin GEMM units), 640 tokens (fat units)."""
    L = synth.make_raw(synth.small_geom(), T, wfmt, seed=500 + T, device="cuda")
    y, ids, tw = run_layer(L)
    ids_g, _ = check_routing(L, ids, tw)
    check_outputs(L, y, ids_g)
    if T <= 4:
        entry_point_chain(L)


TIE_BIAS = {
    "zero": lambda E: np.zeros(E),
    "mod3": lambda E: 0.125 * (np.arange(E) % 3),
    "pairs": lambda E: 0.0625 * ((np.arange(E) * 5) % 4),
}


@pytest.mark.parametrize("bias", sorted(TIE_BIAS))
@pytest.mark.parametrize("T", [1, 3, 37])
def test_exact_router_ties(T, bias):
    """Zero router weights make every sigmoid score exactly 1/2, so the
    selection is decided by biases with exact ties (equal group scores, equal
    biased scores): the ids must equal the oracle's tie-break (lower group,
    lower id) exactly, with no near-tie leniency, and every weight is
    rsf / top_k."""
    geom = synth.small_geom()
    L = synth.make_custom(geom, T, "int4", "zero", seed=600 + T, device="cuda")
    L.router_w.zero_()
    L.bias.copy_(torch.from_numpy(TIE_BIAS[bias](geom["n_routed_experts"])).float())
    y, ids, tw = run_layer(L)
    x, Wr, b, cfg, _, _ = oracle_inputs(L)
    ids_ref, w_ref, info = oracle.route(oracle.bf16_bits_to_f64(x), Wr, b, cfg)
    assert np.all(info["margin"] == 0) or bias != "zero"
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.array_equal(tw.cpu().numpy(), w_ref.astype(np.float32))
    check_outputs(L, y, ids_ref)


@pytest.mark.parametrize("bias", sorted(TIE_BIAS))
@pytest.mark.parametrize("T", [1, 4])
def test_exact_router_ties_split_small(T, bias):
    """The same on the split path at 1 and 4 tokens (per-row int8: routing and
    the sort of the picks in one workgroup).  Every token then picks the same
    experts, so each selected expert holds T picks in token order."""
    geom = synth.small_geom()
    L = synth.make_custom(geom, T, "int8_row", "zero", seed=640 + T, device="cuda")
    L.router_w.zero_()
    L.bias.copy_(torch.from_numpy(TIE_BIAS[bias](geom["n_routed_experts"])).float())
    y, ids, tw = run_layer(L)
    x, Wr, b, cfg, _, _ = oracle_inputs(L)
    ids_ref, w_ref, _ = oracle.route(oracle.bf16_bits_to_f64(x), Wr, b, cfg)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.array_equal(tw.cpu().numpy(), w_ref.astype(np.float32))
    check_outputs(L, y, ids_ref)


def test_exact_router_ties_full_decode():
    """The same at the GLM-5.2 decode shape (one token, fused kernel)."""
    L = layer("decode")
    rw, b0 = L.router_w.clone(), L.bias.clone()
    try:
        L.router_w.zero_()
        E = L.geom["n_routed_experts"]
        L.bias.copy_(torch.from_numpy(0.0625 * ((np.arange(E) * 5) % 4)).float())
        y, ids, tw = run_layer(L)
        x, Wr, b, cfg, _, _ = oracle_inputs(L, lazy=True)
        ids_ref, w_ref, _ = oracle.route(oracle.bf16_bits_to_f64(x), Wr, b, cfg)
        assert np.array_equal(ids.cpu().numpy(), ids_ref)
        assert np.array_equal(tw.cpu().numpy(), w_ref.astype(np.float32))
        check_outputs(L, y, ids_ref)
    finally:
        L.router_w.copy_(rw)
        L.bias.copy_(b0)


# ---------------------------------------------------------------------------
# adaptive expert top-p
# ---------------------------------------------------------------------------

TOP_P = {
    "T1": (1, "int4", 0),
    "T1_split": (1, "int4", q.MOE_OPT_NO_GRID_WAIT),
    "T3": (3, "int4", 0),
    "T4_nvfp4": (4, "nvfp4", 0),
    "T37": (37, "int4", 0),
    "T640": (640, "int4", 0),
    "T40_nvfp4": (40, "nvfp4", 0),
    # the split path's one-workgroup selection and sort (per-row int8)
    "T1_int8": (1, "int8_row", 0),
    "T4_int8": (4, "int8_row", 0),
}


@pytest.mark.parametrize("p", [0.35, 0.7])
@pytest.mark.parametrize("case", sorted(TOP_P))
def test_top_p_paths(case, p):
    """Every kernel path with the adaptive top-p: ids exact (kept ids
    ascending, then -1), weights renormalised over the kept experts, outputs
    against the oracle; some tokens keep fewer than top_k experts."""
    T, wfmt, options = TOP_P[case]
    geom = synth.small_geom(expert_top_p=p, top_k=6, topk_group=4)
    L = synth.make_custom(geom, T, wfmt, "normal0.1", seed=700 + T, device="cuda")
    y, ids, tw = run_layer(L, options=options)
    ids_g, _ = check_routing(L, ids, tw)
    check_outputs(L, y, ids_g)
    n_kept = (ids_g >= 0).sum(1)
    assert n_kept.min() >= 1 and (T < 8 or n_kept.min() < geom["top_k"])


def test_top_p_fused_matches_split_and_entry_points():
    geom = synth.small_geom(expert_top_p=0.6, top_k=6, topk_group=4)
    L = synth.make_custom(geom, 1, "int4", "normal0.1", seed=720, device="cuda")
    a = run_layer(L)
    b = run_layer(L, options=q.MOE_OPT_NO_GRID_WAIT)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    L8 = synth.make_custom(geom, 8, "int4", "normal0.1", seed=721, device="cuda")
    entry_point_chain(L8)


def test_top_p_full_size():
    """The GLM-5.2 decode layer (one token, fused kernel) and the 64-token
    verify batch with expert_top_p 0.7 (the pages' setting): every token."""
    for name in ("decode", "verify64"):
        L = layer(name)
        L.geom["expert_top_p"] = 0.7
        try:
            y, ids, tw = run_layer(L)
            ids_g, _ = check_routing(L, ids, tw)
            _, _, _, _, routed, shared = oracle_inputs(L, lazy=True)
            check_outputs(L, y, ids_g, ffn_map=FFNCache(), srcs=(routed, shared))
            print(f"{name} top-p 0.7: experts kept per token {(ids_g >= 0).sum(1).mean():.2f} "
                  f"of {L.geom['top_k']}", flush=True)
        finally:
            del L.geom["expert_top_p"]
