"""Pins of the fp64 oracle against facts it does not compute itself: library
routines, closed forms, brute force on tiny inputs, invariants and hand-built
byte layouts.  CPU only."""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import oracle_inputs, np_u16, router_cfg


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def test_e4m3_exhaustive_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3fn(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    # a few landmarks of the format: max 448, min subnormal 2^-9, 1.0 = 0x38
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0


def test_e2m1_table():
    # OCP FP4 E2M1 value table, positive codes 0..7 then negative 8..15
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = oracle.decode_e2m1(np.arange(16))
    assert list(got[:8]) == table
    assert list(-got[8:]) == table


def test_e2m1_vs_torch_if_available():
    dt = getattr(torch, "float4_e2m1fn_x2", None)
    if dt is None:
        pytest.skip("torch has no float4_e2m1fn_x2")
    codes = np.arange(256, dtype=np.uint8)   # each byte = two codes
    try:
        ref = torch.from_numpy(codes).view(dt).to(torch.float32)
    except Exception as exc:  # CPU conversion not implemented in this torch
        pytest.skip(f"no CPU conversion for float4_e2m1fn_x2: {exc}")
    ref = ref.double().numpy().reshape(-1)
    lo = oracle.decode_e2m1(codes & 15)
    hi = oracle.decode_e2m1(codes >> 4)
    assert np.array_equal(ref, np.stack([lo, hi], -1).reshape(-1))


def test_bf16_and_fp16_widening():
    x = torch.randn(1000, dtype=torch.float32)
    b = x.to(torch.bfloat16)
    assert np.array_equal(oracle.bf16_bits_to_f64(np_u16(b)), b.double().numpy())
    h = x.to(torch.float16)
    assert np.array_equal(oracle.fp16_bits_to_f64(np_u16(h)), h.double().numpy())
    assert oracle.bf16_bits_to_f64(np.uint16(0x3F80)) == 1.0
    assert oracle.bf16_bits_to_f64(np.uint16(0xC040)) == -3.0


# ---------------------------------------------------------------------------
# Layout probes: bytes built by hand from the documented bit positions
# ---------------------------------------------------------------------------

def _int4_bytes_from_codes_by_position(codes):
    """Place code of input k at the bit position the format documents."""
    N, K = codes.shape
    out = np.zeros((N, K // 2), np.uint8)
    for n in range(N):
        for k in range(K):
            j, r = divmod(k, 8)
            bit = 4 * (r // 2) + 16 * (r % 2)
            byte, sh = 4 * j + bit // 8, bit % 8
            out[n, byte] |= np.uint8(int(codes[n, k]) << sh)
    return out


def test_int4_layout_one_hot_probe():
    K = 64
    for k in range(K):
        codes = np.full((1, K), 8, np.uint8)
        codes[0, k] = 9                       # q = +1 at input k only
        q = _int4_bytes_from_codes_by_position(codes)
        s = np.full((1, K // 32), np.float16(0.5)).view(np.uint16)
        w = oracle.dequant_int4(q, s)
        expect = np.zeros((1, K))
        expect[0, k] = 0.5
        assert np.array_equal(w, expect), k


def test_int4_group_alignment_probe():
    K = 96
    codes = np.full((2, K), 9, np.uint8)          # q = 1 everywhere
    s = np.array([[1.0, 2.0, 4.0], [0.25, 0.5, 8.0]], np.float16).view(np.uint16)
    w = oracle.dequant_int4(_int4_bytes_from_codes_by_position(codes), s)
    assert np.array_equal(w[0], np.repeat([1.0, 2.0, 4.0], 32))
    assert np.array_equal(w[1], np.repeat([0.25, 0.5, 8.0], 32))
    # u = 0 decodes to -8 (the format accepts it even though the encoder never emits it)
    codes[:] = 0
    w = oracle.dequant_int4(_int4_bytes_from_codes_by_position(codes), s)
    assert np.array_equal(w[0], -8.0 * np.repeat([1.0, 2.0, 4.0], 32))


def test_synth_int4_packer_matches_documented_layout():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, size=(3, 64), dtype=np.uint8)
    ref = _int4_bytes_from_codes_by_position(codes)
    got = synth.pack_int4_words(torch.from_numpy(codes)).numpy()
    assert np.array_equal(ref, got)
    assert np.array_equal(oracle.unpack_int4_codes(ref), codes)


def test_nvfp4_layout_probe():
    K = 32
    for k in range(K):
        codes = np.zeros((1, K), np.uint8)
        codes[0, k] = 0xB                       # -1.5
        q = np.zeros((1, K // 2), np.uint8)
        for kk in range(K):
            q[0, kk // 2] |= np.uint8(int(codes[0, kk]) << (4 * (kk % 2)))
        s = np.array([[0x38, 0x40]], np.uint8)  # e4m3 1.0 and 2.0
        w = oracle.dequant_nvfp4(q, s, 0.5)
        expect = np.zeros((1, K))
        expect[0, k] = -1.5 * (1.0 if k < 16 else 2.0) * 0.5
        assert np.array_equal(w, expect), k
        assert np.array_equal(synth.pack_nibbles_natural(torch.from_numpy(codes)).numpy(), q)


# ---------------------------------------------------------------------------
# Quantise / dequantise round trips
# ---------------------------------------------------------------------------

def test_int4_roundtrip_bound():
    W = torch.randn(64, 256) * 0.02
    W[3, :32] = 0.0                              # an all-zero group
    q, s = synth.quantize_int4_g32(W)
    w = oracle.dequant_int4(q.numpy(), np_u16(s))
    sd = oracle.fp16_bits_to_f64(np_u16(s))
    bound = np.repeat(sd, 32, axis=1) / 2 * (1 + 1e-12)
    assert np.all(np.abs(w - W.double().numpy()) <= bound)
    assert np.all(w[3, :32] == 0.0)


def test_int4_on_grid_roundtrip_exact():
    rng = np.random.default_rng(1)
    qv = rng.integers(-7, 8, size=(16, 128)).astype(np.float64)
    qv[:, ::32] = 7                              # every group reaches absmax = 7*s
    s = np.float16(0.0078125) * (1 + np.arange(16)[:, None, None] % 4)   # exact in fp16
    W = (qv.reshape(16, 4, 32) * s.astype(np.float64)).reshape(16, 128)
    q, sc = synth.quantize_int4_g32(torch.from_numpy(W).float())
    assert np.array_equal(oracle.dequant_int4(q.numpy(), np_u16(sc)), W)


def test_nvfp4_roundtrip_bound():
    W = torch.randn(32, 256) * 0.02
    W[0, 16:32] = 0.0
    q, s8, g = synth.quantize_nvfp4(W.unsqueeze(0))
    g = float(g[0])
    w = oracle.dequant_nvfp4(q[0].numpy(), s8[0].numpy(), g)
    sd = np.repeat(oracle.decode_e4m3fn(s8[0].numpy()), 16, axis=1) * np.float64(np.float32(g))
    v = np.abs(W.double().numpy()) / np.where(sd > 0, sd, 1)
    rho = np.where(v <= 2, 0.25, np.where(v <= 4, 0.5, 1.0))
    assert np.all(np.abs(w - W.double().numpy()) <= rho * sd + 1e-15)
    assert np.all(w[0, 16:32] == 0.0)


def test_nvfp4_on_grid_roundtrip_exact():
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -.5, -1, -1.5, -2, -3, -4, -6])
    rng = np.random.default_rng(2)
    v = rng.choice(grid, size=(8, 64))
    v[:, ::16] = 6.0                            # every block reaches |v| = 6
    # W = 1.75 v: tensor absmax 10.5 -> g = 10.5/(6*448) = 2^-8 exactly, and
    # every block's scale is 448 (E4M3 max), so w/(s*g) = v lands on the grid.
    W = v * 1.75
    q, s8, g = synth.quantize_nvfp4(torch.from_numpy(W).float().unsqueeze(0))
    w = oracle.dequant_nvfp4(q[0].numpy(), s8[0].numpy(), float(g[0]))
    assert np.array_equal(w, W)


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------

def _tiny():
    L = synth.make_layer("tiny")
    return L, oracle_inputs(L)


def test_router_invariants_tiny():
    L, (x, Wr, b, cfg, _, _) = _tiny()
    X = oracle.bf16_bits_to_f64(x)
    ids, w, info = oracle.route(X, Wr, b, cfg)
    per = cfg.n_experts // cfg.n_group
    for t in range(ids.shape[0]):
        assert len(set(ids[t])) == cfg.top_k
        assert list(ids[t]) == sorted(ids[t])
        groups = set((ids[t] // per).tolist())
        kept = set(np.nonzero(info["keep"][t])[0].tolist())
        assert groups <= kept and len(kept) == cfg.topk_group
        # kept groups have the highest group scores
        gs = info["gscore"][t]
        assert min(gs[list(kept)]) >= max(gs[[g for g in range(cfg.n_group) if g not in kept]])
        assert np.all(w[t] > 0)
        assert abs(w[t].sum() - cfg.routed_scaling_factor) <= 1e-12 * cfg.routed_scaling_factor


def test_router_brute_force_tiny():
    """Enumerate every group subset and every k-subset of allowed experts."""
    L, (x, Wr, b, cfg, _, _) = _tiny()
    X = oracle.bf16_bits_to_f64(x)
    ids, _, _ = oracle.route(X, Wr, b, cfg)
    E, G, per = cfg.n_experts, cfg.n_group, cfg.n_experts // cfg.n_group
    logits = np.array([[sum(X[t, h] * Wr[e, h] for h in range(X.shape[1])) for e in range(E)]
                       for t in range(X.shape[0])])
    s = np.array([[1 / (1 + math.exp(-v)) for v in row] for row in logits])
    sb = s + b
    for t in range(X.shape[0]):
        gscore = [sum(sorted(sb[t, g * per:(g + 1) * per], reverse=True)[:2]) for g in range(G)]
        best_groups = max(itertools.combinations(range(G), cfg.topk_group),
                          key=lambda c: sum(gscore[g] for g in c))
        allowed = [e for g in best_groups for e in range(g * per, (g + 1) * per)]
        best = max(itertools.combinations(allowed, cfg.top_k), key=lambda c: sum(sb[t, e] for e in c))
        assert sorted(best) == list(ids[t]), t


def test_router_reduces_to_topk_sigmoid():
    """G = TG = 1 and zero bias: plain top-k of sigmoid(logits) (torch.topk)."""
    geom = synth.small_geom(n_group=1, topk_group=1)
    L = synth.make_custom(geom, 64, "int4", "zero", seed=7)
    x, Wr, b, cfg, _, _ = oracle_inputs(L)
    X = oracle.bf16_bits_to_f64(x)
    ids, w, info = oracle.route(X, Wr, b, cfg)
    logits = torch.from_numpy(X) @ torch.from_numpy(Wr).T
    vals, ref = torch.topk(torch.sigmoid(logits), cfg.top_k, dim=1)
    ok = info["margin"] > 1e-12
    assert ok.sum() > 60
    assert np.array_equal(np.sort(ref.numpy(), 1)[ok], ids[ok])
    wref = vals / vals.sum(1, keepdim=True) * cfg.routed_scaling_factor
    order = np.argsort(ref.numpy(), 1)
    assert np.allclose(np.take_along_axis(wref.numpy(), order, 1)[ok], w[ok], rtol=1e-13)


def test_router_all_experts_closed_form():
    """k = E, one group: w = rsf * s / sum(s) over all experts."""
    geom = synth.small_geom(n_group=1, topk_group=1, top_k=16)
    L = synth.make_custom(geom, 8, "int4", "normal0.1", seed=8)
    x, Wr, b, cfg, _, _ = oracle_inputs(L)
    X = oracle.bf16_bits_to_f64(x)
    ids, w, _ = oracle.route(X, Wr, b, cfg)
    assert np.array_equal(ids, np.tile(np.arange(16), (8, 1)))
    s = 1 / (1 + np.exp(-(X @ Wr.T)))
    assert np.allclose(w, 2.5 * s / s.sum(1, keepdims=True), rtol=1e-14)


def test_router_masks_dropped_groups_even_with_negative_scores():
    """A huge negative bias on the kept groups' experts must not leak picks to
    dropped groups: exactly k experts from the kept groups."""
    cfg = oracle.RouterConfig(8, 4, 1, 2, 1.0)
    X = np.zeros((1, 4))
    Wr = np.zeros((8, 4))
    b = np.array([-5.0, -6.0, -9, -9, -9, -9, -9, -9])   # group 0 wins on score
    ids, w, info = oracle.route(X, Wr, b, cfg)
    assert list(ids[0]) == [0, 1]


def test_router_tie_break_lower_index():
    cfg = oracle.RouterConfig(8, 2, 1, 2, 1.0)
    X = np.zeros((1, 4))
    Wr = np.zeros((8, 4))
    b = np.zeros(8)                                     # every score equal
    ids, _, _ = oracle.route(X, Wr, b, cfg)
    assert list(ids[0]) == [0, 1]


def test_valid_under_perturbation():
    cfg = oracle.RouterConfig(8, 2, 1, 2, 1.0)
    sb = np.array([0.9, 0.5, 0.5 - 1e-12, 0.1, 0.2, 0.2, 0.2, 0.2])
    assert oracle.valid_under_perturbation(np.array([0, 1]), sb, cfg, 1e-9)
    assert oracle.valid_under_perturbation(np.array([0, 2]), sb, cfg, 1e-9)   # near tie
    assert not oracle.valid_under_perturbation(np.array([0, 3]), sb, cfg, 1e-9)
    assert not oracle.valid_under_perturbation(np.array([0, 4]), sb, cfg, 1e-9)  # other group


@pytest.mark.slow
def test_hot_skew_share_at_glm_shape():
    """The hot-16 bias recipe puts about 30% of top-8 picks on the hot experts
    at hidden 6144 (the batched-verify workload's skew)."""
    geom = synth.WORKLOADS["verify64"]["geom"]
    seed = synth.BASE_SEED + synth.WORKLOADS["verify64"]["index"]
    Wr = synth.randn((256, 6144), synth.sub_seed(seed, 2), "cpu", synth.WEIGHT_STD).double().numpy()
    b = synth.make_bias("hot16", 256, seed).double().numpy()
    X = synth.to_bf16(synth.randn((2048, 6144), 99, "cpu")).double().numpy()
    ids, _, _ = oracle.route(X, Wr, b, router_cfg(geom))
    hot = np.nonzero(b > 0)[0]
    share = np.isin(ids, hot).mean()
    assert 0.27 <= share <= 0.33, share


# ---------------------------------------------------------------------------
# Permutation
# ---------------------------------------------------------------------------

def test_permute_vs_library():
    rng = np.random.default_rng(3)
    for T, k, E in [(1, 8, 256), (37, 4, 16), (512, 8, 256)]:
        ids = np.sort(rng.choice(E, size=(T, k), replace=True), 1)
        offs, st, inv, act = oracle.permute(ids, E)
        flat = ids.reshape(-1)
        order = np.argsort(flat, kind="stable")
        assert np.array_equal(st, order // k)
        assert np.array_equal(np.diff(offs), np.bincount(flat, minlength=E))
        assert offs[0] == 0 and offs[-1] == T * k and np.all(np.diff(offs) >= 0)
        assert np.array_equal(order[inv], np.arange(T * k))       # inverse
        assert np.array_equal(act, np.unique(flat))


# ---------------------------------------------------------------------------
# FFN and layer
# ---------------------------------------------------------------------------

def test_ffn_one_hot_input_probe():
    """x = e_j picks column j of each dequantised matrix."""
    L, (x, Wr, b, cfg, routed, shared) = _tiny()
    Wg, Wu, Wd = (routed.weight(p, 3) for p in ("gate", "up", "down"))
    H = Wg.shape[1]
    for j in (0, 1, 8, 17, 31, 32, H - 1):
        X = np.zeros((1, H))
        X[0, j] = 1.0
        g, u = Wg[:, j], Wu[:, j]
        h = g / (1 + np.exp(-g)) * u
        ref = np.array([sum(Wd[r, i] * h[i] for i in range(len(h))) for r in range(H)])
        assert np.allclose(oracle.swiglu_ffn(X, Wg, Wu, Wd)[0], ref, rtol=1e-12, atol=1e-15)


def test_ffn_constant_codes():
    """Codes u = 9 (q = +1) everywhere: gate = up = scale * sum(x)."""
    H, I = 64, 32
    codes = np.full((I, H), 9, np.uint8)
    q = synth.pack_int4_words(torch.from_numpy(codes)).numpy()
    s = np.full((I, H // 32), np.float16(0.125)).view(np.uint16)
    W = oracle.dequant_int4(q, s)
    X = np.random.default_rng(4).standard_normal((3, H))
    G = X @ W.T
    assert np.allclose(G, 0.125 * X.sum(1, keepdims=True) * np.ones((1, I)), rtol=1e-13)


def test_ffn_vs_torch_float64():
    rng = np.random.default_rng(5)
    X = rng.standard_normal((5, 64))
    Wg, Wu = rng.standard_normal((2, 32, 64)) * 0.1
    Wd = rng.standard_normal((64, 32)) * 0.1
    t = lambda a: torch.from_numpy(a)
    ref = (torch.nn.functional.silu(t(X) @ t(Wg).T) * (t(X) @ t(Wu).T)) @ t(Wd).T
    assert np.allclose(oracle.swiglu_ffn(X, Wg, Wu, Wd), ref.numpy(), rtol=1e-12, atol=1e-14)


def test_dense_equivalence_tiny():
    L, (x, Wr, b, cfg, routed, shared) = _tiny()
    y, ids, w = oracle.layer(x, Wr, b, cfg, routed, shared)
    yd = oracle.dense_layer(x, Wr, b, cfg, routed, shared)
    assert np.allclose(y, yd, rtol=1e-12, atol=1e-14)


def test_layer_identical_experts():
    """All routed experts identical: y = rsf * FFN(x) + FFN_s(x)."""
    L, (x, Wr, b, cfg, routed, shared) = _tiny()
    same = oracle.ExpertSource("int4", *[tuple(np.repeat(a[:1], a.shape[0], 0) if a is not None else None
                                               for a in getattr(routed, p)) for p in ("gate", "up", "down")])
    y, _, _ = oracle.layer(x, Wr, b, cfg, same, shared)
    X = oracle.bf16_bits_to_f64(x)
    W0 = [routed.weight(p, 0) for p in ("gate", "up", "down")]
    Ws = [shared.weight(p, 0) for p in ("gate", "up", "down")]
    ref = cfg.routed_scaling_factor * oracle.swiglu_ffn(X, *W0) + oracle.swiglu_ffn(X, *Ws)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_layer_zero_shared_zero_input_and_down_scaling():
    L, (x, Wr, b, cfg, routed, shared) = _tiny()
    zero_shared = oracle.ExpertSource("int4", *[(a[0], np.zeros_like(a[1]), None)
                                                for a in (shared.gate, shared.up, shared.down)])
    y0, _, _ = oracle.layer(x, Wr, b, cfg, routed, None)
    y1, _, _ = oracle.layer(x, Wr, b, cfg, routed, zero_shared)
    assert np.array_equal(y0, y1)
    yz, _, _ = oracle.layer(np.zeros_like(x), Wr, b, cfg, routed, shared)
    assert np.all(yz == 0)
    # doubling every down-projection scale doubles the routed part exactly
    d = routed.down
    s2 = (oracle.fp16_bits_to_f64(d[1]) * 2).astype(np.float16).view(np.uint16)
    routed2 = oracle.ExpertSource("int4", routed.gate, routed.up, (d[0], s2, None))
    y2, _, _ = oracle.layer(x, Wr, b, cfg, routed2, None)
    assert np.allclose(y2, 2 * y0, rtol=1e-12, atol=1e-14)


def test_layer_token_subset_matches_full():
    L, (x, Wr, b, cfg, routed, shared) = _tiny()
    y, ids, _ = oracle.layer(x, Wr, b, cfg, routed, shared)
    idx = np.array([1, 5, 6])
    ys, ids_s, _ = oracle.layer(x, Wr, b, cfg, routed, shared, token_idx=idx)
    assert np.array_equal(ids_s, ids[idx])
    assert np.allclose(ys, y[idx], rtol=1e-13, atol=1e-15)


def test_nvfp4_layer_dense_equivalence():
    geom = synth.small_geom()
    L = synth.make_custom(geom, 6, "nvfp4", "zipf", seed=9)
    x, Wr, b, cfg, routed, shared = oracle_inputs(L)
    y, _, _ = oracle.layer(x, Wr, b, cfg, routed, shared)
    assert np.allclose(y, oracle.dense_layer(x, Wr, b, cfg, routed, shared), rtol=1e-12, atol=1e-14)
