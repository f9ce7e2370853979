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


# ---------------------------------------------------------------------------
# Decision margins, routing on given ids, one-expert groups
# ---------------------------------------------------------------------------

def _margin_case(TG, k, G=4):
    """8 experts, zero router weights (every sigmoid score is 1/2), so the
    biased scores are 1/2 + b, chosen by hand."""
    cfg = oracle.RouterConfig(8, G, TG, k, 1.0)
    b = np.array([0.40, 0.10, 0.30, 0.28, 0.05, 0.00, 0.20, 0.15])
    _, _, info = oracle.route(np.ones((1, 4)), np.zeros((8, 4)), b, cfg)
    return info["margin"][0]


def test_route_margins_hand_computed():
    """Biased scores .9 .6 | .8 .78 | .55 .5 | .7 .65 in groups of two: group
    scores 1.5, 1.58, 1.05, 1.35.
      TG=2, k=3: groups 1, 0 kept; group gap 1.5 - 1.35 = .15; allowed
                 scores .9 .8 .78 .6, gap after the 3rd .78 - .6 = .18 -> .15
      TG=2, k=2: expert gap .8 - .78 = .02 -> .02
      TG=4, k=3: no group boundary; all eight allowed, .78 - .7 = .08
      TG=1, k=2: group gap 1.58 - 1.5 = .08; both experts of the kept group
                 are chosen, so no expert boundary -> .08
      TG=4, k=8: no boundary at all -> inf"""
    assert abs(_margin_case(2, 3) - 0.15) < 1e-12
    assert abs(_margin_case(2, 2) - 0.02) < 1e-12
    assert abs(_margin_case(4, 3) - 0.08) < 1e-12
    assert abs(_margin_case(1, 2) - 0.08) < 1e-12
    assert _margin_case(4, 8) == np.inf


@pytest.mark.parametrize("wfmt,bias", [("int4", "normal0.1"), ("nvfp4", "zipf")])
def test_layer_on_given_ids_equals_routed_layer(wfmt, bias):
    """layer(ids=...) with the router's own ids reproduces layer() exactly:
    the weights it recomputes for given ids are the router's weights."""
    L = synth.make_custom(synth.small_geom(), 8, wfmt, bias, seed=31)
    x, Wr, b, cfg, routed, shared = oracle_inputs(L)
    y, ids, w = oracle.layer(x, Wr, b, cfg, routed, shared)
    y2, ids2, w2 = oracle.layer(x, Wr, b, cfg, routed, shared, ids=ids)
    assert np.array_equal(ids, ids2) and np.array_equal(w, w2) and np.array_equal(y, y2)
    # and on a token subset, with the subset's ids (BLAS may block a smaller
    # product differently: equal up to fp64 rounding)
    idx = np.array([0, 3, 7])
    y3, _, _ = oracle.layer(x, Wr, b, cfg, routed, shared, ids=ids[idx], token_idx=idx)
    assert np.allclose(y3, y[idx], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("E,G,TG,k", [(16, 16, 6, 4), (12, 6, 3, 4)])
def test_router_small_groups_brute_force(E, G, TG, k):
    """Groups of one expert (a group's score is its single biased score) and
    of two (the top-two sum is the whole group): brute force over every
    TG-subset of groups and every k-subset of their experts."""
    geom = synth.small_geom(n_routed_experts=E, n_group=G, topk_group=TG, top_k=k)
    L = synth.make_custom(geom, 12, "int4", "normal0.1", seed=32 + G)
    x, Wr, b, cfg, _, _ = oracle_inputs(L)
    X = oracle.bf16_bits_to_f64(x)
    ids, _, info = oracle.route(X, Wr, b, cfg)
    per = E // G
    sb = 1 / (1 + np.exp(-(X @ Wr.T))) + b
    for t in range(X.shape[0]):
        gscore = [sum(sb[t, g * per:(g + 1) * per]) for g in range(G)]   # per <= 2: all of it
        best_groups = max(itertools.combinations(range(G), TG),
                          key=lambda c: sum(gscore[g] for g in c))
        allowed = [e for g in best_groups for e in range(g * per, (g + 1) * per)]
        best = max(itertools.combinations(allowed, k), key=lambda c: sum(sb[t, e] for e in c))
        assert info["margin"][t] > 1e-9
        assert sorted(best) == list(ids[t]), t


# ---------------------------------------------------------------------------
# Adaptive expert top-p
# ---------------------------------------------------------------------------

def test_top_p_hand_example():
    """Chosen experts 0..3 with scores .5, .25, .125, .125 (shares exactly
    1/2, 1/4, 1/8, 1/8): the shortest share-ordered prefix reaching p."""
    s = np.array([[0.5, 0.25, 0.125, 0.125]])
    ids = np.array([[0, 1, 2, 3]])
    cases = {0.5: [0], 0.6: [0, 1], 0.75: [0, 1], 0.76: [0, 1, 2], 0.9: [0, 1, 2, 3],
             0.01: [0]}
    for p, kept in cases.items():
        out, _ = oracle.apply_top_p(s, ids, p)
        assert list(out[0]) == kept + [-1] * (4 - len(kept)), p
    out, _ = oracle.apply_top_p(s, ids, 0.75)
    w = oracle.route_weights(s, out, 2.0)
    assert np.allclose(w[0], [2.0 * 2 / 3, 2.0 / 3, 0, 0], rtol=1e-15)
    # scores given in another id order: ties still go to the lower id
    s2 = np.array([[0.125, 0.25, 0.125, 0.5]])
    out, _ = oracle.apply_top_p(s2, ids, 0.76)
    assert list(out[0]) == [0, 1, 3, -1]


def test_top_p_brute_force():
    """Random tokens: the kept set is the smallest set of chosen experts that
    contains every expert with a larger share than any member and whose
    shares reach p (found by enumerating all subsets)."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        k = int(rng.integers(1, 7))
        E = 12
        ids = np.sort(rng.choice(E, size=k, replace=False))[None, :]
        s = rng.random((1, E)) * 0.9 + 0.05
        p = float(rng.random())
        out, _ = oracle.apply_top_p(s, ids, p)
        chosen = list(ids[0])
        total = sum(s[0, e] for e in chosen)
        best = None
        for r in range(1, k + 1):
            for sub in itertools.combinations(chosen, r):
                rest = [e for e in chosen if e not in sub]
                closed = not rest or min(s[0, e] for e in sub) >= max(s[0, e] for e in rest)
                if closed and sum(s[0, e] for e in sub) / total >= p - 1e-12:
                    best = sorted(sub)
                    break
            if best:
                break
        assert [e for e in out[0] if e >= 0] == best


def test_top_p_off_is_plain_routing_and_layer_is_dense_definition():
    L = synth.make_custom(synth.small_geom(), 8, "int4", "normal0.1", seed=51)
    x, Wr, b, cfg, routed, shared = oracle_inputs(L)
    X = oracle.bf16_bits_to_f64(x)
    ids0, w0, _ = oracle.route(X, Wr, b, cfg)
    for p in (0.0, 1.0):
        c = oracle.RouterConfig(cfg.n_experts, cfg.n_group, cfg.topk_group, cfg.top_k,
                                cfg.routed_scaling_factor, top_p=p)
        ids1, w1, _ = oracle.route(X, Wr, b, c)
        assert np.array_equal(ids0, ids1) and np.array_equal(w0, w1)
    c = oracle.RouterConfig(cfg.n_experts, cfg.n_group, cfg.topk_group, cfg.top_k,
                            cfg.routed_scaling_factor, top_p=0.6)
    ids, w, _ = oracle.route(X, Wr, b, c)
    n_kept = (ids >= 0).sum(1)
    assert n_kept.min() >= 1 and n_kept.max() <= cfg.top_k and (n_kept < cfg.top_k).any()
    assert np.allclose(w.sum(1), cfg.routed_scaling_factor, rtol=1e-13)
    assert np.all((w > 0) == (ids >= 0))
    # kept ids are a subset of the plain choice, in ascending order, -1 after
    for t in range(ids.shape[0]):
        kept = [e for e in ids[t] if e >= 0]
        assert kept == sorted(kept) and set(kept) <= set(ids0[t])
        assert list(ids[t][len(kept):]) == [-1] * (cfg.top_k - len(kept))
    y, _, _ = oracle.layer(x, Wr, b, c, routed, shared)
    assert np.allclose(y, oracle.dense_layer(x, Wr, b, c, routed, shared), rtol=1e-12, atol=1e-14)
    # permutation of the kept picks: stable argsort of the valid ones
    offs, st, inv, act = oracle.permute(ids, cfg.n_experts)
    flat = ids.reshape(-1)
    valid = np.nonzero(flat >= 0)[0]
    order = valid[np.argsort(flat[valid], kind="stable")]
    assert np.array_equal(st, order // cfg.top_k)
    assert offs[-1] == len(valid) and np.all(inv[flat < 0] == -1)
    assert np.array_equal(order[inv[valid]], valid)


def test_valid_top_p():
    s = np.array([0.5, 0.25, 0.125, 0.125])
    chosen = np.array([0, 1, 2, 3])
    assert oracle.valid_top_p(np.array([0, 1, -1, -1]), s, chosen, 0.75, 1e-9)
    assert oracle.valid_top_p(np.array([0, 1, 2, -1]), s, chosen, 0.75, 1e-9)     # at the boundary
    assert not oracle.valid_top_p(np.array([0, 1, 2, -1]), s, chosen, 0.6, 1e-9)
    assert not oracle.valid_top_p(np.array([0, 2, -1, -1]), s, chosen, 0.6, 1e-9)
    assert oracle.valid_top_p(np.array([0, 1, 3, -1]), s, chosen, 0.76, 1e-9)     # tie


def test_repack_int4_natural():
    """Natural-order bytes repacked to the word order decode, through the
    oracle, to the codes they held."""
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 16, size=(3, 64)).astype(np.uint8)
    natural = torch.from_numpy((codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8))
    q = synth.repack_int4_natural(natural).numpy()
    assert np.array_equal(oracle.unpack_int4_codes(q), codes)


# ---------------------------------------------------------------------------
# Per-row-scale formats (int4, int8, packed int2)
# ---------------------------------------------------------------------------

def _int2_bytes_from_codes_by_position(codes):
    """Independent packer for the int2 word layout, bit by bit from the
    layout's statement (input 16j + r: r even in bits r, r+1 of word j; r odd
    in bits 16 + r - 1, 16 + r)."""
    N, K = codes.shape
    out = np.zeros((N, K // 4), np.uint8)
    for n in range(N):
        for k in range(K):
            j, r = divmod(k, 16)
            bit = (r - r % 2) + 16 * (r % 2)
            byte, sh = 4 * j + bit // 8, bit % 8
            out[n, byte] |= np.uint8(int(codes[n, k]) << sh)
    return out


def test_int2_layout_one_hot_probe():
    K = 48
    for k in range(K):
        codes = np.full((1, K), 2, np.uint8)
        codes[0, k] = 3                        # q = +1 at input k only
        q = _int2_bytes_from_codes_by_position(codes)
        w = oracle.dequant_int2_row(q, np.array([0.25], np.float32))
        expect = np.zeros((1, K))
        expect[0, k] = 0.25
        assert np.array_equal(w, expect), k
        assert np.array_equal(synth.pack_int2_words(torch.from_numpy(codes)).numpy(), q)


def test_int2_hand_words():
    """Word 0x00000001: input 0 has code 1 (q = -1), every other input code 0
    (q = -2).  Word 0xC0000000: input 15 has code 3 (q = 1).  Byte order is
    little-endian."""
    q = np.array([[0x01, 0x00, 0x00, 0x00], [0x00, 0x00, 0x00, 0xC0]], np.uint8)
    w = oracle.dequant_int2_row(q, np.array([1.0, 2.0], np.float32))
    assert np.array_equal(w[0], np.array([-1.0] + [-2.0] * 15))
    assert np.array_equal(w[1], np.array([-4.0] * 15 + [2.0]))


def test_int8_hand_bytes():
    q = np.array([[0x00, 0x01, 0x7F, 0x80, 0xFF, 0xFE]], np.uint8)
    w = oracle.dequant_int8_row(q, np.array([0.5], np.float32))
    assert np.array_equal(w[0], 0.5 * np.array([0, 1, 127, -128, -1, -2]))


def test_int4_row_equals_group_scales_when_all_equal():
    """Per-row int4 is int4 g32 with every group scale equal to the row scale
    (scales exact in fp16)."""
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, size=(5, 96)).astype(np.uint8)
    q = _int4_bytes_from_codes_by_position(codes)
    srow = np.array([0.5, 0.25, 2.0, 1.0, 0.125], np.float32)
    sg = np.repeat(srow[:, None], 3, axis=1).astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.dequant_int4_row(q, srow), oracle.dequant_int4(q, sg))
    assert np.array_equal(oracle.dequant_int4_row(q, srow), (codes - 8.0) * srow[:, None])


@pytest.mark.parametrize("fmt,qmax", [("int4_row", 7), ("int8_row", 127)])
def test_row_roundtrip_bound(fmt, qmax):
    W = torch.randn(32, 256) * 0.02
    W[5] = 0.0                                  # an all-zero row
    qp = synth._quantize(W.unsqueeze(0), fmt)
    w = oracle.ROW_FORMATS[fmt](qp.q[0].numpy(), qp.scale[0].numpy())
    s = qp.scale[0].double().numpy()[:, None]
    assert np.all(np.abs(w - W.double().numpy()) <= s / 2 * (1 + 1e-6))
    assert np.all(w[5] == 0.0)
    # the row's absmax is on the grid
    assert np.allclose(np.abs(w).max(1)[s[:, 0] > 0], (qmax * s[:, 0])[s[:, 0] > 0], rtol=1e-6)


def test_int2_on_grid_roundtrip_exact():
    rng = np.random.default_rng(3)
    qv = rng.integers(-2, 2, size=(8, 64)).astype(np.float64)
    qv[:, 0] = -2                                # every row reaches absmax = 2 s
    s = np.float32(2.0 ** -7) * (1 + np.arange(8) % 3)
    W = qv * s.astype(np.float64)[:, None]
    qp = synth._quantize(torch.from_numpy(W).float().unsqueeze(0), "int2_row")
    assert np.array_equal(oracle.dequant_int2_row(qp.q[0].numpy(), qp.scale[0].numpy()), W)


def test_repack_int2_natural():
    rng = np.random.default_rng(13)
    codes = rng.integers(0, 4, size=(3, 64)).astype(np.uint8)
    natural = (codes[:, 0::4] | (codes[:, 1::4] << 2) | (codes[:, 2::4] << 4)
               | (codes[:, 3::4] << 6)).astype(np.uint8)
    q = synth.repack_int2_natural(torch.from_numpy(natural)).numpy()
    assert np.array_equal(oracle.unpack_int2_codes(q), codes)


@pytest.mark.parametrize("fmt", ["int4_row", "int8_row", "int2_row"])
def test_row_format_layer_dense_equivalence(fmt):
    """The batch-union layer equals the dense definition (every expert applied
    to every token, weights zero off the chosen ones) for the per-row formats."""
    geom = synth.small_geom()
    L = synth.make_custom(geom, 5, fmt, "normal0.1", seed=21)
    x, Wr, b, cfg, routed, shared = oracle_inputs(L)
    y, _, _ = oracle.layer(x, Wr, b, cfg, routed, shared)
    assert np.allclose(y, oracle.dense_layer(x, Wr, b, cfg, routed, shared), rtol=1e-12, atol=1e-14)
    # doubling every down-projection row scale doubles the routed part exactly
    d = routed.down
    routed2 = oracle.ExpertSource(fmt, routed.gate, routed.up, (d[0], d[1] * 2, None))
    y0, _, _ = oracle.layer(x, Wr, b, cfg, routed, None)
    y2, _, _ = oracle.layer(x, Wr, b, cfg, routed2, None)
    assert np.allclose(y2, 2 * y0, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# W4A8 integer-dot path: the int8 row quantiser and the FFN
# ---------------------------------------------------------------------------

def test_quantize_rows_int8_hand_values():
    """Row 0: amax 1, so a * 127: 63.5 -> 64 and 31.75 -> 32 (ties to even);
    row 1 all zero; row 2: amax 254, so a * 0.5: 0.5 -> 0, -1.5 -> -2, 2.5 -> 2."""
    a = np.array([[0.5, -1.0, 0.25, 0.0],
                  [0.0, 0.0, 0.0, 0.0],
                  [254.0, 1.0, -3.0, 5.0]], np.float32)
    q, s = oracle.quantize_rows_int8(a)
    assert q.tolist() == [[64, -127, 32, 0], [0, 0, 0, 0], [127, 0, -2, 2]]
    assert s.dtype == np.float32
    assert s[0] == np.float32(1.0) / np.float32(127.0) and s[1] == 0 and s[2] == 2.0


def test_quantize_rows_int8_on_grid_exact():
    """Rows k * 2^-e with integer k in [-127, 127] reaching |k| = 127 come
    back as k exactly, with scale 2^-e."""
    rng = np.random.default_rng(31)
    k = rng.integers(-127, 128, size=(6, 64))
    k[:, 5] = 127 * np.where(np.arange(6) % 2 == 0, 1, -1)
    s = np.float32(2.0) ** -np.arange(3, 9, dtype=np.float32)
    a = (k * s[:, None]).astype(np.float32)
    q, sc = oracle.quantize_rows_int8(a)
    assert np.array_equal(q, k) and np.array_equal(sc, s)


def _a8_source(seed, E=3, H=64, I=32):
    """Per-row int4 experts (as the synthetic encoder makes them) viewed as a
    W4A8 source and as a plain one."""
    torch.manual_seed(seed)
    projs = [synth._quantize(torch.randn(E, n, k) * 0.02, "int4_row") for n, k in ((I, H), (I, H), (H, I))]
    arrs = [(p.q.numpy(), p.scale.numpy(), None) for p in projs]
    return oracle.ExpertSource("int4_row_a8", *arrs), oracle.ExpertSource("int4_row", *arrs)


def test_w4a8_ffn_on_grid_input_bound():
    """Inputs on the int8 grid are quantised exactly, so gate and up equal the
    float64 ones; the result then differs from the float64 FFN only through
    h's fp16 rounding and int8 quantisation: |dO[n]| <= sum_k |Wd[n,k]| (s_h/2 +
    2^-11 |h_k|) per token."""
    a8, plain = _a8_source(41)
    rng = np.random.default_rng(42)
    k = rng.integers(-127, 128, size=(5, 64))
    k[:, 0] = 127
    X = k * np.float64(2.0 ** -6)
    for e in range(3):
        Wg, Wu, Wd = (plain.weight(p, e) for p in ("gate", "up", "down"))
        G, U = X @ Wg.T, X @ Wu.T
        h = G / (1.0 + np.exp(-G)) * U
        ref = h @ Wd.T
        got = oracle.w4a8_ffn(a8, e, X)
        sh = np.abs(h).max(1) / 127.0
        bound = (sh[:, None] / 2 + 2.0 ** -11 * np.abs(h)) @ np.abs(Wd).T
        assert np.all(np.abs(got - ref) <= bound * (1 + 1e-6) + 1e-300), e
        assert not np.allclose(got, ref, rtol=1e-12, atol=0)      # h really was quantised


def test_w4a8_integer_core_brute_force():
    """The integer dot products against a loop over the decoded codes, on a
    two-token example (every step of w4a8_ffn recomputed by hand)."""
    a8, _ = _a8_source(43, E=1, H=32, I=32)
    X = np.random.default_rng(44).standard_normal((2, 32)).astype(np.float32).astype(np.float64)
    q, s = oracle.quantize_rows_int8(X.astype(np.float32))
    codes = {p: oracle.unpack_int4_codes(getattr(a8, p)[0][0]).astype(int) - 8 for p in ("gate", "up", "down")}
    rs = {p: getattr(a8, p)[1][0].astype(np.float64) for p in ("gate", "up", "down")}
    out = np.zeros((2, 32))
    for t in range(2):
        G = [sum(int(q[t, i]) * int(codes["gate"][r, i]) for i in range(32)) * rs["gate"][r] * float(s[t])
             for r in range(32)]
        U = [sum(int(q[t, i]) * int(codes["up"][r, i]) for i in range(32)) * rs["up"][r] * float(s[t])
             for r in range(32)]
        h = np.array([g / (1 + math.exp(-g)) * u for g, u in zip(G, U)])
        h16 = h.astype(np.float16).astype(np.float32)
        amax = np.float32(np.abs(h16).max())
        inv = np.float32(127.0) / amax
        hq = [int(np.clip(np.rint(np.float32(v) * inv), -127, 127)) for v in h16]
        sh = float(amax / np.float32(127.0))
        for n in range(32):
            out[t, n] = sum(hq[i] * int(codes["down"][n, i]) for i in range(32)) * rs["down"][n] * sh
    assert np.allclose(oracle.w4a8_ffn(a8, 0, X), out, rtol=1e-12, atol=1e-15)


def test_w4a8_layer_dense_equivalence():
    geom = synth.small_geom()
    L = synth.make_custom(geom, 5, "int4_row", "normal0.1", seed=47)
    x, Wr, b, cfg, routed, shared = oracle_inputs(L)
    a8 = lambda src: oracle.ExpertSource("int4_row_a8", src.gate, src.up, src.down)
    y, _, _ = oracle.layer(x, Wr, b, cfg, a8(routed), a8(shared))
    yd = oracle.dense_layer(x, Wr, b, cfg, a8(routed), a8(shared))
    assert np.allclose(y, yd, rtol=1e-12, atol=1e-14)
    # and it stays close to the float-activation layer (int8 rounding only)
    y0, _, _ = oracle.layer(x, Wr, b, cfg, routed, shared)
    assert np.abs(y - y0).max() <= 0.05 * np.abs(y0).max()
