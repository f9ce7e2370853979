"""The per-row-scale weight formats (int4, int8, packed int2 with one fp32
scale per output row) on the GPU against the fp64 oracle: moe_layer on every
path they take (grouped GEMV at 1-4 tokens, thin and fat grouped-GEMM units
above), the entry points, raw code bytes covering every code, K not a multiple
of the GEMM's K block, the GLM-5.2 shape, and the expert cache."""
import numpy as np
import pytest
import torch

import oracle
import quantized_moe_02_amd as q
import synth
from gpu_common import (FFNCache, check_outputs, check_routing, cover_tokens, entry_point_chain,
                        qexp, run_layer)

pytestmark = pytest.mark.gpu

FMTS = ["int4_row", "int8_row", "int2_row"]


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T", [1, 2, 4, 8, 40, 300])
def test_row_format_layer(fmt, T):
    """Every token against the oracle: 1-4 tokens take the grouped GEMV, 8 and
    40 the thin GEMM units, 300 (about 75 tokens per expert) the fat units."""
    L = synth.make_custom(synth.small_geom(), T, fmt, "normal0.1", seed=600 + T, device="cuda")
    y, ids, tw = run_layer(L)
    ids_g, _ = check_routing(L, ids, tw)
    check_outputs(L, y, ids_g)
    if T <= 8:
        entry_point_chain(L)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T", [1, 3, 40, 640])
def test_row_format_raw_bytes(fmt, T):
    """Uniformly random code bytes (every code, int8 -128 included) and row
    scales of either sign."""
    L = synth.make_raw(synth.small_geom(), T, fmt, seed=700 + T, device="cuda")
    y, ids, tw = run_layer(L)
    ids_g, _ = check_routing(L, ids, tw)
    check_outputs(L, y, ids_g)
    if T <= 4:
        entry_point_chain(L)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T", [2, 20])
def test_row_format_ragged_k(fmt, T):
    """hidden 160 and inter 96: the GEMM's last K block is partial and the
    GEMV's last lanes hold no group."""
    geom = synth.small_geom(hidden=160, moe_inter=96, shared_inter=96)
    L = synth.make_custom(geom, T, fmt, "normal0.1", seed=800 + T, device="cuda")
    y, ids, tw = run_layer(L)
    ids_g, _ = check_routing(L, ids, tw)
    check_outputs(L, y, ids_g)


@pytest.mark.parametrize("fmt,T", [("int2_row", 1), ("int8_row", 1), ("int4_row", 3)])
def test_row_format_glm_decode(fmt, T):
    """The GLM-5.2 layer shape (hidden 6144, moe_inter 2048, 256 experts) at
    decode sizes, every token."""
    geom = dict(synth.WORKLOADS["decode"]["geom"])
    L = synth.make_custom(geom, T, fmt, "zero", seed=900 + T, device="cuda")
    y, ids, tw = run_layer(L)
    ids_g, _ = check_routing(L, ids, tw)
    check_outputs(L, y, ids_g, ffn_map=FFNCache())


def test_row_format_glm_batch():
    """The GLM-5.2 layer shape at 64 tokens in int8 (thin GEMM units): routing
    on every token, outputs on a few tokens that together touch 24 experts."""
    geom = dict(synth.WORKLOADS["decode"]["geom"])
    L = synth.make_custom(geom, 64, "int8_row", "hot16", seed=950, device="cuda")
    y, ids, tw = run_layer(L)
    ids_g, _ = check_routing(L, ids, tw)
    check_outputs(L, y, ids_g, token_idx=cover_tokens(ids_g, limit=3), ffn_map=FFNCache())


def test_row_format_cached_layer():
    """The expert cache streams per-row-format experts (row scales copied with
    the codes)."""
    geom = dict(hidden=512, moe_inter=256, n_routed_experts=32, n_group=4, topk_group=2, top_k=4,
                n_shared_experts=1, shared_inter=256, routed_scaling_factor=2.5)
    L = synth.make_custom(geom, 4, "int2_row", "normal0.1", seed=960, device="cuda")
    cfg = q.make_config(geom, "int2_row")
    projs = (L.routed.gate, L.routed.up, L.routed.down)
    host = [(p.q.cpu().pin_memory(), p.scale.cpu().pin_memory(), None) for p in projs]
    slots = [(torch.zeros((8,) + tuple(p.q.shape[1:]), dtype=torch.uint8, device="cuda"),
              torch.zeros((8,) + tuple(p.scale.shape[1:]), dtype=torch.float32, device="cuda"), None)
             for p in projs]
    cache = q.moe_cache_create(cfg, 8, q.qexperts(*host), q.qexperts(*slots))
    try:
        for i, T in enumerate([1, 2, 1, 2, 2, 1]):
            x = synth.to_bf16(synth.randn((T, geom["hidden"]), 9600 + i, "cuda"))
            ws = q.workspace(cfg, T)
            y = torch.empty(T, geom["hidden"], device="cuda")
            ids = torch.empty(T, 4, dtype=torch.int32, device="cuda")
            tw = torch.empty(T, 4, dtype=torch.float32, device="cuda")
            q.moe_layer_cached(cache, T, x, L.router_w, L.bias, qexp(L.shared), y, q.MOE_OUT_F32,
                               ids, tw, ws)
            torch.cuda.synchronize()
            x_np = x.view(torch.int16).cpu().numpy().view(np.uint16)
            ids_g, _ = check_routing(L, ids, tw, x_np=x_np)
            check_outputs(L, y, ids_g, x_np=x_np)
        assert q.moe_cache_get_stats(cache)["evictions"] > 0
    finally:
        q.moe_cache_destroy(cache)


@pytest.mark.parametrize("fmt", ["int4_row", "int2_row"])
@pytest.mark.parametrize("shape", ["tiny", "glm"])
def test_row_format_single_token_kernels(fmt, shape):
    """One token in per-row int4 / int2 takes the single-token kernels: the
    fused kernel and the two-launch form (MOE_OPT_NO_GRID_WAIT) agree bit for
    bit, and both match the oracle."""
    geom = synth.small_geom() if shape == "tiny" else dict(synth.WORKLOADS["decode"]["geom"])
    L = synth.make_custom(geom, 1, fmt, "normal0.1", seed=1600 + len(fmt), device="cuda")
    y, ids, tw = run_layer(L)
    y2, ids2, tw2 = run_layer(L, options=q.MOE_OPT_NO_GRID_WAIT)
    assert torch.equal(y, y2) and torch.equal(ids, ids2) and torch.equal(tw, tw2)
    ids_g, _ = check_routing(L, ids, tw)
    check_outputs(L, y, ids_g, ffn_map=FFNCache() if shape == "glm" else None)


@pytest.mark.parametrize("fmt", ["int4_row", "int2_row"])
@pytest.mark.parametrize("T", [2, 3, 4])
def test_row_format_small_batch_kernels(fmt, T):
    """2-4 tokens in per-row int4 / int2 take the small-batch kernels (K2, K3,
    the multi-token down kernel) at the GLM-5.2 shape: every token against the
    oracle."""
    geom = dict(synth.WORKLOADS["verify4"]["geom"])
    L = synth.make_custom(geom, T, fmt, "hot16", seed=1700 + T, device="cuda")
    y, ids, tw = run_layer(L)
    ids_g, _ = check_routing(L, ids, tw)
    check_outputs(L, y, ids_g, ffn_map=FFNCache())
