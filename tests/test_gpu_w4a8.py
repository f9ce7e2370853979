"""The W4A8 integer-dot path (MOE_OPT_INT8_ACTIVATIONS: per-row int4 weights,
int8 activations, int8 matrix cores) on the GPU against the oracle's W4A8 FFN,
which rounds the activations the same way: every token of small layers on the
thin and fat GEMM units, ragged K, raw code bytes, the dense entry point, the
GLM-5.2 shape; at 1-4 tokens the option changes nothing."""
import numpy as np
import pytest
import torch

import oracle
import quantized_moe_02_amd as q
import synth
from gpu_common import FFNCache, check_outputs, check_routing, cover_tokens, qexp, run_layer
from helpers import LazyExperts, expert_source, np_u16, row_rel_err

pytestmark = pytest.mark.gpu
A8 = q.MOE_OPT_INT8_ACTIVATIONS


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


def a8_sources(L, lazy=False):
    """The layer's experts as W4A8 oracle sources: host copies of every expert
    (small layers), or copied on demand for the worker pool (FFNCache)."""
    mk = (lambda qe: LazyExperts(qe, "int4_row_a8")) if lazy else (lambda qe: expert_source(qe, "int4_row_a8"))
    return mk(L.routed), mk(L.shared) if L.shared is not None else None


def check_a8(L, T=None, token_idx=None, ffn_map=None):
    y, ids, tw = run_layer(L, options=A8)
    ids_g, _ = check_routing(L, ids, tw)
    return check_outputs(L, y, ids_g, token_idx=token_idx, srcs=a8_sources(L), ffn_map=ffn_map)


@pytest.mark.parametrize("T", [5, 8, 40, 300])
def test_w4a8_layer(T):
    """Every token: 5, 8 and 40 tokens on thin units, 300 on fat units."""
    L = synth.make_custom(synth.small_geom(), T, "int4_row", "normal0.1", seed=1000 + T, device="cuda")
    err = check_a8(L)
    # the float-activation path differs by the activations' int8 rounding only
    y0, _, _ = run_layer(L)
    y8, _, _ = run_layer(L, options=A8)
    d = row_rel_err(y8.cpu().numpy(), y0.cpu().numpy())
    assert 0 < d.max() < 0.05, d.max()
    assert err <= 2e-3


@pytest.mark.parametrize("T", [1, 3, 4])
def test_w4a8_small_batch_is_float(T):
    """At 1-4 tokens the option leaves the float-activation GEMV path alone:
    the same bits."""
    L = synth.make_custom(synth.small_geom(), T, "int4_row", "normal0.1", seed=1100 + T, device="cuda")
    y0, i0, w0 = run_layer(L)
    y8, i8, w8 = run_layer(L, options=A8)
    assert torch.equal(y0, y8) and torch.equal(i0, i8) and torch.equal(w0, w8)


@pytest.mark.parametrize("T", [6, 70])
def test_w4a8_ragged_k(T):
    """hidden 160 and inter 96: partial K blocks (zero-padded int8 rows)."""
    geom = synth.small_geom(hidden=160, moe_inter=96, shared_inter=96)
    L = synth.make_custom(geom, T, "int4_row", "normal0.1", seed=1200 + T, device="cuda")
    check_a8(L)


@pytest.mark.parametrize("T", [9, 640])
def test_w4a8_raw_bytes(T):
    """Every int4 code (u = 0 included) and row scales of either sign."""
    L = synth.make_raw(synth.small_geom(), T, "int4_row", seed=1300 + T, device="cuda")
    check_a8(L)


def test_w4a8_dense_entry_point():
    """moe_expert_ffn_q4 in dense mode (the shared expert on every token)."""
    L = synth.make_custom(synth.small_geom(), 40, "int4_row", "normal0.1", seed=1400, device="cuda")
    cfg = q.make_config(L.geom, "int4_row", A8)
    T, H = 40, L.geom["hidden"]
    ws = q.workspace(cfg, T)
    out = torch.empty(T, H, device="cuda")
    q.moe_expert_ffn_q4(cfg, T, L.x, qexp(L.shared), None, None, None, None, out, ws)
    torch.cuda.synchronize()
    _, shared = a8_sources(L)
    ref = oracle.w4a8_ffn(shared, 0, oracle.bf16_bits_to_f64(np_u16(L.x)))
    assert row_rel_err(out.cpu().numpy(), ref).max() <= 2e-3


def test_w4a8_glm_shape():
    """The GLM-5.2 layer shape at 512 tokens: routing on every token, outputs
    on tokens that together touch 24 experts."""
    geom = dict(synth.WORKLOADS["decode"]["geom"])
    L = synth.make_custom(geom, 512, "int4_row", "zero", seed=1500, device="cuda")
    y, ids, tw = run_layer(L, options=A8)
    ids_g, _ = check_routing(L, ids, tw)
    check_outputs(L, y, ids_g, token_idx=cover_tokens(ids_g, limit=3), srcs=a8_sources(L, lazy=True),
                  ffn_map=FFNCache())
