"""moe_layer_noalloc -- moe_layer on the library's own device workspace, for
callers that cannot allocate -- against moe_layer with a caller workspace:
bit-identical routing and outputs (the same kernels), and the oracle's bar,
on consecutive calls whose second input is smaller (the buffer keeps the
last call's contents)."""
import numpy as np
import pytest
import torch

import quantized_moe_02_amd as q
import synth
from gpu_common import check_outputs, check_routing, qexp, run_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


def _noalloc(L, x, options=0):
    T = x.shape[0]
    cfg = q.make_config(L.geom, L.wfmt, options)
    H, k = L.geom["hidden"], L.geom["top_k"]
    y = torch.empty(T, H, device="cuda", dtype=torch.float32)
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    tw = torch.empty(T, k, dtype=torch.float32, device="cuda")
    q.moe_layer_noalloc(cfg, T, x, L.router_w, L.bias, qexp(L.routed),
                        qexp(L.shared) if L.shared is not None else None, y, q.MOE_OUT_F32, ids, tw)
    torch.cuda.synchronize()
    return y, ids, tw


def _same(L, Ts):
    for T in Ts:
        x = L.x[:T].contiguous()
        ref = run_layer(L, x=x)
        got = _noalloc(L, x)
        for a, b in zip(ref, got):
            assert torch.equal(a, b), T
        ids_g, _ = check_routing(L, got[1], got[2], x_np=x.cpu().view(torch.int16).numpy().view(np.uint16))
        check_outputs(L, got[0], ids_g, x_np=x.cpu().view(torch.int16).numpy().view(np.uint16))


def test_noalloc_tiny_consecutive_calls():
    """8 tokens (large-batch kernels), then 3 (small-batch), then 1 (the
    single-token kernel with its grid barrier)."""
    _same(synth.make_layer("tiny", "cuda"), (8, 3, 1))


def test_noalloc_full_size_consecutive_calls():
    """The GLM-5.2 layer at 64 tokens (23 MB of workspace), then 4, then 1."""
    _same(synth.make_layer("verify64", "cuda"), (64, 4, 1))


def test_noalloc_flags_and_size_limit():
    L = synth.make_layer("tiny", "cuda")
    x = L.x[:1].contiguous()
    y, _, _ = _noalloc(L, x, options=q.MOE_OPT_GRID_WAIT_NONE)
    assert torch.isnan(y).all()
    assert q.moe_layer_flags(None) == q.MOE_FLAG_GRID_WAIT_TIMEOUT
    _noalloc(L, x)
    assert q.moe_layer_flags(None) == 0
    G = synth.make_layer("verify64", "cuda", tokens=128)
    with pytest.raises(q.QmoeError) as ei:
        _noalloc(G, G.x)
    assert ei.value.status == q.MOE_ERR_UNSUPPORTED
