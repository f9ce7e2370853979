"""The parity tests' own machinery, on the CPU: the oracle's expert FFNs run in
worker processes give the same numbers as in-process, and the token and slot
pickers cover what they promise."""
import numpy as np

import oracle
import synth
from gpu_common import FFNCache, cover_tokens, expert_slots_to_check
from helpers import oracle_inputs


def test_layer_through_worker_pool_is_identical():
    for wfmt, bias in (("int4", "normal0.1"), ("nvfp4", "zipf")):
        L = synth.make_custom(synth.small_geom(), 8, wfmt, bias, seed=41)
        x, Wr, b, cfg, routed, shared = oracle_inputs(L)
        y, ids, _ = oracle.layer(x, Wr, b, cfg, routed, shared)
        cache = FFNCache()
        y2, ids2, _ = oracle.layer(x, Wr, b, cfg, routed, shared, ffn_map=cache)
        assert np.array_equal(ids, ids2) and np.array_equal(y, y2)
        # a second pass is served from the cache, same numbers
        y3, _, _ = oracle.layer(x, Wr, b, cfg, routed, shared, ids=ids[2:5],
                                token_idx=np.arange(2, 5), ffn_map=cache)
        assert np.allclose(y3, y[2:5], rtol=1e-13, atol=1e-15)


def test_cover_tokens_and_slots():
    rng = np.random.default_rng(1)
    ids = np.sort(np.stack([rng.choice(64, 8, replace=False) for _ in range(300)]), 1)
    cov = cover_tokens(ids, always=(0, 299))
    assert 0 in cov and 299 in cov
    assert set(ids[cov].ravel()) == set(ids.ravel())
    offs, _, _, act = oracle.permute(ids, 64)
    sl = expert_slots_to_check(offs)
    assert sorted(sl) == list(act)
    full = [e for e in sl if len(sl[e]) == offs[e + 1] - offs[e] and len(sl[e]) > 3]
    assert len(full) >= 5
    for e, s in sl.items():
        assert s.min() == offs[e] and s.max() == offs[e + 1] - 1
