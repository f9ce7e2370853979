"""Expert streaming from host memory (moe_layer_cached and the moe_cache_*
calls) on the GPU: the routing and the outputs against the fp64 oracle and
against moe_layer with every expert resident, and every hit, miss and slot
against tests/cache_model.py over sequences of calls, with lookahead
prefetches on a second stream, pinned experts and a call that does not fit."""
import numpy as np
import pytest
import torch

import quantized_moe_02_amd as q
import synth
from cache_model import SlotModel
from gpu_common import check_outputs, check_routing, qexp, run_layer
from helpers import np_u16

pytestmark = pytest.mark.gpu

GEOM = dict(hidden=512, moe_inter=256, n_routed_experts=32, n_group=4, topk_group=2, top_k=4,
            n_shared_experts=1, shared_inter=256, routed_scaling_factor=2.5)


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


class Streamed:
    """A layer whose routed experts live in pinned host memory, served by an
    expert cache of n_slots device slots; the model predicts the cache."""

    def __init__(self, geom, wfmt, n_slots, seed):
        self.L = synth.make_custom(geom, 4, wfmt, "normal0.1", seed, device="cuda")
        self.geom, self.wfmt, self.S = geom, wfmt, n_slots
        self.cfg = q.make_config(geom, wfmt)
        r = self.L.routed
        self.host = [self._pinned(p) for p in (r.gate, r.up, r.down)]
        self.slots = [self._slots(p, n_slots) for p in (r.gate, r.up, r.down)]
        self.h_store = q.qexperts(*self.host)
        self.d_slots = q.qexperts(*self.slots)
        self.cache = q.moe_cache_create(self.cfg, n_slots, self.h_store, self.d_slots)
        self.model = SlotModel(geom["n_routed_experts"], n_slots)
        self.last_call = None        # model request number of the latest layer call

    @staticmethod
    def _pinned(p):
        return tuple(None if t is None else t.cpu().pin_memory() for t in (p.q, p.scale, p.gscale))

    @staticmethod
    def _slots(p, S):
        return tuple(None if t is None else torch.zeros((S,) + tuple(t.shape[1:]), dtype=t.dtype,
                                                        device="cuda")
                     for t in (p.q, p.scale, p.gscale))

    def close(self):
        q.moe_cache_destroy(self.cache)

    def tokens(self, T, seed):
        return synth.to_bf16(synth.randn((T, self.geom["hidden"]), seed, "cuda"))

    def call(self, x, stream=None):
        T, k, H = x.shape[0], self.geom["top_k"], self.geom["hidden"]
        ws = q.workspace(self.cfg, T)
        y = torch.empty(T, H, device="cuda")
        ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
        tw = torch.empty(T, k, dtype=torch.float32, device="cuda")
        q.moe_layer_cached(self.cache, T, x, self.L.router_w, self.L.bias, qexp(self.L.shared), y,
                           q.MOE_OUT_F32, ids, tw, ws, stream=stream)
        torch.cuda.synchronize()
        return y, ids, tw

    def predict_call(self, ids):
        need = [e for e in ids.cpu().numpy().ravel().tolist() if e >= 0]
        res = self.model.request(need)
        if res is not None:
            self.last_call = self.model.requests
        return res

    def predict_prefetch(self, experts):
        loaded = 0
        for e in experts:
            res = self.model.request([e], self.last_call)
            if res is not None:
                loaded += len(res[1])
        return loaded

    def check_table(self):
        got = [q.moe_cache_slot_of(self.cache, e) for e in range(self.geom["n_routed_experts"])]
        assert got == self.model.table()


def _check_call(st, x, y, ids, tw, exact_vs_resident):
    x_np = np_u16(x)
    ids_g, _ = check_routing(st.L, ids, tw, x_np=x_np)
    check_outputs(st.L, y, ids_g, x_np=x_np)
    y_res, ids_res, tw_res = run_layer(st.L, x=x)
    assert torch.equal(ids, ids_res)
    if exact_vs_resident:     # same kernels (T > 4): bit for bit
        assert torch.equal(y, y_res)
        assert torch.equal(tw, tw_res)


@pytest.mark.parametrize("wfmt", ["int4", "nvfp4"])
def test_cached_layer_sequence(wfmt):
    """A sequence of calls of 1..4 tokens through 16 slots of 32 experts
    (a call needs at most 16): each call's routing and outputs, and the
    cache's hits, loads, evictions and slots."""
    st = Streamed(GEOM, wfmt, 16, seed=901 if wfmt == "int4" else 902)
    try:
        stats0 = q.moe_cache_get_stats(st.cache)
        for i, T in enumerate([1, 2, 1, 3, 4, 1, 4, 1, 2, 4, 1, 3, 4, 2, 4]):
            x = st.tokens(T, 7000 + i)
            y, ids, tw = st.call(x)
            res = st.predict_call(ids)
            assert res is not None
            hits, loads = res
            s = q.moe_cache_get_stats(st.cache)
            assert s["hits"] - stats0["hits"] == hits, i
            assert s["misses"] - stats0["misses"] == len(loads), i
            assert s["calls"] == i + 1
            assert s["evictions"] == st.model.evictions
            stats0 = s
            st.check_table()
            _check_call(st, x, y, ids, tw, exact_vs_resident=T > 4)
        assert st.model.evictions > 0      # the sequence did evict
    finally:
        st.close()


def test_cached_layer_all_resident_and_large_batch():
    """As many slots as experts: nothing is ever evicted, each expert is
    loaded once; 37 and 130 tokens (the grouped GEMM over the slots) equal
    moe_layer bit for bit."""
    st = Streamed(GEOM, "int4", 32, seed=903)
    try:
        loaded = 0
        for i, T in enumerate([37, 130, 37]):
            x = st.tokens(T, 7100 + i)
            y, ids, tw = st.call(x)
            hits, loads = st.predict_call(ids)
            loaded += len(loads)
            st.check_table()
            _check_call(st, x, y, ids, tw, exact_vs_resident=True)
        s = q.moe_cache_get_stats(st.cache)
        assert s["misses"] == loaded
        assert s["evictions"] == 0
    finally:
        st.close()


def test_lookahead_prefetch_on_second_stream():
    """The next call's experts, predicted by routing its tokens ahead
    (moe_route), are prefetched on a second stream while the current call's
    kernels run; the next call then loads nothing and is exact."""
    st = Streamed(GEOM, "int4", 16, seed=904)
    side = torch.cuda.Stream()
    try:
        cfg, k = st.cfg, GEOM["top_k"]
        x0 = st.tokens(2, 7200)
        y0, ids0, tw0 = st.call(x0)
        st.predict_call(ids0)
        for i in range(1, 6):
            x1 = st.tokens(2, 7200 + i)
            # lookahead: route the next tokens now
            ws = q.workspace(cfg, 2)
            nid = torch.empty(2, k, dtype=torch.int32, device="cuda")
            ntw = torch.empty(2, k, dtype=torch.float32, device="cuda")
            q.moe_route(cfg, 2, x1, st.L.router_w, st.L.bias, nid, ntw, ws)
            torch.cuda.synchronize()
            pred = sorted(set(nid.cpu().numpy().ravel().tolist()))
            n = q.moe_cache_prefetch(st.cache, pred, stream=side)
            assert n == st.predict_prefetch(pred)
            st.check_table()
            y1, ids1, tw1 = st.call(x1)
            hits, loads = st.predict_call(ids1)
            assert loads == []                 # all prefetched
            assert hits == len(pred)
            st.check_table()
            _check_call(st, x1, y1, ids1, tw1, exact_vs_resident=False)
        assert q.moe_cache_get_stats(st.cache)["prefetched"] > 0
    finally:
        st.close()


def test_pinned_experts_stay_and_capacity_error():
    """Pinned experts keep their slots through calls that evict everything
    else; a call needing more experts than the unpinned slots returns
    MOE_ERR_UNSUPPORTED with its routing written and the cache unchanged; a
    pin that does not fit changes nothing."""
    st = Streamed(GEOM, "int4", 8, seed=905)
    try:
        pins = [3, 17, 30]
        q.moe_cache_pin(st.cache, pins)
        res = st.model.request(pins, st.last_call)
        st.model.pin(pins)
        assert res is not None
        slots = [q.moe_cache_slot_of(st.cache, e) for e in pins]
        assert min(slots) >= 0
        for i in range(6):
            x = st.tokens(1, 7300 + i)
            y, ids, tw = st.call(x)
            assert st.predict_call(ids) is not None
            st.check_table()
            assert [q.moe_cache_slot_of(st.cache, e) for e in pins] == slots
            _check_call(st, x, y, ids, tw, exact_vs_resident=False)
        # 16 tokens pick far more than the 5 unpinned slots
        x = st.tokens(16, 7400)
        before = [q.moe_cache_slot_of(st.cache, e) for e in range(GEOM["n_routed_experts"])]
        ids = torch.full((16, GEOM["top_k"]), -7, dtype=torch.int32, device="cuda")
        tw = torch.empty(16, GEOM["top_k"], dtype=torch.float32, device="cuda")
        y = torch.empty(16, GEOM["hidden"], device="cuda")
        with pytest.raises(q.QmoeError) as err:
            q.moe_layer_cached(st.cache, 16, x, st.L.router_w, st.L.bias, qexp(st.L.shared), y,
                               q.MOE_OUT_F32, ids, tw, q.workspace(st.cfg, 16))
        assert err.value.status == q.MOE_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        check_routing(st.L, ids, tw, x_np=np_u16(x))     # the routing was written
        assert st.model.request(ids.cpu().numpy().ravel().tolist()) is None
        assert [q.moe_cache_slot_of(st.cache, e) for e in range(GEOM["n_routed_experts"])] == before
        with pytest.raises(q.QmoeError) as err:
            q.moe_cache_pin(st.cache, list(range(4, 10)))  # 3 pinned + 6 > 8 slots
        assert err.value.status == q.MOE_ERR_UNSUPPORTED
        q.moe_cache_unpin_all(st.cache)
        st.model.unpin_all()
        x = st.tokens(1, 7500)
        y, ids, tw = st.call(x)
        assert st.predict_call(ids) is not None
        st.check_table()
    finally:
        st.close()


def test_cached_layer_adaptive_top_p():
    """Adaptive expert top-p: dropped picks (-1) load nothing and are
    skipped."""
    geom = dict(GEOM, expert_top_p=0.5)
    st = Streamed(geom, "int4", 16, seed=906)
    try:
        for i, T in enumerate([1, 3, 8]):
            x = st.tokens(T, 7600 + i)
            y, ids, tw = st.call(x)
            assert st.predict_call(ids) is not None
            st.check_table()
            x_np = np_u16(x)
            ids_g, _ = check_routing(st.L, ids, tw, x_np=x_np)
            check_outputs(st.L, y, ids_g, x_np=x_np)
        assert (ids.cpu().numpy() < 0).any()
    finally:
        st.close()
