"""Pins against figures the pages print (tests/golden/page_expert_sizes.txt)."""
import os

import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    out = {}
    with open(os.path.join(HERE, "golden", "page_expert_sizes.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, val, tol, *_ = line.split()
                out[key] = (float(val), float(tol))
    return out


def test_int4_container_size_matches_page():
    """One GLM-shaped expert (hidden 6144, moe_inter 2048, gate/up/down) packed
    by the encoder holds about 19 MB of 4-bit codes, and top-8 over 75 MoE
    layers moves about 11 GB per token."""
    g = _golden()
    geom = synth.WORKLOADS["decode"]["geom"]
    H, I = geom["hidden"], geom["moe_inter"]
    e = synth.make_experts(1, 1, H, I, "int4", "cpu", tag=0)
    packed = sum(p.q.numel() for p in (e.gate, e.up, e.down))
    val, tol = g["expert_int4_bytes"]
    assert abs(packed - val) <= tol * val, packed
    per_token = g["moe_layers"][0] * geom["top_k"] * packed
    val, tol = g["routed_bytes_per_token"]
    assert abs(per_token - val) <= tol * val, per_token
    assert geom["n_routed_experts"] == g["experts_per_layer"][0]
