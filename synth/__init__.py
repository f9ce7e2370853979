"""Seeded synthetic inputs for the quantized MoE layer.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It draws random numbers and encodes weights into the two packed
storage formats; it holds none of the layer's arithmetic (no decoding, no
routing, no FFN, no combine).  Everything here is plain PyTorch so that the same
code runs on the CPU (small workloads, CPU-only tests) and on the GPU (full
GLM-5.2-sized workloads, where generating 5 GB of weights on the host would take
minutes).

Shapes and distributions follow the workloads of the colibri / GLM-5.2 pages
(page "Show HN: Menjalankan GLM 5.2 di komputer lambat", sections "Cara kerja
eksekusi MoE berbasis streaming disk" and "Fitur utama": 256 routed experts per
MoE layer, top-8 DeepSeek-V3-style routing, a shared expert, about 19 MB of int4
per expert; page "NVIDIA stellt neues GLM-5.2 NVFP4 Modell vor", section
"Technische Details": expert FFNs in 4-bit with one FP8 scale per 16 elements).

Storage formats (also stated in include/qmoe.h):

int4, group 32, fp16 scale  (QMOE_WFMT_INT4_G32_F16)
    A projection with N output rows and K inputs stores, per row, K/8
    little-endian 32-bit words.  Word j holds inputs 8j..8j+7: input 8j+2i
    (i = 0..3) sits in bits [4i, 4i+4) and input 8j+2i+1 in bits
    [16+4i, 16+4i+4).  A 4-bit code u encodes q = u - 8.  One fp16 scale per
    32 consecutive inputs; the weight is q * scale.

NVFP4  (QMOE_WFMT_NVFP4)
    Per row, K/2 bytes; byte j holds input 2j in its low nibble and input 2j+1
    in its high nibble.  A nibble is an E2M1 code (bit 3 sign, bits 2..1
    exponent with bias 1, bit 0 mantissa).  One E4M3 ("fn": bias 7, no
    infinities) scale byte per 16 consecutive inputs and one fp32 scale per
    (expert, projection); the weight is e2m1 * e4m3 * fp32.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch

BASE_SEED = 20261203

# Layer geometry of the GLM-5.2 MoE layer (hidden 6144, moe_inter 2048, 256
# routed experts in 8 groups, 4 groups kept, top-8, one shared expert,
# routed_scaling_factor 2.5) and of a tiny layer with the same structure.
_GLM = dict(hidden=6144, moe_inter=2048, n_routed_experts=256, n_group=8,
            topk_group=4, top_k=8, n_shared_experts=1, shared_inter=2048,
            routed_scaling_factor=2.5)
# the same layer with the adaptive expert top-p at the pages' setting (0.7)
_GLM_TOPP = dict(_GLM, expert_top_p=0.7)
_TINY = dict(hidden=256, moe_inter=128, n_routed_experts=16, n_group=4,
             topk_group=2, top_k=4, n_shared_experts=1, shared_inter=128,
             routed_scaling_factor=2.5)

# name -> (index used in the seed, geometry, tokens, weight format, bias recipe)
WORKLOADS: Dict[str, dict] = {
    "tiny":       dict(index=0, geom=_TINY, tokens=8,     wfmt="int4",  bias="normal0.1"),
    "decode":     dict(index=1, geom=_GLM,  tokens=1,     wfmt="int4",  bias="zero"),
    "verify4":    dict(index=2, geom=_GLM,  tokens=4,     wfmt="int4",  bias="hot16"),
    "verify64":   dict(index=2, geom=_GLM,  tokens=64,    wfmt="int4",  bias="hot16"),
    "prefill4k":  dict(index=3, geom=_GLM,  tokens=4096,  wfmt="int4",  bias="zero"),
    "prefill16k": dict(index=3, geom=_GLM,  tokens=16384, wfmt="int4",  bias="zero"),
    "nvfp4_512":  dict(index=4, geom=_GLM,  tokens=512,   wfmt="nvfp4", bias="zipf"),
    "decode_topp":   dict(index=1, geom=_GLM_TOPP, tokens=1,  wfmt="int4", bias="zero"),
    "verify64_topp": dict(index=2, geom=_GLM_TOPP, tokens=64, wfmt="int4", bias="hot16"),
    # the per-row-scale formats on the decode and prefill shapes
    "decode_int4_row":    dict(index=1, geom=_GLM, tokens=1,    wfmt="int4_row", bias="zero"),
    "decode_int8_row":    dict(index=1, geom=_GLM, tokens=1,    wfmt="int8_row", bias="zero"),
    "decode_int2_row":    dict(index=1, geom=_GLM, tokens=1,    wfmt="int2_row", bias="zero"),
    "verify4_int2_row":   dict(index=2, geom=_GLM, tokens=4,    wfmt="int2_row", bias="hot16"),
    "prefill4k_int4_row": dict(index=3, geom=_GLM, tokens=4096, wfmt="int4_row", bias="zero"),
    "prefill4k_int8_row": dict(index=3, geom=_GLM, tokens=4096, wfmt="int8_row", bias="zero"),
    # the W4A8 integer-dot path (per-row int4 weights, int8 activations;
    # options = the library's MOE_OPT_INT8_ACTIVATIONS bit)
    "prefill4k_w4a8":     dict(index=3, geom=_GLM, tokens=4096, wfmt="int4_row", bias="zero", options=4),
    "prefill16k_w4a8":    dict(index=3, geom=_GLM, tokens=16384, wfmt="int4_row", bias="zero", options=4),
    "verify64_w4a8":      dict(index=2, geom=_GLM, tokens=64, wfmt="int4_row", bias="hot16", options=4),
}

WEIGHT_STD = 0.02       # expert, shared-expert and router weights ~ N(0, 0.02)
HOT_EXPERTS = 16        # batched-verify skew: 16 hot experts get +HOT_DELTA
HOT_DELTA = 0.13        # gives ~30% of top-8 picks on the hot set at H=6144
ZIPF_S = 1.1            # NVFP4 workload: b_e = ZIPF_BETA * rank_e ** -ZIPF_S
ZIPF_BETA = 2.0


def sub_seed(*parts: int) -> int:
    """Deterministic 63-bit seed from integer parts (splitmix64 chain)."""
    z = 0x9E3779B97F4A7C15
    for p in parts:
        z = (z ^ (int(p) & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        z = (z + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        z ^= z >> 31
    return z & 0x7FFFFFFFFFFFFFFF


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn(shape, seed: int, device="cpu", std: float = 1.0) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(device, seed), device=device,
                       dtype=torch.float32) * std


def to_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round float32 inputs to bfloat16 (round to nearest even)."""
    return x.to(torch.bfloat16)


# ----------------------------------------------------------------------------
# Encoders (weights -> packed bytes).  The layer only ever sees the bytes.
# ----------------------------------------------------------------------------

def pack_int4_words(u: torch.Tensor) -> torch.Tensor:
    """u: uint8 codes in [0, 15], shape [..., K] with K % 8 == 0.
    Returns uint8 [..., K/2] in the interleaved word layout described above."""
    *lead, K = u.shape
    assert K % 8 == 0
    c = u.to(torch.int32).reshape(*lead, K // 8, 8)
    b0 = c[..., 0] | (c[..., 2] << 4)
    b1 = c[..., 4] | (c[..., 6] << 4)
    b2 = c[..., 1] | (c[..., 3] << 4)
    b3 = c[..., 5] | (c[..., 7] << 4)
    out = torch.stack([b0, b1, b2, b3], dim=-1).to(torch.uint8)
    return out.reshape(*lead, K // 2)


def repack_int4_natural(q: torch.Tensor) -> torch.Tensor:
    """int4 codes packed in the natural order (byte j = input 2j in its low
    nibble, input 2j+1 in its high nibble), uint8 [..., K/2] -> the library's
    word order.  A layout change only (no arithmetic on the codes)."""
    c = torch.stack([q & 15, q >> 4], dim=-1).reshape(*q.shape[:-1], q.shape[-1] * 2)
    return pack_int4_words(c)


def pack_nibbles_natural(c: torch.Tensor) -> torch.Tensor:
    """c: uint8 codes in [0, 15], shape [..., K] with K even.  Byte j = c[2j] |
    c[2j+1] << 4."""
    *lead, K = c.shape
    c = c.to(torch.int32).reshape(*lead, K // 2, 2)
    return (c[..., 0] | (c[..., 1] << 4)).to(torch.uint8)


def quantize_int4_g32(W: torch.Tensor):
    """Symmetric int4 with one fp16 scale per 32 inputs.
    scale = fp16(absmax/7); q = clamp(round_half_even(w/scale), -7, 7); u = q+8.
    A group whose scale is zero encodes q = 0.
    W: float [..., N, K].  Returns (packed uint8 [..., N, K/2], fp16 [..., N, K/32])."""
    *lead, N, K = W.shape
    assert K % 32 == 0
    Wg = W.float().reshape(*lead, N, K // 32, 32)
    s16 = (Wg.abs().amax(-1) / 7.0).to(torch.float16)
    s = s16.float().unsqueeze(-1)
    q = torch.where(s > 0, torch.round(Wg / torch.where(s > 0, s, torch.ones_like(s))),
                    torch.zeros_like(Wg)).clamp_(-7, 7)
    u = (q + 8).to(torch.uint8).reshape(*lead, N, K)
    return pack_int4_words(u), s16


def pack_int2_words(u: torch.Tensor) -> torch.Tensor:
    """u: uint8 codes in [0, 3], shape [..., K] with K % 16 == 0.  Returns
    uint8 [..., K/4]: per 16 inputs one little-endian 32-bit word, input
    16j+2i (i = 0..7) in bits [2i, 2i+2), input 16j+2i+1 in bits
    [16+2i, 16+2i+2)."""
    *lead, K = u.shape
    assert K % 16 == 0
    c = u.to(torch.int64).reshape(*lead, K // 16, 8, 2)
    sh = 2 * torch.arange(8, dtype=torch.int64, device=u.device)
    word = ((c[..., 0] << sh) | (c[..., 1] << (sh + 16))).sum(-1)     # disjoint bits
    b = torch.stack([(word >> (8 * j)) & 255 for j in range(4)], dim=-1).to(torch.uint8)
    return b.reshape(*lead, K // 4)


def repack_int2_natural(q: torch.Tensor) -> torch.Tensor:
    """int2 codes packed in the natural order (byte j holds inputs 4j..4j+3 in
    bits 0-1, 2-3, 4-5, 6-7), uint8 [..., K/4] -> the library's word order.
    A layout change only."""
    c = torch.stack([(q >> (2 * i)) & 3 for i in range(4)], dim=-1)
    return pack_int2_words(c.reshape(*q.shape[:-1], q.shape[-1] * 4))


def _row_quantize(W: torch.Tensor, qmin: int, qmax: int, div: float):
    """scale = absmax(row) / div (fp32); q = clamp(round_half_even(w/scale),
    qmin, qmax); a zero row encodes q = 0."""
    Wf = W.float()
    s = Wf.abs().amax(-1) / div
    sd = torch.where(s > 0, s, torch.ones_like(s)).unsqueeze(-1)
    q = torch.where(s.unsqueeze(-1) > 0, torch.round(Wf / sd), torch.zeros_like(Wf))
    return q.clamp_(qmin, qmax), s


def quantize_int4_row(W: torch.Tensor):
    """int4 codes with one fp32 scale per row: scale = absmax/7, q in -7..7,
    u = q + 8, word layout of pack_int4_words.  W: float [..., N, K].
    Returns (uint8 [..., N, K/2], float32 [..., N])."""
    q, s = _row_quantize(W, -7, 7, 7.0)
    return pack_int4_words((q + 8).to(torch.uint8)), s


def quantize_int8_row(W: torch.Tensor):
    """int8 two's-complement codes in input order with one fp32 scale per row:
    scale = absmax/127, q in -127..127.  Returns (uint8 [..., N, K], float32 [..., N])."""
    q, s = _row_quantize(W, -127, 127, 127.0)
    return q.to(torch.int8).view(torch.uint8), s


def quantize_int2_row(W: torch.Tensor):
    """int2 codes with one fp32 scale per row: scale = absmax/2, q in -2..1
    (the positive side saturates at 1), u = q + 2, word layout of
    pack_int2_words.  Returns (uint8 [..., N, K/4], float32 [..., N])."""
    q, s = _row_quantize(W, -2, 1, 2.0)
    return pack_int2_words((q + 2).to(torch.uint8)), s


ROW_FORMATS = ("int4_row", "int8_row", "int2_row")


def _e2m1_encode(v: torch.Tensor) -> torch.Tensor:
    """Round-to-nearest-even onto the E2M1 grid {0,.5,1,1.5,2,3,4,6}, saturating
    at 6; returns uint8 codes (bit 3 = sign)."""
    m = v.abs()
    code = ((m > 0.25).to(torch.int32) + (m >= 0.75).to(torch.int32)
            + (m > 1.25).to(torch.int32) + (m >= 1.75).to(torch.int32)
            + (m > 2.5).to(torch.int32) + (m >= 3.5).to(torch.int32)
            + (m > 5.0).to(torch.int32))
    sign = ((v < 0) & (code > 0)).to(torch.int32) << 3
    return (code | sign).to(torch.uint8)


def quantize_nvfp4(W: torch.Tensor):
    """NVFP4 with one E4M3 scale per 16 inputs and one fp32 scale per tensor.
    g = absmax(W)/(6*448); s = e4m3_rne(min(absmax(block)/(6g), 448));
    q = e2m1_rne(w/(s*g)).  W: float [..., N, K] where the leading dims index
    separate tensors (experts).  Returns (packed uint8 [..., N, K/2], e4m3 bytes
    [..., N, K/16], fp32 [...])."""
    *lead, N, K = W.shape
    assert K % 16 == 0
    Wf = W.float()
    g = Wf.abs().flatten(-2).amax(-1) / (6.0 * 448.0)                    # [...]
    gs = torch.where(g > 0, g, torch.ones_like(g))
    Wb = Wf.reshape(*lead, N, K // 16, 16)
    bmax = Wb.abs().amax(-1) / (6.0 * gs[..., None, None])
    s8 = bmax.clamp(max=448.0).to(torch.float8_e4m3fn)
    s = s8.float()
    denom = (s * gs[..., None, None]).unsqueeze(-1)
    v = torch.where(denom > 0, Wb / torch.where(denom > 0, denom, torch.ones_like(denom)),
                    torch.zeros_like(Wb))
    codes = _e2m1_encode(v).reshape(*lead, N, K)
    return pack_nibbles_natural(codes), s8.view(torch.uint8), g


# ----------------------------------------------------------------------------
# Layers
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class QProj:
    """One projection of E experts: N output rows, K inputs."""
    q: torch.Tensor                   # uint8 [E, N, K * bits / 8]
    scale: torch.Tensor               # int4: float16 [E, N, K/32]; nvfp4: uint8 [E, N, K/16];
                                      # per-row formats: float32 [E, N]
    gscale: Optional[torch.Tensor]    # nvfp4: float32 [E]; otherwise None


@dataclasses.dataclass
class QExperts:
    gate: QProj                       # N = inter, K = hidden
    up: QProj                         # N = inter, K = hidden
    down: QProj                       # N = hidden, K = inter


@dataclasses.dataclass
class LayerInputs:
    name: str
    seed: int
    geom: dict
    wfmt: str
    T: int
    x: torch.Tensor                   # bfloat16 [T, H]
    router_w: torch.Tensor            # float32 [E, H]
    bias: torch.Tensor                # float32 [E]
    routed: QExperts
    shared: Optional[QExperts]


def _quantize(W: torch.Tensor, wfmt: str) -> QProj:
    if wfmt == "int4":
        q, s = quantize_int4_g32(W)
        return QProj(q, s, None)
    if wfmt in ROW_FORMATS:
        q, s = {"int4_row": quantize_int4_row, "int8_row": quantize_int8_row,
                "int2_row": quantize_int2_row}[wfmt](W)
        return QProj(q, s, None)
    q, s, g = quantize_nvfp4(W)
    return QProj(q, s, g)


def make_experts(seed: int, n_experts: int, hidden: int, inter: int, wfmt: str,
                 device="cpu", tag: int = 0) -> QExperts:
    """Generate N(0, 0.02) gate/up/down weights per expert and encode them.
    Each (expert, projection) has its own seed stream, so one expert can be
    regenerated alone."""
    parts = {"gate": [], "up": [], "down": []}
    for e in range(n_experts):
        for p, name in enumerate(("gate", "up", "down")):
            shape = (inter, hidden) if name != "down" else (hidden, inter)
            W = randn(shape, sub_seed(seed, tag, e, p), device, WEIGHT_STD)
            parts[name].append(_quantize(W.unsqueeze(0), wfmt))
            del W

    def cat(lst):
        return QProj(torch.cat([a.q for a in lst]), torch.cat([a.scale for a in lst]),
                     None if lst[0].gscale is None else torch.cat([a.gscale for a in lst]))
    return QExperts(cat(parts["gate"]), cat(parts["up"]), cat(parts["down"]))


def make_bias(recipe: str, n_experts: int, seed: int, device="cpu") -> torch.Tensor:
    if recipe == "zero":
        return torch.zeros(n_experts, dtype=torch.float32, device=device)
    if recipe == "normal0.1":
        return randn((n_experts,), sub_seed(seed, 3), device, 0.1)
    gcpu = _gen("cpu", sub_seed(seed, 4))
    if recipe == "hot16":
        hot = torch.randperm(n_experts, generator=gcpu)[:HOT_EXPERTS]
        b = torch.zeros(n_experts, dtype=torch.float32)
        b[hot] = HOT_DELTA
        return b.to(device)
    if recipe == "hot1":
        # expert 0 far ahead of every other: every token picks it
        b = torch.zeros(n_experts, dtype=torch.float32)
        b[0] = 10.0
        return b.to(device)
    if recipe == "zipf":
        rank = torch.randperm(n_experts, generator=gcpu).to(torch.float64) + 1.0
        return (ZIPF_BETA * rank.pow(-ZIPF_S)).to(torch.float32).to(device)
    raise ValueError(recipe)


def make_layer(name: str, device="cpu", tokens: Optional[int] = None,
               seed: Optional[int] = None) -> LayerInputs:
    """Build the seeded synthetic inputs of one named workload on `device`."""
    w = WORKLOADS[name]
    geom = dict(w["geom"])
    T = w["tokens"] if tokens is None else tokens
    seed = BASE_SEED + w["index"] if seed is None else seed
    H, I, E = geom["hidden"], geom["moe_inter"], geom["n_routed_experts"]
    x = to_bf16(randn((T, H), sub_seed(seed, 1, T), device))
    router_w = randn((E, H), sub_seed(seed, 2), device, WEIGHT_STD)
    bias = make_bias(w["bias"], E, seed, device)
    routed = make_experts(seed, E, H, I, w["wfmt"], device, tag=10)
    shared = None
    if geom["n_shared_experts"]:
        shared = make_experts(seed, 1, H, geom["shared_inter"], w["wfmt"], device, tag=11)
    return LayerInputs(name, seed, geom, w["wfmt"], T, x, router_w, bias, routed, shared)


def make_tokens(name: str, T: int, device="cpu", seed: Optional[int] = None) -> torch.Tensor:
    """Another batch of bf16 N(0,1) activations for an existing layer."""
    w = WORKLOADS[name]
    seed = BASE_SEED + w["index"] if seed is None else seed
    return to_bf16(randn((T, w["geom"]["hidden"]), sub_seed(seed, 1, T), device))


def small_geom(**over) -> dict:
    """A tiny geometry (the 'tiny' workload's) with overrides, for unit tests."""
    g = dict(_TINY)
    g.update(over)
    return g


def make_custom(geom: dict, T: int, wfmt: str, bias: str, seed: int,
                device="cpu") -> LayerInputs:
    """Inputs for an arbitrary (small) geometry; used by edge-case tests."""
    H, E = geom["hidden"], geom["n_routed_experts"]
    x = to_bf16(randn((T, H), sub_seed(seed, 1, T), device))
    router_w = randn((E, H), sub_seed(seed, 2), device, WEIGHT_STD)
    b = make_bias(bias, E, seed, device)
    routed = make_experts(seed, E, H, geom["moe_inter"], wfmt, device, tag=10)
    shared = None
    if geom.get("n_shared_experts", 0):
        shared = make_experts(seed, 1, H, geom["shared_inter"], wfmt, device, tag=11)
    return LayerInputs("custom", seed, dict(geom), wfmt, T, x, router_w, b, routed, shared)


# ----------------------------------------------------------------------------
# Raw packed bytes: every code the formats admit, not only what the encoders
# above emit (int4 code 0, i.e. q = -8; E2M1 -0; negative block scales)
# ----------------------------------------------------------------------------

def raw_int4_proj(E: int, N: int, K: int, seed: int, device="cpu") -> QProj:
    """Uniformly random code bytes and fp16 scales of either sign with
    magnitudes 2^U(-12, -4)."""
    g = _gen("cpu", seed)
    q = torch.randint(0, 256, (E, N, K // 2), generator=g, dtype=torch.int32).to(torch.uint8)
    mag = torch.exp2(torch.rand((E, N, K // 32), generator=g) * 8.0 - 12.0)
    sign = torch.where(torch.rand((E, N, K // 32), generator=g) < 0.5, -1.0, 1.0)
    return QProj(q.to(device), (mag * sign).to(torch.float16).to(device), None)


def raw_nvfp4_proj(E: int, N: int, K: int, seed: int, gscale: float,
                   device="cpu") -> QProj:
    """Uniformly random code bytes (both zeros of E2M1 included) and random
    finite E4M3 scale bytes of either sign (the two NaN codes 0x7F and 0xFF
    excluded); per-tensor scale `gscale` for every expert."""
    g = _gen("cpu", seed)
    q = torch.randint(0, 256, (E, N, K // 2), generator=g, dtype=torch.int32).to(torch.uint8)
    s = torch.randint(0, 254, (E, N, K // 16), generator=g, dtype=torch.int32)
    s = torch.where(s >= 0x7F, s + 1, s)          # skip 0x7F; 0xFF is out of range
    gs = torch.full((E,), gscale, dtype=torch.float32)
    return QProj(q.to(device), s.to(torch.uint8).to(device), gs.to(device))


def raw_row_proj(E: int, N: int, K: int, bits: int, seed: int, device="cpu") -> QProj:
    """Uniformly random code bytes (every code of the format) and fp32 row
    scales of either sign with magnitudes 2^U(-14, -6) / 2^(bits-4)."""
    g = _gen("cpu", seed)
    q = torch.randint(0, 256, (E, N, K * bits // 8), generator=g, dtype=torch.int32).to(torch.uint8)
    mag = torch.exp2(torch.rand((E, N), generator=g) * 8.0 - 14.0 - (bits - 4))
    sign = torch.where(torch.rand((E, N), generator=g) < 0.5, -1.0, 1.0)
    return QProj(q.to(device), (mag * sign).float().to(device), None)


def make_raw(geom: dict, T: int, wfmt: str, seed: int, device="cpu",
             gscale: float = 2e-4) -> LayerInputs:
    """A small layer whose expert weights are raw random bytes (see above);
    router and activations as in make_custom, zero bias."""
    H, E, I = geom["hidden"], geom["n_routed_experts"], geom["moe_inter"]

    def experts(n, inter, tag):
        shapes = ((inter, H), (inter, H), (H, inter))
        ps = []
        for p, (N, K) in enumerate(shapes):
            s = sub_seed(seed, tag, p)
            if wfmt == "int4":
                ps.append(raw_int4_proj(n, N, K, s, device))
            elif wfmt in ROW_FORMATS:
                bits = {"int4_row": 4, "int8_row": 8, "int2_row": 2}[wfmt]
                ps.append(raw_row_proj(n, N, K, bits, s, device))
            else:
                ps.append(raw_nvfp4_proj(n, N, K, s, gscale, device))
        return QExperts(*ps)
    x = to_bf16(randn((T, H), sub_seed(seed, 1, T), device))
    router_w = randn((E, H), sub_seed(seed, 2), device, WEIGHT_STD)
    b = make_bias("zero", E, seed, device)
    shared = experts(1, geom["shared_inter"], 21) if geom.get("n_shared_experts", 0) else None
    return LayerInputs("raw", seed, dict(geom), wfmt, T, x, router_w, b, experts(E, I, 20), shared)
