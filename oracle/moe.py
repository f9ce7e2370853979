"""fp64 reference of the quantized MoE layer (test infrastructure only).

Every step is written from its definition, in float64, with NumPy; no blocking,
fusion or reordering beyond what the definition states.  Page references:

  [P2-Fitur]  page "Show HN: Menjalankan GLM 5.2 di komputer lambat",
              section "Fitur utama yang diimplementasikan" (DeepSeek-V3-style
              sigmoid router, noaux_tc, routed_scaling_factor, shared expert;
              batch-union MoE; int4 kernels with dequant-on-use).
  [P2-Cara]   same page, section "Cara kerja eksekusi MoE berbasis streaming
              disk" (routed experts vs the always-resident shared expert).
  [P2-Unduh]  same page, section "Mengunduh model dan menjalankannya"
              (the --topp 0.7 option: adaptive expert top-p), and section
              "Benchmark komunitas" (its measured effect).
  [P5-Tech]   page "NVIDIA stellt neues GLM-5.2 NVFP4 Modell vor", section
              "Technische Details und Quantisierungsansatz" (expert FFNs in
              NVFP4 with FP8 scales per 16 elements; router kept in BF16/FP32).

Readings taken where the pages are silent are listed in the repository's design
notes; the ones that change results are repeated at the function that takes them.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.  A bf16 number is the upper
    half of an IEEE binary32, so widening is exact."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def fp16_bits_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64 (exact)."""
    return np.asarray(bits).astype(np.uint16).view(np.float16).astype(np.float64)


def decode_e2m1(codes) -> np.ndarray:
    """E2M1 (FP4) code -> value.  Bit 3 is the sign, bits 2..1 the exponent with
    bias 1, bit 0 the mantissa; exponent 0 is subnormal (0 or 0.5).  Magnitudes
    are therefore {0, 0.5, 1, 1.5, 2, 3, 4, 6}.  [P5-Tech: 4-bit elements]"""
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> 3) & 1
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1).astype(np.int64)))
    return np.where(sign == 1, -mag, mag)


def decode_e4m3fn(codes) -> np.ndarray:
    """FP8 E4M3 ("fn": bias 7, no infinities, S.1111.111 is NaN) -> value.
    [P5-Tech: FP8 scale per 16 elements]"""
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6),
                   np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


# ---------------------------------------------------------------------------
# Packed weight layouts
# ---------------------------------------------------------------------------

def unpack_int4_codes(q: np.ndarray) -> np.ndarray:
    """uint8 [..., K/2] in the interleaved word layout -> codes [..., K].
    Each group of 4 bytes is a little-endian 32-bit word covering inputs
    8j..8j+7; input 8j+2i sits in bits [4i, 4i+4) and input 8j+2i+1 in bits
    [16+4i, 16+4i+4)."""
    q = np.asarray(q, dtype=np.uint8)
    *lead, half = q.shape
    K = half * 2
    b = q.reshape(*lead, K // 8, 4).astype(np.uint32)
    word = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)
    out = np.empty((*lead, K // 8, 8), dtype=np.uint8)
    for i in range(4):
        out[..., 2 * i] = (word >> (4 * i)) & 15
        out[..., 2 * i + 1] = (word >> (16 + 4 * i)) & 15
    return out.reshape(*lead, K)


def unpack_nvfp4_codes(q: np.ndarray) -> np.ndarray:
    """uint8 [..., K/2] -> E2M1 codes [..., K]; byte j holds input 2j in the low
    nibble and input 2j+1 in the high nibble."""
    q = np.asarray(q, dtype=np.uint8)
    *lead, half = q.shape
    out = np.empty((*lead, half, 2), dtype=np.uint8)
    out[..., 0] = q & 15
    out[..., 1] = q >> 4
    return out.reshape(*lead, half * 2)


def dequant_int4(q: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Symmetric int4 with one fp16 scale per 32 inputs: w = (u - 8) * scale.
    [P2-Fitur: packed int4, dequant-on-use; group-32 scales per the workload]
    q: uint8 [N, K/2]; scale_bits: uint16/float16 [N, K/32] -> float64 [N, K]."""
    u = unpack_int4_codes(q).astype(np.float64)
    s = fp16_bits_to_f64(np.asarray(scale_bits).view(np.uint16))
    N, K = u.shape
    return ((u - 8.0).reshape(N, K // 32, 32) * s[:, :, None]).reshape(N, K)


def dequant_nvfp4(q: np.ndarray, scale_e4m3: np.ndarray, gscale: float) -> np.ndarray:
    """NVFP4: w = e2m1(code) * e4m3(block scale of 16 inputs) * fp32 per-tensor
    scale.  [P5-Tech]  q: uint8 [N, K/2]; scale_e4m3: uint8 [N, K/16]."""
    v = decode_e2m1(unpack_nvfp4_codes(q))
    s = decode_e4m3fn(scale_e4m3)
    N, K = v.shape
    g = float(np.float32(gscale))
    return (v.reshape(N, K // 16, 16) * s[:, :, None]).reshape(N, K) * g


# Per-row-scale formats.  [P2-Fitur: the quantisation kernels handle int8,
# packed int4 and packed int2 with one scale per row, dequantised on use.]  The
# pages name these formats without a layout; the reading taken: symmetric
# integer codes with one float32 scale per output row, w = q * scale[row];
# int8 codes are two's-complement bytes in input order; int4 codes use the
# int4 word layout above (q = u - 8); int2 codes use the word layout below
# (q = u - 2).

def unpack_int2_codes(q: np.ndarray) -> np.ndarray:
    """uint8 [..., K/4] -> codes [..., K] in 0..3.  Each group of 4 bytes is a
    little-endian 32-bit word covering inputs 16j..16j+15; input 16j+2i
    (i = 0..7) sits in bits [2i, 2i+2) and input 16j+2i+1 in bits
    [16+2i, 16+2i+2)."""
    q = np.asarray(q, dtype=np.uint8)
    *lead, quarter = q.shape
    K = quarter * 4
    b = q.reshape(*lead, K // 16, 4).astype(np.uint32)
    word = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)
    out = np.empty((*lead, K // 16, 16), dtype=np.uint8)
    for i in range(8):
        out[..., 2 * i] = (word >> (2 * i)) & 3
        out[..., 2 * i + 1] = (word >> (16 + 2 * i)) & 3
    return out.reshape(*lead, K)


def _row_scale(scale) -> np.ndarray:
    return np.asarray(scale, dtype=np.float32).astype(np.float64)[:, None]


def dequant_int4_row(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """int4 codes (word layout of unpack_int4_codes), one fp32 scale per row:
    w = (u - 8) * scale[n].  q: uint8 [N, K/2]; scale: float32 [N]."""
    return (unpack_int4_codes(q).astype(np.float64) - 8.0) * _row_scale(scale)


def dequant_int8_row(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """int8 two's-complement codes in input order, one fp32 scale per row:
    w = q * scale[n].  q: uint8/int8 [N, K]; scale: float32 [N]."""
    return np.asarray(q).view(np.int8).astype(np.float64) * _row_scale(scale)


def dequant_int2_row(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """int2 codes (word layout of unpack_int2_codes), one fp32 scale per row:
    w = (u - 2) * scale[n].  q: uint8 [N, K/4]; scale: float32 [N]."""
    return (unpack_int2_codes(q).astype(np.float64) - 2.0) * _row_scale(scale)


ROW_FORMATS = {"int4_row": dequant_int4_row, "int8_row": dequant_int8_row,
               "int2_row": dequant_int2_row}
# W4A8 (integer-dot) sources: per-row int4 weights whose FFN takes int8
# activations (w4a8_ffn); their weights decode as the base format.
A8_FORMATS = {"int4_row_a8": "int4_row"}


@dataclasses.dataclass
class ExpertSource:
    """Packed weights of E experts as NumPy arrays, decoded on demand.
    proj -> (q uint8 [E,N,...], scale [E,N,...], gscale float32 [E] or None)."""
    wfmt: str                      # "int4", "nvfp4" or one of ROW_FORMATS
    gate: tuple
    up: tuple
    down: tuple

    def weight(self, proj: str, e: int) -> np.ndarray:
        q, s, g = getattr(self, proj)
        if self.wfmt == "int4":
            return dequant_int4(q[e], s[e])
        if self.wfmt in ROW_FORMATS:
            return ROW_FORMATS[self.wfmt](q[e], s[e])
        if self.wfmt in A8_FORMATS:
            return ROW_FORMATS[A8_FORMATS[self.wfmt]](q[e], s[e])
        return dequant_nvfp4(q[e], s[e], g[e])

    @property
    def n_experts(self) -> int:
        return self.gate[0].shape[0]


# ---------------------------------------------------------------------------
# Router  [P2-Fitur: DeepSeek-V3-style sigmoid router, noaux_tc,
#          routed_scaling_factor]
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class RouterConfig:
    n_experts: int
    n_group: int
    topk_group: int
    top_k: int
    routed_scaling_factor: float
    group_top: int = 2          # reading: a group's score is the sum of its top-2 biased scores
    top_p: float = 0.0          # adaptive expert top-p; 0 (or >= 1) keeps all top_k


def _router_scores(x: np.ndarray, Wr: np.ndarray, b: np.ndarray):
    logits = np.asarray(x, np.float64) @ np.asarray(Wr, np.float64).T
    s = 1.0 / (1.0 + np.exp(-logits))
    sb = s + np.asarray(b, np.float64)[None, :]
    return logits, s, sb


def _group_scores(sb: np.ndarray, cfg: RouterConfig) -> np.ndarray:
    T, E = sb.shape
    per = E // cfg.n_group
    top = min(cfg.group_top, per)
    desc = -np.sort(-sb.reshape(T, cfg.n_group, per), axis=-1)
    return desc[..., :top].sum(-1)


def route(x: np.ndarray, Wr: np.ndarray, b: np.ndarray, cfg: RouterConfig):
    """Select top_k experts per token.

    1. logits = x . Wr^T (float64; x is bf16 widened exactly, Wr fp32).
    2. s = sigmoid(logits).
    3. s' = s + b  (the score-correction bias steers selection only).
    4. group j = experts [j*E/G, (j+1)*E/G); group score = sum of its top-2 s'.
    5. keep the topk_group best groups (equal scores: lower group index first).
    6. among experts of the kept groups, take the top_k by s' (equal: lower id);
       experts of dropped groups are excluded outright (-inf), so exactly top_k
       experts always come from the kept groups.
    7. report ids in ascending expert id.
    8. weights: w_i = s[id_i] / sum_j s[id_j] * routed_scaling_factor.
    9. adaptive expert top-p (0 < top_p < 1), see `apply_top_p`: only a
       prefix of the chosen experts stays; the others get id -1 and weight 0,
       after the kept ids.
    Returns (ids int64 [T,k], w float64 [T,k], info dict)."""
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    E, G, TG, k = cfg.n_experts, cfg.n_group, cfg.topk_group, cfg.top_k
    logits, s, sb = _router_scores(x, Wr, b)
    gscore = _group_scores(sb, cfg)
    gorder = np.argsort(-gscore, axis=1, kind="stable")
    keep = np.zeros((T, G), dtype=bool)
    np.put_along_axis(keep, gorder[:, :TG], True, axis=1)
    allowed = np.repeat(keep, E // G, axis=1)
    masked = np.where(allowed, sb, -np.inf)
    eorder = np.argsort(-masked, axis=1, kind="stable")
    ids = np.sort(eorder[:, :k], axis=1)
    margin = route_margins(sb, gscore, keep, cfg)
    if 0.0 < cfg.top_p < 1.0:
        ids, pmargin = apply_top_p(s, ids, cfg.top_p)
        margin = np.minimum(margin, pmargin)
    w = route_weights(s, ids, cfg.routed_scaling_factor)
    info = dict(logits=logits, s=s, sb=sb, gscore=gscore, keep=keep, margin=margin)
    return ids, w, info


def apply_top_p(s: np.ndarray, ids: np.ndarray, p: float):
    """Adaptive expert top-p [P2-Unduh: --topp].  The pages name the option
    only; the reading taken: order a token's chosen experts by their share
    s_e / sum(s over the chosen) (descending; equal shares: lower id first),
    keep the shortest prefix whose shares add up to at least p -- at least
    one expert -- and drop the rest (id -1, after the kept ids, which stay in
    ascending order).  The kept weights are renormalised by `route_weights`.
    Also returns each token's decision margin: the smallest distance of a
    prefix sum from p, and the share gap between the last kept and the first
    dropped expert."""
    ids = np.asarray(ids)
    T, k = ids.shape
    out = np.full_like(ids, -1)
    margin = np.full(T, np.inf)
    for t in range(T):
        sel = [int(e) for e in ids[t]]
        sv = [float(s[t, e]) for e in sel]
        total = sum(sv)
        order = sorted(range(k), key=lambda i: (-sv[i], sel[i]))
        shares = [sv[i] / total for i in order]
        csum, keep = 0.0, k
        for j in range(k):
            csum += shares[j]
            margin[t] = min(margin[t], abs(csum - p))
            if csum >= p and keep == k:
                keep = j + 1
        if keep < k:
            margin[t] = min(margin[t], shares[keep - 1] - shares[keep])
        kept = sorted(sel[i] for i in order[:keep])
        out[t, :keep] = kept
    return out, margin


def route_weights(s: np.ndarray, ids: np.ndarray, rsf: float) -> np.ndarray:
    """Renormalised unbiased sigmoid scores of the chosen experts times
    routed_scaling_factor (no epsilon: every s > 0).  Slots with id -1
    (dropped by the adaptive top-p) get weight 0 and do not enter the sum."""
    ids = np.asarray(ids)
    valid = ids >= 0
    sel = np.take_along_axis(np.asarray(s, np.float64), np.where(valid, ids, 0), axis=1)
    sel = np.where(valid, sel, 0.0)
    return sel / sel.sum(axis=1, keepdims=True) * float(rsf)


def route_margins(sb, gscore, keep, cfg: RouterConfig) -> np.ndarray:
    """Per token: the smallest gap at a selection boundary -- between the
    topk_group-th and next group score, and between the top_k-th and next
    allowed s'.  A decision whose margin is tiny may flip under rounding."""
    T, G = gscore.shape
    gdesc = -np.sort(-gscore, axis=1)
    m = np.full(T, np.inf)
    if cfg.topk_group < G:
        m = np.minimum(m, gdesc[:, cfg.topk_group - 1] - gdesc[:, cfg.topk_group])
    allowed = np.repeat(keep, cfg.n_experts // G, axis=1)
    masked = np.where(allowed, sb, -np.inf)
    edesc = -np.sort(-masked, axis=1)
    n_allowed = allowed.sum(1)
    k = cfg.top_k
    has_next = n_allowed > k
    if has_next.any():
        gap = edesc[:, k - 1] - np.where(has_next, edesc[:, min(k, edesc.shape[1] - 1)], -np.inf)
        m = np.minimum(m, np.where(has_next, gap, np.inf))
    return m


def valid_under_perturbation(ids_t: np.ndarray, sb_t: np.ndarray, cfg: RouterConfig,
                             tau: float) -> bool:
    """Whether `ids_t` (one token's chosen experts) is what the selection of
    `route` returns for some biased scores within `tau` of `sb_t` -- the check
    applied to tokens whose decision margin is below rounding level."""
    E, G, TG, k = cfg.n_experts, cfg.n_group, cfg.topk_group, cfg.top_k
    ids_t = np.asarray(ids_t)
    if len(set(ids_t.tolist())) != k or ids_t.min() < 0 or ids_t.max() >= E:
        return False
    # (with the adaptive top-p, check the kept prefix with valid_top_p)
    per = E // G
    gscore = _group_scores(sb_t[None, :], cfg)[0]
    chosen_groups = sorted(set((ids_t // per).tolist()))
    if len(chosen_groups) > TG:
        return False
    rest = [g for g in np.argsort(-gscore, kind="stable") if g not in chosen_groups]
    gsel = chosen_groups + rest[: TG - len(chosen_groups)]
    out = [g for g in range(G) if g not in gsel]
    # each s' may move by tau, so a group score (sum of two) by 2*tau
    if out and min(gscore[gsel]) < max(gscore[out]) - 4 * tau:
        return False
    allowed = np.zeros(E, bool)
    for g in gsel:
        allowed[g * per:(g + 1) * per] = True
    chosen = np.zeros(E, bool)
    chosen[ids_t] = True
    others = allowed & ~chosen
    if others.any() and sb_t[chosen].min() < sb_t[others].max() - 2 * tau:
        return False
    return True


# ---------------------------------------------------------------------------
# Permutation  [P2-Fitur: batch-union MoE]
# ---------------------------------------------------------------------------

def permute(ids: np.ndarray, n_experts: int):
    """Group the T*k picks by expert, keeping pick order (t*k+i) inside an
    expert: a counting sort written out.  Picks with id -1 (dropped by the
    adaptive top-p) take no slot; their inv_perm is -1.
    Returns expert_offsets [E+1], sorted_token [P'] (token of the pick at each
    sorted position, P' valid picks), inv_perm [T*k] (sorted position of pick
    t*k+i), active_experts (ascending ids with at least one pick)."""
    ids = np.asarray(ids)
    T, k = ids.shape
    flat = ids.reshape(-1).tolist()
    counts = [0] * n_experts
    for e in flat:
        if e < 0:
            continue
        counts[e] += 1
    offsets = [0] * (n_experts + 1)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:-1]
    cursor = list(cursor)
    sorted_token = [0] * offsets[n_experts]
    inv_perm = [-1] * (T * k)
    for p, e in enumerate(flat):
        if e < 0:
            continue
        pos = cursor[e]
        cursor[e] += 1
        sorted_token[pos] = p // k
        inv_perm[p] = pos
    active = [e for e in range(n_experts) if counts[e] > 0]
    return (np.array(offsets, np.int64), np.array(sorted_token, np.int64),
            np.array(inv_perm, np.int64), np.array(active, np.int64))


# ---------------------------------------------------------------------------
# Expert FFN and layer  [P2-Fitur, P2-Cara, P5-Tech]
# ---------------------------------------------------------------------------

def swiglu_ffn(X: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """FFN(x) = Wd ( silu(Wg x) * (Wu x) ),  silu(z) = z * sigmoid(z).
    X: [M, H]; Wg, Wu: [I, H]; Wd: [H, I]; all float64."""
    G = X @ Wg.T
    U = X @ Wu.T
    with np.errstate(over="ignore"):
        h = G / (1.0 + np.exp(-G)) * U
    return h @ Wd.T


def _expert_weights(src: ExpertSource, e: int):
    return src.weight("gate", e), src.weight("up", e), src.weight("down", e)


def layer(x_bits, Wr, b, cfg: RouterConfig, routed: ExpertSource,
          shared: Optional[ExpertSource] = None, ids: Optional[np.ndarray] = None,
          token_idx: Optional[np.ndarray] = None, ffn_map=None):
    """y_t = sum_{e in S_t} w_{t,e} FFN_e(x_t) + FFN_shared(x_t).

    (S_t, w_t) come from `route` unless `ids` is given, in which case the
    weights are recomputed for those ids.  `token_idx` restricts the evaluation
    to a subset of tokens (rows of x_bits / ids are then those tokens).
    The shared expert enters with weight 1 (routed_scaling_factor applies to the
    routed experts only).  Each routed expert is dequantised once and applied to
    the tokens that chose it; that only reorders the sum over experts.
    `ffn_map`, if given, evaluates the list of (source, expert, X rows) jobs and
    returns their FFN outputs in order -- e.g. spread over worker processes,
    each calling `expert_ffn`; it only decides where the jobs run.
    Returns (y float64 [T', H], ids, w)."""
    X = bf16_bits_to_f64(x_bits)
    if token_idx is not None:
        X = X[np.asarray(token_idx)]
    _, s, _ = _router_scores(X, Wr, b)
    if ids is None:
        ids, w, _ = route(X, Wr, b, cfg)
    else:
        ids = np.asarray(ids)
        w = route_weights(s, ids, cfg.routed_scaling_factor)
    T, H = X.shape
    experts = [int(e) for e in np.unique(ids) if e >= 0]
    jobs = [(routed, e, X[np.nonzero(ids == e)[0]]) for e in experts]
    if shared is not None:
        jobs.append((shared, 0, X))
    outs = ffn_map(jobs) if ffn_map is not None else [expert_ffn(*j) for j in jobs]
    y = np.zeros((T, H))
    for e, F in zip(experts, outs):
        rows, slots = np.nonzero(ids == e)
        y[rows] += w[rows, slots][:, None] * F
    if shared is not None:
        y += outs[-1]
    return y, ids, w


def expert_ffn(src: ExpertSource, e: int, X: np.ndarray) -> np.ndarray:
    """FFN of expert e of `src` (dequantised from its packed bytes) on rows X;
    W4A8 sources take their integer-dot FFN."""
    if src.wfmt in A8_FORMATS:
        return w4a8_ffn(src, e, X)
    return swiglu_ffn(X, *_expert_weights(src, e))


# ---------------------------------------------------------------------------
# W4A8 integer-dot FFN.  [P2-Fitur: an integer-dot kernel with int8
# activations in the Q8_0 manner (1.4-2.5x faster than float; int4 weights
# 1.8x faster on batches, single rows kept in float).]  Reading: the weights
# are the pages' own container (int4 codes, one scale per row); activations are
# quantised to int8 with one scale per row -- the input x per token, and the
# SwiGLU output h (held in fp16) per (token, expert) row -- instead of Q8_0's one
# scale per 32 inputs, so that both scales factor out of an integer dot product
# over the whole row.  The quantiser's decisions are taken in float32 (the
# precision the kernels use), so both sides form the same codes from the same
# values.
# ---------------------------------------------------------------------------

def quantize_rows_int8(a: np.ndarray):
    """Symmetric int8 codes per row, in float32 arithmetic: amax = max |a|,
    q = clamp(rint(a * (127 / amax)), -127, 127) (ties to even), scale =
    amax / 127; an all-zero row gives q = 0 and scale 0.
    a: float32 [M, K] -> (q int64 [M, K], scale float32 [M])."""
    a = np.asarray(a, dtype=np.float32)
    amax = np.abs(a).max(axis=1)
    safe = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
    inv = np.where(amax > 0, np.float32(127.0) / safe, np.float32(0.0)).astype(np.float32)
    q = np.clip(np.rint(a * inv[:, None]), -127, 127).astype(np.int64)
    return q, (amax / np.float32(127.0)).astype(np.float32)


def _int4_row_codes(src: ExpertSource, proj: str, e: int):
    q, s, _ = getattr(src, proj)
    codes = unpack_int4_codes(q[e]).astype(np.int64) - 8
    return codes, np.asarray(s[e], dtype=np.float32).astype(np.float64)


def w4a8_ffn(src: ExpertSource, e: int, X: np.ndarray) -> np.ndarray:
    """SwiGLU FFN of expert e with int8 activations: G = s_x s_g (q_x . q_g),
    U likewise, h = silu(G) U rounded to fp16, then quantised per row, and
    O = s_h s_d (q_h . q_d); the integer dot products are exact.
    X: float64 rows holding bf16 values."""
    cg, sg = _int4_row_codes(src, "gate", e)
    cu, su = _int4_row_codes(src, "up", e)
    cd, sd = _int4_row_codes(src, "down", e)
    xq, sx = quantize_rows_int8(np.asarray(X, dtype=np.float32))
    sx = sx.astype(np.float64)[:, None]
    G = (xq @ cg.T).astype(np.float64) * sg[None, :] * sx
    U = (xq @ cu.T).astype(np.float64) * su[None, :] * sx
    with np.errstate(over="ignore"):
        h = G / (1.0 + np.exp(-G)) * U
    hq, sh = quantize_rows_int8(h.astype(np.float16).astype(np.float32))
    return (hq @ cd.T).astype(np.float64) * sd[None, :] * sh.astype(np.float64)[:, None]


def dense_layer(x_bits, Wr, b, cfg: RouterConfig, routed: ExpertSource,
                shared: Optional[ExpertSource] = None):
    """The same layer as a dense MoE: every expert on every token, multiplied by
    a gate matrix that is w on the chosen experts and 0 elsewhere.  Small
    shapes only."""
    X = bf16_bits_to_f64(x_bits)
    ids, w, _ = route(X, Wr, b, cfg)
    T, H = X.shape
    gate = np.zeros((T, cfg.n_experts))
    for t in range(T):
        for e, we in zip(ids[t], w[t]):
            if e >= 0:
                gate[t, e] = we
    y = np.zeros((T, H))
    for e in range(cfg.n_experts):
        y += gate[:, e:e + 1] * expert_ffn(routed, e, X)
    if shared is not None:
        y += expert_ffn(shared, 0, X)
    return y


def valid_top_p(ids_t: np.ndarray, s_t: np.ndarray, chosen_t: np.ndarray, p: float,
                tau: float) -> bool:
    """Whether `ids_t` (one token's ids after the adaptive top-p, -1 for
    dropped slots) is what `apply_top_p` keeps from the chosen experts
    `chosen_t` for some shares within `tau` of the exact ones -- the check for
    tokens whose top-p decision margin is below rounding level."""
    kept = [int(e) for e in ids_t if e >= 0]
    chosen = [int(e) for e in chosen_t]
    if not kept or not set(kept) <= set(chosen) or list(ids_t[len(kept):]) != [-1] * (len(ids_t) - len(kept)):
        return False
    if kept != sorted(kept):
        return False
    total = sum(float(s_t[e]) for e in chosen)
    share = {e: float(s_t[e]) / total for e in chosen}
    dropped = [e for e in chosen if e not in kept]
    if dropped and min(share[e] for e in kept) < max(share[e] for e in dropped) - 2 * tau:
        return False
    ks = sorted((share[e] for e in kept), reverse=True)
    csum = sum(ks)
    if csum < p - len(chosen) * tau:
        return False
    return len(kept) == 1 or csum - ks[-1] < p + len(chosen) * tau
