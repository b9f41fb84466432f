"""Seeded synthetic workloads for the batched routed-MoE FFN.

This module only draws random inputs and packs them into the formats the
FFN consumes; it holds none of the FFN's own arithmetic.  Both the HIP path
and the CPU oracle take their inputs from here, and nothing else is shared
between them.

Shapes follow the workloads the SharpInference issue pages benchmark:

* OLMoE-1B-7B layer (issue #406 "Measured", llama.cpp pp2048; issue #408
  names 64 experts / 8 active, norm_topk_prob=false): N=2048, d=2048, E=64,
  k=8, expert ffn 1024.
* A 35B-A3B MoE layer (issue #388, Carnice pp512 with a shared expert behind a
  gate, "shexp-gate" in the router phase): N=512, E=256, k=8, ffn 512 plus a
  512-wide shared expert.
* Decode (issue #408 tg128): N=1 and N=8 on the OLMoE shape.

The trained GGUF weights those pages run are not available, so every tensor
is drawn from a seeded generator: ``numpy.random.default_rng([cfg, layer,
role, index])``.  Roles: 0 hidden states, 1 router matrix, 2 router-bias
permutation, 3 shared-expert gate vector, 4/5/6 expert gate/up/down
(index = expert; index E = the shared expert).

Expert weights are drawn as N(0, 0.02) in fp32 and packed as Q8_0: per
32-element block one IEEE binary16 scale followed by 32 signed bytes
(34 bytes, no padding), rows of ``in/32`` blocks.  The packing rule used here
(scale = fp16(amax/127), code = clamp(rint(w/scale))) is input preparation
only: both sides read the same bytes, so any rule would do.

Workloads with ``fmt="q4_k"`` pack the same draws as Q4_K (the other MMQ
weight format issue #406 names): per 256 values {binary16 d, binary16 dmin,
12 bytes of 6-bit sub-block scales and mins, 128 bytes of 4-bit codes}
(144 bytes), a value being d*sc*q - dmin*m for its 32-value sub-block.  The
choice of d, dmin, sc, m and q below is again input preparation only.

Workloads with ``fmt="q3_k"`` pack the draws as Q3_K (the format of the
Q3_K expert kernel issue #388 names): per 256 values {32 bytes of high bits,
64 bytes of 2-bit codes, 12 bytes of 6-bit sub-block scales, binary16 d}
(110 bytes), a value being d*(sc-32)*q, q in -4..3, for its 16-value
sub-block; the field choice is input preparation only.
"""

from __future__ import annotations

import dataclasses
import math
import os
from typing import Optional

import numpy as np

Q8_BLOCK = 32          # elements per Q8_0 block
Q8_BLOCK_BYTES = 34    # fp16 scale + 32 int8 codes
Q4K_VALUES = 256       # elements per Q4_K super-block
Q4K_BYTES = 144        # fp16 d, fp16 dmin, 12 scale bytes, 128 code bytes
Q3K_BYTES = 110        # 32 high-bit bytes, 64 code bytes, 12 scale bytes, fp16 d

ROLE_X, ROLE_ROUTER, ROLE_BIAS_PERM, ROLE_SHARED_GATE = 0, 1, 2, 3
ROLE_GATE, ROLE_UP, ROLE_DOWN = 4, 5, 6


@dataclasses.dataclass(frozen=True)
class LayerShape:
    d: int                 # hidden size
    n_experts: int         # E
    top_k: int             # k (active experts per token, "na")
    ffn: int               # routed expert intermediate size F
    shared_ffn: int = 0    # shared expert intermediate size (0 = none)
    norm_topk_prob: bool = False
    zipf_bias: float = 0.0  # s of the per-expert Zipf router bias (0 = no bias)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    n_tokens: int
    shape: LayerShape
    n_layers: int = 1
    description: str = ""
    fmt: str = "q8_0"      # expert weight format: "q8_0", "q4_k" or "q3_k"


OLMOE = LayerShape(d=2048, n_experts=64, top_k=8, ffn=1024)
A3B = LayerShape(d=2048, n_experts=256, top_k=8, ffn=512, shared_ffn=512,
                 norm_topk_prob=True, zipf_bias=1.1)

WORKLOADS = {
    "tiny": Workload("tiny", 1, 16, LayerShape(d=128, n_experts=8, top_k=2, ffn=256),
                     description="tiny single MoE FFN layer"),
    "olmoe_n2048": Workload("olmoe_n2048", 2, 2048, OLMOE,
                            description="OLMoE-shaped layer, pp2048"),
    "olmoe_stack16": Workload("olmoe_stack16", 3, 2048, OLMOE, n_layers=16,
                              description="16 OLMoE layers with residual + RMSNorm"),
    "a3b_n512": Workload("a3b_n512", 4, 512, A3B,
                         description="35B-A3B-shaped layer, ubatch 512, shared expert, Zipf-skewed routing"),
    "olmoe_decode1": Workload("olmoe_decode1", 5, 1, OLMOE, description="decode, 1 token"),
    "olmoe_decode8": Workload("olmoe_decode8", 5, 8, OLMOE, description="decode, 8 tokens"),
    "olmoe_n4096": Workload("olmoe_n4096", 5, 4096, OLMOE, description="prefill stress, 4096 tokens"),
    # #388's second comment: a 2048-token logical batch prefilled as ubatch-512
    # chunks on the 35B-A3B shape (same layer seeds as a3b_n512)
    "a3b_n2048": Workload("a3b_n2048", 4, 2048, A3B,
                          description="35B-A3B-shaped layer, logical batch 2048 (ubatch-512 chunking)"),
    # the OLMoE and 35B-A3B layers with their experts in Q4_K
    "olmoe_n2048_q4k": Workload("olmoe_n2048_q4k", 2, 2048, OLMOE, fmt="q4_k",
                                description="OLMoE-shaped layer, pp2048, Q4_K experts"),
    "a3b_n512_q4k": Workload("a3b_n512_q4k", 4, 512, A3B, fmt="q4_k",
                             description="35B-A3B-shaped layer, ubatch 512, Q4_K experts"),
    # the OLMoE layer with its experts in Q3_K
    "olmoe_n2048_q3k": Workload("olmoe_n2048_q3k", 2, 2048, OLMOE, fmt="q3_k",
                                description="OLMoE-shaped layer, pp2048, Q3_K experts"),
}


def rng_for(cfg_id: int, layer: int, role: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg_id, layer, role, index])


def pack_q8_0(w: np.ndarray) -> np.ndarray:
    """Pack an fp32 matrix [rows][cols] (cols % 32 == 0) into Q8_0 bytes
    [rows][cols/32*34]."""
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert cols % Q8_BLOCK == 0
    nb = cols // Q8_BLOCK
    blk = w.reshape(rows, nb, Q8_BLOCK)
    amax = np.max(np.abs(blk), axis=2)
    d16 = (amax / np.float32(127.0)).astype(np.float16)
    d32 = d16.astype(np.float32)
    safe = np.where(d32 > 0, d32, np.float32(1.0))
    q = np.rint(blk / safe[:, :, None])
    q = np.where(d32[:, :, None] > 0, q, 0.0)
    q = np.clip(q, -127, 127).astype(np.int8)
    out = np.empty((rows, nb, Q8_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = d16.view(np.uint8).reshape(rows, nb, 2)
    out[:, :, 2:] = q.view(np.uint8)
    return out.reshape(rows, nb * Q8_BLOCK_BYTES)


def q4k_parts(w: np.ndarray):
    """Choose the Q4_K fields of an fp32 matrix [rows][cols] (cols % 256 == 0):
    returns d, dmin (fp16 [rows][cols/256]), sc, m (uint8 [rows][cols/32], 0..63)
    and q (uint8 [rows][cols], 0..15).  Per 32-value sub-block the codes span
    [min(block, 0), max(block, 0)] in 15 steps; d and dmin take the largest
    sub-block step and offset over 63."""
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert cols % Q4K_VALUES == 0
    nsb = cols // Q4K_VALUES
    sb = w.reshape(rows, nsb, 8, 32).astype(np.float64)
    lo = np.minimum(sb.min(axis=3), 0.0)
    hi = np.maximum(sb.max(axis=3), 0.0)
    step = (hi - lo) / 15.0
    off = -lo
    d16 = (step.max(axis=2) / 63.0).astype(np.float16)
    dmin16 = (off.max(axis=2) / 63.0).astype(np.float16)
    d = d16.astype(np.float64)[:, :, None]
    dmin = dmin16.astype(np.float64)[:, :, None]
    sc = np.clip(np.rint(np.divide(step, d, out=np.zeros_like(step), where=d > 0)), 0, 63)
    m = np.clip(np.rint(np.divide(off, dmin, out=np.zeros_like(off), where=dmin > 0)), 0, 63)
    unit = (d * sc)[..., None]
    base = (dmin * m)[..., None]
    q = np.clip(np.rint(np.divide(sb + base, unit, out=np.zeros_like(sb), where=unit > 0)), 0, 15)
    return (d16, dmin16, sc.astype(np.uint8).reshape(rows, nsb * 8), m.astype(np.uint8).reshape(rows, nsb * 8),
            q.astype(np.uint8).reshape(rows, cols))


def pack_q4_k(w: np.ndarray) -> np.ndarray:
    """Pack an fp32 matrix [rows][cols] (cols % 256 == 0) into Q4_K bytes
    [rows][cols/256*144]."""
    d16, dmin16, sc, m, q = q4k_parts(w)
    rows, cols = q.shape
    nsb = cols // Q4K_VALUES
    sc = sc.reshape(rows, nsb, 8).astype(np.uint16)
    m = m.reshape(rows, nsb, 8).astype(np.uint16)
    out = np.zeros((rows, nsb, Q4K_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = d16.view(np.uint8).reshape(rows, nsb, 2)
    out[:, :, 2:4] = dmin16.view(np.uint8).reshape(rows, nsb, 2)
    # scale bytes: 0..3 = sc_j (6 bits) | high 2 bits of sc_{j+4} << 6;
    # 4..7 = m_j | high 2 bits of m_{j+4} << 6; 8..11 = low 4 bits of
    # sc_{j+4} | low 4 bits of m_{j+4} << 4
    out[:, :, 4:8] = (sc[:, :, 0:4] | ((sc[:, :, 4:8] >> 4) << 6)).astype(np.uint8)
    out[:, :, 8:12] = (m[:, :, 0:4] | ((m[:, :, 4:8] >> 4) << 6)).astype(np.uint8)
    out[:, :, 12:16] = ((sc[:, :, 4:8] & 15) | ((m[:, :, 4:8] & 15) << 4)).astype(np.uint8)
    # code bytes: byte 32c + i = code i of sub-block 2c (low nibble) and of
    # sub-block 2c + 1 (high nibble)
    qs = q.reshape(rows, nsb, 4, 2, 32)
    out[:, :, 16:] = (qs[:, :, :, 0, :] | (qs[:, :, :, 1, :] << 4)).reshape(rows, nsb, 128)
    return out.reshape(rows, nsb * Q4K_BYTES)


def q3k_parts(w: np.ndarray):
    """Choose the Q3_K fields of an fp32 matrix [rows][cols] (cols % 256 ==
    0): returns d (fp16 [rows][cols/256]), sc (uint8 [rows][cols/16], 1..63)
    and q (int8 [rows][cols], -4..3).  Per 16-value sub-block the multiplier
    sc - 32 takes the sign that puts the value of largest magnitude on the
    code -4 side, and its size a quarter of that magnitude over d; d is the
    largest such quarter over 31."""
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert cols % Q4K_VALUES == 0
    nsb = cols // Q4K_VALUES
    sb = w.reshape(rows, nsb, 16, 16).astype(np.float64)
    pos, neg = sb.max(axis=3), -sb.min(axis=3)
    sign = np.where(pos > neg, -1.0, 1.0)
    step = np.maximum(pos, neg) / 4.0
    d16 = (step.max(axis=2) / 31.0).astype(np.float16)
    d = d16.astype(np.float64)[:, :, None]
    k = sign * np.clip(np.rint(np.divide(step, d, out=np.zeros_like(step), where=d > 0)), 0, 31)
    unit = (d * k)[..., None]
    q = np.clip(np.rint(np.divide(sb, unit, out=np.zeros_like(sb), where=unit != 0)), -4, 3)
    return d16, (k + 32).astype(np.uint8).reshape(rows, nsb * 16), q.astype(np.int8).reshape(rows, cols)


def pack_q3_k(w: np.ndarray) -> np.ndarray:
    """Pack an fp32 matrix [rows][cols] (cols % 256 == 0) into Q3_K bytes
    [rows][cols/256*110]."""
    d16, sc, q = q3k_parts(w)
    rows, cols = q.shape
    nsb = cols // Q4K_VALUES
    out = np.zeros((rows, nsb, Q3K_BYTES), dtype=np.uint8)
    # value 128h + 32g + l: 2-bit code in bits 2g of code byte 32h + l, its
    # high bit (set when q >= 0, else the code is q + 4) in bit 4h + g of
    # high-bit byte l
    qv = q.reshape(rows, nsb, 2, 4, 32).astype(np.int16)
    high = (qv >= 0).astype(np.uint16)
    code = np.where(qv >= 0, qv, qv + 4).astype(np.uint16)
    shifts = (2 * np.arange(4)).reshape(1, 1, 1, 4, 1)
    out[:, :, 32:96] = (code << shifts).sum(axis=3).reshape(rows, nsb, 64).astype(np.uint8)
    hb = (4 * np.arange(2).reshape(1, 1, 2, 1, 1) + np.arange(4).reshape(1, 1, 1, 4, 1))
    out[:, :, 0:32] = (high << hb).sum(axis=(2, 3)).astype(np.uint8)
    # sub-block s: low 4 bits in nibble s/8 of byte s%8, high 2 bits in
    # bits 2(s/4) of byte 8 + s%4
    s = sc.reshape(rows, nsb, 16).astype(np.uint16)
    out[:, :, 96:104] = ((s[:, :, 0:8] & 15) | ((s[:, :, 8:16] & 15) << 4)).astype(np.uint8)
    hi2 = ((s >> 4) & 3).reshape(rows, nsb, 4, 4)          # [t][k] for s = 4t + k
    out[:, :, 104:108] = (hi2 << (2 * np.arange(4)).reshape(1, 1, 4, 1)).sum(axis=2).astype(np.uint8)
    out[:, :, 108:110] = d16.view(np.uint8).reshape(rows, nsb, 2)
    return out.reshape(rows, nsb * Q3K_BYTES)


def pack_weights(w: np.ndarray, fmt: str) -> np.ndarray:
    return {"q4_k": pack_q4_k, "q3_k": pack_q3_k}.get(fmt, pack_q8_0)(w)


def row_bytes(fmt: str, in_dim: int) -> int:
    if fmt == "q4_k":
        return in_dim // Q4K_VALUES * Q4K_BYTES
    if fmt == "q3_k":
        return in_dim // Q4K_VALUES * Q3K_BYTES
    return in_dim // Q8_BLOCK * Q8_BLOCK_BYTES


def unpack_q8_0(b: np.ndarray, cols: int):
    """Split Q8_0 bytes [rows][cols/32*34] into (codes int8 [rows][cols],
    scales fp16 [rows][cols/32])."""
    rows = b.shape[0]
    nb = cols // Q8_BLOCK
    blk = np.ascontiguousarray(b).reshape(rows, nb, Q8_BLOCK_BYTES)
    scales = np.ascontiguousarray(blk[:, :, 0:2]).view(np.float16).reshape(rows, nb)
    codes = np.ascontiguousarray(blk[:, :, 2:]).view(np.int8).reshape(rows, cols)
    return codes, scales


@dataclasses.dataclass
class LayerWeights:
    shape: LayerShape
    router_w: np.ndarray                 # fp32 [E][d]
    router_bias: Optional[np.ndarray]    # fp32 [E] or None
    gate_q8: np.ndarray                  # uint8 [E][F][d/32*34]
    up_q8: np.ndarray                    # uint8 [E][F][d/32*34]
    down_q8: np.ndarray                  # uint8 [E][d][F/32*34]
    sh_gate_q8: Optional[np.ndarray] = None   # uint8 [Fs][d/32*34]
    sh_up_q8: Optional[np.ndarray] = None     # uint8 [Fs][d/32*34]
    sh_down_q8: Optional[np.ndarray] = None   # uint8 [d][Fs/32*34]
    sh_gate_vec: Optional[np.ndarray] = None  # fp32 [d]
    fmt: str = "q8_0"    # format of the expert rows above (the *_q8 arrays hold Q4_K / Q3_K rows for those formats)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def _cache_path(tag: str) -> Optional[str]:
    root = os.environ.get("MOE_WORKLOAD_CACHE")
    if not root:
        return None
    os.makedirs(root, exist_ok=True)
    return os.path.join(root, tag + ".npz")


def make_layer(shape: LayerShape, cfg_id: int, layer: int = 0,
               n_experts_override: Optional[int] = None, fmt: str = "q8_0") -> LayerWeights:
    """Draw one layer's weights.  Expert e of role r always comes from
    ``rng_for(cfg_id, layer, r, e)`` so a subset of experts can be drawn alone;
    the expert rows are packed in ``fmt`` ("q8_0", "q4_k" or "q3_k")."""
    E = shape.n_experts if n_experts_override is None else n_experts_override
    d, F, Fs = shape.d, shape.ffn, shape.shared_ffn
    tag = f"layer_c{cfg_id}_l{layer}_d{d}_e{E}_f{F}_s{Fs}_z{shape.zipf_bias}" + ("" if fmt == "q8_0" else "_" + fmt)
    cp = _cache_path(tag)
    if cp and os.path.exists(cp):
        z = np.load(cp, allow_pickle=False)
        get = lambda k: (z[k] if k in z.files else None)
        return LayerWeights(shape, z["router_w"], get("router_bias"), z["gate_q8"], z["up_q8"],
                            z["down_q8"], get("sh_gate_q8"), get("sh_up_q8"), get("sh_down_q8"),
                            get("sh_gate_vec"), fmt)

    router_w = _normal(rng_for(cfg_id, layer, ROLE_ROUTER), (E, d), 0.02)
    router_bias = None
    if shape.zipf_bias:
        # Zipf(s) prior over a seeded random ranking of the experts:
        # bias_e = -s * ln(rank_e), rank_e in 1..E.
        perm = rng_for(cfg_id, layer, ROLE_BIAS_PERM).permutation(E)
        router_bias = (-shape.zipf_bias * np.log(perm.astype(np.float64) + 1.0)).astype(np.float32)
    pack = lambda w: pack_weights(w, fmt)
    gate = np.empty((E, F, row_bytes(fmt, d)), np.uint8)
    up = np.empty((E, F, row_bytes(fmt, d)), np.uint8)
    down = np.empty((E, d, row_bytes(fmt, F)), np.uint8)
    for e in range(E):
        gate[e] = pack(_normal(rng_for(cfg_id, layer, ROLE_GATE, e), (F, d), 0.02))
        up[e] = pack(_normal(rng_for(cfg_id, layer, ROLE_UP, e), (F, d), 0.02))
        down[e] = pack(_normal(rng_for(cfg_id, layer, ROLE_DOWN, e), (d, F), 0.02))
    lw = LayerWeights(shape, router_w, router_bias, gate, up, down, fmt=fmt)
    if Fs:
        se = shape.n_experts
        lw.sh_gate_q8 = pack(_normal(rng_for(cfg_id, layer, ROLE_GATE, se), (Fs, d), 0.02))
        lw.sh_up_q8 = pack(_normal(rng_for(cfg_id, layer, ROLE_UP, se), (Fs, d), 0.02))
        lw.sh_down_q8 = pack(_normal(rng_for(cfg_id, layer, ROLE_DOWN, se), (d, Fs), 0.02))
        lw.sh_gate_vec = _normal(rng_for(cfg_id, layer, ROLE_SHARED_GATE), (d,), 0.02)
    if cp:
        arrs = {k: v for k, v in dataclasses.asdict(lw).items() if isinstance(v, np.ndarray)}
        np.savez(cp, **arrs)
    return lw


def make_tokens(cfg_id: int, n_tokens: int, d: int, layer: int = 0) -> np.ndarray:
    """Hidden states x ~ N(0, 1), fp32 [N][d] (the scale RMSNorm leaves)."""
    return rng_for(cfg_id, layer, ROLE_X).standard_normal((n_tokens, d), dtype=np.float32)


def workload_layer(name: str, layer: int = 0) -> LayerWeights:
    w = WORKLOADS[name]
    return make_layer(w.shape, w.cfg_id, layer, fmt=w.fmt)


def workload_tokens(name: str, n_tokens: Optional[int] = None) -> np.ndarray:
    w = WORKLOADS[name]
    return make_tokens(w.cfg_id, w.n_tokens if n_tokens is None else n_tokens, w.shape.d)


def random_shape_case(seed: int, d: int, E: int, k: int, F: int, Fs: int = 0,
                      norm: bool = False, zipf: float = 0.0, fmt: str = "q8_0"):
    """A small arbitrary-shape case for edge-case tests (cfg id 100 + seed)."""
    shape = LayerShape(d=d, n_experts=E, top_k=k, ffn=F, shared_ffn=Fs,
                       norm_topk_prob=norm, zipf_bias=zipf)
    return shape, make_layer(shape, 100 + seed, fmt=fmt)


def expert_bytes(shape: LayerShape, fmt: str = "q8_0") -> int:
    return 2 * shape.ffn * row_bytes(fmt, shape.d) + shape.d * row_bytes(fmt, shape.ffn)


def describe(name: str) -> dict:
    w = WORKLOADS[name]
    s = w.shape
    return {"workload": name, "n_tokens": w.n_tokens, "d": s.d, "n_experts": s.n_experts,
            "top_k": s.top_k, "ffn": s.ffn, "shared_ffn": s.shared_ffn,
            "norm_topk_prob": bool(s.norm_topk_prob), "n_layers": w.n_layers,
            "router_bias": ("zipf(%.1f)" % s.zipf_bias) if s.zipf_bias else "none",
            "weights": {"q4_k": "Q4_K (4-bit codes, 256-elem super-blocks, 6-bit sub-block scales and mins)",
                        "q3_k": "Q3_K (3-bit codes, 256-elem super-blocks, 6-bit signed 16-elem sub-block scales)"}
                       .get(w.fmt, "Q8_0 (int8, 32-elem blocks, fp16 scale)")}
