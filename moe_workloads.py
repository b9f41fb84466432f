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
"""

from __future__ import annotations

import dataclasses
import math
import os
from typing import Optional

import numpy as np

Q8_BLOCK = 32          # elements per Q8_0 block
Q8_BLOCK_BYTES = 34    # fp16 scale + 32 int8 codes

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


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def _cache_path(tag: str) -> Optional[str]:
    root = os.environ.get("MOE_WORKLOAD_CACHE")
    if not root:
        return None
    os.makedirs(root, exist_ok=True)
    return os.path.join(root, tag + ".npz")


def make_layer(shape: LayerShape, cfg_id: int, layer: int = 0,
               n_experts_override: Optional[int] = None) -> LayerWeights:
    """Draw one layer's weights.  Expert e of role r always comes from
    ``rng_for(cfg_id, layer, r, e)`` so a subset of experts can be drawn alone."""
    E = shape.n_experts if n_experts_override is None else n_experts_override
    d, F, Fs = shape.d, shape.ffn, shape.shared_ffn
    tag = f"layer_c{cfg_id}_l{layer}_d{d}_e{E}_f{F}_s{Fs}_z{shape.zipf_bias}"
    cp = _cache_path(tag)
    if cp and os.path.exists(cp):
        z = np.load(cp, allow_pickle=False)
        get = lambda k: (z[k] if k in z.files else None)
        return LayerWeights(shape, z["router_w"], get("router_bias"), z["gate_q8"], z["up_q8"],
                            z["down_q8"], get("sh_gate_q8"), get("sh_up_q8"), get("sh_down_q8"),
                            get("sh_gate_vec"))

    router_w = _normal(rng_for(cfg_id, layer, ROLE_ROUTER), (E, d), 0.02)
    router_bias = None
    if shape.zipf_bias:
        # Zipf(s) prior over a seeded random ranking of the experts:
        # bias_e = -s * ln(rank_e), rank_e in 1..E.
        perm = rng_for(cfg_id, layer, ROLE_BIAS_PERM).permutation(E)
        router_bias = (-shape.zipf_bias * np.log(perm.astype(np.float64) + 1.0)).astype(np.float32)
    nbd = d // Q8_BLOCK
    nbf = F // Q8_BLOCK
    gate = np.empty((E, F, nbd * Q8_BLOCK_BYTES), np.uint8)
    up = np.empty((E, F, nbd * Q8_BLOCK_BYTES), np.uint8)
    down = np.empty((E, d, nbf * Q8_BLOCK_BYTES), np.uint8)
    for e in range(E):
        gate[e] = pack_q8_0(_normal(rng_for(cfg_id, layer, ROLE_GATE, e), (F, d), 0.02))
        up[e] = pack_q8_0(_normal(rng_for(cfg_id, layer, ROLE_UP, e), (F, d), 0.02))
        down[e] = pack_q8_0(_normal(rng_for(cfg_id, layer, ROLE_DOWN, e), (d, F), 0.02))
    lw = LayerWeights(shape, router_w, router_bias, gate, up, down)
    if Fs:
        se = shape.n_experts
        lw.sh_gate_q8 = pack_q8_0(_normal(rng_for(cfg_id, layer, ROLE_GATE, se), (Fs, d), 0.02))
        lw.sh_up_q8 = pack_q8_0(_normal(rng_for(cfg_id, layer, ROLE_UP, se), (Fs, d), 0.02))
        lw.sh_down_q8 = pack_q8_0(_normal(rng_for(cfg_id, layer, ROLE_DOWN, se), (d, Fs), 0.02))
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
    return make_layer(w.shape, w.cfg_id, layer)


def workload_tokens(name: str, n_tokens: Optional[int] = None) -> np.ndarray:
    w = WORKLOADS[name]
    return make_tokens(w.cfg_id, w.n_tokens if n_tokens is None else n_tokens, w.shape.d)


def random_shape_case(seed: int, d: int, E: int, k: int, F: int, Fs: int = 0,
                      norm: bool = False, zipf: float = 0.0):
    """A small arbitrary-shape case for edge-case tests (cfg id 100 + seed)."""
    shape = LayerShape(d=d, n_experts=E, top_k=k, ffn=F, shared_ffn=Fs,
                       norm_topk_prob=norm, zipf_bias=zipf)
    return shape, make_layer(shape, 100 + seed)


def expert_bytes(shape: LayerShape) -> int:
    per = (2 * shape.ffn * shape.d + shape.d * shape.ffn) // Q8_BLOCK * Q8_BLOCK_BYTES
    return per


def describe(name: str) -> dict:
    w = WORKLOADS[name]
    s = w.shape
    return {"workload": name, "n_tokens": w.n_tokens, "d": s.d, "n_experts": s.n_experts,
            "top_k": s.top_k, "ffn": s.ffn, "shared_ffn": s.shared_ffn,
            "norm_topk_prob": bool(s.norm_topk_prob), "n_layers": w.n_layers,
            "router_bias": ("zipf(%.1f)" % s.zipf_bias) if s.zipf_bias else "none",
            "weights": "Q8_0 (int8, 32-elem blocks, fp16 scale)"}
