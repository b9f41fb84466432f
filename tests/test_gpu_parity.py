"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.

Bar: routing top-k ids, CSR arrays and the int8 activation codes/scales are
bit-exact; the ordered combine is bit-exact given identical inputs; the fp32
outputs are within relative L2 2e-3 and per-element 1e-2 * rms(out) of the
oracle (int8 MMQ, argmax-stable contract of SharpInference #406).
"""
import os
import sys

import numpy as np
import pytest

import moe_workloads as mw
from helpers import moe_close
from oracle import oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def lib_loaded():
    from mixture_experts_ffn_gemm_amd import binding
    binding.lib()   # raises when the library is missing: no fallback
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield


def run_gpu(lw, x, api="prefill", layer=None, keep=False):
    from mixture_experts_ffn_gemm_amd import binding as B
    from mixture_experts_ffn_gemm_amd.layer import MoeLayer
    s = lw.shape
    n = x.shape[0]
    own = layer is None
    if own:
        layer = MoeLayer.from_workload(lw)
    dev = torch.device("cuda")
    kk = s.top_k + (1 if s.shared_ffn else 0)
    P = n * s.top_k + (n if s.shared_ffn else 0)
    bufs = dict(
        topk_ids=torch.full((n, s.top_k), -7, dtype=torch.int32, device=dev),
        topk_w=torch.full((n, s.top_k), -7.0, dtype=torch.float32, device=dev),
        shared_gate=torch.zeros(n, dtype=torch.float32, device=dev),
        exp_start=torch.full((s.n_experts + 1 + (1 if s.shared_ffn else 0),), -7, dtype=torch.int32, device=dev),
        exp_tok_i=torch.full((P,), -7, dtype=torch.int32, device=dev),
        exp_tok_k=torch.full((P,), -7, dtype=torch.int32, device=dev),
        xq=torch.zeros((n, s.d), dtype=torch.int8, device=dev),
        xs=torch.zeros((n, s.d // 32), dtype=torch.int16, device=dev),
        partial=torch.zeros((n, kk, s.d), dtype=torch.float32, device=dev),
    )
    r = B.make_routing(**bufs)
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    out = torch.full((n, s.d), float("nan"), dtype=torch.float32, device=dev)
    if api == "prefill":
        layer.prefill(xt, out=out, routing=r)
    else:
        layer.decode(xt, out=out, routing=r)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in bufs.items()}
    res["xs"] = res["xs"].view(np.uint16)
    res["out"] = out.cpu().numpy()
    if own and not keep:
        layer.close()
    if keep:
        res["layer"] = layer
    return res


def check_routing(lw, x, g):
    s = lw.shape
    o = O.routing(lw, x)
    assert np.array_equal(g["topk_ids"], o["ids"]), "top-k ids differ"
    assert np.array_equal(g["exp_start"], o["exp_start"]), "expStart differs"
    assert np.array_equal(g["exp_tok_i"], o["tok_i"]), "expTokI differs"
    assert np.array_equal(g["exp_tok_k"], o["tok_k"]), "expTokK differs"
    assert np.array_equal(g["xq"], o["xq"]), "int8 activation codes differ"
    assert np.array_equal(g["xs"], o["xs"]), "activation scales differ"
    np.testing.assert_allclose(g["topk_w"], o["w"], rtol=2e-6, atol=1e-7)
    if s.shared_ffn:
        np.testing.assert_allclose(g["shared_gate"], o["gs"], rtol=1e-5, atol=1e-6)
    return o


def check_outputs(lw, x, g, tokens=None):
    n = x.shape[0]
    toks = np.arange(n) if tokens is None else np.asarray(tokens)
    ref = O.moe_tokens(lw, x, tokens=toks, want_partial=True)
    r, e = moe_close(g["out"][toks], ref["out"])
    # Unweighted partials: same L2 bar; per element, one int8 code of h landing
    # on the other side of a rounding boundary (fp32 on the GPU, fp64 in the
    # oracle) moves a partial by |W_down| * (h step) ~ 3/(127 sqrt(F)) of its
    # rms times amax/rms of the h block, i.e. a few percent when F is 32 wide.
    rp, ep = moe_close(g["partial"][toks], ref["partial"], elem=6e-2)
    # the GPU's combine reproduces the fp32 ordered reduce bit for bit
    gs = g["shared_gate"][toks] if lw.shape.shared_ffn else None
    comb = O.combine_f32(g["partial"][toks], g["topk_w"][toks], gs)
    assert np.array_equal(comb, g["out"][toks]), "combine is not the ordered fp32 reduce"
    return r, e


# ------------------------------------------------------------- stage kernels
def test_quantize_stage_bitexact():
    from mixture_experts_ffn_gemm_amd import binding as B
    rng = np.random.default_rng(20)
    v = (rng.standard_normal((37, 256)) * np.exp(rng.standard_normal((37, 1)) * 4)).astype(np.float32)
    v[5, 64:96] = 0.0
    v[6, :32] = np.float32(1e-30)
    v[7, 32:64] = np.array([127.0, 2.5, 3.5, -2.5] + [0.0] * 28, np.float32)
    vt = torch.from_numpy(v).cuda()
    q = torch.empty(v.shape, dtype=torch.int8, device="cuda")
    s = torch.empty((37, 8), dtype=torch.int16, device="cuda")
    B.moe_ffn_quantize(vt, v.size, q, s)
    torch.cuda.synchronize()
    oq, os_ = O.quantize_q8(v)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(s.cpu().numpy().view(np.uint16), os_)


@pytest.mark.parametrize("k,shared,n,d", [(1, False, 3, 64), (8, False, 37, 2048), (8, True, 21, 256),
                                          (16, True, 5, 128), (3, False, 0, 32)])
def test_combine_stage_bitexact(k, shared, n, d):
    from mixture_experts_ffn_gemm_amd import binding as B
    rng = np.random.default_rng(21 + k)
    kk = k + (1 if shared else 0)
    P = rng.standard_normal((n, kk, d)).astype(np.float32)
    w = rng.random((n, k)).astype(np.float32)
    gs = rng.random(n).astype(np.float32) if shared else None
    out = torch.empty((n, d), dtype=torch.float32, device="cuda")
    B.moe_ffn_combine(torch.from_numpy(P).cuda(), torch.from_numpy(w).cuda(),
                      torch.from_numpy(gs).cuda() if shared else None, n, k, d, out)
    torch.cuda.synchronize()
    ref = O.combine_f32(P, w, gs)
    assert np.array_equal(out.cpu().numpy(), ref)


def test_combine_stage_golden_order():
    import json
    from mixture_experts_ffn_gemm_amd import binding as B
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "combine_slot_order.json")))
    for c in g["cases"]:
        k = len(c["weights"])
        # pad d to 4 so the float4 path is exercised with the same value in every column
        P = np.repeat(np.array(c["partials"], np.float32)[None], 1, 0)
        P = np.repeat(P, 4, axis=2)
        w = np.array([c["weights"]], np.float32)
        gs = np.array([c["shared_gate"]], np.float32) if "shared_gate" in c else None
        out = torch.empty((1, 4), dtype=torch.float32, device="cuda")
        B.moe_ffn_combine(torch.from_numpy(P).cuda(), torch.from_numpy(w).cuda(),
                          torch.from_numpy(gs).cuda() if gs is not None else None, 1, k, 4, out)
        torch.cuda.synchronize()
        assert np.all(out.cpu().numpy() == np.float32(c["expected"][0])), c["name"]


# ------------------------------------------------------------- whole layer
def test_tiny_layer_parity():
    lw = mw.workload_layer("tiny")
    x = mw.workload_tokens("tiny")
    g = run_gpu(lw, x)
    check_routing(lw, x, g)
    r, e = check_outputs(lw, x, g)
    say(f"tiny: rel_l2={r:.2e} max_elem={e:.2e}")


SHAPES = [
    dict(d=96, E=5, k=5, F=64, norm=True),             # k = E, paddings everywhere
    dict(d=128, E=8, k=1, F=32),                        # k = 1
    dict(d=160, E=16, k=3, F=96, Fs=64, zipf=1.1),      # shared expert, Fs != F, skew
    dict(d=256, E=70, k=4, F=128, norm=True),           # E not a multiple of 64
    dict(d=64, E=1, k=1, F=64, norm=True),              # a single expert (dense FFN)
    dict(d=128, E=256, k=16, F=64, Fs=32),              # E = 256, k = 16, shared
]


@pytest.mark.parametrize("case", range(len(SHAPES)))
@pytest.mark.parametrize("n", [1, 7, 53])
def test_shape_edge_cases(case, n):
    shape, lw = mw.random_shape_case(case, **SHAPES[case])
    x = mw.make_tokens(200 + case, n, shape.d)
    g = run_gpu(lw, x)
    check_routing(lw, x, g)
    check_outputs(lw, x, g)


# Mid-size cases checked on every token: groups of more than 128 rows (so
# expert groups span several 128-row GEMM tiles and every wavefront of a tile
# computes), an odd k-step count above one (d = 384: 3 gate/up k-steps;
# F = 320 -> 3 down k-steps, ragged against the 64-column gate/up strips), and
# a shared expert of 2-8 tiles.
MID_SHAPES = [
    dict(d=384, E=4, k=2, F=320),
    dict(d=384, E=4, k=2, F=320, Fs=160, zipf=1.1, norm=True),
]


@pytest.mark.parametrize("case", range(len(MID_SHAPES)))
@pytest.mark.parametrize("n", [300, 1000])
def test_mid_size_all_tokens(case, n):
    shape, lw = mw.random_shape_case(20 + case, **MID_SHAPES[case])
    x = mw.make_tokens(700 + case, n, shape.d)
    g = run_gpu(lw, x)
    check_routing(lw, x, g)
    counts = np.diff(g["exp_start"])
    assert counts.max() > 128, "the case must put more than one GEMM tile in a group"
    r, e = check_outputs(lw, x, g)
    say(f"mid case {case} n={n}: max group {int(counts.max())} rows, rel_l2={r:.2e} max_elem={e:.2e}")


def _tied_router(lw, E, bias):
    """The layer with router rows 5 and E-1 duplicating rows 3 and 0 (scaled up
    so that they are usually selected) and, with a bias, equal biases on the
    duplicated pairs: every token has exactly tied logits."""
    import dataclasses
    rw = lw.router_w.copy()
    rw[3] *= 4.0
    rw[0] *= 4.0
    rw[5] = rw[3]
    rw[E - 1] = rw[0]
    b = None
    if bias:
        b = (-0.2 * np.log(np.arange(E, dtype=np.float64)[::-1] % 7 + 1.0)).astype(np.float32)
        b[5] = b[3]
        b[E - 1] = b[0]
    return dataclasses.replace(lw, router_w=rw, router_bias=b)


@pytest.mark.parametrize("api", ["prefill", "decode"])
@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("E", [8, 70])
def test_routing_ties(E, bias, api):
    """Exactly tied logits: duplicated router rows (with and without equal
    biases) and all-zero token rows, whose logits all tie (0, or the bias).
    The top-k must break ties towards the lower expert id exactly as the
    oracle does, on the fused router (E <= 64) and the separate routing
    launch (E > 64), in prefill and in decode."""
    shape, lw = mw.random_shape_case(30 + E, d=128, E=E, k=4, F=64)
    lw = _tied_router(lw, E, bias)
    n = 45 if api == "prefill" else 8
    x = mw.make_tokens(800 + E, n, shape.d)
    x[0] = 0.0
    x[n - 2] = 0.0
    g = run_gpu(lw, x, api=api)
    o = check_routing(lw, x, g)
    logits = o["logits"]
    assert np.any(logits[:, 3] == logits[:, 5]) and np.any(logits[:, 0] == logits[:, E - 1])
    if not bias:
        assert np.array_equal(g["topk_ids"][0], np.arange(4)), "an all-zero token ties every expert"
    check_outputs(lw, x, g)


# ------------------------------------------------------------- GEMM integer core
def _strip_rows(q8, s, strip, gemm, n_rows):
    """The Q8_0 weight rows of strip column c = 0..127 (None past the matrix)."""
    rows = []
    for c in range(128):
        if gemm == 0:
            src, r = (q8[0], 64 * strip + c) if c < 64 else (q8[1], 64 * strip + c - 64)
        else:
            src, r = q8, 128 * strip + c
        rows.append(src[r] if r < n_rows else None)
    return rows


def check_block_sums(lw, x, layer, ws, n, samples):
    """moe_ffn_dbg_block_sums after a prefill on ws: the exact int32 block sums
    of the product GEMMs' int8 MFMA path, compared bit for bit with the
    oracle's block sums of the same codes.  Gate/up: the A codes must be the
    oracle's activation codes of the tile's CSR rows.  Down: the A codes are
    the GPU's own h codes (the oracle's may differ where h sits on a rounding
    boundary), and must be the oracle's h codes of those rows almost
    everywhere."""
    from mixture_experts_ffn_gemm_amd import binding as B
    s = lw.shape
    o = O.routing(lw, x)
    dev = torch.device("cuda")
    sums = torch.empty((128, 128), dtype=torch.int32, device=dev)
    acodes = torch.empty((128, 32), dtype=torch.int8, device=dev)
    info = torch.empty(4, dtype=torch.int32, device=dev)
    checked = 0
    flips = []
    for gemm, tile, strip, kb in samples:
        sums.fill_(-7)
        B.moe_ffn_dbg_block_sums(layer.handle, ws, ws.numel(), n, gemm, tile, strip, kb, sums, acodes, info)
        torch.cuda.synchronize()
        g, row0, row_end, n_tiles = (int(v) for v in info.cpu().numpy())
        assert g >= 0, (gemm, tile, strip, kb, g)
        m = min(128, row_end - row0)
        toks = o["tok_i"][row0:row0 + m]
        slots = o["tok_k"][row0:row0 + m]
        got, ac = sums.cpu().numpy()[:m], acodes.cpu().numpy()[:m]
        shared = g == s.n_experts
        Fg = s.shared_ffn if shared else s.ffn
        if gemm == 0:
            kbs = s.d // 32
            want_a = o["xq"][toks, 32 * kb:32 * kb + 32] if kb < kbs else np.zeros((m, 32), np.int8)
            assert np.array_equal(ac, want_a), f"gate/up A codes of tile {tile} differ"
            q8 = (lw.sh_gate_q8, lw.sh_up_q8) if shared else (lw.gate_q8[g], lw.up_q8[g])
            rows = _strip_rows(q8, s, strip, 0, Fg)
        else:
            kbs = Fg // 32
            q8 = lw.sh_down_q8 if shared else lw.down_q8[g]
            rows = _strip_rows(q8, s, strip, 1, s.d)
            if kb < kbs:
                hq = []
                for t, sl in zip(toks, slots):
                    gw = (lw.sh_gate_q8, lw.sh_up_q8, lw.sh_down_q8) if shared else \
                        (lw.gate_q8[g], lw.up_q8[g], lw.down_q8[g])
                    _, hq_t, _, _ = O.expert_ffn(s.d, Fg, o["xq"][t], o["xs"][t], *gw)
                    hq.append(hq_t[32 * kb:32 * kb + 32])
                same = np.mean(np.asarray(hq) == ac)
                flips.append((int(np.sum(np.asarray(hq) != ac)), int(ac.size)))
                assert same >= 0.98, f"down A codes of tile {tile} match the oracle's h codes in {same:.3f}"
            else:
                assert np.all(ac == 0), "K-padding blocks of h must hold zero codes"
        want = np.zeros((m, 128), np.int64)
        if kb < kbs:
            for c, row in enumerate(rows):
                if row is not None:
                    want[:, c] = O.q8_block_sums(ac, row[None, :], kb)[:, 0]
        assert np.array_equal(got, want), f"block sums differ: gemm {gemm} tile {tile} strip {strip} k-block {kb}"
        checked += 1
    if flips:
        nf, nt = sum(f for f, _ in flips), sum(t for _, t in flips)
        say(f"h codes differing from the oracle's (rounding-boundary flips): {nf} of {nt} ({nf / nt:.2e})")
    return checked


@pytest.mark.parametrize("which", ["tiny", "mid", "a3b_n512", "olmoe_n2048"])
def test_gemm_block_sums_bitexact(which):
    from mixture_experts_ffn_gemm_amd.layer import MoeLayer
    if which == "mid":
        shape, lw = mw.random_shape_case(21, **MID_SHAPES[1])
        x = mw.make_tokens(701, 300, shape.d)
    else:
        lw = mw.workload_layer(which)
        x = mw.workload_tokens(which)
    s = lw.shape
    n = x.shape[0]
    layer = MoeLayer.from_workload(lw)
    try:
        xt = torch.from_numpy(x).cuda()
        layer.prefill(xt)
        ws = layer.workspace(n)
        o = O.routing(lw, x)
        counts = np.diff(o["exp_start"])
        ntiles = int(sum((c + 127) // 128 for c in counts))
        gu_strips = max(s.ffn, s.shared_ffn) // 64
        dn_strips = (s.d + 127) // 128
        kb_gu, kb_dn = (s.d + 127) // 128 * 4, (max(s.ffn, s.shared_ffn) + 127) // 128 * 4
        rng = np.random.default_rng(31)
        tiles = sorted({0, ntiles - 1, int(rng.integers(0, ntiles))})
        samples = []
        for t in tiles:
            samples += [(0, t, 0, 0), (0, t, int(rng.integers(0, gu_strips)), kb_gu - 1),
                        (0, t, 0, int(rng.integers(0, kb_gu))),
                        (1, t, 0, 0), (1, t, dn_strips - 1, int(rng.integers(0, kb_dn))),
                        (1, t, int(rng.integers(0, dn_strips)), kb_dn - 1)]
        # the shared expert's F may differ: keep only strips / k-blocks inside the tile's group
        from mixture_experts_ffn_gemm_amd import binding as B
        ok = []
        for gemm, t, st, kb in samples:
            grp = _tile_group(counts, t)
            Fg = s.shared_ffn if grp == s.n_experts else s.ffn
            Fg_pad = (Fg + 127) // 128 * 128
            if gemm == 0 and st >= Fg_pad // 64:
                continue
            if gemm == 1 and kb >= Fg_pad // 32:
                continue
            ok.append((gemm, t, st, kb))
        checked = check_block_sums(lw, x, layer, ws, n, ok)
        say(f"{which}: {checked} (tile, strip, k-block) block-sum dumps bit-exact")
        assert checked >= 6
    finally:
        layer.close()


def _tile_group(counts, t):
    """Group of 128-row tile t in the tile table (groups in order, each cut into ceil(c/128) tiles)."""
    for g, c in enumerate(counts):
        nt = (int(c) + 127) // 128
        if t < nt:
            return g
        t -= nt
    raise AssertionError("tile past the table")


# ------------------------------------------------------------- Q4_K weights
# The Q4_K grouped GEMMs (#406 "References": Q4_K beside Q8_0 in the int8
# MMQ path) against the oracle's Q4_K expert path (per value the dequantised
# activation times the dequantised super-block value, summed in fp64).  d, F
# and Fs are multiples of 256 (one super-block = two 128-value k-steps).
Q4K_SHAPES = [
    dict(d=256, E=8, k=2, F=256),                                 # one super-block per row
    dict(d=512, E=16, k=3, F=256, Fs=512, zipf=1.1, norm=True),   # shared expert, Fs != F, skew
    dict(d=256, E=70, k=4, F=512),                                # E > 64: routing in its own launch
    dict(d=256, E=1, k=1, F=256, norm=True),                      # a single expert (dense FFN)
    dict(d=256, E=5, k=5, F=256, norm=True),                      # k = E
    dict(d=256, E=256, k=16, F=256, Fs=256),                      # E = 256, k = 16, shared
]


@pytest.mark.parametrize("case", range(len(Q4K_SHAPES)))
@pytest.mark.parametrize("n", [1, 53])
def test_q4k_shapes(case, n):
    shape, lw = mw.random_shape_case(40 + case, fmt="q4_k", **Q4K_SHAPES[case])
    say(f"q4k case {case}: {Q4K_SHAPES[case]} n={n}")
    x = mw.make_tokens(900 + case, n, shape.d)
    g = run_gpu(lw, x)
    check_routing(lw, x, g)
    r, e = check_outputs(lw, x, g)
    say(f"q4k case {case} n={n}: rel_l2={r:.2e} max_elem={e:.2e}")


def test_q4k_mid_size_all_tokens():
    """Groups of several 128-row tiles (every wavefront of a tile computes),
    6 gate/up and 4 down k-steps, a shared expert of a different width."""
    shape, lw = mw.random_shape_case(45, d=768, E=4, k=2, F=512, Fs=256, zipf=1.1, fmt="q4_k")
    x = mw.make_tokens(945, 600, shape.d)
    say("q4k mid: d=768 E=4 k=2 F=512 Fs=256 n=600")
    g = run_gpu(lw, x)
    check_routing(lw, x, g)
    counts = np.diff(g["exp_start"])
    assert counts.max() > 128, "the case must put more than one GEMM tile in a group"
    r, e = check_outputs(lw, x, g)
    say(f"q4k mid: max group {int(counts.max())} rows, rel_l2={r:.2e} max_elem={e:.2e}")


@pytest.mark.parametrize("n", [1, 8])
def test_q4k_decode_runs_the_prefill_launches(n):
    """moe_ffn_decode on a Q4_K handle (the gathered matvecs read Q8_0 planes
    only, so the call runs the prefill launches): routing bit-exact, outputs
    against the oracle."""
    shape, lw = mw.random_shape_case(41, fmt="q4_k", **Q4K_SHAPES[1])
    x = mw.make_tokens(941 + n, n, shape.d)
    g = run_gpu(lw, x, api="decode")
    check_routing(lw, x, g)
    r, e = check_outputs(lw, x, g)
    say(f"q4k decode n={n}: rel_l2={r:.2e} max_elem={e:.2e}")


def test_q4k_chunked_residual_and_static():
    """The Q4_K GEMMs through the other prefill entry points: chunked (100
    tokens per chunk, serpentine) against the oracle, the stack form bit for
    bit against prefill + residual RMSNorm, and the no-alloc entry point bit
    for bit against prefill."""
    from mixture_experts_ffn_gemm_amd import binding as B
    from mixture_experts_ffn_gemm_amd.layer import MoeLayer
    shape, lw = mw.random_shape_case(42, fmt="q4_k", **Q4K_SHAPES[1])
    n, d, eps = 300, shape.d, 1e-5
    x_np = mw.make_tokens(942, n, d)
    layer = MoeLayer.from_workload(lw)
    try:
        x = torch.from_numpy(x_np).cuda()
        full = layer.prefill(x)
        ws = torch.empty(layer.workspace_size(100), dtype=torch.uint8, device="cuda")
        ch = torch.full((n, d), float("nan"), dtype=torch.float32, device="cuda")
        B.moe_ffn_prefill_chunked(layer.handle, x, n, 100, B.CHUNK_SERPENTINE, ch, ws, ws.numel())
        h0 = torch.from_numpy(mw.make_tokens(943, n, d)).cuda()
        h_ref, xn_ref = h0.clone(), torch.empty_like(h0)
        B.moe_ffn_residual_rmsnorm(h_ref, full, xn_ref, n, d, eps)
        h1, xn1 = h0.clone(), torch.empty_like(h0)
        layer.prefill_residual(x, h1, xn1, eps)
        st = torch.empty_like(full)
        B.moe_ffn_prefill_static(layer.handle, x, n, st)
        torch.cuda.synchronize()
    finally:
        layer.close()
    r, e = moe_close(ch.cpu().numpy(), O.moe_tokens(lw, x_np)["out"])
    assert torch.equal(h1, h_ref) and torch.equal(xn1, xn_ref)
    assert torch.equal(st, full)
    say(f"q4k chunked: rel_l2={r:.2e} max_elem={e:.2e}; stack form and no-alloc entry bit-identical")


def test_q4k_unsupported_entry_points():
    """The Q8_0 block-sum dump rejects a Q4_K handle before enqueueing
    anything; prefill and decode on the same handle work."""
    from mixture_experts_ffn_gemm_amd import binding as B
    from mixture_experts_ffn_gemm_amd.layer import MoeLayer
    shape, lw = mw.random_shape_case(40, fmt="q4_k", **Q4K_SHAPES[0])
    x = mw.make_tokens(940, 4, shape.d)
    layer = MoeLayer.from_workload(lw)
    try:
        xt = torch.from_numpy(x).cuda()
        dec = layer.decode(xt)
        layer.prefill(xt)
        ws = layer.workspace(4)
        sums = torch.empty((128, 128), dtype=torch.int32, device="cuda")
        ac = torch.empty((128, 32), dtype=torch.int8, device="cuda")
        info = torch.empty(4, dtype=torch.int32, device="cuda")
        with pytest.raises(B.MoeFfnError) as ei:
            B.moe_ffn_dbg_block_sums(layer.handle, ws, ws.numel(), 4, 0, 0, 0, 0, sums, ac, info)
        assert ei.value.status == B.MOE_FFN_UNSUPPORTED
        out = layer.prefill(xt)
        torch.cuda.synchronize()
        ref = O.moe_tokens(lw, x)["out"]
        moe_close(out.cpu().numpy(), ref)
        moe_close(dec.cpu().numpy(), ref)
    finally:
        layer.close()


def test_q4k_scale_overflow_is_rejected():
    """A super-block whose d * sc exceeds the binary16 range cannot be held by
    the kernels' binary16 scale pairs: weights create returns
    MOE_FFN_UNSUPPORTED (and allocates nothing that outlives the call)."""
    import dataclasses
    from mixture_experts_ffn_gemm_amd import binding as B
    from mixture_experts_ffn_gemm_amd.layer import MoeLayer
    shape, lw = mw.random_shape_case(40, fmt="q4_k", **Q4K_SHAPES[0])
    up = lw.up_q8.copy()
    up[3, 5, 0:2] = np.array([60000.0], np.float16).view(np.uint8)   # d of row 5, super-block 0
    up[3, 5, 4] = (up[3, 5, 4] & 0xC0) | 63                          # sc of sub-block 0 = 63
    with pytest.raises(B.MoeFfnError) as ei:
        MoeLayer.from_workload(dataclasses.replace(lw, up_q8=up))
    assert ei.value.status == B.MOE_FFN_UNSUPPORTED


@pytest.mark.slow
def test_q4k_olmoe_layer_full_size():
    """OLMoE-shaped layer at N=2048 on Q4_K experts, in the launch
    configuration the benchmark times: every token's routing bit-exact, every
    token's output and partials against the oracle."""
    lw = mw.workload_layer("olmoe_n2048_q4k")
    x = mw.workload_tokens("olmoe_n2048_q4k")
    say("olmoe_n2048_q4k: weights generated")
    g = run_gpu(lw, x)
    check_routing(lw, x, g)
    r, e = check_outputs(lw, x, g)
    say(f"olmoe_n2048_q4k: rel_l2={r:.2e} max_elem={e:.2e} on all 2048 tokens")


@pytest.mark.slow
def test_q4k_a3b_layer_full_size():
    """35B-A3B-shaped layer on Q4_K experts (E=256, shared expert, Zipf-skewed
    routing): every token against the oracle."""
    lw = mw.workload_layer("a3b_n512_q4k")
    x = mw.workload_tokens("a3b_n512_q4k")
    say("a3b_n512_q4k: weights generated")
    g = run_gpu(lw, x)
    check_routing(lw, x, g)
    r, e = check_outputs(lw, x, g)
    say(f"a3b_n512_q4k: rel_l2={r:.2e} max_elem={e:.2e} on all 512 tokens")


# ------------------------------------------------------------- Q3_K weights
# Q3_K rows (#388 "Key references": the Q3_K expert GEMM) expanded at load
# into the Q8_0 planes; prefill and decode against the oracle's Q3_K path.
Q3K_SHAPES = [
    dict(d=256, E=8, k=2, F=256),
    dict(d=512, E=16, k=3, F=256, Fs=512, zipf=1.1, norm=True),
    dict(d=256, E=70, k=4, F=512),
    dict(d=256, E=1, k=1, F=256, norm=True),
    dict(d=256, E=256, k=16, F=256, Fs=256),
]


@pytest.mark.parametrize("case", range(len(Q3K_SHAPES)))
@pytest.mark.parametrize("api,n", [("prefill", 1), ("prefill", 53), ("prefill", 300), ("decode", 1), ("decode", 8)])
def test_q3k_shapes(case, api, n):
    shape, lw = mw.random_shape_case(50 + case, fmt="q3_k", **Q3K_SHAPES[case])
    say(f"q3k case {case}: {Q3K_SHAPES[case]} {api} n={n}")
    x = mw.make_tokens(950 + case, n, shape.d)
    g = run_gpu(lw, x, api=api)
    check_routing(lw, x, g)
    r, e = check_outputs(lw, x, g)
    say(f"q3k case {case} {api} n={n}: rel_l2={r:.2e} max_elem={e:.2e}")


def test_q3k_extreme_products():
    """Sub-blocks with scale field 0 (multiplier -32) and codes -4: the
    product 128 whose negation, -128, is the one expanded code at the edge of
    int8; also multiplier +31 against codes 3 and -1.  Rows 0-63 of expert
    0's gate, up and down matrices get these sub-blocks in super-block 0."""
    import dataclasses
    shape, lw = mw.random_shape_case(50, fmt="q3_k", **Q3K_SHAPES[0])
    gate, up, down = lw.gate_q8.copy(), lw.up_q8.copy(), lw.down_q8.copy()
    for arr, rows in ((gate[0], slice(0, 64)), (up[0], slice(0, 64)), (down[0], slice(0, 64))):
        blk = arr[rows, 0:110]
        blk[:, 96:108] = 0            # every scale field 0 -> multiplier -32
        blk[:, 104:108] = 0
        blk[:, 32:96] = 0             # codes 0 ...
        blk[:, 0:32] = 0              # ... with the high bit clear: q = -4
        # sub-blocks 8..15 (second half): scale 63 (+31), codes alternating 3 and -1
        blk[:, 96:104] |= 0xF0
        blk[:, 104:108] |= 0xF0
        blk[:, 64:96] = 0xFF                     # code 3 in every group ...
        blk[:, 0:32:2] |= 0xF0                   # ... with the high bit set on even l (q = 3), clear on odd (q = -1)
        arr[rows, 0:110] = blk
    lw = dataclasses.replace(lw, gate_q8=gate, up_q8=up, down_q8=down)
    dq = O.q3k_dequant(gate[0, 0:1], shape.d)[0]
    d0 = float(np.frombuffer(gate[0, 0, 108:110].tobytes(), np.float16)[0])
    assert dq[0] == d0 * -32 * -4 and dq[128] == d0 * 31 * 3 and dq[129] == d0 * 31 * -1
    x = mw.make_tokens(960, 64, shape.d)
    g = run_gpu(lw, x)
    check_routing(lw, x, g)
    assert (g["topk_ids"] == 0).any(), "expert 0 must be selected"
    r, e = check_outputs(lw, x, g)
    say(f"q3k extreme products: rel_l2={r:.2e} max_elem={e:.2e}")


@pytest.mark.slow
def test_q3k_olmoe_layer_full_size():
    """OLMoE-shaped layer at N=2048 on Q3_K experts: every token's routing
    bit-exact, every token's output and partials against the oracle."""
    lw = mw.workload_layer("olmoe_n2048_q3k")
    x = mw.workload_tokens("olmoe_n2048_q3k")
    say("olmoe_n2048_q3k: weights generated")
    g = run_gpu(lw, x)
    check_routing(lw, x, g)
    r, e = check_outputs(lw, x, g)
    say(f"olmoe_n2048_q3k: rel_l2={r:.2e} max_elem={e:.2e} on all 2048 tokens")


# ------------------------------------------------------------- chunked prefill
@pytest.mark.parametrize("flags", [0, 1])
@pytest.mark.parametrize("case,n,chunk", [(0, 300, 128), (1, 300, 100), (1, 37, 512)])
def test_chunked_prefill(case, n, chunk, flags):
    """moe_ffn_prefill_chunked: consecutive chunks on one workspace sized for
    one chunk, in forward and serpentine tile order; every token's output
    against the oracle to the fp32 bar, and against the unchunked call's."""
    from mixture_experts_ffn_gemm_amd import binding as B
    from mixture_experts_ffn_gemm_amd.layer import MoeLayer
    shape, lw = mw.random_shape_case(20 + case, **MID_SHAPES[case])
    x = mw.make_tokens(750 + case, n, shape.d)
    layer = MoeLayer.from_workload(lw)
    try:
        xt = torch.from_numpy(x).cuda()
        full = layer.prefill(xt)
        ws = torch.empty(layer.workspace_size(min(chunk, n)), dtype=torch.uint8, device="cuda")
        out = torch.full((n, shape.d), float("nan"), dtype=torch.float32, device="cuda")
        B.moe_ffn_prefill_chunked(layer.handle, xt, n, chunk, flags, out, ws, ws.numel())
        torch.cuda.synchronize()
        got, ref_full = out.cpu().numpy(), full.cpu().numpy()
    finally:
        layer.close()
    ref = O.moe_tokens(lw, x)
    r, e = moe_close(got, ref["out"])
    moe_close(got, ref_full)
    say(f"chunked case {case} n={n} chunk={chunk} flags={flags}: rel_l2={r:.2e} max_elem={e:.2e}")


@pytest.mark.slow
def test_chunked_prefill_olmoe_ubatch512():
    """The OLMoE-shaped N=2048 layer as four ubatch-512 chunks in serpentine
    order: every token against the oracle."""
    from mixture_experts_ffn_gemm_amd import binding as B
    from mixture_experts_ffn_gemm_amd.layer import MoeLayer
    lw = mw.workload_layer("olmoe_n2048")
    x = mw.workload_tokens("olmoe_n2048")
    n, d = x.shape
    layer = MoeLayer.from_workload(lw)
    try:
        xt = torch.from_numpy(x).cuda()
        ws = torch.empty(layer.workspace_size(512), dtype=torch.uint8, device="cuda")
        out = torch.full((n, d), float("nan"), dtype=torch.float32, device="cuda")
        B.moe_ffn_prefill_chunked(layer.handle, xt, n, 512, B.CHUNK_SERPENTINE, out, ws, ws.numel())
        torch.cuda.synchronize()
        got = out.cpu().numpy()
    finally:
        layer.close()
    r, e = moe_close(got, O.moe_tokens(lw, x)["out"])
    say(f"olmoe_n2048 in 4 serpentine chunks of 512: rel_l2={r:.2e} max_elem={e:.2e} on all 2048 tokens")


# ------------------------------------------------------------- stack form
@pytest.mark.parametrize("case", [1, 2, 5])
def test_prefill_residual_matches_unfused(case):
    """moe_ffn_prefill_residual (combine fused with the residual add and the
    RMSNorm) against moe_ffn_prefill followed by moe_ffn_residual_rmsnorm: h
    and xn bit for bit, also with xn written over the layer's own input.
    Cases: top-1, shared expert with skewed routing, and E = 256 (routing in
    its own launch)."""
    from mixture_experts_ffn_gemm_amd import binding as B
    from mixture_experts_ffn_gemm_amd.layer import MoeLayer
    shape, lw = mw.random_shape_case(case, **SHAPES[case])
    n, d, eps = 53, shape.d, 1e-5
    dev = torch.device("cuda")
    say(f"prefill_residual case {case}: d={d} E={shape.n_experts} k={shape.top_k} n={n}")
    x = torch.from_numpy(mw.make_tokens(300 + case, n, d)).to(dev)
    h0 = torch.from_numpy(mw.make_tokens(400 + case, n, d)).to(dev)
    layer = MoeLayer.from_workload(lw)
    try:
        y = layer.prefill(x)
        h_ref, xn_ref = h0.clone(), torch.empty_like(h0)
        B.moe_ffn_residual_rmsnorm(h_ref, y, xn_ref, n, d, eps)
        h1, xn1 = h0.clone(), torch.full_like(h0, float("nan"))
        layer.prefill_residual(x, h1, xn1, eps)
        h2, x2 = h0.clone(), x.clone()
        layer.prefill_residual(x2, h2, x2, eps)
        torch.cuda.synchronize()
    finally:
        layer.close()
    assert torch.equal(h1, h_ref) and torch.equal(h2, h_ref)
    assert torch.equal(xn1, xn_ref) and torch.equal(x2, xn_ref)


def test_stack_graph_replays_match_eager():
    """Two layers in the stack form captured in one HIP graph (no memset
    nodes: the library issues kernels only) and replayed three times, with
    eager passes and host synchronisations in between; every replay gives the
    eager pass's residual stream and next input bit for bit."""
    from mixture_experts_ffn_gemm_amd.layer import MoeLayer
    shapes = [mw.random_shape_case(2, **SHAPES[2]), mw.random_shape_case(12, **SHAPES[2])]
    d, n, eps = SHAPES[2]["d"], 37, 1e-5
    dev = torch.device("cuda")
    layers = [MoeLayer.from_workload(lw) for _, lw in shapes]
    try:
        h_in = torch.from_numpy(mw.make_tokens(500, n, d)).to(dev)
        x_in = torch.from_numpy(mw.make_tokens(501, n, d)).to(dev)
        h, x = torch.empty_like(h_in), torch.empty_like(x_in)
        for lay in layers:
            lay.workspace(n)   # allocated before the capture

        def stack_pass(stream=None):
            h.copy_(h_in)
            x.copy_(x_in)
            for lay in layers:
                lay.prefill_residual(x, h, x, eps, stream=stream)

        stack_pass()
        torch.cuda.synchronize()
        h_eager, x_eager = h.clone(), x.clone()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                stack_pass(stream=torch.cuda.current_stream())
        torch.cuda.synchronize()
        for rep in range(3):
            h.zero_()
            x.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(h, h_eager) and torch.equal(x, x_eager), f"replay {rep} differs"
            say(f"graph replay {rep}: bit-identical to the eager pass")
            stack_pass()
            torch.cuda.synchronize()
            assert torch.equal(h, h_eager) and torch.equal(x, x_eager)
    finally:
        for lay in layers:
            lay.close()


def test_decode_graph_replays_match_eager():
    """A moe_ffn_decode call captured in a HIP graph and replayed three times,
    with eager calls and host synchronisations in between: every replay's
    output is the eager call's, bit for bit."""
    from mixture_experts_ffn_gemm_amd import binding as B
    from mixture_experts_ffn_gemm_amd.layer import MoeLayer
    shape, lw = mw.random_shape_case(2, **SHAPES[2])
    n = 3
    dev = torch.device("cuda")
    layer = MoeLayer.from_workload(lw)
    try:
        x = torch.from_numpy(mw.make_tokens(600, n, shape.d)).to(dev)
        out = torch.empty((n, shape.d), dtype=torch.float32, device=dev)
        ws = layer.workspace(n)
        B.moe_ffn_decode(layer.handle, x, n, out, ws, ws.numel(), None)
        torch.cuda.synchronize()
        ref = out.clone()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                B.moe_ffn_decode(layer.handle, x, n, out, ws, ws.numel(), None, torch.cuda.current_stream())
        torch.cuda.synchronize()
        for rep in range(3):
            out.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), f"replay {rep} differs"
            B.moe_ffn_decode(layer.handle, x, n, out, ws, ws.numel(), None)
            torch.cuda.synchronize()
            assert torch.equal(out, ref)
        say("decode graph: 3 replays bit-identical to the eager call")
    finally:
        layer.close()


# Decode: the same shapes through moe_ffn_decode, plus one whose K spans
# several staged activation passes of the decode matvecs (d and F above 2048,
# both ragged against the 128-value k-step) and whose router runs three
# passes of 2048 j (the last one a single block).
DECODE_SHAPES = SHAPES + [dict(d=4160, E=8, k=2, F=2080, Fs=96)]


@pytest.mark.parametrize("case", range(len(DECODE_SHAPES)))
@pytest.mark.parametrize("n", [1, 3, 8])
def test_decode_shapes(case, n):
    shape, lw = mw.random_shape_case(case, **DECODE_SHAPES[case])
    x = mw.make_tokens(300 + case, n, shape.d)
    g = run_gpu(lw, x, api="decode")
    check_routing(lw, x, g)
    check_outputs(lw, x, g)


def test_decode_repeat_is_bitwise_identical():
    lw = mw.workload_layer("tiny")
    x = mw.make_tokens(2, 8, 128)
    a = run_gpu(lw, x, api="decode")
    b = run_gpu(lw, x, api="decode")
    for key in ("out", "partial", "topk_w", "exp_tok_i", "xq", "xs"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("case", range(len(DECODE_SHAPES)))
def test_decode_single_token_out_is_the_combine_of_its_partials(case):
    """One token with at most 9 slots (k plus the shared expert) runs the down
    matvec and the ordered combine in one launch.  Its output must equal, bit
    for bit, the standalone combine stage applied to the partials, weights and
    shared gate the same call reports (the same fp32 chain over the slots);
    shapes with more slots take the two-launch path, which must satisfy the
    same identity."""
    from mixture_experts_ffn_gemm_amd import binding as B
    shape, lw = mw.random_shape_case(case, **DECODE_SHAPES[case])
    s = lw.shape
    say(f"decode n=1 combine identity case {case}: d={s.d} E={s.n_experts} k={s.top_k} shared={bool(s.shared_ffn)}")
    x = mw.make_tokens(700 + case, 1, shape.d)
    g = run_gpu(lw, x, api="decode")
    check_routing(lw, x, g)
    check_outputs(lw, x, g)
    out = torch.full((1, s.d), float("nan"), dtype=torch.float32, device="cuda")
    B.moe_ffn_combine(torch.from_numpy(g["partial"]).cuda(), torch.from_numpy(g["topk_w"]).cuda(),
                      torch.from_numpy(g["shared_gate"]).cuda() if s.shared_ffn else None,
                      1, s.top_k, s.d, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), g["out"])


def test_empty_batch_is_a_noop():
    from mixture_experts_ffn_gemm_amd.layer import MoeLayer
    lw = mw.workload_layer("tiny")
    layer = MoeLayer.from_workload(lw)
    out = torch.full((1, 128), 3.0, device="cuda")
    x = torch.zeros((0, 128), device="cuda")
    layer.prefill(x, out=out[:0])
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    layer.close()


def test_repeat_runs_are_bitwise_identical():
    lw = mw.workload_layer("tiny")
    x = mw.make_tokens(1, 300, 128)
    a = run_gpu(lw, x)
    b = run_gpu(lw, x)
    for key in ("out", "partial", "topk_w", "exp_tok_i"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.slow
def test_olmoe_layer_full_size():
    """OLMoE-shaped layer at N=2048, in the launch configuration the benchmark
    times: routing, CSR and activation codes of every token bit-exact, and the
    output and the unweighted partials of every token against the oracle."""
    lw = mw.workload_layer("olmoe_n2048")
    x = mw.workload_tokens("olmoe_n2048")
    say("olmoe_n2048: weights generated")
    g = run_gpu(lw, x)
    check_routing(lw, x, g)
    say("olmoe_n2048: routing bit-exact")
    r, e = check_outputs(lw, x, g)
    say(f"olmoe_n2048: rel_l2={r:.2e} max_elem={e:.2e} on all 2048 tokens")
    counts = np.diff(g["exp_start"])
    assert counts.sum() == 2048 * 8 and counts.min() > 0


@pytest.mark.slow
def test_repeated_calls_are_bitwise_identical():
    """Four prefill calls on one OLMoE-shaped N=2048 batch give bitwise
    identical routing weights, CSR and outputs.  Every stage is deterministic
    by construction, so any difference is a synchronisation bug (a read of an
    LDS buffer before its copy landed): the softmax weights of an affected
    token change even where its top-k ids do not."""
    lw = mw.workload_layer("olmoe_n2048")
    x = mw.workload_tokens("olmoe_n2048")
    first = run_gpu(lw, x, keep=True)
    layer = first.pop("layer")
    try:
        for i in range(3):
            g = run_gpu(lw, x, layer=layer)
            for key in ("topk_ids", "topk_w", "exp_start", "exp_tok_i", "xq", "xs", "out"):
                assert np.array_equal(g[key].view(np.uint8), first[key].view(np.uint8)), f"call {i + 2}: {key} differs"
    finally:
        layer.close()
    say("olmoe_n2048: 4 calls bitwise identical")


@pytest.mark.slow
def test_a3b_layer_full_size():
    """35B-A3B-shaped layer: E=256, shared expert + gate, Zipf-skewed routing."""
    lw = mw.workload_layer("a3b_n512")
    x = mw.workload_tokens("a3b_n512")
    g = run_gpu(lw, x)
    check_routing(lw, x, g)
    counts = np.diff(g["exp_start"][:257])
    say(f"a3b_n512: experts touched {int((counts > 0).sum())}, max load {int(counts.max())}")
    r, e = check_outputs(lw, x, g)
    say(f"a3b_n512: rel_l2={r:.2e} max_elem={e:.2e} on all 512 tokens")


@pytest.mark.slow
@pytest.mark.parametrize("n", [1, 8])
def test_decode(n):
    lw = mw.workload_layer("olmoe_decode1")
    x = mw.make_tokens(5, n, 2048)
    g = run_gpu(lw, x, api="decode")
    check_routing(lw, x, g)
    check_outputs(lw, x, g)


@pytest.mark.slow
def test_n4096_prefill_all_tokens():
    """N=4096 prefill on the OLMoE shape: every token's routing bit-exact and
    every token's output and partials against the oracle."""
    lw = mw.workload_layer("olmoe_n4096")
    x = mw.workload_tokens("olmoe_n4096")
    g = run_gpu(lw, x)
    check_routing(lw, x, g)
    r, e = check_outputs(lw, x, g)
    say(f"olmoe_n4096: rel_l2={r:.2e} max_elem={e:.2e} on all 4096 tokens")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_olmoe_stack16():
    """The 16-layer OLMoE-shaped stack in the form the benchmark times: each
    layer is one moe_ffn_prefill_residual call, h += MoE_l(xn) and
    xn <- RMSNorm(h) written over the layer's own input, independent seeded
    weights per layer.  Every layer is checked against the oracle fed the
    GPU's own normalised input: routing of all 2048 tokens bit-exact; the
    residual update is exactly h + y, where y is the fp32 ordered combine of
    the layer's reported partials and weights (the fused kernel's combine);
    y of every token within the fp32 bar of the oracle's layer output; and
    the next input against the oracle's RMSNorm of the updated h."""
    from mixture_experts_ffn_gemm_amd import binding as B
    from mixture_experts_ffn_gemm_amd.layer import MoeLayer
    wl = mw.WORKLOADS["olmoe_stack16"]
    s = wl.shape
    n, d, eps = wl.n_tokens, s.d, 1e-5
    dev = torch.device("cuda")
    h = torch.from_numpy(mw.workload_tokens("olmoe_stack16")).to(dev)
    xn = torch.empty_like(h)
    B.moe_ffn_residual_rmsnorm(h, None, xn, n, d, eps)
    for layer_idx in range(wl.n_layers):
        lw = mw.workload_layer("olmoe_stack16", layer=layer_idx)
        layer = MoeLayer.from_workload(lw)
        try:
            ids = torch.full((n, s.top_k), -7, dtype=torch.int32, device=dev)
            tw = torch.full((n, s.top_k), float("nan"), dtype=torch.float32, device=dev)
            part = torch.full((n, s.top_k, d), float("nan"), dtype=torch.float32, device=dev)
            r = B.make_routing(topk_ids=ids, topk_w=tw, partial=part)
            torch.cuda.synchronize()
            xn_np = xn.cpu().numpy()
            h_before = h.cpu().numpy()
            layer.prefill_residual(xn, h, xn, eps, routing=r)
            torch.cuda.synchronize()
            h_np, xn_next = h.cpu().numpy(), xn.cpu().numpy()
            ids_np, tw_np, part_np = ids.cpu().numpy(), tw.cpu().numpy(), part.cpu().numpy()
        finally:
            layer.close()
        o = O.routing(lw, xn_np)
        assert np.array_equal(ids_np, o["ids"]), f"layer {layer_idx}: top-k ids differ"
        y = O.combine_f32(part_np, tw_np)
        assert np.array_equal(h_np, h_before + y), f"layer {layer_idx}: residual update is not h + y"
        ref = O.moe_tokens(lw, xn_np)
        rel, emax = moe_close(y, ref["out"])
        np.testing.assert_allclose(xn_next, O.rmsnorm(h_np, eps), rtol=2e-6, atol=1e-6)
        say(f"olmoe_stack16 layer {layer_idx}: routing bit-exact, rel_l2={rel:.2e} max_elem={emax:.2e} "
            f"(all {n} tokens)")
