"""Pins of the CPU oracle against facts fixed outside it: hand-derived golden
cases, library routines (numpy / scipy), closed forms, error bounds and
brute force.  A plausible slip anywhere in the oracle (a dropped term, a
wrong sign, index or order, a transposed operand) fails one of these.

The oracle follows the SharpInference issue pages: #388 "Remaining levers"
item 1 (router, top-k, CSR), #408 "Hypothesis" (norm_topk_prob, int8 block
activations), #406 "The work" item 2 (grouped expert GEMM) and #129 "Scope"
(ordered weighted combine).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import moe_workloads as mw
from oracle import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ fp16
def test_half_conversion_matches_numpy():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-9, 6, 20000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, np.inf, -np.inf,
                  6.1035156e-05, 6.0e-8, 2.9e-8, 3.0e-8, 5.96e-8, 1e-9,
                  1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0], np.float32)]).astype(np.float32)
    ours = O.float_to_half(vals)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    back = O.half_to_float(allh)
    refb = allh.view(np.float16).astype(np.float32)
    finite = np.isfinite(refb)
    assert np.array_equal(back[finite].view(np.uint32), refb[finite].view(np.uint32))
    assert np.all(np.isnan(back[np.isnan(refb)]))


# ---------------------------------------------------------------- router
def test_router_golden_cases():
    g = load("router_topk.json")
    for c in g["cases"]:
        x = np.array([c["x"]], np.float32)
        w = np.array(c["w"], np.float32)
        l = O.router_logits(x, w)
        if "expected_logits" in c:
            assert np.array_equal(l[0], np.array(c["expected_logits"], np.float32)), c["name"]
        if "expected_ids" in c:
            ids = O.topk(l, c["k"])
            assert ids[0].tolist() == c["expected_ids"], c["name"]


def test_router_single_product_is_rounded_once():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 1)).astype(np.float32)
    w = rng.standard_normal((5, 1)).astype(np.float32)
    l = O.router_logits(x, w)
    assert np.array_equal(l, (x * w[:, 0][None, :]).astype(np.float32))


def test_router_error_bound_vs_fp64():
    rng = np.random.default_rng(3)
    n, d, E = 32, 512, 16
    x = rng.standard_normal((n, d)).astype(np.float32)
    w = (rng.standard_normal((E, d)) * 0.02).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    l = O.router_logits(x, w, b).astype(np.float64)
    exact = x.astype(np.float64) @ w.astype(np.float64).T + b.astype(np.float64)
    u = 2.0 ** -24
    gam = (d + 1) * u / (1 - (d + 1) * u)
    bound = gam * (np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T + np.abs(b)) + 1e-30
    assert np.all(np.abs(l - exact) <= bound)
    # a one-hot row picks one column exactly, bias added in fp32
    oh = np.zeros((1, d), np.float32)
    oh[0, 7] = 1.0
    l1 = O.router_logits(oh, w, b)
    assert np.array_equal(l1[0], (w[:, 7] + b).astype(np.float32))


# ----------------------------------------------------------------- top-k
def test_topk_brute_force_and_stable_argsort():
    rng = np.random.default_rng(4)
    for trial in range(30):
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, E + 1))
        # coarse values so that ties are frequent
        l = rng.integers(-3, 4, size=(20, E)).astype(np.float32) * np.float32(0.5)
        ids = O.topk(l, k)
        ref = np.argsort(-l, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref)
        for t in range(l.shape[0]):
            sel = set(ids[t].tolist())
            assert len(sel) == k
            for s in range(k):
                a = ids[t, s]
                for b in range(E):
                    if b in sel:
                        continue
                    assert l[t, a] > l[t, b] or (l[t, a] == l[t, b] and a < b)
                if s:
                    p = ids[t, s - 1]
                    assert l[t, p] > l[t, a] or (l[t, p] == l[t, a] and p < a)


def test_all_zero_router_gives_ids_in_order_and_uniform_weights():
    x = np.random.default_rng(5).standard_normal((6, 64)).astype(np.float32)
    w = np.zeros((16, 64), np.float32)
    l = O.router_logits(x, w)
    ids = O.topk(l, 4)
    assert np.array_equal(ids, np.tile(np.arange(4, dtype=np.int32), (6, 1)))
    rw = O.route_weights(l, ids, False)
    assert np.all(rw == 1.0 / 16)
    rn = O.route_weights(l, ids, True)
    assert np.all(rn == 0.25)


# --------------------------------------------------------------- weights
def test_route_weights_match_scipy_softmax():
    rng = np.random.default_rng(6)
    l = (rng.standard_normal((50, 64)) * 3).astype(np.float32)
    ids = O.topk(l, 8)
    p = scipy.special.softmax(l.astype(np.float64), axis=1)
    w = O.route_weights(l, ids, False)
    ref = np.take_along_axis(p, ids, axis=1)
    np.testing.assert_allclose(w, ref, rtol=1e-13, atol=0)
    assert np.all(np.diff(w, axis=1) <= 0)   # slots are rank ordered
    wn = O.route_weights(l, ids, True)
    np.testing.assert_allclose(wn, ref / ref.sum(1, keepdims=True), rtol=1e-13)
    np.testing.assert_allclose(wn.sum(1), 1.0, rtol=1e-14)
    allw = O.route_weights(l, O.topk(l, 64), False)
    np.testing.assert_allclose(allw.sum(1), 1.0, rtol=1e-14)


def test_shared_gate_matches_expit():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((10, 256)).astype(np.float32)
    g = (rng.standard_normal(256) * 0.02).astype(np.float32)
    gs = O.shared_gate(x, g)
    ref = scipy.special.expit(x.astype(np.float64) @ g.astype(np.float64))
    np.testing.assert_allclose(gs, ref, rtol=1e-13)


# ------------------------------------------------------------------- CSR
def test_csr_golden():
    for c in load("csr_small.json")["cases"]:
        start, ti, tk = O.csr(np.array(c["ids"], np.int32), c["n_experts"], c["has_shared"])
        assert start.tolist() == c["expected_exp_start"]
        assert ti.tolist() == c["expected_tok_i"]
        assert tk.tolist() == c["expected_tok_k"]


@pytest.mark.parametrize("shared", [False, True])
def test_csr_matches_stable_argsort_and_invariants(shared):
    rng = np.random.default_rng(8)
    N, E, k = 300, 37, 5
    l = rng.standard_normal((N, E)).astype(np.float32)
    ids = O.topk(l, k)
    start, ti, tk = O.csr(ids, E, shared)
    order = np.argsort(ids.ravel(), kind="stable")
    P = N * k
    assert np.array_equal(ti[:P], order // k)
    assert np.array_equal(tk[:P], order % k)
    cnt = np.bincount(ids.ravel(), minlength=E)
    assert np.array_equal(start[:E + 1], np.concatenate([[0], np.cumsum(cnt)]))
    assert start[E] == P
    seen = set()
    for e in range(E):
        rows = range(start[e], start[e + 1])
        toks = [ti[p] for p in rows]
        assert toks == sorted(toks) and len(set(toks)) == len(toks)
        for p in rows:
            assert ids[ti[p], tk[p]] == e
            seen.add((ti[p], tk[p]))
    assert len(seen) == P
    if shared:
        assert start[E + 1] == P + N
        assert np.array_equal(ti[P:], np.arange(N)) and np.all(tk[P:] == k)


# ------------------------------------------------------------- quantiser
def test_quantiser_golden():
    for c in load("quantize_blocks.json")["cases"]:
        v = np.full(32, c["pad"], np.float32)
        v[:len(c["x_head"])] = c["x_head"]
        q, s = O.quantize_q8(v)
        assert q[:len(c["expected_codes_head"])].tolist() == c["expected_codes_head"], c["name"]
        assert int(s[0]) == c["expected_scale_bits"], c["name"]
        if not c["x_head"]:
            assert np.all(q == 0)


def test_quantiser_bounds():
    rng = np.random.default_rng(9)
    v = (rng.standard_normal((40, 256)) * np.exp(rng.standard_normal((40, 1)) * 3)).astype(np.float32)
    v[3, 32:64] = 0.0
    q, s = O.quantize_q8(v)
    blk = v.reshape(40, 8, 32).astype(np.float64)
    qb = q.reshape(40, 8, 32).astype(np.float64)
    amax = np.abs(blk).max(2)
    nz = amax > 0
    # code is within 1/2 (+ fp32 rounding slack) of x*127/amax
    ideal = blk * (127.0 / np.where(nz, amax, 1.0))[:, :, None]
    assert np.all(np.abs(qb - ideal)[nz] <= 0.5 + 1e-4)
    assert np.all(np.abs(qb) <= 127)
    # the largest magnitude maps to +-127 with its sign
    idx = np.abs(blk).argmax(2)
    top = np.take_along_axis(qb, idx[:, :, None], 2)[:, :, 0]
    sgn = np.sign(np.take_along_axis(blk, idx[:, :, None], 2)[:, :, 0])
    assert np.all((top == 127 * sgn)[nz])
    # stored scale is binary16 of the fp32 quotient (numpy's conversion)
    ref = (amax.astype(np.float32) / np.float32(127)).astype(np.float16).view(np.uint16)
    assert np.array_equal(s.reshape(40, 8), np.where(nz, ref, 0))
    assert np.all(q.reshape(40, 8, 32)[3, 1] == 0) and s.reshape(40, 8)[3, 1] == 0


# ----------------------------------------------------------------- Q8 dot
def _dequant_rows(b, cols):
    codes, sc = mw.unpack_q8_0(b, cols)
    return codes.astype(np.float64) * np.repeat(sc.astype(np.float64), 32, axis=1)


def test_q8_dot_matches_numpy_dequantised_dot():
    rng = np.random.default_rng(10)
    d = 512
    x = rng.standard_normal((8, d)).astype(np.float32)
    xq, xs = O.quantize_q8(x)
    W = mw.pack_q8_0((rng.standard_normal((16, d)) * 0.02).astype(np.float32))
    Wd = _dequant_rows(W, d)
    xd = xq.astype(np.float64) * np.repeat(xs.view(np.float16).astype(np.float64), 32, axis=1)
    for t in range(8):
        for r in range(16):
            got = O.q8_dot(xq[t], xs[t], W[r])
            ref = float(xd[t] @ Wd[r])
            assert abs(got - ref) <= 1e-12 * (np.abs(xd[t]) @ np.abs(Wd[r]))


def test_q8_dot_block_sums_are_exact_integers():
    rng = np.random.default_rng(11)
    d = 256
    qa = rng.integers(-127, 128, d).astype(np.int8)
    qw = rng.integers(-127, 128, (3, d)).astype(np.int8)
    one = np.float16(1.0).view(np.uint16)
    sa = np.full(d // 32, one, np.uint16)
    rows = np.empty((3, d // 32, 34), np.uint8)
    rows[:, :, 0:2] = np.full((3, d // 32), one, np.uint16).view(np.uint8).reshape(3, d // 32, 2)
    rows[:, :, 2:] = qw.view(np.uint8).reshape(3, d // 32, 32)
    for r in range(3):
        got = O.q8_dot(qa, sa, rows[r].reshape(-1))
        assert got == float(int(qa.astype(np.int64) @ qw[r].astype(np.int64)))
    # block scales multiply their own block only
    sa2 = sa.copy()
    sa2[2] = np.float16(2.0).view(np.uint16)
    got = O.q8_dot(qa, sa2, rows[0].reshape(-1))
    prod = qa.astype(np.int64) * qw[0].astype(np.int64)
    assert got == float(prod.sum() + prod[64:96].sum())


def test_q8_block_sums_match_int64_matmul():
    """The integer core: per-block int32 sums equal numpy's int64 product of
    the unpacked int8 codes, block by block; extreme codes (+-127 everywhere,
    the largest |sum| a block can reach) stay exact."""
    rng = np.random.default_rng(16)
    d, m, n = 256, 7, 5
    W = mw.pack_q8_0((rng.standard_normal((n, d)) * 0.02).astype(np.float32))
    codes, _ = mw.unpack_q8_0(W, d)
    qa = rng.integers(-127, 128, (m, d)).astype(np.int8)
    for kb in range(d // 32):
        got = O.q8_block_sums(qa[:, 32 * kb:32 * kb + 32], W, kb)
        ref = qa[:, 32 * kb:32 * kb + 32].astype(np.int64) @ codes[:, 32 * kb:32 * kb + 32].astype(np.int64).T
        assert np.array_equal(got, ref)
    # block kb reads its own 32 codes only: an extreme block next to zeros
    Wx = W.copy().reshape(n, d // 32, 34)
    Wx[:, :, 2:] = 0
    Wx[:, 3, 2:] = np.int8(-127).view(np.uint8)
    Wx = Wx.reshape(n, -1)
    qx = np.full((1, 32), 127, np.int8)
    assert np.all(O.q8_block_sums(qx, Wx, 3) == -127 * 127 * 32)
    assert np.all(O.q8_block_sums(qx, Wx, 2) == 0)
    # the scaled Q8 dot is the sum of these integers times the block scales
    xs = np.full(d // 32, np.float16(1.0).view(np.uint16), np.uint16)
    tot = sum(int(O.q8_block_sums(qa[0:1, 32 * kb:32 * kb + 32], W[0:1], kb)[0, 0]) *
              float(np.float16(W[0].reshape(-1, 34)[kb, :2].view(np.float16)[0]))
              for kb in range(d // 32))
    assert abs(O.q8_dot(qa[0], xs, W[0]) - tot) <= 1e-12 * abs(tot) + 1e-15


# ---------------------------------------------------------------- expert
def test_expert_ffn_against_numpy():
    rng = np.random.default_rng(12)
    d, F = 256, 128
    x = rng.standard_normal((1, d)).astype(np.float32)
    xq, xs = O.quantize_q8(x)
    G = mw.pack_q8_0((rng.standard_normal((F, d)) * 0.02).astype(np.float32))
    U = mw.pack_q8_0((rng.standard_normal((F, d)) * 0.02).astype(np.float32))
    D = mw.pack_q8_0((rng.standard_normal((d, F)) * 0.02).astype(np.float32))
    y, hq, hs, h = O.expert_ffn(d, F, xq[0], xs[0], G, U, D)
    xd = xq[0].astype(np.float64) * np.repeat(xs[0].view(np.float16).astype(np.float64), 32)
    g = _dequant_rows(G, d) @ xd
    u = _dequant_rows(U, d) @ xd
    href = g * scipy.special.expit(g) * u          # silu(gate) * up
    np.testing.assert_allclose(h, href, rtol=1e-12, atol=1e-15)
    # gate and up are not interchangeable
    assert np.max(np.abs(h - u * scipy.special.expit(u) * g)) > 1e-3 * np.max(np.abs(h))
    hd = hq.astype(np.float64) * np.repeat(hs.view(np.float16).astype(np.float64), 32)
    amax = np.abs(h.astype(np.float32)).reshape(-1, 32).max(1).astype(np.float64)
    step = np.repeat(amax / 127.0, 32)
    # requantisation error: half a step plus the binary16 rounding of the scale
    assert np.all(np.abs(hd - h) <= 0.5 * step * (1 + 1e-3) + 127 * np.abs(
        np.repeat(hs.view(np.float16).astype(np.float64), 32) - step) + 1e-12)
    yref = _dequant_rows(D, F) @ hd                  # down rows are [d][F]
    np.testing.assert_allclose(y, yref, rtol=1e-11, atol=1e-14)


# ----------------------------------------------------------------- layer
def test_single_expert_layer_is_the_dense_ffn():
    shape, lw = mw.random_shape_case(1, d=128, E=1, k=1, F=64, norm=True)
    x = mw.make_tokens(101, 5, 128)
    r = O.moe_tokens(lw, x, want_partial=True)
    assert np.all(r["ids"] == 0) and np.all(r["w"] == 1.0)
    xq, xs = O.quantize_q8(x)
    for t in range(5):
        y, *_ = O.expert_ffn(128, 64, xq[t], xs[t], lw.gate_q8[0], lw.up_q8[0], lw.down_q8[0])
        assert np.array_equal(r["out"][t], y)


def test_identical_experts_scale_by_weight_sum():
    shape, lw = mw.random_shape_case(2, d=128, E=6, k=3, F=64)
    for arr in (lw.gate_q8, lw.up_q8, lw.down_q8):
        arr[:] = arr[0]
    x = mw.make_tokens(102, 7, 128)
    r = O.moe_tokens(lw, x, want_partial=True)
    y = r["partial"][:, 0, :]
    np.testing.assert_allclose(r["out"], r["w"].sum(1, keepdims=True) * y, rtol=1e-13, atol=1e-18)
    for s in range(3):
        assert np.array_equal(r["partial"][:, s, :], y)


def test_output_is_weighted_sum_of_partials_plus_gated_shared():
    shape, lw = mw.random_shape_case(3, d=128, E=8, k=2, F=64, Fs=96, norm=True, zipf=1.1)
    x = mw.make_tokens(103, 9, 128)
    r = O.moe_tokens(lw, x, want_partial=True)
    P = r["partial"]
    ref = np.einsum("ts,tsd->td", r["w"], P[:, :2]) + r["gs"][:, None] * P[:, 2]
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(r["w"].sum(1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(r["gs"], scipy.special.expit(
        x.astype(np.float64) @ lw.sh_gate_vec.astype(np.float64)), rtol=1e-13)
    # the shared row is the shared expert evaluated on the token
    xq, xs = O.quantize_q8(x)
    y, *_ = O.expert_ffn(128, 96, xq[4], xs[4], lw.sh_gate_q8, lw.sh_up_q8, lw.sh_down_q8)
    assert np.array_equal(P[4, 2], y)
    # a routed slot is the chosen expert evaluated on the token
    e = r["ids"][4, 1]
    y, *_ = O.expert_ffn(128, 64, xq[4], xs[4], lw.gate_q8[e], lw.up_q8[e], lw.down_q8[e])
    assert np.array_equal(P[4, 1], y)


@pytest.mark.parametrize("norm", [False, True])
def test_layer_routing_follows_the_biased_logits(norm):
    """The whole-layer loop routes each token by its biased fp32 logits: the
    ids it reports are numpy's stable argsort of those logits (largest first,
    lower id on ties) and its weights are scipy's softmax over all experts,
    renormalised over the picks when norm_topk_prob is set.  Zipf-biased
    router, so that dropping the bias changes the selection."""
    shape, lw = mw.random_shape_case(5, d=128, E=32, k=4, F=32, Fs=32, norm=norm, zipf=1.1)
    x = mw.make_tokens(105, 40, 128)
    r = O.moe_tokens(lw, x)
    logits = O.router_logits(x, lw.router_w, lw.router_bias)
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :4]
    assert np.array_equal(r["ids"], ids)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    w = np.take_along_axis(p, ids, axis=1)
    if norm:
        w = w / w.sum(1, keepdims=True)
    np.testing.assert_allclose(r["w"], w, rtol=1e-13, atol=0)
    # the bias is load-bearing for this workload: without it the picks differ
    unbiased = O.router_logits(x, lw.router_w)
    assert not np.array_equal(np.argsort(-unbiased, axis=1, kind="stable")[:, :4], ids)
    # the grouped evaluation routes the same way: its output is the per-token one
    assert np.array_equal(O.moe_grouped(lw, x), r["out"])


@pytest.mark.parametrize("case", [
    dict(d=128, E=8, k=2, F=256),
    dict(d=64, E=5, k=5, F=32, norm=True),
    dict(d=96, E=16, k=3, F=64, Fs=32, zipf=1.1),
])
def test_grouped_equals_per_token_bitwise(case):
    shape, lw = mw.random_shape_case(4, **case)
    x = mw.make_tokens(104, 23, case["d"])
    a = O.moe_tokens(lw, x)["out"]
    b = O.moe_grouped(lw, x)
    assert np.array_equal(a, b)
    sub = O.moe_tokens(lw, x, tokens=[22, 3, 3, 0])["out"]
    assert np.array_equal(sub, a[[22, 3, 3, 0]])


def test_tiny_workload_close_to_unquantised_dense_definition():
    """Informational bound: the int8 method stays near the exact fp64 FFN on
    dequantised weights and unquantised activations."""
    lw = mw.workload_layer("tiny")
    x = mw.workload_tokens("tiny")
    r = O.moe_tokens(lw, x)
    s = lw.shape
    ref = np.zeros_like(r["out"])
    for t in range(x.shape[0]):
        for k in range(s.top_k):
            e = r["ids"][t, k]
            g = _dequant_rows(lw.gate_q8[e], s.d) @ x[t].astype(np.float64)
            u = _dequant_rows(lw.up_q8[e], s.d) @ x[t].astype(np.float64)
            h = g * scipy.special.expit(g) * u
            ref[t] += r["w"][t, k] * (_dequant_rows(lw.down_q8[e], s.ffn) @ h)
    rel = np.linalg.norm(r["out"] - ref) / np.linalg.norm(ref)
    assert rel < 2e-2


# --------------------------------------------------------------- combine
def test_combine_golden():
    for c in load("combine_slot_order.json")["cases"]:
        k = len(c["weights"])
        P = np.array(c["partials"], np.float32)[None]
        w = np.array([c["weights"]], np.float32)
        gs = None
        if "shared_gate" in c:
            gs = np.array([c["shared_gate"]], np.float32)
        out = O.combine_f32(P, w, gs)
        assert np.array_equal(out[0], np.array(c["expected"], np.float32)), c["name"]
        assert P.shape[1] == k + (1 if gs is not None else 0)


def test_combine_single_slot_is_identity_and_exact_products_match_numpy():
    rng = np.random.default_rng(13)
    P = rng.standard_normal((7, 1, 64)).astype(np.float32)
    out = O.combine_f32(P, np.ones((7, 1), np.float32))
    assert np.array_equal(out, P[:, 0])
    # power-of-two weights make each product exact, so the fused chain equals
    # numpy's sequential float32 sum in slot order
    P = rng.standard_normal((7, 5, 64)).astype(np.float32)
    w = (2.0 ** rng.integers(-4, 3, (7, 5))).astype(np.float32)
    out = O.combine_f32(P, w)
    acc = np.zeros((7, 64), np.float32)
    for s in range(5):
        acc = (acc + w[:, s:s + 1] * P[:, s]).astype(np.float32)
    assert np.array_equal(out, acc)


def test_combine_fused_step_exact_rational():
    # o = fma(a, b, c) must equal the exactly rounded a*b + c
    rng = np.random.default_rng(14)
    a = rng.standard_normal(200).astype(np.float32)
    b = rng.standard_normal(200).astype(np.float32)
    c = rng.standard_normal(200).astype(np.float32)
    P = np.stack([np.ones(200, np.float32) * 0 + c, b], 1)[:, :, None]   # [n][2][1]
    w = np.stack([np.ones(200, np.float32), a], 1)
    out = O.combine_f32(P, w)[:, 0]
    for i in range(200):
        exact = Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i]))
        lo = np.float32(float(exact))
        # correct rounding of the exact value: no float32 lies strictly between
        cands = [np.nextafter(lo, np.float32(-np.inf)), lo, np.nextafter(lo, np.float32(np.inf))]
        best = min(cands, key=lambda v: (abs(Fraction(float(v)) - exact),
                                         int(np.float32(v).view(np.uint32)) & 1))
        assert out[i] == best


# ---------------------------------------------------------------- rmsnorm
def test_rmsnorm_closed_forms():
    x = np.array([[3.0] * 64, [-0.5] * 64], np.float32)
    out = O.rmsnorm(x, 1e-5)
    for r, c in enumerate([3.0, -0.5]):
        np.testing.assert_allclose(out[r], np.sign(c) / np.sqrt(1 + 1e-5 / c ** 2), rtol=1e-15)
    rng = np.random.default_rng(15)
    x = rng.standard_normal((4, 256)).astype(np.float32) * 7
    out = O.rmsnorm(x, 1e-5)
    ms = (x.astype(np.float64) ** 2).mean(1)
    np.testing.assert_allclose((out ** 2).mean(1), ms / (ms + 1e-5), rtol=1e-13)
    np.testing.assert_allclose(out / x, np.broadcast_to((1 / np.sqrt(ms + 1e-5))[:, None], x.shape),
                               rtol=1e-13)


# ------------------------------------------------------------------- Q4_K
# Q4_K weight rows (#406 "References" names Q4_K MMQ next to Q8_0): the byte
# layout is pinned by the packer's own field choice (numpy), the dot product
# by an integer decomposition of the same sum, the expert by a numpy matmul
# of dequantised rows.

def _q4k_matrix(rng, rows, cols):
    """Weights with the awkward cases: an all-zero sub-block, an all-positive
    and an all-negative one, and rows of very different magnitude."""
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    w[0, 0:32] = 0.0
    w[0, 32:64] = np.abs(w[0, 32:64]) + 0.01
    w[0, 64:96] = -np.abs(w[0, 64:96]) - 0.01
    if rows > 2:
        w[2] *= np.float32(40.0)
    return w


def _q4k_represented(w):
    """The values the Q4_K fields chosen for w stand for, d*sc*q - dmin*m in
    fp64 (from the fields, not from the packed bytes)."""
    d16, dmin16, sc, m, q = mw.q4k_parts(w)
    d = np.repeat(d16.astype(np.float64), 8, axis=1)
    dmin = np.repeat(dmin16.astype(np.float64), 8, axis=1)
    return np.repeat(d * sc, 32, axis=1) * q.astype(np.float64) - np.repeat(dmin * m, 32, axis=1)


def test_q4k_dequant_matches_the_packed_fields():
    rng = np.random.default_rng(40)
    w = _q4k_matrix(rng, 5, 768)
    b = mw.pack_q4_k(w)
    assert b.shape == (5, 3 * 144)
    dq = O.q4k_dequant(b, 768)
    assert np.array_equal(dq, _q4k_represented(w))
    # the represented values stay within a few code steps of the draw
    d16, dmin16, sc, m, q = mw.q4k_parts(w)
    step = np.repeat(np.repeat(d16.astype(np.float64), 8, axis=1) * sc, 32, axis=1)
    slack = np.repeat(np.repeat(dmin16.astype(np.float64), 8, axis=1), 32, axis=1)
    assert np.all(np.abs(dq - w) <= step + slack + 1e-9)
    assert np.all(dq[0, 0:32] == 0.0)


def test_q4k_layout_of_one_super_block_by_hand():
    """One super-block written byte by byte: d = 1, dmin = 0.5, sub-block j
    scale j+1 and min 2j (six-bit fields split as the format packs them), code
    i of sub-block j equal to (i + j) % 16."""
    blk = np.zeros(144, np.uint8)
    blk[0:2] = np.array([1.0], np.float16).view(np.uint8)
    blk[2:4] = np.array([0.5], np.float16).view(np.uint8)
    sc = [j + 1 for j in range(8)]
    m = [2 * j for j in range(8)]
    sc[5], m[7] = 45, 63   # values that need the high two bits
    for j in range(4):
        blk[4 + j] = sc[j] | ((sc[j + 4] >> 4) << 6)
        blk[8 + j] = m[j] | ((m[j + 4] >> 4) << 6)
        blk[12 + j] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    for c in range(4):
        for i in range(32):
            blk[16 + 32 * c + i] = ((i + 2 * c) % 16) | (((i + 2 * c + 1) % 16) << 4)
    got = O.q4k_dequant(blk[None, :], 256)[0]
    want = np.array([1.0 * sc[j] * ((i + j) % 16) - 0.5 * m[j] for j in range(8) for i in range(32)])
    assert np.array_equal(got, want)


def test_q4k_dot_integer_decomposition():
    rng = np.random.default_rng(41)
    d = 1024
    w = _q4k_matrix(rng, 3, d)
    b = mw.pack_q4_k(w)
    d16, dmin16, sc, m, q = mw.q4k_parts(w)
    x = (rng.standard_normal((1, d)) * 3).astype(np.float32)
    qa, sa = O.quantize_q8(x)
    qa, sa = qa[0], sa[0]
    saf = sa.view(np.float16).astype(np.float64)
    for r in range(3):
        got = O.q4k_dot(qa, sa, b[r])
        # per 32-block: sa * (d*sc * sum(qa*q) - dmin*m * sum(qa)), the sums in int64
        cq = (qa.astype(np.int64) * q[r].astype(np.int64)).reshape(-1, 32).sum(1)
        ca = qa.astype(np.int64).reshape(-1, 32).sum(1)
        dd = np.repeat(d16[r].astype(np.float64), 8)
        dm = np.repeat(dmin16[r].astype(np.float64), 8)
        ref = float(np.sum(saf * (dd * sc[r] * cq - dm * m[r] * ca)))
        assert abs(got - ref) <= 1e-12 * np.sum(np.abs(saf * (dd * sc[r] * cq) + saf * (dm * m[r] * ca))) + 1e-300
    # a row whose codes are all zero leaves only the mins
    w0 = np.full((1, 256), -0.05, np.float32)
    b0 = mw.pack_q4_k(w0)
    d0, dmin0, sc0, m0, q0 = mw.q4k_parts(w0)
    assert not q0.any()
    ref0 = -float(np.sum(saf[:8] * dmin0[0, 0].astype(np.float64) * m0[0] * qa[:256].astype(np.int64).reshape(8, 32).sum(1)))
    assert O.q4k_dot(qa[:256], sa[:8], b0[0]) == pytest.approx(ref0, rel=1e-12, abs=1e-300)


def test_q4k_expert_ffn_against_numpy():
    rng = np.random.default_rng(42)
    d, F = 512, 256
    x = rng.standard_normal((1, d)).astype(np.float32)
    xq, xs = O.quantize_q8(x)
    G = mw.pack_q4_k((rng.standard_normal((F, d)) * 0.02).astype(np.float32))
    U = mw.pack_q4_k((rng.standard_normal((F, d)) * 0.02).astype(np.float32))
    D = mw.pack_q4_k((rng.standard_normal((d, F)) * 0.02).astype(np.float32))
    y, hq, hs, h = O.expert_ffn(d, F, xq[0], xs[0], G, U, D, fmt="q4_k")
    xd = xq[0].astype(np.float64) * np.repeat(xs[0].view(np.float16).astype(np.float64), 32)
    g = O.q4k_dequant(G, d) @ xd
    u = O.q4k_dequant(U, d) @ xd
    np.testing.assert_allclose(h, g * scipy.special.expit(g) * u, rtol=1e-12, atol=1e-15)
    hd = hq.astype(np.float64) * np.repeat(hs.view(np.float16).astype(np.float64), 32)
    np.testing.assert_allclose(y, O.q4k_dequant(D, F) @ hd, rtol=1e-11, atol=1e-14)
    # the same draws in Q8_0 give a different (but close) expert
    y8, _, _, _ = O.expert_ffn(d, F, xq[0], xs[0], mw.pack_q8_0(O.q4k_dequant(G, d).astype(np.float32)),
                               mw.pack_q8_0(O.q4k_dequant(U, d).astype(np.float32)),
                               mw.pack_q8_0(O.q4k_dequant(D, F).astype(np.float32)))
    assert np.linalg.norm(y8 - y) < 0.05 * np.linalg.norm(y)


@pytest.mark.parametrize("case", [
    dict(d=256, E=8, k=2, F=256),
    dict(d=512, E=6, k=3, F=256, Fs=256, zipf=1.1, norm=True),
])
def test_q4k_grouped_equals_per_token_bitwise(case):
    shape, lw = mw.random_shape_case(5, fmt="q4_k", **case)
    assert lw.fmt == "q4_k" and lw.gate_q8.shape[-1] == case["d"] // 256 * 144
    x = mw.make_tokens(105, 19, case["d"])
    a = O.moe_tokens(lw, x)["out"]
    b = O.moe_grouped(lw, x)
    assert np.array_equal(a, b)


# ------------------------------------------------------------- Q3_K
def _q3k_represented(w):
    """d*(sc-32)*q in fp64 from the Q3_K fields chosen for w."""
    d16, sc, q = mw.q3k_parts(w)
    d = np.repeat(d16.astype(np.float64), 16, axis=1)
    return np.repeat(d * (sc.astype(np.float64) - 32.0), 16, axis=1) * q.astype(np.float64)


def test_q3k_dequant_matches_the_packed_fields():
    rng = np.random.default_rng(50)
    w = _q4k_matrix(rng, 5, 768)
    b = mw.pack_q3_k(w)
    assert b.shape == (5, 3 * 110)
    dq = O.q3k_dequant(b, 768)
    assert np.array_equal(dq, _q3k_represented(w))
    d16, sc, q = mw.q3k_parts(w)
    assert q.min() == -4 and q.max() == 3 and sc.min() < 32 < sc.max()   # both code signs, both scale signs
    # every value within one step (d*|sc-32|) of the draw, except the top of
    # a sub-block whose largest value sits on the 3 side
    step = np.repeat(np.repeat(d16.astype(np.float64), 16, axis=1) * np.abs(sc.astype(np.float64) - 32), 16, axis=1)
    assert np.mean(np.abs(dq - w) <= step + 1e-9) > 0.98
    assert np.all(dq[0, 0:32] == 0.0)


def test_q3k_layout_of_one_super_block_by_hand():
    """One super-block written byte by byte: d = 0.25, sub-block s scale
    field sc_s (0 and 63 included: multipliers -32 and +31), and value i of
    the super-block q_i = (i * 5 + 3) % 8 - 4, placed as the format places
    it: value 128h + 32g + l has its 2-bit code in bits 2g of code byte
    32h + l and its high bit (q >= 0) in bit 4h + g of high-bit byte l."""
    blk = np.zeros(110, np.uint8)
    sc = [(7 * s + 5) % 64 for s in range(16)]
    sc[3], sc[12] = 0, 63
    for s in range(16):
        blk[96 + s % 8] |= (sc[s] & 15) << (4 * (s // 8))
        blk[104 + s % 4] |= ((sc[s] >> 4) & 3) << (2 * (s // 4))
    qv = [(i * 5 + 3) % 8 - 4 for i in range(256)]
    for i in range(256):
        h, g, l = i // 128, (i % 128) // 32, i % 32
        code = qv[i] if qv[i] >= 0 else qv[i] + 4
        blk[32 + 32 * h + l] |= code << (2 * g)
        if qv[i] >= 0:
            blk[l] |= 1 << (4 * h + g)
    blk[108:110] = np.array([0.25], np.float16).view(np.uint8)
    got = O.q3k_dequant(blk[None, :], 256)[0]
    want = np.array([0.25 * (sc[i // 16] - 32) * qv[i] for i in range(256)])
    assert np.array_equal(got, want)
    assert got[3 * 16] == 0.25 * -32 * qv[48] and qv[48] != 0


def test_q3k_dot_integer_decomposition():
    """Per 32-block: sa * d * sum over its two 16-value sub-blocks of
    (sc - 32) * sum(qa * q), the sums in int64."""
    rng = np.random.default_rng(51)
    d = 1024
    w = _q4k_matrix(rng, 3, d)
    b = mw.pack_q3_k(w)
    d16, sc, q = mw.q3k_parts(w)
    x = (rng.standard_normal((1, d)) * 3).astype(np.float32)
    qa, sa = O.quantize_q8(x)
    qa, sa = qa[0], sa[0]
    saf = sa.view(np.float16).astype(np.float64)
    for r in range(3):
        got = O.q3k_dot(qa, sa, b[r])
        c16 = (qa.astype(np.int64) * q[r].astype(np.int64)).reshape(-1, 16).sum(1)
        per32 = (c16 * (sc[r].astype(np.int64) - 32)).reshape(-1, 2).sum(1)
        dd = np.repeat(d16[r].astype(np.float64), 8)
        ref = float(np.sum(saf * dd * per32))
        assert abs(got - ref) <= 1e-12 * np.sum(np.abs(saf * dd * per32)) + 1e-300


def test_q3k_expert_ffn_against_numpy():
    rng = np.random.default_rng(52)
    d, F = 512, 256
    x = rng.standard_normal((1, d)).astype(np.float32)
    xq, xs = O.quantize_q8(x)
    G = mw.pack_q3_k((rng.standard_normal((F, d)) * 0.02).astype(np.float32))
    U = mw.pack_q3_k((rng.standard_normal((F, d)) * 0.02).astype(np.float32))
    D = mw.pack_q3_k((rng.standard_normal((d, F)) * 0.02).astype(np.float32))
    y, hq, hs, h = O.expert_ffn(d, F, xq[0], xs[0], G, U, D, fmt="q3_k")
    xd = xq[0].astype(np.float64) * np.repeat(xs[0].view(np.float16).astype(np.float64), 32)
    g = O.q3k_dequant(G, d) @ xd
    u = O.q3k_dequant(U, d) @ xd
    np.testing.assert_allclose(h, g * scipy.special.expit(g) * u, rtol=1e-12, atol=1e-15)
    hd = hq.astype(np.float64) * np.repeat(hs.view(np.float16).astype(np.float64), 32)
    np.testing.assert_allclose(y, O.q3k_dequant(D, F) @ hd, rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("case", [
    dict(d=256, E=8, k=2, F=256),
    dict(d=512, E=6, k=3, F=256, Fs=256, zipf=1.1, norm=True),
])
def test_q3k_grouped_equals_per_token_bitwise(case):
    shape, lw = mw.random_shape_case(6, fmt="q3_k", **case)
    assert lw.fmt == "q3_k" and lw.gate_q8.shape[-1] == case["d"] // 256 * 110
    x = mw.make_tokens(106, 19, case["d"])
    a = O.moe_tokens(lw, x)["out"]
    b = O.moe_grouped(lw, x)
    assert np.array_equal(a, b)
