"""moe_ffn_prefill_static, the prefill entry point that allocates nothing (its
workspace is the library's static per-device scratch array), against
moe_ffn_prefill with a caller workspace: two calls in a row, the second
smaller than the first, each bit for bit equal to the workspace form in its
output, routing and partials; and a batch too large for the array is
rejected before anything is enqueued."""
import numpy as np
import pytest

import moe_workloads as mw

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _routing(B, shape, n, dev):
    kk = shape.top_k + (1 if shape.shared_ffn else 0)
    P = n * shape.top_k + (n if shape.shared_ffn else 0)
    bufs = dict(topk_ids=torch.full((n, shape.top_k), -7, dtype=torch.int32, device=dev),
                topk_w=torch.full((n, shape.top_k), -7.0, dtype=torch.float32, device=dev),
                exp_start=torch.full((shape.n_experts + 2,), -7, dtype=torch.int32, device=dev),
                exp_tok_i=torch.full((P,), -7, dtype=torch.int32, device=dev),
                partial=torch.full((n, kk, shape.d), float("nan"), dtype=torch.float32, device=dev))
    return bufs, B.make_routing(**bufs)


def test_static_prefill_matches_workspace_prefill():
    from mixture_experts_ffn_gemm_amd import binding as B
    from mixture_experts_ffn_gemm_amd.layer import MoeLayer
    dev = torch.device("cuda")
    shape, lw = mw.random_shape_case(21, d=384, E=4, k=2, F=320, Fs=160, zipf=1.1, norm=True)
    layer = MoeLayer.from_workload(lw)
    try:
        for n in (300, 37):   # the second call is smaller: the first call's scratch contents stay behind
            assert layer.workspace_size(n) <= B.STATIC_SCRATCH_BYTES
            print(f"[no-alloc] n={n}", flush=True)
            x = torch.from_numpy(mw.make_tokens(900 + n, n, shape.d)).to(dev)
            bufs_a, ra = _routing(B, shape, n, dev)
            bufs_b, rb = _routing(B, shape, n, dev)
            ref = layer.prefill(x, routing=ra)
            out = torch.full((n, shape.d), float("nan"), dtype=torch.float32, device=dev)
            B.moe_ffn_prefill_static(layer.handle, x, n, out, rb)
            torch.cuda.synchronize()
            assert torch.equal(out, ref), f"n={n}: output differs from moe_ffn_prefill"
            for key in bufs_a:
                assert torch.equal(bufs_a[key], bufs_b[key]), f"n={n}: {key} differs"
        # a batch whose workspace exceeds the array: rejected on the host (x is
        # never read, so a dummy address is fine)
        with pytest.raises(B.MoeFfnError) as err:
            B.moe_ffn_prefill_static(layer.handle, 256, 1 << 20, 4096, None)
        assert err.value.status == B.MOE_FFN_SCRATCH_TOO_SMALL
    finally:
        layer.close()
