"""A small owner of one weights handle plus its workspace (torch supplies the
device memory and the stream; the library does the work)."""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as B


def _dev(a, device, dtype=None):
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        t = a.to(device)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a)).to(device)
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous()


class MoeLayer:
    """Weights handle for one MoE FFN layer.

    Arguments follow moe_ffn_weights_create_fmt: router_w [E][d] fp32,
    router_bias [E] or None, gate/up rows [E][F][...], down rows [E][d][...]
    and the optional shared expert (sh_gate/sh_up [Fs][...], sh_down [d][...],
    sh_gate_vec [d]), the rows in format ``fmt``: "q8_0" (d/32 or F/32 blocks
    of 34 bytes), "q4_k" or "q3_k" (d/256 or F/256 super-blocks of 144 or 110
    bytes).  Host or device arrays are accepted.
    """

    def __init__(self, d_model, n_experts, top_k, d_ffn, router_w, gate_q8, up_q8, down_q8,
                 router_bias=None, d_shared_ffn=0, norm_topk_prob=False, sh_gate_q8=None,
                 sh_up_q8=None, sh_down_q8=None, sh_gate_vec=None, device="cuda", fmt="q8_0"):
        self.device = torch.device(device)
        self.fmt = fmt
        self.dims = B.make_dims(d_model, n_experts, top_k, d_ffn, d_shared_ffn, norm_topk_prob)
        up = dict(router_w=_dev(router_w, self.device, torch.float32),
                  router_bias=_dev(router_bias, self.device, torch.float32),
                  gate=_dev(gate_q8, self.device), up=_dev(up_q8, self.device),
                  down=_dev(down_q8, self.device), sh_gate=_dev(sh_gate_q8, self.device),
                  sh_up=_dev(sh_up_q8, self.device), sh_down=_dev(sh_down_q8, self.device),
                  sh_gate_vec=_dev(sh_gate_vec, self.device, torch.float32))
        with torch.cuda.device(self.device):
            self.handle = B.moe_ffn_weights_create_fmt(self.dims, B.FORMATS[fmt], **up)
        del up  # the call synchronised its stream; the library holds its own copy
        self._ws = None

    @classmethod
    def from_workload(cls, lw, device="cuda"):
        s = lw.shape
        return cls(s.d, s.n_experts, s.top_k, s.ffn, lw.router_w, lw.gate_q8, lw.up_q8, lw.down_q8,
                   router_bias=lw.router_bias, d_shared_ffn=s.shared_ffn,
                   norm_topk_prob=s.norm_topk_prob, sh_gate_q8=lw.sh_gate_q8, sh_up_q8=lw.sh_up_q8,
                   sh_down_q8=lw.sh_down_q8, sh_gate_vec=lw.sh_gate_vec, device=device,
                   fmt=getattr(lw, "fmt", "q8_0"))

    @property
    def d(self):
        return self.dims.d_model

    def workspace_size(self, max_tokens: int) -> int:
        return B.moe_ffn_workspace_size(self.handle, max_tokens)

    def workspace(self, n_tokens: int) -> torch.Tensor:
        need = self.workspace_size(n_tokens)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def _run(self, fn, x, out, routing, stream):
        n = x.shape[0]
        if out is None:
            out = torch.empty((n, self.d), dtype=torch.float32, device=self.device)
        ws = self.workspace(n)
        fn(self.handle, x, n, out, ws, ws.numel(), routing, stream)
        return out

    def prefill(self, x: torch.Tensor, out: Optional[torch.Tensor] = None, routing=None, stream=None):
        return self._run(B.moe_ffn_prefill, x, out, routing, stream)

    def prefill_residual(self, x: torch.Tensor, h: torch.Tensor, xn: torch.Tensor, eps: float = 1e-5,
                         routing=None, stream=None):
        """The layer inside a residual stack: h += layer(x), xn = RMSNorm(h); xn may be x."""
        n = x.shape[0]
        ws = self.workspace(n)
        B.moe_ffn_prefill_residual(self.handle, x, n, h, xn, eps, ws, ws.numel(), routing, stream)

    def decode(self, x: torch.Tensor, out: Optional[torch.Tensor] = None, routing=None, stream=None):
        return self._run(B.moe_ffn_decode, x, out, routing, stream)

    def close(self):
        if getattr(self, "handle", None):
            B.moe_ffn_weights_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
