"""Device-side plumbing around the library: upload inputs, pack the argument tensors the
C ABI expects, run the layer, and read back the per-step tensors from the workspace.

Packing is layout only: text keys and values are stacked into text_kv [2,L,H,d], the two
gate logit tensors into gates [2,N,H,d], the two projection weights side by side into
w_out [D, 2*H*d] (row o = W_s[o] followed by W_l[o]), and the linear branch's own q/k/v
(when given) into qkv_lin [3,N,H,d].
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

from . import binding
from .synth import LayerInputs

_ACT = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class DeviceLayer:
    cfg: binding.Cfg
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    text_kv: torch.Tensor
    gates: torch.Tensor
    rms_weight: torch.Tensor
    w_out: torch.Tensor
    residual: torch.Tensor
    out: torch.Tensor
    workspace: torch.Tensor
    qkv_lin: Optional[torch.Tensor] = None
    o_soft_dbg: Optional[torch.Tensor] = None
    u_lin_dbg: Optional[torch.Tensor] = None
    extra: dict = field(default_factory=dict)

    def run(self, stream=None) -> None:
        binding.hybrid_attn_fwd(self.q, self.k, self.v, self.text_kv, self.gates, self.rms_weight, self.w_out,
                                self.residual, self.out, self.cfg, qkv_lin=self.qkv_lin,
                                o_soft_dbg=self.o_soft_dbg, u_lin_dbg=self.u_lin_dbg, workspace=self.workspace,
                                stream=stream)

    def run_train(self, stream=None) -> None:
        """The forward, keeping its training record for backward(dout, saved=True)."""
        if "saved" not in self.extra:
            self.extra["saved"] = torch.empty(binding.saved_bytes(self.cfg), dtype=torch.uint8, device=self.q.device)
        binding.hybrid_attn_fwd_train(self.q, self.k, self.v, self.text_kv, self.gates, self.rms_weight, self.w_out,
                                      self.residual, self.out, self.cfg, self.extra["saved"],
                                      workspace=self.workspace, stream=stream)

    def backward(self, dout: torch.Tensor, stream=None, saved: bool = False) -> dict:
        """Layer backward for the upstream gradient dout [N, D]; returns float32 gradients
        (dq, dk, dv, dtext_k, dtext_v, dg_s, dg_l, dw_rms, dw_s, dw_l).  saved: use the
        record of the last run_train instead of recomputing the forward."""
        c = self.cfg
        N, H, d, L, D = c.frames * c.tokens_per_frame, c.heads, c.head_dim, c.text_len, c.model_dim
        dev = self.q.device
        f32 = dict(dtype=torch.float32, device=dev)
        dqkv = torch.empty(3, N, H, d, **f32)
        dtext = torch.empty(2, L, H, d, **f32)
        dgates = torch.empty(2, N, H, d, **f32)
        dw = torch.empty(H, d, **f32)
        dwo = torch.empty(D, 2 * H * d, **f32)
        if "bwd_ws" not in self.extra:
            self.extra["bwd_ws"] = torch.empty(binding.bwd_workspace_bytes(c), dtype=torch.uint8, device=dev)
        binding.hybrid_attn_bwd(self.q, self.k, self.v, self.text_kv, self.gates, self.rms_weight, self.w_out,
                                dout.contiguous(), c, dqkv, dtext if L > 0 else None, dgates, dw, dwo,
                                workspace=self.extra["bwd_ws"], stream=stream,
                                saved=self.extra["saved"] if saved else None)
        hd = H * d
        return dict(dq=dqkv[0], dk=dqkv[1], dv=dqkv[2], dtext_k=dtext[0], dtext_v=dtext[1], dg_s=dgates[0],
                    dg_l=dgates[1], dw_rms=dw, dw_s=dwo[:, :hd], dw_l=dwo[:, hd:])

    def workspace_tensors(self) -> dict:
        """Views into the workspace (valid after run): frame_states [F,H,d,d],
        text_state [H,d,d], fwd_states/bwd_states [nC,H,d,d] float32 and
        branch_out [N, 2*H*d] in the activation dtype."""
        c = self.cfg
        L = binding.workspace_layout(c)
        F, H, d = c.frames, c.heads, c.head_dim
        nC = -(-F // c.chunk_frames)
        N = F * c.tokens_per_frame
        ws = self.workspace

        def view(off, shape, dtype):
            n = 1
            for s in shape:
                n *= s
            nbytes = n * torch.tensor([], dtype=dtype).element_size()
            return ws[off:off + nbytes].view(dtype).view(*shape)

        act = torch.float32 if c.act_dtype == binding.F32 else torch.bfloat16
        return dict(frame_states=view(L.frame_states, (F, H, d, d), torch.float32),
                    text_state=view(L.text_state, (H, d, d), torch.float32),
                    fwd_states=view(L.fwd_states, (nC, H, d, d), torch.float32),
                    bwd_states=view(L.bwd_states, (nC, H, d, d), torch.float32),
                    branch_out=view(L.branch_out, (N, 2 * H * d), act))


def upload(inp: LayerInputs, device="cuda", debug: bool = False, out_aliases_residual: bool = False,
           sentinel: Optional[float] = None) -> DeviceLayer:
    """Copy LayerInputs to the device in the layout the library takes.

    debug: also allocate the float32 o_soft / u_lin outputs.  sentinel: fill every output
    (and the workspace) with this value first, so a test can see that all of it is
    overwritten.
    """
    s = inp.shape
    act = _ACT[s.act_dtype]

    def dev(t):
        return t.to(device, non_blocking=False).contiguous()

    cfg = binding.make_cfg(s, inp.q_scale, inp.k_scale, inp.v_scale)
    text_kv = dev(torch.stack([inp.text_k, inp.text_v]))
    gates = dev(torch.stack([inp.g_s, inp.g_l]))
    w_out = dev(torch.cat([inp.w_s, inp.w_l], dim=1))
    residual = dev(inp.x)
    out = residual if out_aliases_residual else torch.empty_like(residual)
    qkv_lin = None
    if inp.q_lin is not None:
        qkv_lin = dev(torch.stack([inp.q_lin, inp.k_lin, inp.v_lin]).to(act))
    ws = torch.empty(binding.workspace_bytes(cfg), dtype=torch.uint8, device=device)
    N, H, d = s.tokens, s.heads, s.head_dim
    o_dbg = torch.empty(N, H, d, dtype=torch.float32, device=device) if debug else None
    u_dbg = torch.empty(N, H, d, dtype=torch.float32, device=device) if debug else None
    if sentinel is not None:
        for t in (o_dbg, u_dbg):
            if t is not None:
                t.fill_(sentinel)
        if not out_aliases_residual:
            out.fill_(sentinel)
        ws.view(torch.uint8).fill_(0xFF)  # NaN pattern in float32 and bf16
    return DeviceLayer(cfg=cfg, q=dev(inp.q), k=dev(inp.k), v=dev(inp.v), text_kv=text_kv, gates=gates,
                       rms_weight=dev(inp.w_rms), w_out=w_out, residual=residual, out=out, workspace=ws,
                       qkv_lin=qkv_lin, o_soft_dbg=o_dbg, u_lin_dbg=u_dbg)
