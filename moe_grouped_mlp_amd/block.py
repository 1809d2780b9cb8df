"""ExpertBlock: the buffers and call order of one MoE expert layer on one GPU.

It owns device buffers (allocated once with torch) and issues the C-ABI calls
of a training step on the current stream:

  forward   moe_permute(BUILD_MAP | GATHER) -> moe_grouped_mlp_fwd (FC1 + GLU
            epilogue, FC2) -> moe_unpermute
  backward  moe_permute(GATHER of dOut, map reused) -> moe_grouped_mlp_bwd
            (FC2 dgrad + dGLU epilogue, FC1 dgrad) -> moe_unpermute (dX and
            dprobs)

No call reads device memory back or synchronises, so a whole step can be
captured in a HIP graph.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import binding as B


class ExpertBlock:
    def __init__(self, E: int, H: int, I: int, T: int, k: int, *,
                 act: Optional[B.ActParams] = None, first_expert: int = 0,
                 M_cap: Optional[int] = None, cu_margin: int = 0,
                 device="cuda"):
        self.E, self.H, self.I, self.T, self.k = E, H, I, T, k
        self.act = act or B.act_params()
        self.gated = self.act.act != B.ACT_SRELU
        self.N1 = 2 * I if self.gated else I
        self.first_expert = first_expert
        self.M_cap = M_cap if M_cap is not None else T * k + E * (B.GROUP_ALIGN - 1)
        self.cu_margin = cu_margin
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        bf = dict(dtype=torch.bfloat16, device=dev)
        M = self.M_cap
        self.split_sizes = torch.zeros(E, **i32)
        self.offsets = torch.zeros(E + 1, **i32)
        self.padded_offsets = torch.zeros(E + 1, **i32)
        self.row_id_map = torch.zeros(T, k, **i32)
        self.row_src = torch.zeros(M, **i32)
        self.probs_p = torch.zeros(M, **f32)
        self.err_flag = torch.zeros(1, **i32)
        self.ws_route = torch.empty(max(1, B.moe_permute_workspace_size(T, E)),
                                    dtype=torch.uint8, device=dev)
        self.xp = torch.empty(M, H, **bf)
        self.z = torch.empty(M, self.N1, **bf)
        self.a = torch.empty(M, I, **bf)
        self.yp = torch.empty(M, H, **bf)
        self.out = torch.empty(T, H, **bf)
        self.amax = torch.zeros(1, **f32)
        self.dyp = torch.empty(M, H, **bf)
        self.dz = torch.empty(M, self.N1, **bf)
        self.dprobs_p = torch.zeros(M, **f32)
        self.dxp = torch.empty(M, H, **bf)
        self.dx = torch.empty(T, H, **bf)
        self.dprobs = torch.zeros(T, k, **f32)
        self.ws_bwd = torch.empty(
            max(1, B.moe_grouped_mlp_workspace_size(E, H, I, M, B.PREC_BF16,
                                                    self.act.act)),
            dtype=torch.uint8, device=dev)
        self.w1i = torch.empty(E, self.N1, H, **bf)
        self.w2 = torch.empty(E, H, I, **bf)

    # ------------------------------------------------------------ weights --
    def load_weights(self, w1: torch.Tensor, w2: torch.Tensor) -> None:
        """w1: bf16 [E][N1][H] (gate rows then up rows), w2: bf16 [E][H][I].
        The gated FC1 weight is repacked into the interleaved layout."""
        if self.gated:
            B.moe_weight_repack_interleave(w1, self.w1i, self.E, self.I,
                                           self.H)
        else:
            self.w1i.copy_(w1)
        self.w2.copy_(w2)

    # ------------------------------------------------------------ forward --
    def route(self, expert_idx: torch.Tensor, probs: torch.Tensor,
              x: Optional[torch.Tensor] = None) -> None:
        flags = B.PERMUTE_BUILD_MAP | (B.PERMUTE_GATHER if x is not None else 0)
        B.moe_permute(flags=flags, T=self.T, k=self.k, E=self.E, H=self.H,
                      M_cap=self.M_cap, first_expert=self.first_expert,
                      expert_idx=expert_idx, probs=probs,
                      split_sizes=self.split_sizes, offsets=self.offsets,
                      padded_offsets=self.padded_offsets,
                      row_id_map=self.row_id_map, row_src=self.row_src,
                      probs_p=self.probs_p, x=x, xp=self.xp,
                      err_flag=self.err_flag, workspace=self.ws_route)

    def gather(self, src: torch.Tensor, dst: torch.Tensor) -> None:
        B.moe_permute(flags=B.PERMUTE_GATHER, T=self.T, k=self.k, E=self.E,
                      H=self.H, M_cap=self.M_cap,
                      first_expert=self.first_expert,
                      split_sizes=self.split_sizes,
                      padded_offsets=self.padded_offsets,
                      row_id_map=self.row_id_map, x=src, xp=dst)

    def experts_forward(self, timing_events=None) -> None:
        B.moe_grouped_mlp_fwd(E=self.E, H=self.H, I=self.I, M_cap=self.M_cap,
                              split_sizes=self.split_sizes,
                              padded_offsets=self.padded_offsets,
                              probs_p=self.probs_p, xp=self.xp, w1i=self.w1i,
                              w2=self.w2, z=self.z, a=self.a, yp=self.yp,
                              amax=self.amax, act=self.act,
                              cu_margin=self.cu_margin,
                              err_flag=self.err_flag,
                              timing_events=timing_events)

    def combine(self, yp: torch.Tensor, out: torch.Tensor,
                dprobs: bool = False) -> None:
        B.moe_unpermute(T=self.T, k=self.k, H=self.H, M_cap=self.M_cap,
                        row_id_map=self.row_id_map, yp=yp, out=out,
                        dprobs_p=self.dprobs_p if dprobs else None,
                        dprobs=self.dprobs if dprobs else None)

    def forward(self, x, expert_idx, probs, timing_events=None):
        self.route(expert_idx, probs, x)
        self.experts_forward(timing_events)
        self.combine(self.yp, self.out)
        return self.out

    # ----------------------------------------------------------- backward --
    def experts_backward(self, timing_events=None) -> None:
        B.moe_grouped_mlp_bwd(E=self.E, H=self.H, I=self.I, M_cap=self.M_cap,
                              split_sizes=self.split_sizes,
                              padded_offsets=self.padded_offsets,
                              probs_p=self.probs_p, dyp=self.dyp, w2=self.w2,
                              z=self.z, w1i=self.w1i, dz=self.dz,
                              dprobs_p=self.dprobs_p, dxp=self.dxp,
                              workspace=self.ws_bwd, act=self.act,
                              cu_margin=self.cu_margin,
                              err_flag=self.err_flag,
                              timing_events=timing_events)

    def backward(self, dout, timing_events=None):
        self.gather(dout, self.dyp)
        self.experts_backward(timing_events)
        self.combine(self.dxp, self.dx, dprobs=True)
        return self.dx, self.dprobs
