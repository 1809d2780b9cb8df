"""ExpertBlock: the buffers and call order of one MoE expert layer on one GPU.

It owns device buffers (allocated once with torch) and issues the C-ABI calls
of a training step on the current stream:

  forward   moe_permute(BUILD_MAP | GATHER) -> moe_grouped_mlp_fwd (FC1 + GLU
            epilogue, FC2) -> moe_unpermute
  backward  moe_permute(GATHER of dOut, map reused) -> moe_grouped_mlp_bwd
            (FC2 dgrad + dGLU epilogue, FC1 dgrad) -> moe_unpermute (dX and
            dprobs)

With prec=PREC_MXFP8 the permutes write MXFP8 rows (no bf16 copy), the four
GEMMs take MXFP8 operands, and quantize_weights() (after every weight update;
load_weights() calls it) makes the four weight copies the GEMMs read, each
blocked along its K.  A training step whose optimizer has just changed the
bf16 weights calls quantize_weights(live_only=True) between route() and the
GEMMs: it then skips the experts that received no rows this step.  The
epilogues then write only the MXFP8 copies of a and dz that the next GEMMs
(and weight-gradient GEMMs) read, unless bf16_copies=True also asks for the
bf16 tensors.

With wgrad=True, weight_grads() adds the weight-gradient grouped GEMMs
(moe_grouped_mlp_wgrad): dW1 [E][N1][H] in the interleaved row order of w1i
and dW2 [E][H][I].  bf16 reads dz, Xp, dYp and a as stored; MXFP8 reads the
transposed copies of a and dz the epilogues wrote and makes those of Xp and
dYp with moe_quantize_mxfp8 (the permutes then also keep bf16 Xp and dYp).

With prec=PREC_MXFP4 the layer is fused the same way with MXFP4 operands:
the permutes write MXFP4 rows, the GLU and dGLU epilogues write the MXFP4
copies of a and dz (rowwise and transposed), quantize_weights() makes the
four MXFP4 weight copies (rowwise and, for the dgrads, along N1 / H), and
weight_grads() runs the MXFP4 weight-gradient GEMMs on the transposed
copies (those of Xp and dYp made by moe_quantize_mxfp4).  No bias path.
unfused=True runs the same layer
as separate passes instead (bf16 permutes and activation passes,
moe_quantize_mxfp4 before each of the four grouped GEMMs): the baseline the
fused path is measured against, which needs the bf16 copies.

With recompute=True (activation recompute) the forward stores no z and the
backward first rebuilds it with moe_grouped_gemm from the saved Xp and W1
(recompute_z): z's write moves from the forward to the backward, at the cost
of one more FC1-sized GEMM, and gradients are bit for bit those of the path
that keeps z.  The block then holds no z between its forward and its
backward: z lives in `z_scratch` (a bf16 tensor of at least M_cap * N1
elements that many blocks may share, as their backwards run one after the
other) or, without one, in a buffer allocated at the start of the backward
and released at its end.

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
                 prec: int = B.PREC_BF16, transposed_copies: bool = True,
                 bf16_copies: Optional[bool] = None, wgrad: bool = False,
                 recompute: bool = False, z_scratch: Optional[torch.Tensor] = None,
                 unfused: bool = False, device="cuda"):
        self.E, self.H, self.I, self.T, self.k = E, H, I, T, k
        self.act = act or B.act_params()
        self.gated = self.act.act != B.ACT_SRELU
        self.N1 = 2 * I if self.gated else I
        self.first_expert = first_expert
        self.prec = prec
        # activation recompute: the forward keeps no z; the backward rebuilds
        # it from xp and W1 before the dActivation pass (recompute_z)
        self.recompute = recompute
        self._z_valid = False
        # tests may keep the rebuilt z after the backward, to compare it
        self.keep_recomputed_z = False
        self.mx = prec == B.PREC_MXFP8
        # MXFP4: fused like MXFP8 -- the permutes and the GLU / dGLU
        # epilogues write the MXFP4 rowwise operands of the next GEMM -- or,
        # through the *_unfused methods (bf16 copies needed), as separate
        # passes with every operand quantized by moe_quantize_mxfp4
        self.mx4 = prec == B.PREC_MXFP4
        # forward() / backward() run the unfused passes (the baseline the
        # fused kernels are measured against; bf16 copies are then needed)
        self.unfused = unfused
        M_cap = M_cap if M_cap is not None else T * k + E * (B.GROUP_ALIGN - 1)
        if self.mx or self.mx4:
            M_cap = -(-M_cap // B.GROUP_ALIGN) * B.GROUP_ALIGN
        self.M_cap = M_cap
        self.cu_margin = cu_margin
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        bf = dict(dtype=torch.bfloat16, device=dev)
        u8 = dict(dtype=torch.uint8, device=dev)
        M, N1 = self.M_cap, self.N1
        self.split_sizes = torch.zeros(E, **i32)
        self.offsets = torch.zeros(E + 1, **i32)
        self.padded_offsets = torch.zeros(E + 1, **i32)
        self.row_id_map = torch.zeros(T, k, **i32)
        self.row_src = torch.zeros(M, **i32)
        self.probs_p = torch.zeros(M, **f32)
        self.err_flag = torch.zeros(1, **i32)
        self.bias1 = None            # optional FC1 bias, fp32 [E][N1] (load_weights)
        self.ws_route = torch.empty(max(1, B.moe_permute_workspace_size(T, E)),
                                    dtype=torch.uint8, device=dev)
        # bf16 a and dz (and, in MXFP4, Xp and dYp): operands of the bf16
        # GEMMs; optional with MX operands, kept by default only for the
        # unfused layer, whose separate passes read them
        mx_any = self.mx or self.mx4
        keep = ((not mx_any or unfused) if bf16_copies is None
                else (bf16_copies or not mx_any))
        if self.mx4 and unfused and (wgrad or recompute):
            raise ValueError("the unfused MXFP4 layer has no weight-gradient or recompute path")
        if recompute:
            # z exists only while the backward runs (see recompute_z)
            if z_scratch is not None:
                if (z_scratch.dtype != torch.bfloat16 or not z_scratch.is_contiguous()
                        or z_scratch.numel() < M * N1):
                    raise ValueError("z_scratch must be a contiguous bf16 tensor of at "
                                     f"least M_cap * N1 = {M * N1} elements")
            self._z_scratch = z_scratch
            self.z = None
        else:
            self.z = torch.empty(M, N1, **bf)
        self.a = torch.empty(M, I, **bf) if keep else None
        self.yp = torch.empty(M, H, **bf)
        self.out = torch.empty(T, H, **bf)
        self.amax = torch.zeros(1, **f32)
        self.dz = torch.empty(M, N1, **bf) if keep else None
        self.dprobs_p = torch.zeros(M, **f32)
        self.dxp = torch.empty(M, H, **bf)
        self.dx = torch.empty(T, H, **bf)
        self.dprobs = torch.zeros(T, k, **f32)
        self.ws = torch.empty(
            max(1, B.moe_grouped_mlp_workspace_size(E, H, I, M, prec,
                                                    self.act.act)),
            dtype=torch.uint8, device=dev)
        self.w1i = torch.empty(E, N1, H, **bf)
        self.w2 = torch.empty(E, H, I, **bf)

        def mx_pair(*shape):
            n = 1
            for d in shape:
                n *= d
            return torch.empty(*shape, **u8), torch.empty(n // B.MX_BLOCK, **u8)

        if self.mx4 and not keep:
            self.xp = self.dyp = None
        if self.mx:
            self.xp = self.dyp = None
            self.xp_q, self.xp_s = mx_pair(M, H)
            self.dyp_q, self.dyp_s = mx_pair(M, H)
            self.w1_q, self.w1_s = mx_pair(E, N1, H)      # along H
            self.w2_q, self.w2_s = mx_pair(E, H, I)       # along I
            self.w2t_q, self.w2t_s = mx_pair(E, I, H)     # along H
            self.w1t_q, self.w1t_s = mx_pair(E, H, N1)    # along N1
            self.a_q, self.a_s = mx_pair(M, I)
            self.dz_q, self.dz_s = mx_pair(M, N1)
            if transposed_copies:
                self.aT_q, self.aT_s = mx_pair(I, M)
                self.dzT_q, self.dzT_s = mx_pair(N1, M)
            else:
                self.aT_q = self.aT_s = self.dzT_q = self.dzT_s = None
        elif not self.mx4 or keep:
            self.xp = torch.empty(M, H, **bf)
            self.dyp = torch.empty(M, H, **bf)
        if self.mx4:
            def fp4_pair(*shape):
                n = 1
                for d in shape:
                    n *= d
                return (torch.empty(n // 2, **u8), torch.empty(n // B.MX_BLOCK, **u8))
            self.xp_q4, self.xp_s4 = fp4_pair(M, H)
            self.a_q4, self.a_s4 = fp4_pair(M, I)
            self.dyp_q4, self.dyp_s4 = fp4_pair(M, H)
            self.dz_q4, self.dz_s4 = fp4_pair(M, N1)
            if transposed_copies and not unfused:
                self.aT_q4, self.aT_s4 = fp4_pair(I, M)      # along M
                self.dzT_q4, self.dzT_s4 = fp4_pair(N1, M)
            else:
                self.aT_q4 = self.aT_s4 = self.dzT_q4 = self.dzT_s4 = None
            self.w1_q4, self.w1_s4 = fp4_pair(E, N1, H)     # along H
            self.w2_q4, self.w2_s4 = fp4_pair(E, H, I)      # along I
            self.w2t_q4, self.w2t_s4 = fp4_pair(E, I, H)    # along H
            self.w1t_q4, self.w1t_s4 = fp4_pair(E, H, N1)   # along N1
        self.wgrad = wgrad
        if wgrad:
            if self.mx or self.mx4:
                if not transposed_copies:
                    raise ValueError("MX weight gradients read the transposed "
                                     "copies of a and dz (transposed_copies=True)")
                if self.xp is None:
                    self.xp = torch.empty(M, H, **bf)
                    self.dyp = torch.empty(M, H, **bf)
            if self.mx:
                self.xpT_q, self.xpT_s = mx_pair(H, M)
                self.dypT_q, self.dypT_s = mx_pair(H, M)
            elif self.mx4:
                self.xpT_q4, self.xpT_s4 = fp4_pair(H, M)
                self.dypT_q4, self.dypT_s4 = fp4_pair(H, M)
            self.dw1 = torch.empty(E, N1, H, **bf)
            self.dw2 = torch.empty(E, H, I, **bf)

    # ------------------------------------------------------------ weights --
    def load_weights(self, w1: torch.Tensor, w2: torch.Tensor,
                     bias1: Optional[torch.Tensor] = None) -> None:
        """w1: bf16 [E][N1][H] (gate rows then up rows), w2: bf16 [E][H][I].
        The gated FC1 weight is repacked into the interleaved layout; with
        MXFP8 the weight copies are then quantized.  bias1: optional FC1
        bias, [E][N1] in the same logical order as w1's rows (kept as fp32;
        the fused forward and backward add it to the activation's input)."""
        if bias1 is None:
            self.bias1 = None
        else:
            if tuple(bias1.shape) != (self.E, self.N1):
                raise ValueError(f"bias1 must be [{self.E}][{self.N1}]")
            self.bias1 = bias1.detach().to(device=self.w2.device,
                                           dtype=torch.float32).contiguous()
        if self.gated:
            B.moe_weight_repack_interleave(w1, self.w1i, self.E, self.I,
                                           self.H)
        else:
            self.w1i.copy_(w1)
        self.w2.copy_(w2)
        if self.mx or self.mx4:
            self.quantize_weights()

    def quantize_weights(self, live_only: bool = False) -> None:
        """MX copies of the bf16 weights, each blocked along the K of the
        GEMM that reads it: W1i along H (FC1), W2 along I (FC2), W2 along H
        (FC2 dgrad, stored [E][I][H]) and W1i along N1 (FC1 dgrad, stored
        [E][H][N1]).  In training the bf16 master weights change every step,
        so a step makes them anew (bench.py times it inside the step).
        live_only: after route(), skip the experts with no routed rows (this
        step's GEMMs read none of their weights; their copies are left as
        they were)."""
        E, H, I, N1 = self.E, self.H, self.I, self.N1
        # one pass per weight writes both of its copies (ROW into q / s, COL
        # into qT / sT), reading the bf16 weight once
        if self.mx4:
            sfx, quant = "4", B.moe_quantize_mxfp4
        else:
            sfx, quant = "", B.moe_quantize_mxfp8
        for x, rows, cols, row_copy, col_copy in ((self.w1i, N1, H, "w1", "w1t"),
                                                  (self.w2, H, I, "w2", "w2t")):
            quant(mode=B.QUANT_BOTH, batch=E, rows=rows, cols=cols, x=x,
                  q=getattr(self, row_copy + "_q" + sfx), s=getattr(self, row_copy + "_s" + sfx),
                  qT=getattr(self, col_copy + "_q" + sfx), sT=getattr(self, col_copy + "_s" + sfx),
                  live=self.split_sizes if live_only else None)

    # ------------------------------------------------------------ forward --
    def route(self, expert_idx: torch.Tensor, probs: torch.Tensor,
              x: Optional[torch.Tensor] = None) -> None:
        flags = B.PERMUTE_BUILD_MAP
        xq, xs = self._mx_dst("xp")
        if x is not None:
            flags |= B.PERMUTE_GATHER
            if xq is not None:
                flags |= B.PERMUTE_WRITE_MX4 if self.mx4 else B.PERMUTE_WRITE_MX
        B.moe_permute(flags=flags, T=self.T, k=self.k, E=self.E, H=self.H,
                      M_cap=self.M_cap, first_expert=self.first_expert,
                      expert_idx=expert_idx, probs=probs,
                      split_sizes=self.split_sizes, offsets=self.offsets,
                      padded_offsets=self.padded_offsets,
                      row_id_map=self.row_id_map, row_src=self.row_src,
                      probs_p=self.probs_p, x=x, xp=self.xp, xp_q=xq, xp_s=xs,
                      err_flag=self.err_flag, workspace=self.ws_route)

    def _mx_dst(self, name):
        """The MX copy (codes, scales) the permutes write for xp or dyp:
        MXFP8 or MXFP4, or (None, None) in bf16 and in the unfused MXFP4
        layer (which quantizes the bf16 rows itself)."""
        if self.mx:
            return getattr(self, name + "_q"), getattr(self, name + "_s")
        if self.mx4 and not self.unfused:
            return getattr(self, name + "_q4"), getattr(self, name + "_s4")
        return None, None

    def route_logits(self, logits: torch.Tensor,
                     x: Optional[torch.Tensor] = None, fused: bool = True) -> None:
        """Top-k router on the device (softmax over the experts of fp32
        logits [T][E_total], k largest, ties to the lower id) into
        self.expert_idx / self.probs, and the routing metadata of the local
        experts.  fused: router and metadata in one launch
        (moe_router_route), then the gather of x if given; else
        moe_router_topk followed by route() (four launches before the
        gather).  Both give the same bits."""
        T, E_all = logits.shape
        if not hasattr(self, "expert_idx"):
            dev = logits.device
            self.expert_idx = torch.empty(T, self.k, dtype=torch.int32, device=dev)
            self.probs = torch.empty(T, self.k, dtype=torch.float32, device=dev)
        if not fused:
            B.moe_router_topk(T=T, E=E_all, k=self.k, logits=logits,
                              expert_idx=self.expert_idx, probs=self.probs)
            self.route(self.expert_idx, self.probs, x)
            return
        if getattr(self, "ws_router", None) is None:
            # its counters start at zero; every call leaves them at zero
            self.ws_router = torch.zeros(B.moe_router_route_workspace_size(T, E_all, self.E),
                                         dtype=torch.uint8, device=logits.device)
        B.moe_router_route(T=T, E_total=E_all, k=self.k, E=self.E,
                           first_expert=self.first_expert, M_cap=self.M_cap,
                           logits=logits, expert_idx=self.expert_idx, probs=self.probs,
                           split_sizes=self.split_sizes, offsets=self.offsets,
                           padded_offsets=self.padded_offsets, row_id_map=self.row_id_map,
                           row_src=self.row_src, probs_p=self.probs_p,
                           err_flag=self.err_flag, workspace=self.ws_router)
        if x is not None:
            self.gather(x, self.xp, *self._mx_dst("xp"))

    def gather(self, src: torch.Tensor, dst: Optional[torch.Tensor],
               dst_q: Optional[torch.Tensor] = None,
               dst_s: Optional[torch.Tensor] = None) -> None:
        flags = B.PERMUTE_GATHER
        if dst_q is not None:
            flags |= B.PERMUTE_WRITE_MX4 if self.mx4 else B.PERMUTE_WRITE_MX
        B.moe_permute(flags=flags, T=self.T, k=self.k, E=self.E,
                      H=self.H, M_cap=self.M_cap,
                      first_expert=self.first_expert,
                      split_sizes=self.split_sizes,
                      padded_offsets=self.padded_offsets,
                      row_id_map=self.row_id_map, x=src, xp=dst, xp_q=dst_q,
                      xp_s=dst_s)

    def experts_forward(self, timing_events=None) -> None:
        kw = {}
        if self.mx:
            kw = dict(xp_q=self.xp_q, xp_s=self.xp_s, w1_q=self.w1_q,
                      w1_s=self.w1_s, w2_q=self.w2_q, w2_s=self.w2_s,
                      a_q=self.a_q, a_s=self.a_s, aT_q=self.aT_q,
                      aT_s=self.aT_s)
        elif self.mx4:
            kw = dict(xp_q=self.xp_q4, xp_s=self.xp_s4, w1_q=self.w1_q4,
                      w1_s=self.w1_s4, w2_q=self.w2_q4, w2_s=self.w2_s4,
                      a_q=self.a_q4, a_s=self.a_s4, aT_q=self.aT_q4, aT_s=self.aT_s4)
        else:
            kw = dict(xp=self.xp, w1i=self.w1i, w2=self.w2)
        B.moe_grouped_mlp_fwd(E=self.E, H=self.H, I=self.I, M_cap=self.M_cap,
                              split_sizes=self.split_sizes,
                              padded_offsets=self.padded_offsets,
                              probs_p=self.probs_p,
                              z=None if self.recompute else self.z, a=self.a,
                              yp=self.yp, amax=self.amax, act=self.act,
                              prec=self.prec, cu_margin=self.cu_margin,
                              err_flag=self.err_flag, workspace=self.ws,
                              timing_events=timing_events, bias1=self.bias1, **kw)
        self._z_valid = not self.recompute

    def recompute_z(self) -> None:
        """Rebuilds z = xp . W1i^T after a forward that kept none: FC1's
        grouped GEMM without its epilogue and without split-K, so every tile
        sums K in the order FC1 used and z is bit for bit the one FC1 would
        have stored (MXFP8: from the same xp and W1 codes and scales)."""
        if self.recompute and self.z is None:
            if self._z_scratch is not None:
                self.z = self._z_scratch.view(-1)[:self.M_cap * self.N1].view(self.M_cap,
                                                                               self.N1)
            else:
                self.z = torch.empty(self.M_cap, self.N1, dtype=torch.bfloat16,
                                     device=self.yp.device)
        if self.mx:
            self._gemm(self.N1, self.H, self.xp_q, self.w1_q, self.z, self.xp_s,
                       self.w1_s, split=False)
        elif self.mx4:
            self._gemm(self.N1, self.H, self.xp_q4, self.w1_q4, self.z, self.xp_s4,
                       self.w1_s4, split=False)
        else:
            self._gemm(self.N1, self.H, self.xp, self.w1i, self.z, split=False)
        self._z_valid = True

    def release_z(self) -> None:
        """With recompute, drop the rebuilt z (the backward no longer needs
        it); experts_backward calls it at its end."""
        if self.recompute:
            self.z = None
            self._z_valid = False

    def combine(self, yp: torch.Tensor, out: torch.Tensor,
                dprobs: bool = False) -> None:
        B.moe_unpermute(T=self.T, k=self.k, H=self.H, M_cap=self.M_cap,
                        row_id_map=self.row_id_map, yp=yp, out=out,
                        dprobs_p=self.dprobs_p if dprobs else None,
                        dprobs=self.dprobs if dprobs else None)

    def forward(self, x, expert_idx, probs, timing_events=None):
        self.route(expert_idx, probs, x)
        if self.unfused:
            self.experts_forward_unfused()
        else:
            self.experts_forward(timing_events)
        self.combine(self.yp, self.out)
        return self.out

    # ----------------------------------------------------------- backward --
    def experts_backward(self, timing_events=None) -> None:
        if self.recompute and not self._z_valid:
            self.recompute_z()
        if self.mx:
            kw = dict(dyp_q=self.dyp_q, dyp_s=self.dyp_s, w2t_q=self.w2t_q,
                      w2t_s=self.w2t_s, w1t_q=self.w1t_q, w1t_s=self.w1t_s,
                      dz_q=self.dz_q, dz_s=self.dz_s, dzT_q=self.dzT_q,
                      dzT_s=self.dzT_s)
        elif self.mx4:
            kw = dict(dyp_q=self.dyp_q4, dyp_s=self.dyp_s4, w2t_q=self.w2t_q4,
                      w2t_s=self.w2t_s4, w1t_q=self.w1t_q4, w1t_s=self.w1t_s4,
                      dz_q=self.dz_q4, dz_s=self.dz_s4, dzT_q=self.dzT_q4,
                      dzT_s=self.dzT_s4)
        else:
            kw = dict(dyp=self.dyp, w2=self.w2, w1i=self.w1i)
        B.moe_grouped_mlp_bwd(E=self.E, H=self.H, I=self.I, M_cap=self.M_cap,
                              split_sizes=self.split_sizes,
                              padded_offsets=self.padded_offsets,
                              probs_p=self.probs_p, z=self.z, dz=self.dz,
                              dprobs_p=self.dprobs_p, dxp=self.dxp,
                              workspace=self.ws, act=self.act,
                              prec=self.prec, cu_margin=self.cu_margin,
                              err_flag=self.err_flag,
                              timing_events=timing_events, bias1=self.bias1, **kw)
        if self.recompute and not self.keep_recomputed_z:
            self.release_z()

    def backward(self, dout, timing_events=None):
        self.gather(dout, self.dyp, *self._mx_dst("dyp"))
        if self.unfused:
            self.experts_backward_unfused()
        else:
            self.experts_backward(timing_events)
        self.combine(self.dxp, self.dx, dprobs=True)
        return self.dx, self.dprobs

    # ------------------------------------------------- unfused baseline --
    # The same layer without the fused epilogues: FC1 and FC2 dgrad as plain
    # grouped GEMMs, the activation and its gradient as separate passes
    # (moe_glu_unfused) and, with MXFP8, the rowwise and transposed copies of
    # a and dz made by moe_quantize_mxfp8.  It measures what the fused path
    # gains; outputs have the meaning of the fused ones (dA is stored in bf16
    # in between).  MXFP8 needs the block built with bf16_copies=True.
    def _gemm(self, N, K, a, b, c, a_s=None, b_s=None, b_kn=False, split=True):
        B.moe_grouped_gemm(E=self.E, N=N, K=K, M_cap=self.M_cap,
                           split_sizes=self.split_sizes,
                           padded_offsets=self.padded_offsets, a=a, b=b, c=c,
                           b_kn=b_kn, cu_margin=self.cu_margin,
                           workspace=self.ws if split else None,
                           prec=self.prec, a_s=a_s, b_s=b_s, err_flag=self.err_flag)

    def _quantize4(self, x, cols, q, s):
        B.moe_quantize_mxfp4(batch=1, rows=self.M_cap, cols=cols, x=x, q=q, s=s)

    def _quantize(self, x, cols, q, s, qT, sT):
        B.moe_quantize_mxfp8(mode=B.QUANT_ROW, batch=1, rows=self.M_cap, cols=cols,
                             x=x, q=q, s=s)
        if qT is not None:
            B.moe_quantize_mxfp8(mode=B.QUANT_COL, batch=1, rows=self.M_cap,
                                 cols=cols, x=x, q=qT, s=sT)

    def experts_forward_unfused(self, events=None) -> None:
        if self.bias1 is not None:
            raise RuntimeError("the FC1 bias is applied by the fused path only")
        # MXFP8 reads the permute's MXFP8 Xp; MXFP4 quantizes the bf16 Xp
        if (self.mx and self.a is None) or (self.mx4 and (self.a is None or self.xp is None)):
            raise RuntimeError("the MX unfused baseline needs bf16_copies=True")
        rec = (lambda i: events.record(i)) if events else (lambda i: None)
        rec(0)
        if self.mx4:
            self._quantize4(self.xp, self.H, self.xp_q4, self.xp_s4)
            self._gemm(self.N1, self.H, self.xp_q4, self.w1_q4, self.z, self.xp_s4,
                       self.w1_s4)
        elif self.mx:
            self._gemm(self.N1, self.H, self.xp_q, self.w1_q, self.z, self.xp_s, self.w1_s)
        else:
            self._gemm(self.N1, self.H, self.xp, self.w1i, self.z)
        rec(1)
        B.moe_glu_unfused(direction=0, E=self.E, I=self.I, M_cap=self.M_cap,
                          split_sizes=self.split_sizes,
                          padded_offsets=self.padded_offsets, probs_p=self.probs_p,
                          z=self.z, a=self.a, amax=self.amax, act=self.act)
        if self.mx4:
            self._quantize4(self.a, self.I, self.a_q4, self.a_s4)
        elif self.mx:
            self._quantize(self.a, self.I, self.a_q, self.a_s, self.aT_q, self.aT_s)
        rec(2)
        if self.mx4:
            self._gemm(self.H, self.I, self.a_q4, self.w2_q4, self.yp, self.a_s4, self.w2_s4)
        elif self.mx:
            self._gemm(self.H, self.I, self.a_q, self.w2_q, self.yp, self.a_s, self.w2_s)
        else:
            self._gemm(self.H, self.I, self.a, self.w2, self.yp)
        rec(3)

    def experts_backward_unfused(self, events=None) -> None:
        if (self.mx and self.dz is None) or (self.mx4 and (self.dz is None or self.dyp is None)):
            raise RuntimeError("the MX unfused baseline needs bf16_copies=True")
        if getattr(self, "da", None) is None:
            self.da = torch.empty(self.M_cap, self.I, dtype=torch.bfloat16,
                                  device=self.z.device)
        rec = (lambda i: events.record(i)) if events else (lambda i: None)
        rec(0)
        if self.mx4:
            self._quantize4(self.dyp, self.H, self.dyp_q4, self.dyp_s4)
            self._gemm(self.I, self.H, self.dyp_q4, self.w2t_q4, self.da, self.dyp_s4,
                       self.w2t_s4)
        elif self.mx:
            self._gemm(self.I, self.H, self.dyp_q, self.w2t_q, self.da, self.dyp_s,
                       self.w2t_s)
        else:
            self._gemm(self.I, self.H, self.dyp, self.w2, self.da, b_kn=True)
        rec(1)
        B.moe_glu_unfused(direction=1, E=self.E, I=self.I, M_cap=self.M_cap,
                          split_sizes=self.split_sizes,
                          padded_offsets=self.padded_offsets, probs_p=self.probs_p,
                          z=self.z, da=self.da, dz=self.dz,
                          dprobs_p=self.dprobs_p, act=self.act)
        if self.mx4:
            self._quantize4(self.dz, self.N1, self.dz_q4, self.dz_s4)
        elif self.mx:
            self._quantize(self.dz, self.N1, self.dz_q, self.dz_s, self.dzT_q, self.dzT_s)
        rec(2)
        if self.mx4:
            self._gemm(self.H, self.N1, self.dz_q4, self.w1t_q4, self.dxp, self.dz_s4,
                       self.w1t_s4)
        elif self.mx:
            self._gemm(self.H, self.N1, self.dz_q, self.w1t_q, self.dxp, self.dz_s,
                       self.w1t_s)
        else:
            self._gemm(self.H, self.N1, self.dz, self.w1i, self.dxp, b_kn=True)
        rec(3)

    def weight_grads(self, timing_events=None):
        """dW1 (rows in w1i's interleaved order) and dW2 of the last
        forward + backward; needs wgrad=True."""
        if not self.wgrad:
            raise RuntimeError("ExpertBlock was built without wgrad=True")
        kw = {}
        if self.mx:
            for src, q, s in ((self.xp, self.xpT_q, self.xpT_s),
                              (self.dyp, self.dypT_q, self.dypT_s)):
                B.moe_quantize_mxfp8(mode=B.QUANT_COL, batch=1, rows=self.M_cap,
                                     cols=self.H, x=src, q=q, s=s)
            kw = dict(dzT_q=self.dzT_q, dzT_s=self.dzT_s, xpT_q=self.xpT_q,
                      xpT_s=self.xpT_s, dypT_q=self.dypT_q, dypT_s=self.dypT_s,
                      aT_q=self.aT_q, aT_s=self.aT_s)
        elif self.mx4:
            for src, q, s in ((self.xp, self.xpT_q4, self.xpT_s4),
                              (self.dyp, self.dypT_q4, self.dypT_s4)):
                B.moe_quantize_mxfp4(mode=B.QUANT_COL, batch=1, rows=self.M_cap,
                                     cols=self.H, x=src, q=q, s=s)
            kw = dict(dzT_q=self.dzT_q4, dzT_s=self.dzT_s4, xpT_q=self.xpT_q4,
                      xpT_s=self.xpT_s4, dypT_q=self.dypT_q4, dypT_s=self.dypT_s4,
                      aT_q=self.aT_q4, aT_s=self.aT_s4)
        else:
            kw = dict(dz=self.dz, xp=self.xp, dyp=self.dyp, a=self.a)
        B.moe_grouped_mlp_wgrad(E=self.E, H=self.H, I=self.I, M_cap=self.M_cap,
                                gated=self.gated, split_sizes=self.split_sizes,
                                padded_offsets=self.padded_offsets,
                                prec=self.prec, cu_margin=self.cu_margin,
                                dw1=self.dw1, dw2=self.dw2,
                                timing_events=timing_events, err_flag=self.err_flag,
                                **kw)
        return self.dw1, self.dw2
