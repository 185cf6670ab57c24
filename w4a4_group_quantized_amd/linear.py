"""A W4A4 linear layer and a synthetic LLaMA-shaped decoder layer built on it.

The APEX4 page (aiqbench news page, Abstract) presents the method as a
drop-in replacement for a model's linear layers: weights quantized ahead of
time to INT4 with per-group scales, activations quantized on the fly, one
W4A4 GEMM with per-group dequantization.  `W4A4Linear` is that layer over the
library's C ABI (include/apex4.h): `forward` runs apex4_linear_w4a4 (the
activation quantization and the GEMM; for 1-2 rows one fused launch) on
torch's current stream, nothing else.

`LlamaLayerW4A4` strings four of them together the way one LLaMA decoder layer
uses its linear layers (fused QKV, O, fused gate+up, down) with random
weights, so that the layers run back to back on each other's outputs, as in a
model.  The operations between them are not part of the method and run as
plain torch ops on the GPU: the V third of the QKV output stands in for the
attention output (attention itself is not a W4A4 GEMM), two residual adds and
the SwiGLU product silu(gate) * up.  There are no trained weights here: the
layer measures speed, not model quality.
"""
from __future__ import annotations

import torch

from . import apex4


class W4A4Linear(torch.nn.Module):
    """y = x W^T with W held as packed INT4 codes and fp32 group scales.

    qw: uint8 [N, K/2] packed weight codes, sw: float32 [N, K/group_w]
    (apex4_pack_weight's outputs), group_a: activation group size used by the
    on-the-fly quantization (group_w == group_a, or group_w == K for
    per-channel weight scales with activation groups).  Inputs: fp16
    [..., K] on the GPU; output fp16 [..., N].  The call's workspace (the
    activation codes and scales, and the GEMM's K-split partials) is kept per
    row count, so repeated calls at one shape allocate only the output.
    """

    def __init__(self, qw: torch.Tensor, sw: torch.Tensor, group_w: int, group_a: int | None = None):
        super().__init__()
        if qw.dtype != torch.uint8 or qw.dim() != 2 or not qw.is_cuda:
            raise ValueError("qw must be a uint8 [N, K/2] GPU tensor (apex4_pack_weight output)")
        self.out_features = qw.shape[0]
        self.in_features = 2 * qw.shape[1]
        self.group_w = group_w
        self.group_a = group_w if group_a is None else group_a
        self.register_buffer("qw", qw)
        self.register_buffer("sw", sw)
        self._ws = {}

    @classmethod
    def from_weight(cls, w: torch.Tensor, group_w: int = 128, group_a: int | None = None) -> "W4A4Linear":
        """Quantize and pack an fp16 [N, K] GPU weight (the offline step)."""
        qw, sw = apex4.pack_weight(w.contiguous(), group_w)
        return cls(qw, sw, group_w, group_a)

    def _workspace(self, M: int, device):
        ws = self._ws.get(M)
        if ws is None:
            need = apex4.linear_workspace_size(M, self.out_features, self.in_features, self.group_a, self.group_w)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
            self._ws[M] = ws
        return ws

    def forward(self, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected [..., {self.in_features}] input, got {tuple(x.shape)}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features)
        if not x2.is_contiguous():
            x2 = x2.contiguous()
        M = x2.shape[0]
        y16 = None
        if out is not None:
            # the library writes M x out_features contiguous values: `out` must be
            # exactly that memory (a reshape that copies would leave it unwritten)
            if tuple(out.shape) != (*lead, self.out_features) or not out.is_contiguous():
                raise ValueError(f"out must be a contiguous {(*lead, self.out_features)} tensor, "
                                 f"got {tuple(out.shape)} (contiguous: {out.is_contiguous()})")
            y16 = out.view(M, self.out_features)
        y = apex4.linear(x2, self.group_a, self.qw, self.sw, self.group_w, y16=y16,
                         workspace=self._workspace(M, x2.device))
        return y.reshape(*lead, self.out_features)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"group_a={self.group_a}, group_w={self.group_w}")


class LlamaLayerW4A4(torch.nn.Module):
    """The four linear layers of one LLaMA decoder layer, W4A4.

    weights: fp16 GPU tensors "qkv" [3h, h], "o" [h, h], "gate_up" [2i, h]
    (gate rows first) and "down" [h, i], with h the hidden and i the
    intermediate size (LLaMA-2-7B: 4096 and 11008); each is quantized and
    packed with groups of `group` (the offline step).
    """

    NAMES = ("qkv", "o", "gate_up", "down")

    def __init__(self, weights: dict, group: int = 128):
        super().__init__()
        self.hidden = weights["o"].shape[0]
        self.intermediate = weights["down"].shape[1]
        for name in self.NAMES:
            setattr(self, name, W4A4Linear.from_weight(weights[name], group))

    @classmethod
    def random(cls, hidden: int = 4096, intermediate: int = 11008, group: int = 128, seed: int = 0,
               device="cuda") -> "LlamaLayerW4A4":
        """Random N(0, 0.02) fp16 weights from the seeded generator of
        w4a4_group_quantized_amd.inputs (numpy PCG64, seed `seed`)."""
        import numpy as np

        from . import inputs
        rng = np.random.default_rng(seed)
        shapes = {"qkv": (3 * hidden, hidden), "o": (hidden, hidden),
                  "gate_up": (2 * intermediate, hidden), "down": (hidden, intermediate)}
        w = {n: torch.from_numpy(inputs.weights(rng, *shapes[n])).to(device) for n in cls.NAMES}
        return cls(w, group)

    def linear_shapes(self):
        """(K, N) of the four W4A4 GEMMs, in call order."""
        return [(m.in_features, m.out_features) for m in (self.qkv, self.o, self.gate_up, self.down)]

    def forward(self, x: torch.Tensor, return_inputs: bool = False):
        """x: fp16 [M, h].  With return_inputs, also returns the fp16 input of
        each linear layer and its output, in call order (for checking every
        GEMM against a reference on the inputs it actually saw)."""
        h, i = self.hidden, self.intermediate
        seen = []
        qkv = self.qkv(x)
        seen.append((x, qkv))
        attn = qkv[:, 2 * h:].contiguous()          # V: stand-in for the attention output
        o = self.o(attn)
        seen.append((attn, o))
        x = x + o
        gu = self.gate_up(x)
        seen.append((x, gu))
        mid = torch.nn.functional.silu(gu[:, :i]) * gu[:, i:]      # fp16 in, fp16 out
        d = self.down(mid)
        seen.append((mid, d))
        x = x + d
        return (x, seen) if return_inputs else x
