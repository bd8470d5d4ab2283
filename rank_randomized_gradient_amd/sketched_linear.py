"""A bf16 linear layer trained through the sketch instead of a dense weight gradient.

[RGC, "How it works"] (page "Randomized Gradient Compression"): the forward
keeps X P instead of X; the backward adds D^T (X P) to an fp32 sketch C while
the input gradient D W flows on as usual; after the step's microbatches the
weights take the normalized update with stochastic rounding and a new P is
drawn. [LoGRA-M, "Minimal Causal Code"] (page "LoGRA: Low-Rank Gradient
Sketches") runs the same loop with a caller-chosen step (`apply_update(...,
alpha=...)`).

Every step runs in the library's kernels: the forward is one
rgc_linear_forward call ([Y | XP] = X [W^T | P], one tile grid, so the
projection adds no pass over X); the backward one rgc_linear_backward call
(dX = D W, then C += D^T XP on the same stream); the update rgc_apply /
rgc_apply_scaled / rgc_apply_carried; P from rgc_sample_projection. W never
receives a .grad: the sketch replaces it.
"""
from __future__ import annotations

import torch

from . import rgc


class SketchedLinearFunction(torch.autograd.Function):
    """Y = X W^T and XP = X P from one call; saves XP (T x r), not X; backward:
    dX = D W and C += D^T XP from one call (C alone when X needs no gradient)."""

    @staticmethod
    def forward(ctx, x, weight, proj, sketch, workspace):
        x2 = x.reshape(-1, x.shape[-1])
        if not x2.is_contiguous():
            x2 = x2.contiguous()
        y, xp = rgc.rgc_linear_forward(x2, weight, proj)
        ctx.save_for_backward(xp, weight)
        ctx.sketch = sketch
        ctx.workspace = workspace
        ctx.in_shape = x.shape
        return y.reshape(*x.shape[:-1], weight.shape[0])

    @staticmethod
    def backward(ctx, dy):
        xp, weight = ctx.saved_tensors
        d2 = dy.reshape(-1, dy.shape[-1])
        if d2.dtype != torch.bfloat16:
            d2 = d2.to(torch.bfloat16)
        if not d2.is_contiguous():
            d2 = d2.contiguous()
        if ctx.needs_input_grad[0]:
            dx = rgc.rgc_linear_backward(d2, weight, xp, ctx.sketch, workspace=ctx.workspace).reshape(ctx.in_shape)
        else:
            rgc.rgc_accumulate(d2, xp, ctx.sketch, workspace=ctx.workspace)
            dx = None
        return dx, None, None, None, None


class SketchedLinear(torch.nn.Module):
    """out x in bf16 linear layer (no bias) with a rank-r sketch in place of its gradient.

    Per update: begin_update(seed) draws P and zeroes C; every microbatch's
    forward/backward adds its D^T (X P) to C; apply_update(...) changes the
    weights in place. P and C live on the layer (k x r bf16 and d x r fp32).

    carry_norm=True: the normalized update hands ||W||^2 of the weights it
    writes to the next one (rgc_apply_carried), so each later update reads W
    once. The value is streamed from W again (fresh) after a fixed-step
    update, after load_state_dict, whenever the weight's version counter moved
    since the last carried update (any torch in-place op on the Parameter,
    e.g. `with torch.no_grad(): layer.weight.copy_(...)`), and after
    invalidate_weight_norm(). Writes that bypass the version counter
    (through `weight.data`, or raw pointers) are not seen: a caller making
    them must call invalidate_weight_norm().
    """

    def __init__(self, in_features: int, out_features: int, rank: int, kind: str = "qr", device=None,
                 weight: torch.Tensor | None = None, carry_norm: bool = False):
        super().__init__()
        device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        if weight is None:
            weight = torch.empty((out_features, in_features), dtype=torch.bfloat16, device=device)
            torch.nn.init.normal_(weight, std=0.02)
        if tuple(weight.shape) != (out_features, in_features) or weight.dtype != torch.bfloat16:
            raise rgc.RgcError("weight must be a bf16 out_features x in_features tensor")
        self.weight = torch.nn.Parameter(weight.to(device), requires_grad=False)
        self.rank, self.kind = rank, kind
        self.register_buffer("proj", torch.empty((in_features, rank), dtype=torch.bfloat16, device=device))
        self.register_buffer("sketch", torch.zeros((out_features, rank), dtype=torch.float32, device=device))
        self.workspace = rgc.Workspace(device)
        self.proj_seed = None
        self.carry_norm = carry_norm
        self.register_buffer("weight_norm2", torch.zeros(1, dtype=torch.float64, device=device))
        self._norm_fresh = True  # weight_norm2 does not hold ||W||^2 yet
        self._norm_version = None  # the weight's version counter when weight_norm2 was last written

    def invalidate_weight_norm(self) -> None:
        """The weights changed outside apply_update: the next update streams ||W|| again."""
        self._norm_fresh = True

    def _norm_is_stale(self) -> bool:
        return self._norm_fresh or self._norm_version != self.weight._version

    def _load_from_state_dict(self, *args, **kwargs):
        # the loaded weights (and a loaded weight_norm2) need not match each other
        super()._load_from_state_dict(*args, **kwargs)
        self._norm_fresh = True

    def begin_update(self, proj_seed: int) -> None:
        """Draws P from its seed (fixed for the whole accumulation) and zeroes C."""
        rgc.rgc_sample_projection(self.kind, proj_seed, self.weight.shape[1], self.rank, out=self.proj,
                                  workspace=self.workspace)
        self.sketch.zero_()
        self.proj_seed = proj_seed

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if self.proj_seed is None:
            raise rgc.RgcError("begin_update(seed) must draw the projection before the first forward")
        return SketchedLinearFunction.apply(x, self.weight, self.proj, self.sketch, self.workspace)

    def apply_update(self, seed: int, tau: float | None = None, alpha: float | None = None,
                     stats: torch.Tensor | None = None) -> None:
        """Normalized update with tau [RGC], or the fixed step alpha [LoGRA-M]; one of the two."""
        if (tau is None) == (alpha is None):
            raise rgc.RgcError("give exactly one of tau (normalized update) or alpha (fixed step)")
        w = self.weight.data
        if tau is not None and self.carry_norm:
            rgc.rgc_apply_carried(w, self.sketch, self.proj, tau, seed, self.weight_norm2, fresh=self._norm_is_stale(),
                                  stats=stats, workspace=self.workspace)
            # the library writes W through its pointer, which leaves the version counter as it is
            self._norm_fresh = False
            self._norm_version = self.weight._version
        elif tau is not None:
            rgc.rgc_apply(w, self.sketch, self.proj, tau, seed, stats=stats, workspace=self.workspace)
        else:
            rgc.rgc_apply_scaled(w, self.sketch, self.proj, alpha, seed)
            self._norm_fresh = True
