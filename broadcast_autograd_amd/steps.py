"""The five workloads as sequences of library calls (forward, then backward).

Each workload holds its device inputs, preallocated outputs and workspaces, so
a step only issues ``zk`` calls.  The backward replays by hand the graph the
"Zero" book builds (Autograd chapter): add hands its upstream gradient to both
inputs, so a gradient that passes through an add is the same buffer (no
copy), and a tensor reached along two paths gets the second path accumulated
onto the first (``acc``).

Algorithmic bytes of a call = 4 x (distinct elements of every input the call
reads + every element it writes); a repeated operand counts once, and an acc
that is the same buffer as the upstream gradient is not counted twice.
"""
import numpy as np

from . import workloads as W
from . import zk


def _n(shape):
    return int(np.prod(shape, dtype=np.int64))


class Call:
    """One library call of a step.  ``reduce``: the call sums a gradient back
    to a broadcast operand's shape, and this many reduced elements are
    written (by the call's last kernel when it has a separate stage 2)."""

    def __init__(self, name, kind, fn, reads, writes, reduce=None):
        self.name, self.kind, self.fn = name, kind, fn
        self.bytes = 4 * (sum(reads) + sum(writes))
        self.elements = max(writes)  # elements of the largest output
        self.reduce = reduce

    def __call__(self):
        return self.fn()


class Workload:
    """Base: ``calls`` lists Call objects in step order."""
    name = ""

    def run(self):
        for c in self.calls:
            c()

    @property
    def fwd_calls(self):
        return [c for c in self.calls if c.kind == "fwd"]

    @property
    def bwd_calls(self):
        return [c for c in self.calls if c.kind == "bwd"]

    def step_bytes(self, kind=None):
        return sum(c.bytes for c in self.calls if kind is None or c.kind == kind)


def _ws(bytes_, torch):
    return torch.empty(max(256, int(bytes_)), dtype=torch.uint8, device="cuda")


class XYPlusX(Workload):
    """z = x*y + x with x[64,128,256], y[128,1]."""
    name = "xy_plus_x"

    def __init__(self, host=None, scale=1):
        import torch
        h = host or W.xy_plus_x(scale)
        self.host = h
        d = {k: torch.from_numpy(v).to("cuda") for k, v in h.items()}
        self.x, self.y, self.g = d["x"], d["y"], d["g"]
        e = torch.empty_like
        self.t, self.z = e(self.x), e(self.x)
        self.grad_x, self.grad_y = e(self.x), e(self.y)
        self.ws = _ws(zk.bwd_workspace_bytes("mul", self.x, self.y), torch)
        nx, ny = _n(self.x.shape), _n(self.y.shape)
        self.calls = [
            Call("mul(x,y)->t", "fwd",
                 lambda: zk.binary_fwd("mul", self.x, self.y, out=self.t), [nx, ny], [nx]),
            Call("add(t,x)->z", "fwd",
                 lambda: zk.binary_fwd("add", self.t, self.x, out=self.z), [nx, nx], [nx]),
            # add passes g to t and to x; mul's rule then adds x's second path
            Call("mul_bwd(g;x,y)->grad_x(acc=g),grad_y", "bwd",
                 lambda: zk.binary_bwd("mul", self.g, self.x, self.y, grad_a=self.grad_x,
                                       grad_b=self.grad_y, acc_a=self.g, workspace=self.ws),
                 [nx, nx, ny], [nx, ny], reduce=ny),
        ]


class MLPBiasGelu(Workload):
    """y = GeLU(act[4096,1024] + bias[1024])."""
    name = "mlp_bias_gelu"

    def __init__(self, host=None, rows=4096, cols=1024):
        import torch
        h = host or W.mlp_bias_gelu(rows, cols)
        self.host = h
        d = {k: torch.from_numpy(v).to("cuda") for k, v in h.items()}
        self.act, self.bias, self.g = d["act"], d["bias"], d["g"]
        self.y = torch.empty_like(self.act)
        self.grad_act = torch.empty_like(self.act)
        self.grad_bias = torch.empty_like(self.bias)
        self.ws = _ws(zk.bwd_workspace_bytes("add", self.act, self.bias, epi="gelu"), torch)
        na, nb = _n(self.act.shape), _n(self.bias.shape)
        self.calls = [
            Call("add+gelu(act,bias)->y", "fwd",
                 lambda: zk.binary_fwd("add", self.act, self.bias, out=self.y, epi="gelu"),
                 [na, nb], [na]),
            Call("add_bwd+gelu(g;act,bias)->grad_act,grad_bias", "bwd",
                 lambda: zk.binary_bwd("add", self.g, self.act, self.bias,
                                       grad_a=self.grad_act, grad_b=self.grad_bias,
                                       epi="gelu", workspace=self.ws),
                 [na, na, nb], [na, nb], reduce=nb),
        ]


class AttnScaleMask(Workload):
    """scores[8,16,1024,1024] * scale[1,16,1,1] + mask[1,1,1024,1024]."""
    name = "attn_scale_mask"

    def __init__(self, host=None, b=8, h=16, t=1024):
        import torch
        hh = host or W.attn_scale_mask(b, h, t)
        self.host = hh
        d = {k: torch.from_numpy(v).to("cuda") for k, v in hh.items()}
        self.scores, self.scale, self.mask, self.g = d["scores"], d["scale"], d["mask"], d["g"]
        e = torch.empty_like
        self.t, self.out = e(self.scores), e(self.scores)
        self.grad_scores, self.grad_scale = e(self.scores), e(self.scale)
        self.ws = _ws(zk.bwd_workspace_bytes("mul", self.scores, self.scale), torch)
        ns, nc, nm = _n(self.scores.shape), _n(self.scale.shape), _n(self.mask.shape)
        self.calls = [
            Call("mul(scores,scale)->t", "fwd",
                 lambda: zk.binary_fwd("mul", self.scores, self.scale, out=self.t),
                 [ns, nc], [ns]),
            Call("add(t,mask)->out", "fwd",
                 lambda: zk.binary_fwd("add", self.t, self.mask, out=self.out),
                 [ns, nm], [ns]),
            # the gradient of t is g itself (add); mul's rule gives scores / scale
            Call("mul_bwd(g;scores,scale)->grad_scores,grad_scale", "bwd",
                 lambda: zk.binary_bwd("mul", self.g, self.scores, self.scale,
                                       grad_a=self.grad_scores, grad_b=self.grad_scale,
                                       workspace=self.ws),
                 [ns, ns, nc], [ns, nc], reduce=nc),
        ]


class AttnMaskGrad(Workload):
    """The attention mask's gradient: g[8,16,1024,1024] summed back to the
    mask's shape [1,1,1024,1024] (a column reduction over 128 rows)."""
    name = "attn_mask_grad"

    def __init__(self, host=None, b=8, h=16, t=1024):
        import torch
        hh = host or W.attn_mask_grad(b, h, t)
        self.host = hh
        self.g = torch.from_numpy(hh["g"]).to("cuda")
        self.target = (1, 1) + tuple(self.g.shape[2:])
        self.grad_mask = torch.empty(self.target, dtype=torch.float32, device="cuda")
        self.ws = _ws(zk.reduce_workspace_bytes(self.g, self.target), torch)
        ng, nm = _n(self.g.shape), _n(self.target)
        self.calls = [
            Call("reduce_to_shape(g->[1,1,%d,%d])" % self.target[2:], "bwd",
                 lambda: zk.reduce_to_shape(self.g, self.target, out=self.grad_mask,
                                            workspace=self.ws),
                 [ng], [nm], reduce=nm),
        ]


class StridedTransposed(Workload):
    """a[4096,4096] as a transposed view (strides [1,4096]) * b[4096]."""
    name = "strided_transposed"

    def __init__(self, host=None, n=4096):
        import torch
        h = host or W.strided_transposed(n)
        self.host = h
        self.a_storage = torch.from_numpy(h["a_storage"]).to("cuda")
        self.a = torch.as_strided(self.a_storage, h["a_sizes"], h["a_strides"])
        self.b = torch.from_numpy(h["b"]).to("cuda")
        self.g = torch.from_numpy(h["g"]).to("cuda")
        self.out = torch.empty(h["a_sizes"], dtype=torch.float32, device="cuda")
        self.grad_a = torch.empty_like(self.out)
        self.grad_b = torch.empty_like(self.b)
        self.ws = _ws(zk.bwd_workspace_bytes("mul", self.a, self.b), torch)
        na, nb = n * n, n
        self.calls = [
            Call("mul(aT,b)->out", "fwd",
                 lambda: zk.binary_fwd("mul", self.a, self.b, out=self.out), [na, nb], [na]),
            Call("mul_bwd(g;aT,b)->grad_a,grad_b", "bwd",
                 lambda: zk.binary_bwd("mul", self.g, self.a, self.b, grad_a=self.grad_a,
                                       grad_b=self.grad_b, workspace=self.ws),
                 [na, na, nb], [na, nb], reduce=nb),
        ]


class Rank8(Workload):
    """a[2,3,4,5,6,7,8,9] / b[1,3,1,5,1,7,1,9]."""
    name = "rank8_div"

    def __init__(self, host=None):
        import torch
        h = host or W.rank8()
        self.host = h
        d = {k: torch.from_numpy(v).to("cuda") for k, v in h.items()}
        self.a, self.b, self.g = d["a"], d["b"], d["g"]
        e = torch.empty_like
        self.out, self.grad_a, self.grad_b = e(self.a), e(self.a), e(self.b)
        self.ws = _ws(zk.bwd_workspace_bytes("div", self.a, self.b), torch)
        na, nb = _n(self.a.shape), _n(self.b.shape)
        self.calls = [
            Call("div(a,b)->out", "fwd",
                 lambda: zk.binary_fwd("div", self.a, self.b, out=self.out), [na, nb], [na]),
            Call("div_bwd(g;a,b)->grad_a,grad_b", "bwd",
                 lambda: zk.binary_bwd("div", self.g, self.a, self.b, grad_a=self.grad_a,
                                       grad_b=self.grad_b, workspace=self.ws),
                 [na, na, nb], [na, nb], reduce=nb),
        ]


class GPTResidual(Workload):
    """h[16,2048,4096] * gamma[4096] + resid[16,2048,4096]."""
    name = "gpt_residual"

    def __init__(self, host=None, b=16, t=2048, c=4096):
        import torch
        hh = host or W.gpt_residual(b, t, c)
        self.host = hh
        d = {k: torch.from_numpy(v).to("cuda") for k, v in hh.items()}
        self.h, self.gamma, self.resid, self.g = d["h"], d["gamma"], d["resid"], d["g"]
        e = torch.empty_like
        self.t, self.out = e(self.h), e(self.h)
        self.grad_h, self.grad_gamma, self.grad_resid = e(self.h), e(self.gamma), e(self.h)
        self.ws = _ws(zk.bwd_workspace_bytes("mul", self.h, self.gamma), torch)
        self.ws2 = _ws(zk.bwd_workspace_bytes("add", self.t, self.resid, need_a=False), torch)
        nh, ng = _n(self.h.shape), _n(self.gamma.shape)
        self.calls = [
            Call("mul(h,gamma)->t", "fwd",
                 lambda: zk.binary_fwd("mul", self.h, self.gamma, out=self.t), [nh, ng], [nh]),
            Call("add(t,resid)->out", "fwd",
                 lambda: zk.binary_fwd("add", self.t, self.resid, out=self.out),
                 [nh, nh], [nh]),
            Call("mul_bwd(g;h,gamma)->grad_h,grad_gamma", "bwd",
                 lambda: zk.binary_bwd("mul", self.g, self.h, self.gamma, grad_a=self.grad_h,
                                       grad_b=self.grad_gamma, workspace=self.ws),
                 [nh, nh, ng], [nh, ng], reduce=ng),
            # add's gradient of t is g itself; resid's is materialised
            Call("add_bwd(g)->grad_resid", "bwd",
                 lambda: zk.binary_bwd("add", self.g, self.t, self.resid, need_a=False,
                                       grad_b=self.grad_resid, workspace=self.ws2),
                 [nh], [nh]),
        ]


# ------------------------------------------------------------------ fused
# The same expressions as one fused call each way (Operator chapter, "fusion":
# merged operators, same math): out = (a op1 b) op2 c forward, and the
# backward of all inputs from one pass over g.


class XYPlusXFused(Workload):
    """z = x*y + x as one fused call; x's two paths land in one buffer."""
    name = "xy_plus_x_fused"

    def __init__(self, host=None, scale=1):
        import torch
        h = host or W.xy_plus_x(scale)
        self.host = h
        d = {k: torch.from_numpy(v).to("cuda") for k, v in h.items()}
        self.x, self.y, self.g = d["x"], d["y"], d["g"]
        e = torch.empty_like
        self.z, self.grad_x, self.grad_y = e(self.x), e(self.x), e(self.y)
        self.ws = _ws(zk.bwd2_workspace_bytes("mul", "add", self.x, self.y, self.x,
                                              tie="a"), torch)
        nx, ny = _n(self.x.shape), _n(self.y.shape)
        self.calls = [
            Call("fused mul,add(x,y,x)->z", "fwd",
                 lambda: zk.binary2_fwd("mul", "add", self.x, self.y, self.x, out=self.z),
                 [nx, ny], [nx]),
            Call("fused bwd(g;x,y,x)->grad_x(both paths),grad_y", "bwd",
                 lambda: zk.binary2_bwd("mul", "add", self.g, self.x, self.y, self.x,
                                        need=(True, True, True),
                                        grads=(self.grad_x, self.grad_y, None), tie="a",
                                        workspace=self.ws),
                 [nx, nx, ny], [nx, ny], reduce=ny),
        ]


class AttnScaleMaskFused(Workload):
    """scores * scale + mask as one fused call; the mask gets no gradient."""
    name = "attn_scale_mask_fused"

    def __init__(self, host=None, b=8, h=16, t=1024):
        import torch
        hh = host or W.attn_scale_mask(b, h, t)
        self.host = hh
        d = {k: torch.from_numpy(v).to("cuda") for k, v in hh.items()}
        self.scores, self.scale, self.mask, self.g = d["scores"], d["scale"], d["mask"], d["g"]
        e = torch.empty_like
        self.out, self.grad_scores, self.grad_scale = e(self.scores), e(self.scores), e(self.scale)
        self.ws = _ws(zk.bwd2_workspace_bytes("mul", "add", self.scores, self.scale, self.mask,
                                              need=(True, True, False)), torch)
        ns, nc, nm = _n(self.scores.shape), _n(self.scale.shape), _n(self.mask.shape)
        self.calls = [
            Call("fused mul,add(scores,scale,mask)->out", "fwd",
                 lambda: zk.binary2_fwd("mul", "add", self.scores, self.scale, self.mask,
                                        out=self.out),
                 [ns, nc, nm], [ns]),
            Call("fused bwd(g;scores,scale,mask)->grad_scores,grad_scale", "bwd",
                 lambda: zk.binary2_bwd("mul", "add", self.g, self.scores, self.scale,
                                        self.mask, need=(True, True, False),
                                        grads=(self.grad_scores, self.grad_scale, None),
                                        workspace=self.ws),
                 [ns, ns, nc], [ns, nc], reduce=nc),
        ]


class GPTResidualFused(Workload):
    """h * gamma + resid as one fused call; grad_resid from the same pass."""
    name = "gpt_residual_fused"

    def __init__(self, host=None, b=16, t=2048, c=4096):
        import torch
        hh = host or W.gpt_residual(b, t, c)
        self.host = hh
        d = {k: torch.from_numpy(v).to("cuda") for k, v in hh.items()}
        self.h, self.gamma, self.resid, self.g = d["h"], d["gamma"], d["resid"], d["g"]
        e = torch.empty_like
        self.out, self.grad_h, self.grad_gamma = e(self.h), e(self.h), e(self.gamma)
        self.grad_resid = e(self.h)
        self.ws = _ws(zk.bwd2_workspace_bytes("mul", "add", self.h, self.gamma, self.resid),
                      torch)
        nh, ng = _n(self.h.shape), _n(self.gamma.shape)
        self.calls = [
            Call("fused mul,add(h,gamma,resid)->out", "fwd",
                 lambda: zk.binary2_fwd("mul", "add", self.h, self.gamma, self.resid,
                                        out=self.out),
                 [nh, ng, nh], [nh]),
            Call("fused bwd(g;h,gamma,resid)->grad_h,grad_gamma,grad_resid", "bwd",
                 lambda: zk.binary2_bwd("mul", "add", self.g, self.h, self.gamma, self.resid,
                                        grads=(self.grad_h, self.grad_gamma, self.grad_resid),
                                        workspace=self.ws),
                 [nh, nh, ng], [nh, ng, nh], reduce=ng),
        ]


# ------------------------------------------------------ other reductions


class GPTLossMeanClip(Workload):
    """The tail of the GPT chapter's training loop: the per-token loss
    averaged to a scalar and its gradient, then ClipGradNorm(1.0) over every
    parameter gradient.  The gradients live in one flat buffer (one tensor
    view per parameter); each step first rewrites them from a pristine copy,
    standing in for the backward pass that produces them, so that every
    step's clip scales (the clip leaves the norm just under the threshold)."""
    name = "gpt_loss_mean_clip"

    def __init__(self, host=None, b=64, t=256, max_norm=1.0):
        import torch
        hh = host or W.gpt_loss_mean_clip(b, t)
        self.host = hh
        self.loss = torch.from_numpy(hh["loss"]).to("cuda")
        self.g = torch.from_numpy(np.array(hh["g"], dtype=np.float32)).to("cuda")
        self.pristine = torch.from_numpy(hh["grads"]).to("cuda")
        self.grad_params = torch.empty_like(self.pristine)
        shapes = W.gpt_param_shapes(ctx=t)
        offs, _ = W.grad_arena_offsets(shapes)
        self.views = [self.grad_params[o:o + _n(s)].view(s) for o, s in zip(offs, shapes)]
        self.out = torch.empty((), dtype=torch.float32, device="cuda")
        self.grad_loss = torch.empty_like(self.loss)
        self.norm = torch.empty((), dtype=torch.float32, device="cuda")
        self.ws = _ws(zk.reduce_workspace_bytes(self.loss, ()), torch)
        self.ws_norm = _ws(zk.norm_workspace_bytes([v.numel() for v in self.views]), torch)
        nl, na = _n(self.loss.shape), _n(self.pristine.shape)
        npar = sum(v.numel() for v in self.views)
        self.calls = [
            Call("mean(per_token_loss[%d])->loss" % nl, "fwd",
                 lambda: zk.mean_to_shape(self.loss, (), out=self.out, workspace=self.ws),
                 [nl], [1]),
            Call("mean_bwd(g[])->grad_per_token_loss", "bwd",
                 lambda: zk.mean_bwd(self.g, self.loss.shape, out=self.grad_loss), [1], [nl]),
            Call("gradients rewritten from a pristine copy (stands in for backward)", "aux",
                 lambda: zk.materialize(self.pristine, out=self.grad_params), [na], [na]),
            # distinct elements: each gradient read (the kernels read it twice)
            # and written once, plus the norm
            Call("clip_grad_norm(%d grads, %g)" % (len(self.views), max_norm), "bwd",
                 lambda: zk.clip_grad_norm(self.views, max_norm, norm_out=self.norm,
                                           workspace=self.ws_norm),
                 [npar], [npar, 1]),
        ]


class GPTRowStats(Workload):
    """Per-row statistics of the GPT configuration: a LayerNorm's row mean
    and variance of x[64*256, 384] and a softmax's row max and sum of
    exponentials over the causal attention scores [64*6*256, 256]."""
    name = "gpt_row_stats"

    def __init__(self, host=None):
        import torch
        hh = host or W.gpt_row_stats()
        self.host = hh
        self.x = torch.from_numpy(hh["x"]).to("cuda")
        self.scores = torch.from_numpy(hh["scores"]).to("cuda")
        rx, cx = self.x.shape
        rs, cs = self.scores.shape
        e = torch.empty
        self.out_mean, self.out_var = e(rx, device="cuda"), e(rx, device="cuda")
        self.out_max, self.out_sumexp = e(rs, device="cuda"), e(rs, device="cuda")
        self.calls = [
            Call("row_moments(x[%d,%d])->mean,var" % (rx, cx), "fwd",
                 lambda: zk.row_moments(self.x, mean=self.out_mean, var=self.out_var),
                 [rx * cx], [rx, rx]),
            Call("row_softmax_stats(scores[%d,%d])->max,sumexp" % (rs, cs), "fwd",
                 lambda: zk.row_softmax_stats(self.scores, rowmax=self.out_max,
                                              sumexp=self.out_sumexp),
                 [rs * cs], [rs, rs]),
        ]


WORKLOAD_CLASSES = {c.name: c for c in (XYPlusX, MLPBiasGelu, AttnScaleMask,
                                        AttnMaskGrad, StridedTransposed, Rank8, GPTResidual,
                                        XYPlusXFused, AttnScaleMaskFused,
                                        GPTResidualFused, GPTLossMeanClip, GPTRowStats)}
