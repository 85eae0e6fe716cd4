"""Every workload's step captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: each replay, and each eager step run between replays, must
reproduce the eager result bit for bit (every tensor of the step, inputs
and outputs).  The library issues no memset or copy, only kernels on the
caller's stream, so a captured step is the same kernels with the same
arguments; the backward's binary64 partials are rewritten by every step.
The no-alloc backward (its partials in the library's own device scratch)
is captured the same way."""
import ctypes
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from broadcast_autograd_amd import steps, zk  # noqa: E402
from gpu_util import dev  # noqa: E402


@pytest.fixture(autouse=True)
def _name(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


# (workload class, generator arguments): reduced sizes of every workload
CASES = [
    ("xy_plus_x", {}),
    ("mlp_bias_gelu", {"rows": 256, "cols": 1024}),
    ("attn_scale_mask", {"b": 2, "h": 16, "t": 128}),
    ("attn_mask_grad", {"b": 2, "h": 16, "t": 128}),
    ("strided_transposed", {"n": 512}),
    ("rank8_div", {}),
    ("gpt_residual", {"b": 1, "t": 64, "c": 4096}),
    ("xy_plus_x_fused", {}),
    ("attn_scale_mask_fused", {"b": 2, "h": 16, "t": 128}),
    ("gpt_residual_fused", {"b": 1, "t": 64, "c": 4096}),
    ("gpt_loss_mean_clip", {"b": 4, "t": 256}),
    ("gpt_row_stats", {}),
]


def _snapshot(wl):
    return {k: v.detach().clone() for k, v in vars(wl).items()
            if isinstance(v, torch.Tensor) and v.is_cuda and not k.startswith("ws")}


def _same(ref, got, what):
    for k, v in ref.items():
        a = v.reshape(-1).contiguous().view(torch.uint8)
        b = got[k].reshape(-1).contiguous().view(torch.uint8)
        assert torch.equal(a, b), f"{what}: {k} differs"


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_step_graph_replays(name, kw):
    cls = steps.WORKLOAD_CLASSES[name]
    wl = cls(**kw)
    wl.run()
    torch.cuda.synchronize()
    ref = _snapshot(wl)
    g = _capture(wl.run)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        _same(ref, _snapshot(wl), f"{name} replay {rep}")
        wl.run()  # eager work between replays
        torch.cuda.synchronize()
        _same(ref, _snapshot(wl), f"{name} eager after replay {rep}")


def test_noalloc_backward_graph_replays():
    """zk_binary_bwd_noalloc captured: replays match the workspace call."""
    rng = np.random.default_rng(77)
    a = dev(rng.standard_normal((2048, 1024)).astype(np.float32))
    b = dev(rng.standard_normal(1024).astype(np.float32))
    gr = dev(rng.standard_normal((2048, 1024)).astype(np.float32))
    ga_ref, gb_ref = zk.binary_bwd("mul", gr, a, b, epi="gelu")
    ga, gb = torch.empty_like(a), torch.empty_like(b)
    da, db = zk.desc_of(a), zk.desc_of(b)

    def call():
        s = torch.cuda.current_stream()
        rc = zk.lib().zk_binary_bwd_noalloc(
            zk.OPS["mul"], zk.EPIS["gelu"], zk._ptr(gr), zk._ptr(a), ctypes.byref(da),
            zk._ptr(b), ctypes.byref(db), zk._ptr(ga), None, zk._ptr(gb), None,
            ctypes.c_void_p(s.cuda_stream))
        assert rc == 0

    g = _capture(call)
    for rep in range(3):
        ga.fill_(0.0)
        gb.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ga.view(torch.int32), ga_ref.view(torch.int32)), rep
        assert torch.equal(gb.view(torch.int32), gb_ref.view(torch.int32)), rep
        call()  # an eager no-alloc call between replays shares the scratch
        torch.cuda.synchronize()
