"""The allocation-free entry point, ns_orthogonalize_noalloc, through the C ABI.

It runs the same kernels as ns_orthogonalize on the library's fixed device
scratch array instead of an allocated workspace, so its results must equal
ns_orthogonalize's bitwise, call after call (the array keeps the previous
call's contents, so a larger call followed by a smaller one checks that
nothing stale is read), and it must make no workspace allocation.
"""

import ctypes

import numpy as np
import pytest
import torch

import newton_schulz_07_amd as ns
from ns_inputs import gaussian
from oracle import newton_schulz_batched
from tests.gpu_util import device, rel_err, to64

pytestmark = pytest.mark.gpu

# (first call, second smaller call) shapes and dtype
PAIRS = [
    (((4, 264, 392), torch.bfloat16), ((1, 256, 512), torch.bfloat16)),
    (((1, 1024, 2048), torch.bfloat16), ((2, 392, 264), torch.bfloat16)),
    (((2, 512, 768), torch.float32), ((3, 45, 70), torch.float32)),
    (((1, 4096, 4096), torch.bfloat16), ((16, 136, 200), torch.bfloat16)),
]


def raw_noalloc(x, out, steps=5):
    # the C ABI itself, as a caller without the Python wrapper would call it
    L = ns.lib()
    batch, rows, cols = ns._brc(x)
    st = L.ns_orthogonalize_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()), batch, rows,
                                    cols, ns._dtype_code(x), steps, *ns.DEFAULT_COEFFS,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_equals_ns_orthogonalize_twice(first, second):
    dev = device()
    for k, (shape, dtype) in enumerate((first, second)):
        print(f"noalloc call {k}: {shape} {dtype}", flush=True)
        x = gaussian(shape, 1500 + sum(shape), dtype).to(dev)
        out = torch.full_like(x, float("nan"))
        n0 = ns.ns_workspace_allocations()
        assert raw_noalloc(x, out) == 0, ns.lib().ns_last_error().decode()
        assert "fixed scratch" in ns.ns_query_last_config()
        torch.cuda.synchronize()
        assert ns.ns_workspace_allocations() == n0, "the no-alloc entry point allocated a workspace"
        want = ns.orthogonalize(x)
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"call {k} ({shape}) differs from ns_orthogonalize"


def test_noalloc_matches_the_oracle_and_runs_in_place():
    dev = device()
    x = gaussian((3, 200, 136), 1550, torch.float32)
    ref = newton_schulz_batched(x.double().numpy(), steps=3)
    xg = x.to(dev)
    ns.ns_orthogonalize_noalloc(xg, xg, ns_steps=3)  # in place, odd step count: input copy in the scratch
    torch.cuda.synchronize()
    assert rel_err(to64(xg), ref).max() <= 1e-4
    xb = x.to(torch.bfloat16).to(dev)
    yb = ns.ns_orthogonalize_noalloc(xb, torch.empty_like(xb), ns_steps=3)
    torch.cuda.synchronize()
    assert np.all(rel_err(to64(yb), ref) <= 1e-2)


def test_noalloc_rejects_a_call_larger_than_the_scratch():
    dev = device()
    need = ns.ns_workspace_bytes(1, 8192, 8192, ns.NS_DTYPE_BF16)
    assert need > ns.NS_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(8192, 8192, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ns.NSError) as ei:
        ns.ns_orthogonalize_noalloc(x, torch.empty_like(x))
    assert ei.value.status == 7 and "fixed scratch" in str(ei.value)


def test_noalloc_call_replays_from_a_graph_without_warm_up():
    # no warm-up call on the capture stream: the scratch needs none.  (The
    # first call on a device looks the scratch's address up once; that call
    # is made eagerly here, on the default stream, with another shape.)
    dev = device()
    x = gaussian((2, 256, 384), 1560, torch.bfloat16).to(dev)
    out = torch.empty_like(x)
    e = gaussian((1, 64, 128), 1561, torch.bfloat16).to(dev)
    ns.ns_orthogonalize_noalloc(e, torch.empty_like(e))
    want = ns.orthogonalize(x)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    n0 = ns.ns_workspace_allocations()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ns.ns_orthogonalize_noalloc(x, out)
    for r in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r}"
    assert ns.ns_workspace_allocations() == n0
    del g
