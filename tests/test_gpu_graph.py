"""The streams contract: once the workspace of (device, stream) is warm, a call
makes no allocation and no synchronisation and enqueues only kernels (and,
in place with an odd step count, one device copy), so it can be captured into
a HIP graph and replayed.

Each case warms the workspace on a side stream, captures one call on that
stream, and replays the graph several times with eager work and
synchronisations between the replays; every replay must equal the eager
result bitwise, and the library's workspace-allocation count must not move.
"""

import pytest
import torch

import newton_schulz_07_amd as ns
from ns_inputs import gaussian
from tests.gpu_util import device

pytestmark = pytest.mark.gpu

CASES = [
    ((1, 256, 512), torch.bfloat16, 5, False),
    ((4, 264, 392), torch.bfloat16, 5, False),
    ((2, 392, 264), torch.float32, 3, False),
    ((1, 1024, 1024), torch.bfloat16, 5, False),
    ((3, 45, 70), torch.bfloat16, 5, False),   # zero-padded path
    ((2, 256, 384), torch.bfloat16, 3, True),  # in place, odd step count: input copy
]


@pytest.mark.parametrize("shape,dtype,steps,in_place", CASES)
def test_warm_call_replays_from_a_graph(shape, dtype, steps, in_place):
    dev = device()
    print(f"graph case {shape} {dtype} steps={steps} in_place={in_place}", flush=True)
    x0 = gaussian(shape, 1300 + sum(shape) + steps, dtype).to(dev)
    other = gaussian((2, 128, 256), 1399, dtype).to(dev)
    s = torch.cuda.Stream()
    x = x0.clone()
    out = x if in_place else torch.empty_like(x)
    with torch.cuda.stream(s):
        ns.orthogonalize(x, steps=steps, out=out)  # warms the workspace of (device, s)
    s.synchronize()
    want = out.clone()
    n0 = ns.ns_workspace_allocations()

    x.copy_(x0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ns.orthogonalize(x, steps=steps, out=out)
    assert ns.ns_workspace_allocations() == n0, "the captured call allocated"

    for r in range(4):
        # eager work between the replays: refill the input, poison the
        # output, and an unrelated eager call on the default stream
        x.copy_(x0)
        if not in_place:
            out.fill_(float("nan"))
        ns.orthogonalize(other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r} differs from the eager call"
    assert ns.ns_workspace_allocations() == n0
    del g


def test_grouped_call_replays_from_a_graph():
    dev = device()
    shapes = [(2, 256, 512), (1, 512, 256), (3, 136, 200)]
    xs = [gaussian(sh, 1450 + i, torch.bfloat16).to(dev) for i, sh in enumerate(shapes)]
    outs = [torch.empty_like(x) for x in xs]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ns.orthogonalize_grouped(xs, outs=outs)
    s.synchronize()
    want = [o.clone() for o in outs]
    n0 = ns.ns_workspace_allocations()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ns.orthogonalize_grouped(xs, outs=outs)
    for r in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o, w), f"replay {r}"
    assert ns.ns_workspace_allocations() == n0
    del g


def test_warm_calls_do_not_allocate():
    # the counter itself: a first call on a new stream allocates once, a
    # smaller call after it does not, a larger one allocates once more
    dev = device()
    s = torch.cuda.Stream()
    big = gaussian((2, 512, 768), 1470, torch.bfloat16).to(dev)
    small = gaussian((1, 256, 512), 1471, torch.bfloat16).to(dev)
    n0 = ns.ns_workspace_allocations()
    with torch.cuda.stream(s):
        ns.orthogonalize(small)
        n1 = ns.ns_workspace_allocations()
        ns.orthogonalize(small)
        n2 = ns.ns_workspace_allocations()
        ns.orthogonalize(big)
        n3 = ns.ns_workspace_allocations()
        ns.orthogonalize(small)
        n4 = ns.ns_workspace_allocations()
    s.synchronize()
    assert (n1 - n0, n2 - n1, n3 - n2, n4 - n3) == (1, 0, 1, 0)
