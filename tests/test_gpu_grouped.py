"""ns_orthogonalize_grouped: several stacks of different shapes in one call.

Every slice's result must be bitwise the one ns_orthogonalize gives for its
own stack (the grouped launches only change which workgroups run together
and, through the shared tile counts, which tile class runs; each output
element's accumulation order is the same in every tile class), and within
the oracle bars: relative Frobenius error per slice <= 1e-4 (fp32) and
<= 1e-2 (bf16).
"""

import pytest
import torch

import newton_schulz_07_amd as ns
from ns_inputs import gaussian
from oracle import newton_schulz
from tests.gpu_util import device, rel_err, report, to64

pytestmark = pytest.mark.gpu

MIXED = [(2, 264, 520), (3, 520, 264), (1, 100, 37), (4, 128, 128), (1, 1024, 3072), (2, 3072, 1024)]


def make(shapes, dtype, seed0=900):
    dev = device()
    return [gaussian(s, seed0 + i, dtype).to(dev) for i, s in enumerate(shapes)]


def singles(xs, steps=5):
    return [ns.orthogonalize(x, steps=steps) for x in xs]


def assert_bitwise(ys, refs):
    torch.cuda.synchronize()
    for i, (y, r) in enumerate(zip(ys, refs)):
        assert y.shape == r.shape and y.dtype == r.dtype
        assert torch.equal(y, r), f"stack {i} differs from its own call"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_mixed_stacks_match_single_calls_and_oracle(dtype):
    xs = make(MIXED, dtype)
    ys = ns.orthogonalize_grouped(xs)
    assert "grouped: 6 stacks (3 wide, 3 tall)" in ns.ns_query_last_config()
    assert_bitwise(ys, singles(xs))
    bar = 1e-4 if dtype == torch.float32 else 1e-2
    errs = {}
    for i in (0, 1, 2, 4):  # one slice of several stacks (the oracle runs slice by slice)
        e = float(rel_err(to64(ys[i][0]), newton_schulz(to64(xs[i][0])))[0])
        errs[i] = e
        assert e <= bar, (i, e)
    report({"case": f"grouped_mixed_{dtype}", "errs": errs})


def test_more_than_sixteen_stacks():
    # 20 stacks: the launches split into groups of at most 16 stacks
    shapes = [(1 + i % 3, 8 + 8 * i, 16 + 8 * ((i * 7) % 13)) for i in range(20)]
    xs = make(shapes, torch.bfloat16, 950)
    ys = ns.orthogonalize_grouped(xs)
    assert_bitwise(ys, singles(xs))


def test_tile_classes_differ_from_the_single_calls():
    # alone, the 6-slice stack runs its Gram and poly on 192 tiles; grouped
    # with 200 tall slices the poly launch takes 128 tiles; the 400-slice
    # stack takes the 256 Gram tile and A as its lower block triangle
    shapes = [(6, 264, 520), (200, 520, 264), (400, 264, 520)]
    xs = make(shapes, torch.bfloat16, 970)
    ys = ns.orthogonalize_grouped(xs)
    cfg = ns.ns_query_last_config()
    assert "poly: lower-tri tile=128x128" in cfg, cfg
    assert_bitwise(ys, singles(xs))
    ys2 = ns.orthogonalize_grouped(xs[:2])
    assert "A read as its lower block triangle" not in ns.ns_query_last_config()  # 192 Gram tiles beside it
    assert_bitwise(ys2, singles(xs[:2]))


@pytest.mark.parametrize("steps", [0, 1, 3])
def test_in_place_odd_steps_padding_and_empty_stacks(steps):
    shapes = [(2, 264, 520), (0, 64, 64), (3, 9, 13), (1, 520, 264)]
    xs = make(shapes, torch.bfloat16, 990)
    want = [ns.orthogonalize(x, steps=steps) if x.numel() else x.clone() for x in xs]
    work = [x.clone() for x in xs]
    outs = ns.orthogonalize_grouped(work, steps=steps, outs=work)  # in place
    assert all(o is w for o, w in zip(outs, work))
    assert_bitwise(work, want)


def test_one_launch_per_stage_kind():
    xs = make(MIXED, torch.bfloat16, 1010)
    ns.orthogonalize_grouped(xs)  # warm
    torch.cuda.synchronize()
    ns.ns_timing_enable((1 << ns.NS_KIND_SUMSQ) | (1 << ns.NS_KIND_GRAM) | (1 << ns.NS_KIND_POLY)
                        | (1 << ns.NS_KIND_UPDATE))
    ns.ns_timing_reset()
    try:
        ns.orthogonalize_grouped(xs, steps=5)
        torch.cuda.synchronize()
        counts = {k: ns.ns_timing_query(k)[1] for k in (ns.NS_KIND_SUMSQ, ns.NS_KIND_GRAM, ns.NS_KIND_POLY,
                                                         ns.NS_KIND_UPDATE)}
    finally:
        ns.ns_timing_enable(0)
        ns.ns_timing_reset()
    # wide and tall stacks: two Gram and two update launches per step; the
    # sums of squares: one launch over the stacks whose sides are multiples
    # of 8, and for each other stack its zero-padded copy pass, which
    # computes them (here the 100 x 37 stack)
    padded = sum(1 for _, r, c in MIXED if r % 8 or c % 8)
    assert padded == 1
    assert counts == {ns.NS_KIND_SUMSQ: 1 + padded, ns.NS_KIND_GRAM: 10, ns.NS_KIND_POLY: 5,
                      ns.NS_KIND_UPDATE: 10}, counts


def test_grouped_errors_raise():
    dev = device()
    x = torch.zeros(2, 64, 64, device=dev, dtype=torch.bfloat16)
    with pytest.raises(ns.NSError):
        ns.orthogonalize_grouped([x, x[0:1]], outs=[x, x[1:2]])  # out 1 overlaps stack 0
    with pytest.raises(ValueError):
        ns.orthogonalize_grouped([x, x.float()])
