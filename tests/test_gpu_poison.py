"""Every workspace read is of an element the same call wrote: with the
workspace filled with NaN bytes before each call (ns_set_workspace_poison),
results stay bitwise what they are without the fill, and finite.  The output
buffer is pre-filled with NaN too, so an output element the last kernel
missed would show.  The cases cover each layout the driver sets up: the
mirrored Gram (192 and 128 tiles), the lower-block-triangle Gram of large
stacks (128 and 256 tiles), tall and wide inputs, zero-padded odd shapes, an
in-place call with an odd step count (the input copy), zero steps, fp32, and
a grouped call."""

import pytest
import torch

import newton_schulz_07_amd as ns
from ns_inputs import gaussian
from tests.gpu_util import device

pytestmark = pytest.mark.gpu

CASES = [
    ((1, 4096, 4096), torch.bfloat16, 5),   # 192 triangle tiles, mirrored Gram
    ((3, 264, 520), torch.bfloat16, 5),     # ragged 128 tiles
    ((400, 264, 520), torch.bfloat16, 2),   # lower-triangle Gram, 128 tiles
    ((200, 520, 264), torch.bfloat16, 2),   # same, tall
    ((64, 1536, 2048), torch.bfloat16, 2),  # lower-triangle Gram, 256 tiles
    ((3, 100, 37), torch.bfloat16, 3),      # padded copy in and out
    ((2, 264, 520), torch.float32, 3),      # fp32 path
    ((2, 136, 72), torch.bfloat16, 0),      # normalisation only
]


def poisoned(fn):
    ns.ns_set_workspace_poison(True)
    try:
        return fn()
    finally:
        ns.ns_set_workspace_poison(False)


def nan_like(x):
    return torch.full_like(x, float("nan"))


@pytest.mark.parametrize("shape,dtype,steps", CASES)
def test_poisoned_workspace_changes_nothing(shape, dtype, steps):
    dev = device()
    x = gaussian(shape, 900 + sum(shape)).to(dtype).to(dev)
    ref = ns.orthogonalize(x, steps=steps)
    y = poisoned(lambda: ns.orthogonalize(x, steps=steps, out=nan_like(x)))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()), f"{shape}: NaN reached the output"
    assert torch.equal(y, ref), f"{shape}: result differs with a poisoned workspace"


def test_poisoned_workspace_in_place_odd_steps():
    dev = device()
    x = gaussian((4, 264, 520), 77).to(torch.bfloat16).to(dev)
    ref = ns.orthogonalize(x, steps=3)
    y = x.clone()
    poisoned(lambda: ns.orthogonalize(y, steps=3, out=y))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    assert torch.equal(y, ref)


def test_poisoned_workspace_grouped():
    dev = device()
    shapes = [(2, 264, 520), (3, 520, 264), (1, 100, 37), (5, 512, 512)]
    xs = [gaussian(s, 31 + i).to(torch.bfloat16).to(dev) for i, s in enumerate(shapes)]
    refs = [ns.orthogonalize(x) for x in xs]
    outs = [nan_like(x) for x in xs]
    poisoned(lambda: ns.orthogonalize_grouped(xs, outs=outs))
    torch.cuda.synchronize()
    for s, y, r in zip(shapes, outs, refs):
        assert bool(torch.isfinite(y).all()), s
        assert torch.equal(y, r), s
