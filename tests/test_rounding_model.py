"""Pins of the bf16 rounding-placement model (oracle/rounding_model.py).

The model sets the floors of the bf16 parity bars on the two inputs where no
bf16-iterate NS reaches 1e-2, so it is pinned to things other than itself:

  * algebra: with every bf16 rounding replaced by the identity and all
    arithmetic in float64, each placement is the oracle's iteration regrouped,
    so it must equal the fp64 oracle to float64 rounding; planted slips in the
    diagonal restoration or in the folded normalisation's scalings fail it;
  * an exact identity: when ||x||_F is a power of two, x / ||x|| is exact in
    bf16, so folding the normalisation into the first step must give the same
    bits as normalising first;
  * independent earlier CPU probes of the three placements with a stored
    bf16 X0 (literal / fold / diagAC on a 256x512 fp32 matrix cast to bf16, a
    1536x2048 iid slice and a tall 7168x2048 iid slice), within ±10%.  Those
    probes record no seed for the two iid slices (any iid draw of the shape
    lands within a few percent), so fixed seeds are used here.

Reference for the placements: prime-rl PR #3873, the note under the NS
microbenchmark table (an fp32 alpha/beta epilogue as the accuracy reason).
"""

import json
import os

import numpy as np
import pytest
import torch

from ns_inputs import gaussian, make_workload
from oracle import newton_schulz
from oracle import rounding_model as rm
from oracle.rounding_model import PLACEMENTS, ns_bf16_model

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rounding_floor.json")


def rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def exact(x, **kw):
    return ns_bf16_model(x, rounding=False, work=torch.float64, **kw)


@pytest.mark.parametrize("shape", [(24, 40), (40, 24), (16, 16), (8, 8)])
@pytest.mark.parametrize("placement", PLACEMENTS)
@pytest.mark.parametrize("fold_norm", [False, True])
@pytest.mark.parametrize("steps", [0, 1, 5])
def test_identity_rounding_equals_oracle(shape, placement, fold_norm, steps):
    x = gaussian(shape, 40 + sum(shape) + steps).double().numpy() * 3.0
    y = exact(x, placement=placement, fold_norm=fold_norm, steps=steps)
    assert y.shape == x.shape
    assert rel(y, newton_schulz(x, steps)) <= 1e-12


def test_identity_rounding_float32_is_the_fp32_path():
    # float32 arithmetic without bf16 storage: the fp32 path's error level
    x = make_workload("iid_256x512").double().numpy()
    y = ns_bf16_model(x, rounding=False, work=torch.float32)
    assert rel(y, newton_schulz(x)) <= 1e-5


MUTANTS_SPLIT = {
    "dropped (d_i + d_j) O_A": lambda OA, dA, a, b, c: (
        b * OA + c * (OA @ OA), a + b * dA + c * (torch.diagonal(OA @ OA) + dA * dA)),
    "2 d_i for d_i + d_j": lambda OA, dA, a, b, c: (
        b * OA + c * (OA @ OA + 2 * dA[:, None] * OA), a + b * dA + c * (torch.diagonal(OA @ OA) + dA * dA)),
    "dropped d_i² on the diagonal": lambda OA, dA, a, b, c: (
        b * OA + c * (OA @ OA + (dA[:, None] + dA[None, :]) * OA), a + b * dA + c * torch.diagonal(OA @ OA)),
    "a missing from d_C": lambda OA, dA, a, b, c: (
        b * OA + c * (OA @ OA + (dA[:, None] + dA[None, :]) * OA), b * dA + c * (torch.diagonal(OA @ OA) + dA * dA)),
    "b and c swapped on the diagonal": lambda OA, dA, a, b, c: (
        b * OA + c * (OA @ OA + (dA[:, None] + dA[None, :]) * OA), a + c * dA + b * (torch.diagonal(OA @ OA) + dA * dA)),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS_SPLIT))
def test_planted_restoration_mistakes_fail(mutant, monkeypatch):
    x = gaussian((24, 40), 77).double().numpy()
    ref = newton_schulz(x)
    assert rel(exact(x, placement="diagAC"), ref) <= 1e-12
    monkeypatch.setattr(rm, "_split_poly", MUTANTS_SPLIT[mutant])
    assert not rel(exact(x, placement="diagAC"), ref) <= 1e-6


@pytest.mark.parametrize("mutant", [lambda inv: (inv, inv), lambda inv: (inv * inv, 1.0),
                                    lambda inv: (inv * inv, inv * inv)])
def test_planted_folded_norm_mistakes_fail(mutant, monkeypatch):
    x = gaussian((24, 40), 78).double().numpy() * 5.0
    ref = newton_schulz(x)
    monkeypatch.setattr(rm, "_first_step_scales", mutant)
    assert not rel(exact(x, fold_norm=True), ref) <= 1e-6  # (a diverging mutant gives NaN)


def _power_of_two_norm_matrix(shape, nnz, seed):
    # entries in {-1, 0, 1} with nnz nonzeros: ||x||_F = sqrt(nnz)
    rng = np.random.default_rng(seed)
    x = np.zeros(shape)
    pos = rng.choice(shape[0] * shape[1], size=nnz, replace=False)
    x.flat[pos] = rng.choice([-1.0, 1.0], size=nnz)
    return x


@pytest.mark.parametrize("shape,nnz", [((16, 24), 64), ((24, 16), 64), ((32, 64), 256)])
@pytest.mark.parametrize("placement", PLACEMENTS)
def test_folded_norm_is_exact_when_the_norm_is_a_power_of_two(shape, nnz, placement):
    # 1/(||x|| + 1e-7) rounds to 2^-k in float32, so X0 = x 2^-k is exact in
    # bf16 and every float32 product of the folded first step is the
    # unfolded one times a power of two
    x = _power_of_two_norm_matrix(shape, nnz, nnz + shape[0])
    y0 = ns_bf16_model(x, placement=placement, fold_norm=False)
    y1 = ns_bf16_model(x, placement=placement, fold_norm=True)
    assert np.array_equal(y0, y1)


def test_folded_norm_differs_on_a_general_input():
    # the contrapositive: a general bf16 input is not exact after scaling,
    # so the two placements must differ (the flag is not a no-op)
    x = make_workload("iid_256x512").to(torch.bfloat16).double().numpy()
    assert not np.array_equal(ns_bf16_model(x, fold_norm=False), ns_bf16_model(x, fold_norm=True))


# The recorded probes (stored bf16 X0): relative Frobenius error vs fp64.
PROBES = {
    "cfg1": {"literal": 1.11e-2, "fold": 8.57e-3, "diagAC": 5.89e-3},
    "iid_1536x2048": {"literal": 8.46e-3, "fold": 8.13e-3, "diagAC": 5.86e-3},
    "iid_7168x2048": {"literal": 9.54e-3, "diagAC": 4.84e-3},
}


def _probe_input(case):
    if case == "cfg1":
        x = make_workload("iid_256x512")  # fp32; the bf16 path casts it
        return x.double().numpy(), x.to(torch.bfloat16).double().numpy()
    shape = {"iid_1536x2048": (1536, 2048), "iid_7168x2048": (7168, 2048)}[case]
    x = gaussian(shape, {"iid_1536x2048": 11, "iid_7168x2048": 12}[case], torch.bfloat16)
    xd = x.double().numpy()
    return xd, xd


@pytest.fixture(scope="module")
def probes():
    cache = {}

    def get(case):
        if case not in cache:
            x_ref, x_in = _probe_input(case)
            cache[case] = (x_in, newton_schulz(x_ref))
        return cache[case]
    return get


@pytest.mark.parametrize("case,placement", [(c, p) for c in PROBES for p in PROBES[c]])
def test_recorded_probes_within_10_percent(case, placement, probes):
    x_in, ref = probes(case)
    e = rel(ns_bf16_model(x_in, placement=placement, fold_norm=False), ref)
    want = PROBES[case][placement]
    assert abs(e - want) <= 0.10 * want, (e, want)


def test_golden_floor_is_the_shipped_placement():
    # the stored floors must come from the current model (diagAC, folded
    # normalisation): recompute the small case and compare
    with open(GOLDEN) as f:
        golden = json.load(f)["workloads"]["iid_256x512"]["0"]
    x = make_workload("iid_256x512")
    ref = newton_schulz(x.double().numpy())
    xb = x.to(torch.bfloat16).double().numpy()
    assert golden["shipped"] == pytest.approx(rel(ns_bf16_model(xb), ref), rel=1e-9)
    assert golden["literal"] == pytest.approx(rel(ns_bf16_model(xb, placement="literal", fold_norm=False), ref),
                                              rel=1e-9)
