"""Full-size parity: every named workload at its real shape, in the launch
configuration the benchmark times (the whole stack in one call), against the
fp64 oracle on every slice (the oracle computes slices one by one).

Bars (relative Frobenius error per slice):
  * bf16 path: <= 1e-2, and on the slices the CPU rounding model covers
    (tests/golden/rounding_floor.json, 'shipped': the placement the library
    uses) <= 1.1 x the model's error.  Two workloads cannot meet 1e-2 with ANY
    bf16 iterate: on the rank-64-plus-noise square and the rank-32-plus-noise
    MLP weight the low-rank part dominates every entry, so rounding X to bf16
    perturbs the noise subspace by about the noise itself, and NS amplifies
    small singular values (about a^5 ≈ 485).  The model puts their floor above
    1e-2; for those only the 1.1 x model bar applies, and a strict xfail
    records the 1e-2 miss.  The kernels are bitwise deterministic, so these
    numbers do not move from run to run.
  * fp32 path on the same inputs: <= 1e-4, which checks every tile of the
    kernels at full size.
"""

import json
import os

import numpy as np
import pytest
import torch

import newton_schulz_07_amd as ns
from ns_inputs import WORKLOADS, make_workload
from oracle import newton_schulz, newton_schulz_batched
from oracle.ns_oracle import DEFAULT_COEFFS, EPS, ns_iteration
from ns_inputs import gaussian
from tests.gpu_util import device, rel_err, report, to64

pytestmark = pytest.mark.gpu

FLOOR = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rounding_floor.json")))["workloads"]
FLOORED = {"lowrank64_4096x4096", "mlp_4096x14336", "mlp_14336x4096"}

_oracle_cache = {}


def oracle_slice(name, x, i):
    key = (name, i)
    if key not in _oracle_cache:
        if name == "mlp_14336x4096" and ("mlp_4096x14336", i) in _oracle_cache:
            _oracle_cache[key] = _oracle_cache[("mlp_4096x14336", i)].T
        else:
            _oracle_cache[key] = newton_schulz(x.double().numpy())
    return _oracle_cache[key]


def run(name, dtype):
    """One whole-stack call; the error of every slice against the oracle."""
    w = WORKLOADS[name]
    x = make_workload(name)
    xg = x.to(dtype).to(device())
    y = ns.orthogonalize(xg)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    xs = x.reshape(-1, w.rows, w.cols)
    ys = y.reshape(-1, w.rows, w.cols).cpu()
    del xg, y
    errs = {}
    for i in range(w.batch):
        errs[i] = float(rel_err(to64(ys[i]), oracle_slice(name, xs[i], i))[0])
    return errs


NAMES = ["lowrank64_4096x4096", "mlp_4096x14336", "mlp_14336x4096", "experts16_1536x2048",
         "experts128_1536x2048", "experts32_7168x2048", "square_8192x8192", "experts128_2048x768"]


def summary(errs):
    v = np.array(list(errs.values()))
    return {"slices": len(v), "max": float(v.max()), "mean": float(v.mean()), "argmax": int(v.argmax())}


@pytest.mark.parametrize("name", NAMES)
def test_full_size_bf16(name):
    errs = run(name, torch.bfloat16)
    floors = {int(k): v["shipped"] for k, v in FLOOR[name].items()}
    report({"case": f"full_bf16_{name}", **summary(errs), "model_floor": floors})
    for i, e in errs.items():
        if i in floors:
            assert e <= 1.1 * floors[i], (i, e, floors[i])
        if name not in FLOORED:
            assert e <= 1e-2, (i, e)


@pytest.mark.parametrize("name", sorted(FLOORED))
@pytest.mark.xfail(strict=True, reason="inherent bf16-iterate floor above 1e-2 on this input "
                                       "(see tests/golden/rounding_floor.json)")
def test_full_size_bf16_meets_1e_2_on_floored_inputs(name):
    errs = run(name, torch.bfloat16)
    assert max(errs.values()) <= 1e-2


@pytest.mark.parametrize("name", NAMES)
def test_full_size_fp32(name):
    errs = run(name, torch.float32)
    report({"case": f"full_fp32_{name}", **summary(errs)})
    assert max(errs.values()) <= 1e-4


@pytest.mark.parametrize("name,slices", [("experts128_1536x2048", (0, 63, 127)),
                                         ("experts128_2048x768", (0, 64, 127)),
                                         ("experts32_7168x2048", (0, 31))])
def test_full_size_batch_invariance(name, slices):
    # slice i of the whole-stack call (lower-block-triangle A, stack tile
    # classes, XCD-remapped grid) equals the single-slice call bitwise
    w = WORKLOADS[name]
    xg = make_workload(name).to(device())
    y = ns.orthogonalize(xg)
    for i in slices:
        yi = ns.orthogonalize(xg[i:i + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(yi[0], y[i]), f"slice {i} of {w.shape} differs from its single-slice call"


@pytest.mark.parametrize("name", ["iid_256x512", "lowrank64_4096x4096", "experts16_1536x2048",
                                  "experts128_2048x768"])
def test_bf16_at_least_as_accurate_as_dense_bf16(name):
    # [p1] NS microbenchmark table: the symmetric path is no less accurate than
    # the dense bf16 routine.  The comparator is the same method with dense
    # bf16 PyTorch matmuls (bench.dense_ns), on the same bf16 input.
    from bench import dense_ns
    w = WORKLOADS[name]
    x = make_workload(name)
    xg = x.to(torch.bfloat16).to(device())
    y = ns.orthogonalize(xg)
    yd = dense_ns(xg)
    torch.cuda.synchronize()
    xs = x.reshape(-1, w.rows, w.cols)
    ys, yds = y.reshape(-1, w.rows, w.cols), yd.reshape(-1, w.rows, w.cols)
    errs = {}
    for i in range(w.batch):
        ref = oracle_slice(name, xs[i], i)
        errs[i] = (float(rel_err(to64(ys[i]), ref)[0]), float(rel_err(to64(yds[i]), ref)[0]))
    report({"case": f"vs_dense_{name}", "max_ours": max(e for e, _ in errs.values()),
            "max_dense": max(d for _, d in errs.values())})
    for i, (e, ed) in errs.items():
        assert e <= ed, (i, e, ed)


@pytest.mark.parametrize("dtype,bar", [(torch.bfloat16, 1e-2), (torch.float32, 1e-4)])
def test_max_slice_block_diagonal(dtype, bar):
    # a 16384 x 16384 slice (2^28 elements, the largest power-of-two square
    # under the 2^29-element slice limit), block diagonal with four 4096 x
    # 4096 blocks.  A = X Xᵀ, C and every iterate stay block diagonal, so the
    # off-diagonal blocks of the result are exactly zero, and diagonal block
    # b is the oracle's iteration applied to X_b / (||X||_F + eps): the
    # normalisation is the whole matrix's, so each block is checked with the
    # oracle's step function at that global scale.
    n, k = 16384, 4096
    blocks = [gaussian((k, k), 1700 + b, torch.float32) * (0.5 + b) for b in range(4)]
    x = torch.zeros(n, n, dtype=torch.float32)
    for b, xb in enumerate(blocks):
        x[b * k:(b + 1) * k, b * k:(b + 1) * k] = xb
    x = x.to(dtype)
    y = ns.orthogonalize(x.to(device()))
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    mask = torch.ones(n, n, dtype=torch.bool, device=y.device)
    for b in range(4):
        mask[b * k:(b + 1) * k, b * k:(b + 1) * k] = False
    assert int(torch.count_nonzero(y[mask])) == 0, "off-diagonal blocks are not exactly zero"
    xd = x.double().numpy()
    nrm = float(np.sqrt(sum(float((x[b * k:(b + 1) * k, b * k:(b + 1) * k].double() ** 2).sum()) for b in range(4))))
    a, bb, c = DEFAULT_COEFFS
    errs = []
    for b in range(4):
        z = xd[b * k:(b + 1) * k, b * k:(b + 1) * k] / (nrm + EPS)
        for _ in range(5):
            z = ns_iteration(z, a, bb, c)
        got = to64(y[b * k:(b + 1) * k, b * k:(b + 1) * k])
        errs.append(float(np.linalg.norm(got - z) / np.linalg.norm(z)))
    report({"case": f"max_slice_block_diagonal_{dtype}", "errs": errs})
    assert max(errs) <= bar, errs


def test_max_batch():
    # 65535 slices (the batch limit) of 8 x 16, bf16: every slice finite,
    # sampled slices against the oracle
    x = gaussian((65535, 8, 16), 1750, torch.float32)
    y = ns.orthogonalize(x.to(torch.bfloat16).to(device()))
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    idx = [0, 1, 4095, 32767, 65534]
    ref = newton_schulz_batched(x.to(torch.bfloat16).double().numpy(), slices=idx)
    e = rel_err(to64(y[idx]), ref)
    report({"case": "max_batch", "errs": e.tolist()})
    assert e.max() <= 1e-2, e
