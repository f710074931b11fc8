"""Single-kernel parity: each stage export against the oracle's per-step
helpers evaluated in float64 on exactly the values the GPU received.

Error bounds per element (u = 2^-24, fp32 unit roundoff):
  * float32 accumulation of K exact products: K u sum_k |p_k|
  * one bf16 store (round to nearest even): 2^-9 relative, taken as 2^-8
"""

import numpy as np
import pytest
import torch

import newton_schulz_07_amd as ns
from ns_inputs import gaussian
from oracle import ns_oracle
from tests.gpu_util import device, to64

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
DTYPES = [torch.bfloat16, torch.float32]
SHAPES = [(3, 264, 520), (2, 520, 264), (1, 256, 512), (1, 8, 8), (2, 136, 1032), (1, 1032, 136)]


def store_rel(dtype):
    return 2.0 ** -8 if dtype == torch.bfloat16 else 4 * U


def sym_offdiag(batch, m, seed, dtype, scale):
    g = torch.Generator("cpu").manual_seed(seed)
    o = torch.randn(batch, m, m, generator=g) * scale
    o = (o + o.transpose(1, 2)) / 2
    o.diagonal(dim1=1, dim2=2).zero_()
    return o.to(dtype)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", SHAPES)
def test_normalize(dtype, shape):
    dev = device()
    x = gaussian(shape, 100 + shape[1], dtype, scale=3.0)
    xg = x.to(dev)
    norms = torch.empty(shape[0], dtype=torch.float32, device=dev)
    x0 = ns.ns_stage_normalize(xg, norms=norms)
    torch.cuda.synchronize()
    X = to64(x)
    for s in range(shape[0]):
        ref = ns_oracle.frobenius_normalize(X[s])
        got = to64(x0[s])
        assert np.all(np.abs(got - ref) <= store_rel(dtype) * np.abs(ref) + 1e-30)
        assert abs(norms[s].item() - np.linalg.norm(X[s])) <= 1e-5 * np.linalg.norm(X[s])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", SHAPES)
def test_gram(dtype, shape):
    dev = device()
    x = gaussian(shape, 200 + shape[2], dtype, scale=0.05)
    a_off, a_diag = ns.ns_stage_gram(x.to(dev))
    torch.cuda.synchronize()
    X = to64(x)
    K = max(shape[1:])
    assert torch.equal(a_off, a_off.transpose(1, 2)), "Gram must be bitwise symmetric"
    assert torch.all(a_off.diagonal(dim1=1, dim2=2) == 0)
    for s in range(shape[0]):
        A = ns_oracle.gram_matrix(X[s])
        S = ns_oracle.gram_matrix(np.abs(X[s]))
        off = to64(a_off[s])
        m = A.shape[0]
        mask = ~np.eye(m, dtype=bool)
        tol = store_rel(dtype) * np.abs(A) + K * U * S
        assert np.all(np.abs(off - A)[mask] <= tol[mask])
        d = to64(a_diag[s])
        assert np.all(np.abs(d - np.diag(A)) <= K * U * np.diag(S))


@pytest.mark.parametrize("shape", [(400, 264, 520), (400, 520, 264)])
def test_gram_large_stack(shape):
    # 400 slices with m = 264 give 1200 lower-triangle tiles at 256 x 256:
    # the bf16 Gram then runs its 256-tile instance (ragged: 264 = 256 + 8)
    dev = device()
    x = gaussian(shape, 250 + shape[1], torch.bfloat16, scale=0.05)
    a_off, a_diag = ns.ns_stage_gram(x.to(dev))
    torch.cuda.synchronize()
    assert torch.equal(a_off, a_off.transpose(1, 2)), "Gram must be bitwise symmetric"
    assert torch.all(a_off.diagonal(dim1=1, dim2=2) == 0)
    X = to64(x)
    K = max(shape[1:])
    for s in (0, 1, 199, 398, 399):
        A = ns_oracle.gram_matrix(X[s])
        S = ns_oracle.gram_matrix(np.abs(X[s]))
        off = to64(a_off[s])
        mask = ~np.eye(A.shape[0], dtype=bool)
        tol = store_rel(torch.bfloat16) * np.abs(A) + K * U * S
        assert np.all(np.abs(off - A)[mask] <= tol[mask]), s
        assert np.all(np.abs(to64(a_diag[s]) - np.diag(A)) <= K * U * np.diag(S)), s


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("m,batch", [(256, 1), (264, 3), (8, 2), (520, 1), (136, 4)])
def test_poly(dtype, m, batch):
    dev = device()
    a, b, c = ns.DEFAULT_COEFFS
    o = sym_offdiag(batch, m, 300 + m, dtype, 0.02)
    g = torch.Generator("cpu").manual_seed(301 + m)
    d = (0.1 + 0.9 * torch.rand(batch, m, generator=g)).float()
    c_off, c_diag = ns.ns_stage_poly(o.to(dev), d.to(dev), a, b, c)
    torch.cuda.synchronize()
    assert torch.equal(c_off, c_off.transpose(1, 2))
    assert torch.all(c_off.diagonal(dim1=1, dim2=2) == 0)
    O, D = to64(o), to64(d)
    for s in range(batch):
        A = O[s] + np.diag(D[s])
        C = ns_oracle.poly_matrix(A, a, b, c)
        S = np.abs(O[s]) @ np.abs(O[s])
        mag = abs(b) * np.abs(O[s]) + abs(c) * (S + np.abs(D[s][:, None] + D[s][None, :]) * np.abs(O[s]))
        tol = store_rel(dtype) * np.abs(C) + (m * abs(c)) * U * S + 8 * U * mag
        mask = ~np.eye(m, dtype=bool)
        got = to64(c_off[s])
        assert np.all(np.abs(got - C)[mask] <= tol[mask])
        dmag = abs(a) + abs(b) * D[s] + abs(c) * (np.diag(S) + D[s] ** 2)
        assert np.all(np.abs(to64(c_diag[s]) - np.diag(C)) <= (m + 8) * U * dmag)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", SHAPES)
def test_update(dtype, shape):
    dev = device()
    batch, rows, cols = shape
    m = min(rows, cols)
    x = gaussian(shape, 400 + rows, dtype, scale=0.05)
    o = sym_offdiag(batch, m, 401 + m, dtype, 0.03)
    g = torch.Generator("cpu").manual_seed(402)
    d = (1.0 + torch.rand(batch, m, generator=g)).float()
    y = ns.ns_stage_update(x.to(dev), o.to(dev), d.to(dev))
    torch.cuda.synchronize()
    X, O, D = to64(x), to64(o), to64(d)
    for s in range(batch):
        C = O[s] + np.diag(D[s])
        ref = ns_oracle.apply_update(X[s], C)
        S = ns_oracle.apply_update(np.abs(X[s]), np.abs(O[s]))
        tol = store_rel(dtype) * np.abs(ref) + (m + 4) * U * (S + np.abs(ns_oracle.apply_update(X[s], np.diag(D[s]))))
        assert np.all(np.abs(to64(y[s]) - ref) <= tol)
