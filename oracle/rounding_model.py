"""bf16 rounding-placement model of Newton–Schulz (a diagnostic, NOT the oracle).

TEST INFRASTRUCTURE ONLY.  The parity reference is ns_oracle (float64).  This
module answers a different question: how far from the float64 result can an
implementation land whose iterate X is stored in bf16, given where it rounds?
It is written from the description of each placement below, not from the HIP
code, and it shares no code with it.

Common to every placement:
  * products are float32 sums of exact bf16 x bf16 products (emulated as
    float32 matmuls of bf16-valued operands);
  * every named matrix is rounded to bf16 (round-to-nearest-even) once, when
    its producer stores it; epilogue arithmetic is float32.

Placements (the step X -> X' of A = X Xᵀ, B = b A + c A A, X' = a X + B X):
  * "literal": A = bf16(X Xᵀ); B = bf16(b A + c A A); X' = bf16(a X + B X).
  * "fold":    A = bf16(X Xᵀ); C = bf16(a I + b A + c A A); X' = bf16(C X).
  * "diagAC":  A = X Xᵀ is kept as a bf16 off-diagonal part O_A (zero
    diagonal) plus a float32 diagonal vector d_A.  A A is formed from O_A
    only, its diagonal terms restored in float32:
        (A A)_ij = (O_A O_A)_ij + (d_i + d_j) O_A,ij + δ_ij d_i²
    C = a I + b A + c A A is kept the same way (bf16 O_C, float32 d_C, which
    absorbs a), and X' = bf16(O_C X + d_C ⊙ X).
    The prime-rl PR #3873 page credits its accuracy to an fp32 alpha/beta
    epilogue (the note under its NS microbenchmark table); keeping the two
    diagonals in float32 is one use of that freedom: near convergence the
    diagonal of C dominates C X, and rounding it to bf16 costs most of the
    error budget.

Normalisation (X0 = x / (||x||_F + eps)):
  * fold_norm=False: X0 is computed in float32 and rounded to bf16 before the
    first step (the plain reading: a normalisation pass that stores X0).
  * fold_norm=True: X0 is never stored.  The first Gram is formed on the raw
    bf16 input x and scaled by inv² = 1/(||x|| + eps)² in float32 before its
    rounding; the first update forms its product on x and scales it by inv
    before X1 is rounded.  This is the placement the HIP library uses.

rounding=False replaces every bf16 rounding by the identity, and work=float64
runs every product and epilogue in float64.  With both, every placement is
algebraically the oracle's iteration, so the model must equal the oracle to
float64 rounding: that is the pin of the restoration terms above.
"""

import numpy as np
import torch

PLACEMENTS = ("literal", "fold", "diagAC")
_ALIASES = {"plain": "literal", "diag": "diagAC"}


def _bf16(t):
    return t.to(torch.bfloat16).to(t.dtype)


def _ident(t):
    return t


def _split_poly(OA, dA, a, b, c):
    """C = a I + b A + c A A for A = O_A + diag(d_A), with A A formed from O_A
    only and its diagonal terms restored:
        (A A)_ij = (O_A O_A)_ij + (d_i + d_j) O_A,ij   (i != j)
        (A A)_ii = (O_A O_A)_ii + d_i²                 (O_A,ii = 0)
    Returns the off-diagonal part of C (its diagonal entries are to be
    dropped) and the diagonal d_C = a + b d_A + c (A A)_ii."""
    P = OA @ OA
    C_off = b * OA + c * (P + (dA[:, None] + dA[None, :]) * OA)
    dC = a + b * dA + c * (torch.diagonal(P) + dA * dA)
    return C_off, dC


def _first_step_scales(inv):
    """With the normalisation folded into the first step: the factor on the
    first Gram (A of X0 = inv² · x xᵀ) and on the first update's product
    (X1 = inv · (C x), C being a polynomial of A alone)."""
    return inv * inv, inv


def ns_bf16_model(x, steps=5, coeffs=(3.4445, -4.7750, 2.0315), eps=1e-7,
                  placement="diagAC", fold_norm=True, rounding=True, work=torch.float32):
    """Return, in float64, the modelled bf16 NS of one 2-D matrix x.

    x is taken as given (the caller passes the bf16-valued input of the bf16
    path); it is not rounded again here.
    """
    placement = _ALIASES.get(placement, placement)
    if placement not in PLACEMENTS:
        raise ValueError(f"unknown placement {placement!r}")
    if steps < 0:
        raise ValueError("steps must be >= 0")
    rnd = _bf16 if rounding else _ident
    X = torch.as_tensor(np.asarray(x, dtype=np.float64)).to(work).clone()
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T.contiguous()
    a, b, c = (float(v) for v in coeffs)
    # norm: a float32 sum of squares in the kernels; its own rounding is far
    # below bf16's, so it is taken in float64 and cast to the work type
    nrm = torch.sqrt(torch.sum(X.double() * X.double())).to(work)
    inv = 1.0 / (nrm + eps)
    scale_first = fold_norm and steps > 0
    if not scale_first:
        X = rnd(X * inv)
    m = X.shape[0]
    eye = torch.eye(m, dtype=work)
    off = 1 - eye
    for s in range(steps):
        g_scale, x_scale = _first_step_scales(inv) if (scale_first and s == 0) else (1.0, 1.0)
        G = (X @ X.T) * g_scale
        if placement == "literal":
            A = rnd(G)
            B = rnd(b * A + c * (A @ A))
            X = rnd((a * X + B @ X) * x_scale)
        elif placement == "fold":
            A = rnd(G)
            C = rnd(a * eye + b * A + c * (A @ A))
            X = rnd((C @ X) * x_scale)
        else:
            dA = torch.diagonal(G).clone()
            OA = rnd(G * off)
            C_off, dC = _split_poly(OA, dA, a, b, c)
            OC = rnd(C_off * off)
            X = rnd((OC @ X + dC[:, None] * X) * x_scale)
    X = X.double().numpy()
    return X.T.copy() if tall else X
