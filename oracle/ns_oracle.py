"""Plain fp64 CPU oracle of Muon's quintic Newton–Schulz orthogonalization.

TEST INFRASTRUCTURE ONLY: this module is the parity reference for the HIP
library.  Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it; the product path never does, and this file shares no
code with the HIP path (no kernels, headers, helpers or constants are common).

What is computed (per matrix X, in float64):

  1. If X is tall (more rows than columns) work on its transpose, so that the
     Gram matrix is min(rows, cols) square; transpose the result back at the
     end.  The prime-rl PR #3873 page, section "Tests", checks the method on
     both wide and tall 2-D shapes; the transposition is the usual way the
     dense routine it builds on handles tall inputs.
  2. Divide X by its Frobenius norm plus eps (eps = 1e-7 added to the norm,
     outside the square root).  The pages do not print this step; it is part of
     the dense routine the prime-rl page ("Summary", item 1) names as its base,
     Dion's zeropower_via_newtonschulz5.
  3. Repeat ns_steps times (default 5: param-decomp PR #978, section "What",
     the ns_steps setting):
         A = X Xᵀ
         B = b A + c A A
         X = a X + B X
     These are the three products the prime-rl page ("Summary", item 1) maps
     onto the symmetric GEMM (the first two) and addmm/baddbmm (the third).
  4. A stack [E, rows, cols] is a batch of independent matrices along the
     leading axis (prime-rl page, "Summary", item 2: the leading axis is
     treated as a batch; param-decomp page, "What": same-shape leaves batched
     into one NS).

The coefficients (a, b, c) = (3.4445, -4.7750, 2.0315) are the standard Muon
quintic ones; the prime-rl microbenchmark only says that every path uses the
same coefficients.

Nothing here is blocked, fused or reordered: each step is written as the
definition above, with numpy's matmul as the only library primitive.
"""

import numpy as np

DEFAULT_COEFFS = (3.4445, -4.7750, 2.0315)
DEFAULT_STEPS = 5
EPS = 1e-7


def frobenius_normalize(x, eps=EPS):
    """X / (||X||_F + eps) in float64 (step 2 above)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (np.sqrt(np.sum(x * x)) + eps)


def ns_iteration(x, a, b, c):
    """One quintic step: A = X Xᵀ, B = bA + cA·A, X' = aX + B·X (step 3)."""
    A = x @ x.T
    B = b * A + c * (A @ A)
    return a * x + B @ x


def gram_matrix(x):
    """A = X Xᵀ of a wide (or square) matrix; Xᵀ X of a tall one (step 1 above
    applied: the Gram side is always the short side)."""
    x = np.asarray(x, dtype=np.float64)
    return x.T @ x if x.shape[0] > x.shape[1] else x @ x.T


def poly_matrix(A, a, b, c):
    """C = a I + b A + c A A: the step's left factor, since aX + BX = (aI + B) X
    with B = bA + cAA (step 3 above, regrouped)."""
    A = np.asarray(A, dtype=np.float64)
    return a * np.eye(A.shape[0]) + b * A + c * (A @ A)


def apply_update(x, C):
    """X' = C X for a wide X; X' = X C for a tall X (the transpose of
    Cᵀ Xᵀ = C Xᵀ, C symmetric), so a tall X is updated without transposing."""
    x = np.asarray(x, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    return x @ C if x.shape[0] > x.shape[1] else C @ x


def newton_schulz(x, steps=DEFAULT_STEPS, coeffs=DEFAULT_COEFFS, eps=EPS):
    """Orthogonalize one 2-D matrix; returns float64 of the input's shape."""
    X = np.array(x, dtype=np.float64, copy=True)
    if X.ndim != 2:
        raise ValueError(f"expected a 2-D matrix, got shape {X.shape}")
    if steps < 0:
        raise ValueError("steps must be >= 0")
    a, b, c = (float(v) for v in coeffs)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    X = frobenius_normalize(X, eps)
    for _ in range(steps):
        X = ns_iteration(X, a, b, c)
    return X.T.copy() if tall else X


def newton_schulz_batched(x, steps=DEFAULT_STEPS, coeffs=DEFAULT_COEFFS,
                          eps=EPS, slices=None):
    """Apply newton_schulz to every matrix of a [..., rows, cols] stack.

    `slices` optionally restricts the work to the listed flat slice indices
    (the result then holds only those slices, in the given order).  Slices are
    processed one at a time so that large stacks never need a float64 copy of
    the whole stack.
    """
    arr = np.asarray(x)
    if arr.ndim < 2:
        raise ValueError("need at least 2 dimensions")
    r, c = arr.shape[-2:]
    flat = arr.reshape(-1, r, c)
    idx = range(flat.shape[0]) if slices is None else list(slices)
    out = np.empty((len(idx), r, c), dtype=np.float64)
    for k, i in enumerate(idx):
        out[k] = newton_schulz(flat[i], steps, coeffs, eps)
    if slices is None:
        return out.reshape(arr.shape[:-2] + (r, c))
    return out


def dense_equivalent_flops(batch, rows, cols, steps=DEFAULT_STEPS):
    """Dense-GEMM FLOPs of one call: per step 2m²n (X Xᵀ) + 2m³ (A·A) + 2m²n
    (B·X) with m = min(rows, cols), n = max(rows, cols).  This is the basis the
    prime-rl microbenchmark compares implementations on (time per call for the
    same work), used here to turn ms/call into effective FLOP/s."""
    m, n = min(rows, cols), max(rows, cols)
    return batch * steps * (4 * m * m * n + 2 * m ** 3)
