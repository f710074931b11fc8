"""bf16 rounding-placement model of Newton–Schulz (a diagnostic, NOT the oracle).

TEST INFRASTRUCTURE ONLY.  The parity reference is ns_oracle (float64).  This
module answers a different question: how far from the float64 result can ANY
implementation land whose iterate X is stored in bf16, given where it rounds?
It is written from the description of the placement, not from the HIP code.

Placement modelled ("diagonal-split"):
  * X is stored in bf16 (round-to-nearest-even) after every producer.
  * products are float32 sums of exact bf16 x bf16 products;
  * A = X Xᵀ is stored as a bf16 off-diagonal part O_A (zero diagonal) plus a
    float32 diagonal vector d_A;
  * A·A is formed from O_A only, its diagonal terms restored in float32:
        (A A)_ij = (O_A O_A)_ij + (d_i + d_j) O_A,ij + δ_ij d_i²
  * C = a I + b A + c A A is stored the same way (bf16 off-diagonal O_C plus a
    float32 diagonal d_C, which absorbs a);
  * X' = bf16(O_C X + d_C ⊙ X).
The prime-rl PR #3873 microbenchmark note credits its better accuracy to an
fp32 alpha/beta epilogue; keeping the two diagonals in float32 is this
implementation's use of that freedom (the diagonal of C is ≈ a + ... and
dominates C X, so rounding it to bf16 costs most of the error budget).

The "plain" placement (bf16 A, bf16 B = b A + c A A, X' = bf16(a X + B X)) is
also provided for comparison.
"""

import numpy as np
import torch


def _bf16(t):
    return t.to(torch.bfloat16).to(torch.float32)


def _normalize_bf16(x, eps):
    # float32 sum of squares, multiply by float32 reciprocal of (norm + eps)
    s = torch.sqrt(torch.sum(x.double() * x.double())).float()
    inv = 1.0 / (s + eps)
    return _bf16(x * inv)


def ns_bf16_model(x, steps=5, coeffs=(3.4445, -4.7750, 2.0315), eps=1e-7,
                  placement="diag"):
    """Return the float64 result of the modelled bf16 NS of one 2-D matrix."""
    X = torch.as_tensor(np.asarray(x, dtype=np.float32)).clone()
    X = _bf16(X)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T.contiguous()
    a, b, c = (float(v) for v in coeffs)
    X = _normalize_bf16(X, eps)
    m = X.shape[0]
    eye = torch.eye(m, dtype=torch.float32)
    for _ in range(steps):
        G = X @ X.T
        if placement == "plain":
            A = _bf16(G)
            B = _bf16(b * A + c * (A @ A))
            X = _bf16(a * X + B @ X)
            continue
        dA = torch.diagonal(G).clone()
        OA = _bf16(G * (1 - eye))
        P = OA @ OA
        C = b * OA + c * (P + (dA[:, None] + dA[None, :]) * OA)
        dC = a + b * dA + c * (torch.diagonal(P) + dA * dA)
        OC = _bf16(C * (1 - eye))
        X = _bf16(OC @ X + dC[:, None] * X)
    X = X.double().numpy()
    return X.T.copy() if tall else X
