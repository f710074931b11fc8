"""Helpers shared by the GPU tests (no method arithmetic here)."""

import numpy as np
import pytest
import torch


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU test needs a ROCm device")  # never skipped silently
    return torch.device("cuda:0")


def to64(t):
    return t.detach().double().cpu().numpy()


def rel_err(y, ref):
    """Relative Frobenius error per slice of [..., r, c] arrays."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    r, c = ref.shape[-2:]
    y = y.reshape(-1, r, c)
    ref = ref.reshape(-1, r, c)
    num = np.sqrt(((y - ref) ** 2).sum(axis=(1, 2)))
    den = np.sqrt((ref ** 2).sum(axis=(1, 2)))
    return num / np.where(den == 0, 1.0, den)


def report(record):
    """Append a JSON record to $NS_REPORT_DIR/parity.jsonl when that is set."""
    import json
    import os
    d = os.environ.get("NS_REPORT_DIR")
    if d:
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, "parity.jsonl"), "a") as f:
            f.write(json.dumps(record) + "\n")
