"""Measurement helpers on the GPU.

* The roofline calibration loop (ns_peak_mfma): it runs, its rate stays under
  the spec peak at the clock it reports, and that clock is a plausible shader
  clock.  The spec figures: 256 CUs, 2.4 GHz peak engine clock, 4096 dense
  bf16 and 256 fp32 matrix FLOPs per CU per clock.
* Per-kernel timing (ns_timing_*): the sampled launches are the ones timed,
  and timing leaves every result bitwise unchanged.
"""

import pytest
import torch

import newton_schulz_07_amd as ns
from ns_inputs import gaussian
from tests.gpu_util import device

pytestmark = pytest.mark.gpu

FLOPS_PER_CU_CLK = {"bf16": 4096, "fp32": 256}


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_peak_loop_rate_and_clock(dtype):
    device()
    tf, mhz = ns.ns_peak_mfma(dtype, 1 << 16)
    print(f"{dtype}: {tf:.1f} TFLOP/s at {mhz:.0f} MHz", flush=True)
    assert 500.0 < mhz < 2600.0
    # no faster than every CU's matrix cores at the measured clock (10% slack
    # for the clock average over workgroups and the event timing; the loop
    # itself runs at about 98-99% of this bound)
    bound = 256 * FLOPS_PER_CU_CLK[dtype] * mhz * 1e6 / 1e12
    assert 0.0 < tf <= 1.10 * bound


def test_timing_samples_the_chosen_launches_and_changes_nothing():
    dev = device()
    x = gaussian((3, 512, 768), 4242).to(torch.bfloat16).to(dev)
    ref = ns.orthogonalize(x)
    kinds = (ns.NS_KIND_SUMSQ, ns.NS_KIND_GRAM, ns.NS_KIND_POLY, ns.NS_KIND_UPDATE)
    mask = sum(1 << k for k in kinds)
    try:
        for every, offset, want in ((1, 0, {0: 2, 2: 10, 3: 10, 4: 10}), (5, 2, {0: 0, 2: 2, 3: 2, 4: 2})):
            ns.ns_timing_reset()
            ns.ns_timing_sample(every, offset)
            ns.ns_timing_enable(mask)
            ys = [ns.orthogonalize(x) for _ in range(2)]
            ns.ns_timing_enable(0)
            torch.cuda.synchronize()
            for y in ys:
                assert torch.equal(y, ref)
            for k in kinds:
                ms, n = ns.ns_timing_query(k)
                assert n == want[k], (every, offset, k, n)
                assert (ms > 0.0) == (n > 0)
    finally:
        ns.ns_timing_enable(0)
        ns.ns_timing_sample(1, 0)
        ns.ns_timing_reset()
