"""The seeded input recipes: deterministic, right shape and dtype, right structure."""

import math

import torch

from ns_inputs import WORKLOADS, gaussian, make_workload


def test_gaussian_is_deterministic_and_seeded():
    a = gaussian((33, 17), 5)
    b = gaussian((33, 17), 5)
    c = gaussian((33, 17), 6)
    assert torch.equal(a, b) and not torch.equal(a, c)
    assert gaussian((4, 4), 1, torch.bfloat16).dtype == torch.bfloat16


def test_small_workload_shape_and_dtype():
    x = make_workload("iid_256x512")
    assert x.shape == (256, 512) and x.dtype == torch.float32
    assert abs(x.std().item() - 1.0) < 0.02
    assert torch.equal(x, make_workload("iid_256x512"))


def test_expert_shard_scales_are_log_uniform_in_range():
    x = make_workload("experts16_1536x2048")
    assert x.shape == (16, 1536, 2048) and x.dtype == torch.bfloat16
    rms = x.float().pow(2).mean(dim=(1, 2)).sqrt()
    assert rms.min() > 0.9e-3 and rms.max() < 1.01
    # per-slice scales differ: a global norm would mix them
    assert rms.max() / rms.min() > 10


def test_lowrank_square_is_dominated_by_its_rank64_part():
    x = make_workload("lowrank64_4096x4096").float()
    s = torch.linalg.svdvals(x[:1024, :1024])
    assert s[0] / s[200] > 5  # a few dominant directions over a noise floor


def test_mlp_transpose_pair():
    w = make_workload("mlp_4096x14336")
    t = make_workload("mlp_14336x4096")
    assert w.shape == (4096, 14336) and t.shape == (14336, 4096)
    assert t.is_contiguous() and torch.equal(t, w.T)


def test_registry_metadata():
    for name, w in WORKLOADS.items():
        assert w.batch * w.rows * w.cols == math.prod(w.shape), name
        assert w.rows % 8 == 0 and w.cols % 8 == 0
