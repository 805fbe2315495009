"""The seeded generators produce the shapes and laws the workloads ask for."""
import numpy as np
import pytest
import torch

import workloads as W


def test_workload_shapes():
    q = W.get("qwen3_235b")
    assert (q.num_experts, q.top_k, q.num_ranks, q.tokens_per_rank, q.num_plans) == (128, 8, 64, 8192, 94)
    assert q.num_spare == 64 and q.num_phys == 192 and q.pairs_per_plan == 4194304
    assert q.bytes_per_expert == 3 * 4096 * 1536 * 2
    d = W.get("deepseek_v3")
    assert d.num_phys == 288 and d.spare_count[:32] == (1,) * 32 and d.spare_count[32:] == (0,) * 32
    g = W.get("glm_4_5")
    assert g.num_ranks == 40 and g.native_count == (4,) * 40 and g.num_phys == 200
    s = W.get("stress")
    assert s.num_plans == 256 and s.num_spare == 128 and s.num_phys == 512
    t = W.get("tiny")
    assert t.native_count == (2, 2, 2, 2, 1, 1, 1, 1) and t.spare_count == (0, 0, 0, 0, 1, 1, 1, 1)
    assert t.num_phys == 16 and t.pairs_per_plan == 512
    # Qwen3 per-slot memory: bf16 weight + fp32 grad of one expert is 108 MiB
    assert q.bytes_per_expert // 2 * 6 == 108 * 2**20


@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_ids_distinct_per_token_and_in_range(name):
    wl = W.get(name).scaled(tokens_per_rank=16, layers=2, microbatches=1)
    ids = W.make_ids(wl)
    assert ids.dtype == torch.int32 and ids.shape == (2, wl.pairs_per_plan)
    a = ids.numpy().reshape(2, -1, wl.top_k)
    assert a.min() >= 0 and a.max() < wl.num_experts
    s = np.sort(a, axis=-1)
    assert np.all(np.diff(s, axis=-1) > 0)
    again = W.make_ids(wl)
    assert torch.equal(ids, again)


def test_dsv3_group_limited():
    wl = W.get("deepseek_v3").scaled(tokens_per_rank=8, layers=1)
    a = W.make_ids(wl).numpy().reshape(-1, wl.top_k)
    groups = a // 32
    assert max(len(set(g)) for g in groups.tolist()) <= 4


def test_inject_invalid():
    ids = torch.zeros((2, 1000), dtype=torch.int32)
    out = W.inject_invalid(ids, 5, 0.1, 0.05)
    a = out.numpy()
    assert (a < 0).sum() == 200 and (a >= 5).sum() == 100
