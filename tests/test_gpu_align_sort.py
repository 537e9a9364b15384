"""Align-and-sort on the GPU, bit-exact against the oracle on the defined
range: sorted_token_ids[:npp], expert_ids[:npp/BS], expert_offsets, npp."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import align_sort as A

pytestmark = pytest.mark.gpu


def _flat_ids(ids, num_experts, num_shared):
    if not num_shared:
        return ids.reshape(-1)
    t = ids.shape[0]
    return np.concatenate([ids, np.full((t, 1), num_experts, dtype=ids.dtype)], axis=1).reshape(-1)


def _check(lib, ids, num_experts, num_shared, bs):
    out = lib.align_sort(torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda(),
                         num_experts, num_shared, bs)
    torch.cuda.synchronize()
    ref = A.align_sort(_flat_ids(ids, num_experts, num_shared), num_experts + num_shared, bs)
    npp = int(out["num_tokens_post_padded"].item())
    assert npp == ref["num_tokens_post_padded"]
    assert np.array_equal(out["expert_offsets"].cpu().numpy(), ref["expert_offsets"])
    assert np.array_equal(out["sorted_token_ids"][:npp].cpu().numpy(), ref["sorted_token_ids"])
    assert np.array_equal(out["expert_ids"][:npp // bs].cpu().numpy(), ref["expert_ids"])
    assert npp <= out["capacity"]
    return out


@pytest.mark.parametrize("bs", [16, 32, 64])
def test_tiny_config(lib, bs):
    cfg = W.TINY_FP32
    ids, _ = W.routing(cfg, 4)
    _check(lib, ids, cfg.num_experts, 0, bs)


@pytest.mark.parametrize("bs", [64, 128])
def test_prefill_zipf_full_size(lib, bs):
    cfg = W.PREFILL_ZIPF_MXFP8
    ids, _ = W.routing(cfg, 16384)
    _check(lib, ids, cfg.num_experts, 0, bs)


@pytest.mark.parametrize("t,bs", [(1, 32), (7, 16), (256, 64), (1000, 128)])
def test_shared_expert_entries(lib, t, bs):
    cfg = W.DEEPSEEK_V3_FP8_BLK128
    ids, _ = W.routing(cfg, t)
    _check(lib, ids, cfg.num_experts, 1, bs)


@pytest.mark.parametrize("t", [1, 3, 64, 333, 4096])
def test_uniform_ragged(lib, t):
    cfg = W.QWEN3_DECODE_MXFP8
    ids, _ = W.routing(cfg, t)
    _check(lib, ids, cfg.num_experts, 0, 32)


def test_edge_cases(lib):
    # every entry on one expert, block size 1, a single block, empty batch
    ids = np.full((50, 2), 3, dtype=np.int32)
    _check(lib, ids, 8, 0, 1)
    _check(lib, ids, 8, 0, 128)
    out = _check(lib, np.zeros((0, 8), dtype=np.int32), 16, 0, 64)
    assert int(out["num_tokens_post_padded"].item()) == 0
    # the largest expert count the kernels stage on chip
    rng = np.random.default_rng(0)
    ids = rng.integers(0, 1024, size=(300, 3)).astype(np.int32)
    _check(lib, ids, 1024, 0, 16)


def test_repeatable(lib):
    cfg = W.PREFILL_ZIPF_MXFP8
    ids, _ = W.routing(cfg, 4096)
    d = torch.from_numpy(ids).cuda()
    a = lib.align_sort(d, cfg.num_experts, 0, 64)
    b = lib.align_sort(d, cfg.num_experts, 0, 64)
    torch.cuda.synchronize()
    n = int(a["num_tokens_post_padded"].item())
    assert torch.equal(a["sorted_token_ids"][:n], b["sorted_token_ids"][:n])


@pytest.mark.parametrize("t", [4095, 4096, 4097])
@pytest.mark.parametrize("bs", [1, 32, 1024])
def test_single_workgroup_limit(lib, t, bs):
    """Up to 8192 entries one workgroup does the whole sort; one entry pair
    past it the three-launch path runs.  Both sides of the limit, bit-exact."""
    rng = np.random.default_rng(7 + t)
    ids = rng.integers(0, 64, size=(t, 2)).astype(np.int32)
    _check(lib, ids, 64, 0, bs)


def test_random_shapes(lib):
    """Seeded random (T, k, E, S, block) combinations across both launch
    shapes, bit-exact against the oracle."""
    rng = np.random.default_rng(2024)
    for _ in range(24):
        t = int(rng.integers(1, 3000))
        e = int(rng.integers(1, 300))
        k = int(rng.integers(1, min(8, e) + 1))    # k <= E (the entry point's contract)
        s = int(rng.integers(0, 2))
        bs = int(rng.choice([1, 16, 32, 64, 128, 256, 1024]))
        ids = rng.integers(0, e, size=(t, k)).astype(np.int32)
        _check(lib, ids, e, s, bs)
