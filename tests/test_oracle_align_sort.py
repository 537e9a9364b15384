"""Pins of oracle/align_sort.py: the hand-worked example under tests/golden/,
numpy's stable argsort plus padding as an independent route, structural
invariants, and brute force over every id assignment of tiny shapes."""

import itertools
import os

import numpy as np
import pytest

import workloads as W
from oracle import align_sort as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_worked_example():
    d = {}
    with open(os.path.join(GOLDEN, "align_sort_worked_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            d[key] = [int(v) for v in vals]
    return d


def test_worked_example():
    g = _load_worked_example()
    r = A.align_sort(np.array(g["topk_ids"]), g["E"][0], g["BS"][0])
    assert r["sorted_token_ids"].tolist() == g["sorted_token_ids"]
    assert r["expert_ids"].tolist() == g["expert_ids"]
    assert r["expert_offsets"].tolist() == g["expert_offsets"]
    assert r["num_tokens_post_padded"] == g["num_tokens_post_padded"][0]


def _via_argsort(ids, e_n, bs):
    """Independent route: numpy stable argsort on the ids, then per-expert
    padding."""
    ids = np.asarray(ids).reshape(-1)
    n = len(ids)
    order = np.argsort(ids, kind="stable")
    counts = np.bincount(ids, minlength=e_n)
    padded = (counts + bs - 1) // bs * bs
    offs = np.concatenate([[0], np.cumsum(padded)])
    out = np.full(offs[-1], n, dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(counts)])
    for e in range(e_n):
        out[offs[e]: offs[e] + counts[e]] = order[starts[e]: starts[e + 1]]
    blocks = np.repeat(np.arange(e_n), padded // bs)
    return out, blocks, offs


def check_invariants(ids, e_n, bs, r):
    ids = np.asarray(ids).reshape(-1)
    n = len(ids)
    s = r["sorted_token_ids"]
    off = r["expert_offsets"]
    npp = r["num_tokens_post_padded"]
    assert off[0] == 0 and off[-1] == npp and len(off) == e_n + 1
    assert npp % bs == 0 and len(s) == npp and len(r["expert_ids"]) == npp // bs
    real = s[s != n]
    assert sorted(real.tolist()) == list(range(n))          # a permutation of the entries
    for e in range(e_n):
        seg = s[off[e]: off[e + 1]]
        c = int(np.sum(ids == e))
        assert len(seg) == -(-c // bs) * bs                   # padded length
        assert np.all(seg[:c] != n) and np.all(seg[c:] == n)  # sentinels only at the tail
        assert np.all(ids[seg[:c]] == e)                      # grouped by expert
        assert np.all(np.diff(seg[:c]) > 0)                   # stable (ascending entry)
        assert np.all(r["expert_ids"][off[e] // bs: off[e + 1] // bs] == e)
    assert np.all(np.diff(r["expert_ids"]) >= 0)
    assert A.capacity(n, e_n, bs) >= npp


@pytest.mark.parametrize("name,t,bs,kind", [("tiny_fp32", 4, 16, None), ("prefill_zipf_mxfp8", 2048, 64, "zipf"),
                                            ("prefill_zipf_mxfp8", 2048, 128, "zipf"),
                                            ("qwen3_decode_mxfp8", 32, 16, None)])
def test_matches_stable_argsort_and_invariants(name, t, bs, kind):
    cfg = W.CONFIGS[name]
    ids, _ = W.routing(cfg, t, kind=kind)
    r = A.align_sort(ids, cfg.num_experts, bs)
    s, b, off = _via_argsort(ids, cfg.num_experts, bs)
    assert np.array_equal(r["sorted_token_ids"], s)
    assert np.array_equal(r["expert_ids"], b)
    assert np.array_equal(r["expert_offsets"], off)
    check_invariants(ids, cfg.num_experts, bs, r)


def test_brute_force_all_assignments():
    """Every id assignment for T <= 3, k <= 2, E <= 3, BS in {1, 2, 4}: the
    output equals one built by placing entries one at a time from the counts."""
    for t, k, e_n, bs in itertools.product((1, 2, 3), (1, 2), (1, 2, 3), (1, 2, 4)):
        n = t * k
        for ids in itertools.product(range(e_n), repeat=n):
            r = A.align_sort(np.array(ids), e_n, bs)
            # per-expert cursor placement (counting-sort formulation)
            counts = [ids.count(e) for e in range(e_n)]
            starts, acc = [], 0
            for c in counts:
                starts.append(acc)
                acc += -(-c // bs) * bs
            want = [n] * acc
            cur = list(starts)
            for i, e in enumerate(ids):
                want[cur[e]] = i
                cur[e] += 1
            assert r["sorted_token_ids"].tolist() == want
            check_invariants(ids, e_n, bs, r)


def test_empty_and_single_expert():
    r = A.align_sort(np.zeros(0, dtype=np.int32), 4, 16)
    assert r["num_tokens_post_padded"] == 0 and len(r["sorted_token_ids"]) == 0
    r = A.align_sort(np.full(5, 2), 4, 4)
    assert r["sorted_token_ids"].tolist() == [0, 1, 2, 3, 4, 5, 5, 5]
    assert r["expert_ids"].tolist() == [2, 2]
    assert r["expert_offsets"].tolist() == [0, 0, 0, 8, 8]
