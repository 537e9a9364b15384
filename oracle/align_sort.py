"""Oracle of MoE align-and-sort: (token, slot) entries grouped by expert and
padded per expert to the grouped-GEMM block size.

Test infrastructure (see the package docstring): nothing on the product path
imports this module.

Definition (align-and-sort article: background section -- entries are sorted
by expert id, and the alignment pads each expert's run to whole blocks so the
grouped GEMM takes tokens block by block; D-C-P section -- counts, then a
cumulative sum of the block-aligned counts, then placement):

    entry i = t*k + j for i in [0, T*k), with expert id_i
    c_e     = #{i : id_i = e}
    P_e     = ceil(c_e / BS) * BS               (0 for an unused expert)
    off_0   = 0,  off_{e+1} = off_e + P_e
    sorted[off_e + r]               = the r-th smallest i with id_i = e
    sorted[off_e + c_e : off_e+P_e] = sentinel T*k
    expert_ids[b]                   = e for every block b in [off_e/BS, off_{e+1}/BS)
    num_tokens_post_padded          = off_E

Readings of the pages taken here: the order inside an expert's run is ascending
entry index (the stable order; the article's placement uses atomics and fixes
no order, and a bit-exact comparison needs one); experts appear in ascending
id; an expert with no entries gets no block; the sentinel is T*k; only
[0, off_E) of ``sorted`` and [0, off_E/BS) of ``expert_ids`` are defined.
"""

import numpy as np


def capacity(n_entries, num_experts, block):
    """Worst-case padded length: every expert may waste block-1 slots."""
    return n_entries + num_experts * (block - 1)


def align_sort(flat_ids, num_experts, block):
    """flat_ids: int [N] expert id per entry (N = T*k).  Returns a dict with
    sorted_token_ids [off_E], expert_ids [off_E/BS], expert_offsets [E+1],
    num_tokens_post_padded (int), counts [E]."""
    ids = [int(v) for v in np.asarray(flat_ids).reshape(-1)]
    n = len(ids)
    sentinel = n
    per_expert = [[] for _ in range(num_experts)]
    for i, e in enumerate(ids):              # ascending i: the stable order
        if not 0 <= e < num_experts:
            raise ValueError("expert id out of range")
        per_expert[e].append(i)
    offsets = [0]
    for e in range(num_experts):
        c = len(per_expert[e])
        padded = -(-c // block) * block
        offsets.append(offsets[-1] + padded)
    total = offsets[-1]
    sorted_ids = [sentinel] * total
    expert_ids = [0] * (total // block)
    for e in range(num_experts):
        for r, i in enumerate(per_expert[e]):
            sorted_ids[offsets[e] + r] = i
        for b in range(offsets[e] // block, offsets[e + 1] // block):
            expert_ids[b] = e
    return {
        "sorted_token_ids": np.array(sorted_ids, dtype=np.int32),
        "expert_ids": np.array(expert_ids, dtype=np.int32),
        "expert_offsets": np.array(offsets, dtype=np.int32),
        "num_tokens_post_padded": int(total),
        "counts": np.array([len(p) for p in per_expert], dtype=np.int32),
    }
