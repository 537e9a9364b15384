"""Router front-end: gating scores -> (topk_ids, topk_weights).

Test infrastructure (see the package docstring): nothing on the product path
imports this module.

Source: the align-and-sort article ("AMD GPU性能暴涨7倍..."), background
section: the gate activates the experts with the top-k gating scores, with a
per-expert bias added for the selection in DeepSeek V3/R1 (auxiliary-loss-
free balancing); its FasterTransformer section names the fused top-k gating
softmax and biased top-k gating softmax operators.

Readings of the pages taken here:
* selection key = score + bias, taken in float32 (the precision the kernel
  decides in); the k largest keys, ties to the lower expert index, listed in
  descending key order;
* weights = softmax over the k selected raw scores (the bias only steers the
  selection).  This equals the renormalised top-k of a softmax over all
  experts, since a softmax is monotone and renormalising cancels its
  normaliser.
"""

import numpy as np


def topk_route(scores, k, bias=None):
    """scores [T][E] (float32), bias [E] or None -> (ids int32 [T][k],
    weights float64 [T][k])."""
    s32 = np.asarray(scores, dtype=np.float32)
    key = s32 if bias is None else (s32 + np.asarray(bias, dtype=np.float32)[None, :])
    t, e = key.shape
    ids = np.empty((t, k), dtype=np.int32)
    for i in range(t):
        # largest key first; among equal keys the lower expert index first
        order = sorted(range(e), key=lambda j: (-float(key[i, j]), j))
        ids[i] = order[:k]
    sel = np.take_along_axis(s32.astype(np.float64), ids.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return ids, z / z.sum(axis=1, keepdims=True)


def check_routing(ids, num_experts):
    """(number of routed ids outside [0, num_experts), first such flat entry
    t*k + j or -1).  The routed ids index k of the E experts a token activates
    (align-and-sort article, background section), so [0, E) is their range."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    bad = np.flatnonzero((flat < 0) | (flat >= num_experts))
    return int(bad.size), (int(bad[0]) if bad.size else -1)
