"""Shared helpers for the GPU parity tests: upload of the seeded inputs,
oracle access per config, and the comparison metrics."""

import functools

import numpy as np
import torch

import workloads as W
from oracle import layer as L


def to_device_x(cfg, x):
    if cfg.act == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_bits_to_f64(t):
    return L.activations_f64(t.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")


def to_f64(t):
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(t)
    return t.detach().cpu().double().numpy()


@functools.lru_cache(maxsize=4)
def host_weights(cfg):
    return W.all_experts(cfg)


@functools.lru_cache(maxsize=2)
def device_weights(cfg):
    import mixture_experts_decode_amd as moe
    return moe.Weights.from_arrays(cfg, host_weights(cfg))


def expert_getter(cfg):
    arrays = host_weights(cfg)

    def get(e):
        return {k: (None if v is None else v[e]) for k, v in arrays.items()}
    return get


def oracle_kw(cfg):
    return dict(fmt=cfg.fmt, num_experts=cfg.num_experts, num_shared=cfg.num_shared,
                get_expert=expert_getter(cfg))


def inputs(cfg, t, kind=None, variant=0):
    x = W.activations(cfg, t, variant)
    ids, w = W.routing(cfg, t, kind=kind, variant=variant)
    return x, ids, w


def device_routing(ids, w):
    return torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()


def metrics(y, ref):
    """Per-token cosine and relative L2 of y against the float64 oracle."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    dot = np.sum(y * ref, axis=1)
    cos = dot / (np.linalg.norm(y, axis=1) * np.linalg.norm(ref, axis=1))
    rel = np.linalg.norm(y - ref, axis=1) / np.linalg.norm(ref, axis=1)
    return {"min_cos": float(np.min(cos)), "max_rel_l2": float(np.max(rel)),
            "rel_l2": float(np.linalg.norm(y - ref) / np.linalg.norm(ref)),
            "max_abs": float(np.max(np.abs(y - ref)))}


# Layer-output tolerance: per-token cosine >= 0.99999 and relative L2 <= 5e-3
# against the float64 oracle.
COS_MIN = 0.99999
REL_L2_MAX = 5e-3


def assert_layer_close(y, ref, what=""):
    m = metrics(y, ref)
    assert m["min_cos"] >= COS_MIN and m["max_rel_l2"] <= REL_L2_MAX, (what, m)
    return m
