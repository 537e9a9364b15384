"""The C-ABI library loads and exports every function the public headers
declare; host-side argument checks return their status codes before any
launch.  No compute call is made here (no GPU needed)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("moe_mi355x.h", "moe_mi355x_util.h")]


def declared_functions():
    names = []
    for h in HEADERS:
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    import mixture_experts_decode_amd as moe
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail("libmoe_mi355x.so is not built (run python -m mixture_experts_decode_amd.build)")
    return moe.load()


def test_headers_declare_the_boundary():
    names = declared_functions()
    for need in ("moe_align_sort", "moe_gate_up", "moe_down", "moe_layer", "moe_status_string",
                 "moe_quant_rows", "moe_grouped_gate_up", "moe_grouped_down", "moe_combine",
                 "moe_choose_path", "moe_layer_workspace_bytes", "moe_util_copy"):
        assert need in names


def test_library_exports_every_declared_symbol(lib):
    import mixture_experts_decode_amd as moe
    names = declared_functions()
    for n in names:
        assert hasattr(lib, n), n
    # the binding knows every one of them too
    assert set(names) == set(moe.EXPORTS)


def test_status_strings_and_sizes(lib):
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(3) == b"MOE_ERR_WORKSPACE_TOO_SMALL"
    assert lib.moe_abi_version() == 3
    # capacity = T*(k+S) + (E+S)*(BS-1)
    assert lib.moe_align_sort_capacity(16384, 8, 256, 0, 128) == 131072 + 256 * 127
    assert lib.moe_align_sort_capacity(3, 2, 4, 0, 4) == 6 + 4 * 3
    assert lib.moe_align_sort_capacity(4, 8, 256, 1, 64) == 36 + 257 * 63


def _weights(moe, **kw):
    d = dict(hidden=2048, inter=768, num_experts=128, num_shared=0, format=1,
             w13=16, w13_scale=16, w2=16, w2_scale=16)
    d.update(kw)
    return moe._Weights(**d)


def test_host_argument_errors(lib):
    import mixture_experts_decode_amd as moe
    P = ctypes.c_void_p
    dummy = P(4096)
    # null weights
    assert lib.moe_gate_up(None, dummy, 1, dummy, 4, 8, dummy, 0, None) == moe.ERR_INVALID_ARG
    w = _weights(moe)
    # bad dtype enum, negative T, k > E
    assert lib.moe_gate_up(ctypes.byref(w), dummy, 7, dummy, 4, 8, dummy, 0, None) == moe.ERR_INVALID_ARG
    assert lib.moe_gate_up(ctypes.byref(w), dummy, 1, dummy, -1, 8, dummy, 0, None) == moe.ERR_INVALID_ARG
    assert lib.moe_gate_up(ctypes.byref(w), dummy, 1, dummy, 4, 200, dummy, 0, None) == moe.ERR_INVALID_ARG
    # too many entries for the decode kernels
    assert lib.moe_gate_up(ctypes.byref(w), dummy, 1, dummy, 4096, 8, dummy, 0, None) == moe.ERR_UNSUPPORTED
    # f32 activations with quantised weights
    assert lib.moe_gate_up(ctypes.byref(w), dummy, 0, dummy, 4, 8, dummy, 0, None) == moe.ERR_UNSUPPORTED
    # FP32 weights take an FP32 h in both products (a BF16 h is refused)
    w32 = _weights(moe, format=0, w13_scale=None, w2_scale=None)
    assert lib.moe_gate_up(ctypes.byref(w32), dummy, 0, dummy, 4, 8, dummy, 1, None) == moe.ERR_UNSUPPORTED
    assert lib.moe_down(ctypes.byref(w32), dummy, 1, dummy, dummy, 4, 8, dummy, 0, 1, None, 0,
                        None) == moe.ERR_UNSUPPORTED
    # misaligned weight pointer, bad format, non-multiple-of-32 hidden
    assert lib.moe_down(ctypes.byref(_weights(moe, w13=17)), dummy, 0, dummy, dummy, 4, 8, dummy, 0,
                        0, None, 0, None) == moe.ERR_INVALID_ARG
    assert lib.moe_down(ctypes.byref(_weights(moe, format=9)), dummy, 0, dummy, dummy, 4, 8, dummy, 0,
                        0, None, 0, None) == moe.ERR_INVALID_ARG
    assert lib.moe_down(ctypes.byref(_weights(moe, hidden=2050)), dummy, 0, dummy, dummy, 4, 8, dummy,
                        0, 0, None, 0, None) == moe.ERR_UNSUPPORTED
    # missing scales for a quantised format
    assert lib.moe_down(ctypes.byref(_weights(moe, w2_scale=None)), dummy, 0, dummy, dummy, 4, 8, dummy,
                        0, 0, None, 0, None) == moe.ERR_INVALID_ARG
    # bad variant; the expert-major variant's workspace missing or too small
    assert lib.moe_down(ctypes.byref(w), dummy, 0, dummy, dummy, 4, 8, dummy, 0, 3, None, 0,
                        None) == moe.ERR_INVALID_ARG
    assert lib.moe_down(ctypes.byref(w), dummy, 0, dummy, dummy, 4, 8, dummy, 0, 2, None, 0,
                        None) == moe.ERR_INVALID_ARG
    assert lib.moe_down(ctypes.byref(w), dummy, 0, dummy, dummy, 4, 8, dummy, 0, 2, dummy, 64,
                        None) == moe.ERR_WORKSPACE_TOO_SMALL
    # AUTO runs expert-major from 112 entries up here, which needs the workspace
    assert lib.moe_down(ctypes.byref(w), dummy, 0, dummy, dummy, 32, 8, dummy, 0, 0, None, 0,
                        None) == moe.ERR_INVALID_ARG
    assert lib.moe_down_workspace_bytes(ctypes.byref(w), 4, 8) == 4 * 8 * 2048 * 4
    # T == 0 is a no-op
    assert lib.moe_gate_up(ctypes.byref(w), dummy, 1, dummy, 0, 8, dummy, 0, None) == moe.OK
    # routing check: sizes and pointers refused before any launch
    assert lib.moe_check_routing(dummy, -1, 8, 128, dummy, None) == moe.ERR_INVALID_ARG
    assert lib.moe_check_routing(dummy, 4, 0, 128, dummy, None) == moe.ERR_INVALID_ARG
    assert lib.moe_check_routing(dummy, 4, 8, 0, dummy, None) == moe.ERR_INVALID_ARG
    assert lib.moe_check_routing(dummy, 4, 8, 128, None, None) == moe.ERR_INVALID_ARG
    assert lib.moe_check_routing(None, 4, 8, 128, dummy, None) == moe.ERR_INVALID_ARG
    assert lib.moe_check_routing(dummy, 1 << 28, 16, 128, dummy, None) == moe.ERR_UNSUPPORTED
    # align-sort: block size, workspace
    assert lib.moe_align_sort(dummy, 4, 8, 128, 0, 0, dummy, dummy, dummy, dummy, dummy, 1 << 20,
                              None) == moe.ERR_INVALID_ARG
    assert lib.moe_align_sort(dummy, 4, 8, 128, 0, 64, dummy, dummy, dummy, dummy, dummy, 4,
                              None) == moe.ERR_WORKSPACE_TOO_SMALL
    assert lib.moe_align_sort(dummy, 4, 8, 2000, 0, 64, dummy, dummy, dummy, dummy, dummy, 1 << 20,
                              None) == moe.ERR_UNSUPPORTED
    # layer: FP32 activations with quantised weights, on either path
    for path in (1, 2):
        assert lib.moe_layer(ctypes.byref(w), dummy, 0, dummy, dummy, 4, 8, dummy, 0, path, 32, dummy,
                             1 << 30, None, None) == moe.ERR_UNSUPPORTED
    # layer: workspace too small, bad path, grouped with a bad block size
    assert lib.moe_layer(ctypes.byref(w), dummy, 1, dummy, dummy, 4, 8, dummy, 0, 1, 64, dummy, 16,
                         None, None) == moe.ERR_WORKSPACE_TOO_SMALL
    assert lib.moe_layer(ctypes.byref(w), dummy, 1, dummy, dummy, 4, 8, dummy, 0, 5, 64, dummy, 16,
                         None, None) == moe.ERR_INVALID_ARG
    assert lib.moe_layer(ctypes.byref(w), dummy, 1, dummy, dummy, 4, 8, dummy, 0, 2, 48, dummy,
                         1 << 30, None, None) == moe.ERR_UNSUPPORTED
    # router: sizes, null pointers, T == 0 is a no-op
    assert lib.moe_topk_route(dummy, None, 4, 128, 0, dummy, dummy, None) == moe.ERR_INVALID_ARG
    assert lib.moe_topk_route(dummy, None, 4, 128, 129, dummy, dummy, None) == moe.ERR_INVALID_ARG
    assert lib.moe_topk_route(dummy, None, 4, 2048, 8, dummy, dummy, None) == moe.ERR_INVALID_ARG
    assert lib.moe_topk_route(dummy, None, 4, 128, 65, dummy, dummy, None) == moe.ERR_INVALID_ARG
    assert lib.moe_topk_route(None, None, 4, 128, 8, dummy, dummy, None) == moe.ERR_INVALID_ARG
    assert lib.moe_topk_route(dummy, None, 4, 128, 8, dummy, None, None) == moe.ERR_INVALID_ARG
    assert lib.moe_topk_route(None, None, 0, 128, 8, None, None, None) == moe.OK
    # grouped steps reject fp32 weights
    assert lib.moe_grouped_gate_up(ctypes.byref(_weights(moe, format=0)), dummy, dummy, 4, 8, dummy,
                                   dummy, dummy, 64, 64, dummy, dummy, None) == moe.ERR_UNSUPPORTED
    # quant_rows: H must be a multiple of 32; T == 0 is a no-op
    assert lib.moe_quant_rows(dummy, 1, 4, 100, dummy, dummy, None) == moe.ERR_UNSUPPORTED
    assert lib.moe_quant_rows(None, 1, 0, 128, None, None, None) == moe.OK
    assert lib.moe_quant_rows(dummy, 1, 4, 128, None, dummy, None) == moe.ERR_INVALID_ARG


def test_path_choice_host_logic(lib):
    w = _weights(__import__("mixture_experts_decode_amd"))
    DEC, GRP = 1, 2
    assert lib.moe_choose_path(ctypes.byref(w), 1, 8) == DEC
    assert lib.moe_choose_path(ctypes.byref(w), 32, 8) == DEC
    assert lib.moe_choose_path(ctypes.byref(w), 16384, 8) == GRP
    # the regime follows the sweeps of both paths on MI355X where one was
    # clearly faster (whole-layer microseconds replayed from a HIP graph,
    # decode vs grouped with 32-row blocks)
    moe = __import__("mixture_experts_decode_amd")
    qwen = _weights(moe)
    assert lib.moe_choose_path(ctypes.byref(qwen), 16, 8) == DEC       # 79 vs 108
    assert lib.moe_choose_path(ctypes.byref(qwen), 128, 8) == GRP      # 273 vs 149
    assert lib.moe_choose_path(ctypes.byref(qwen), 256, 8) == GRP      # 446 vs 153
    ds = _weights(moe, hidden=7168, inter=2048, num_experts=256, num_shared=1, format=3)
    assert lib.moe_choose_path(ctypes.byref(ds), 1, 8) == DEC          # 77 vs 108
    assert lib.moe_choose_path(ctypes.byref(ds), 64, 8) == GRP         # 1836 vs 982
    fp4 = _weights(moe, hidden=4096, inter=1536, format=2)
    assert lib.moe_choose_path(ctypes.byref(fp4), 8, 8) == DEC         # 118 vs 152
    assert lib.moe_choose_path(ctypes.byref(fp4), 32, 8) == DEC        # 262 vs 275
    assert lib.moe_choose_path(ctypes.byref(fp4), 48, 8) == GRP        # 295 vs 284
    assert lib.moe_choose_path(ctypes.byref(fp4), 128, 8) == GRP       # 366 vs 301
    # the choice is monotone in the batch: decode up to one crossover, then grouped
    for wt in (qwen, ds, fp4):
        picks = [lib.moe_choose_path(ctypes.byref(wt), t, 8) for t in range(0, 300)]
        first = picks.index(GRP)
        assert all(p == DEC for p in picks[:first]) and all(p == GRP for p in picks[first:])
    # fp32 weights have no grouped path
    w32 = _weights(__import__("mixture_experts_decode_amd"), format=0)
    assert lib.moe_choose_path(ctypes.byref(w32), 16384, 8) == DEC
    # workspace sizes: decode = h (T*slots*I, BF16), plus the FP32 slot
    # outputs of the expert-major down, which AUTO runs from 112 entries up
    # when a W_down row spans 16 lanes (I = 768) and from 18 entries up at 32
    # lanes (the measured crossovers)
    assert lib.moe_layer_workspace_bytes(ctypes.byref(w), 32, 8, DEC, 64) == 32 * 8 * (768 * 2 + 2048 * 4)
    assert lib.moe_layer_workspace_bytes(ctypes.byref(w), 14, 8, DEC, 64) == 14 * 8 * (768 * 2 + 2048 * 4)
    assert lib.moe_layer_workspace_bytes(ctypes.byref(w), 13, 8, DEC, 64) == 13 * 8 * 768 * 2
    ds = _weights(moe, hidden=7168, inter=2048, num_experts=256, num_shared=1, format=3)
    assert lib.moe_layer_workspace_bytes(ctypes.byref(ds), 1, 8, DEC, 64) == 9 * 2048 * 2
    assert lib.moe_layer_workspace_bytes(ctypes.byref(ds), 2, 8, DEC, 64) == 18 * (2048 * 2 + 7168 * 4)
    assert lib.moe_layer_workspace_bytes(ctypes.byref(w), 32, 8, GRP, 64) > 0
    assert lib.moe_layer_workspace_bytes(ctypes.byref(w), 32, 8, GRP, 48) == 0
    # block 0: the library picks by expected entries per expert (32 at 2 per
    # expert, 64 at 64, 128 at 1024)
    for t, bs in ((32, 32), (1024, 64), (16384, 128)):
        assert (lib.moe_layer_workspace_bytes(ctypes.byref(w), t, 8, GRP, 0) ==
                lib.moe_layer_workspace_bytes(ctypes.byref(w), t, 8, GRP, bs))


def test_layer_refuses_unsupported_decode_shapes_before_any_launch(lib):
    """Every decode-kernel limit is checked before the first launch: on a
    host without a GPU a call that reached a launch would return
    MOE_ERR_HIP, so MOE_ERR_UNSUPPORTED proves nothing was enqueued."""
    moe = __import__("mixture_experts_decode_amd")
    P = ctypes.c_void_p
    dummy = P(4096)
    big = 1 << 40
    DEC, GRP = 1, 2
    # a W_down row of 64 E4M3 bytes has no compiled lane split
    narrow = _weights(moe, inter=64)
    assert lib.moe_layer(ctypes.byref(narrow), dummy, 1, dummy, dummy, 4, 8, dummy, 0, DEC, 0,
                         dummy, big, None, None) == moe.ERR_UNSUPPORTED
    # no grouped path for it either (I is not a multiple of 128): AUTO keeps
    # decode and the call is refused the same way
    assert lib.moe_choose_path(ctypes.byref(narrow), 4, 8) == DEC
    assert lib.moe_layer(ctypes.byref(narrow), dummy, 1, dummy, dummy, 4, 8, dummy, 0, 0, 0,
                         dummy, big, None, None) == moe.ERR_UNSUPPORTED
    # more than 64 slots: the token-major down kernel keeps one slot per lane
    w = _weights(moe)
    assert lib.moe_layer(ctypes.byref(w), dummy, 1, dummy, dummy, 2, 65, dummy, 0, DEC, 0,
                         dummy, big, None, None) == moe.ERR_UNSUPPORTED
    assert lib.moe_down(ctypes.byref(w), dummy, 1, dummy, dummy, 2, 65, dummy, 0, 0, None, 0,
                        None) == moe.ERR_UNSUPPORTED
    # AUTO never picks a path that cannot run
    assert lib.moe_choose_path(ctypes.byref(w), 2, 65) == GRP
    # more entries than the decode kernels stage on chip
    assert lib.moe_layer(ctypes.byref(w), dummy, 1, dummy, dummy, 257, 8, dummy, 0, DEC, 0,
                         dummy, big, None, None) == moe.ERR_UNSUPPORTED
    assert lib.moe_choose_path(ctypes.byref(w), 257, 8) == GRP
    # F32 activations with quantised weights, refused by moe_layer itself
    assert lib.moe_layer(ctypes.byref(w), dummy, 0, dummy, dummy, 4, 8, dummy, 0, DEC, 0,
                         dummy, big, None, None) == moe.ERR_UNSUPPORTED


def test_library_reads_no_tuning_environment(lib):
    """Launch shapes are fixed in the library: it reads no environment
    variables, so no setting can pick a shape that was not compiled."""
    import mixture_experts_decode_amd as moe
    blob = open(moe.LIB_PATH, "rb").read()
    assert b"MOE_TUNE" not in blob and b"getenv" not in blob


def test_noalloc_entry_point_host_checks(lib):
    """moe_layer_noalloc checks its arguments and the size of its array on
    the host: on a GPU-less host these return before any device call."""
    moe = __import__("mixture_experts_decode_amd")
    P = ctypes.c_void_p
    dummy = P(4096)
    assert lib.moe_layer_noalloc_max_bytes() == 32 << 20
    w = _weights(moe)
    assert lib.moe_layer_noalloc(None, dummy, 1, dummy, dummy, 4, 8, dummy, 0, 0, 0, None,
                                 None) == moe.ERR_INVALID_ARG
    assert lib.moe_layer_noalloc(ctypes.byref(w), dummy, 1, dummy, dummy, 4, 8, dummy, 0, 7, 0,
                                 None, None) == moe.ERR_INVALID_ARG
    # the grouped path at a prefill size needs far more than the array
    assert lib.moe_layer_workspace_bytes(ctypes.byref(w), 16384, 8, 2, 128) > 32 << 20
    assert lib.moe_layer_noalloc(ctypes.byref(w), dummy, 1, dummy, dummy, 16384, 8, dummy, 0, 2,
                                 128, None, None) == moe.ERR_WORKSPACE_TOO_SMALL
    chosen = ctypes.c_int32(-1)
    assert lib.moe_layer_noalloc(ctypes.byref(w), None, 1, None, None, 0, 8, None, 0, 0, 0,
                                 ctypes.byref(chosen), None) == moe.OK
    assert chosen.value == 1


def test_path_choice_and_workspace_rules_over_random_shapes(lib):
    """Host rules over a seeded spread of layer shapes (no GPU): the regime
    choice is monotone in the batch, the decode workspace is h plus, exactly
    when the down product runs expert-major, the FP32 slot outputs, and every
    shape AUTO sends to the decode path (quantised weights) is one the decode
    entry points accept."""
    import numpy as np
    moe = __import__("mixture_experts_decode_amd")
    DEC, GRP = 1, 2
    rng = np.random.default_rng(2024)
    align = lambda n: (n + 255) // 256 * 256
    for _ in range(120):
        fmt = int(rng.choice([0, 1, 2, 3]))
        hidden = int(rng.choice([512, 1024, 2048, 4096, 7168]))
        inter = int(rng.choice([256, 512, 768, 1024, 1536, 2048]))
        e = int(rng.choice([8, 16, 64, 128, 256]))
        s = int(rng.integers(0, 2))
        k = int(rng.choice([1, 2, 4, 6, 8]))
        if k > e:
            continue
        w = _weights(moe, hidden=hidden, inter=inter, num_experts=e, num_shared=s, format=fmt)
        picks = [lib.moe_choose_path(ctypes.byref(w), t, k) for t in range(0, 260, 3)]
        if GRP in picks:
            first = picks.index(GRP)
            assert all(p == DEC for p in picks[:first]) and all(p == GRP for p in picks[first:])
        h_el = 4 if fmt == 0 else 2
        dummy = ctypes.c_void_p(4096)
        for t in (1, 2, 7, 13, 14, 32, 100):
            if lib.moe_choose_path(ctypes.byref(w), t, k) != DEC:
                continue
            ws = lib.moe_layer_workspace_bytes(ctypes.byref(w), t, k, DEC, 0)
            h_bytes = align(t * (k + s) * inter * h_el)
            slot = align(t * (k + s) * hidden * 4)
            assert ws in (h_bytes, h_bytes + slot), (fmt, hidden, inter, e, s, k, t, ws)
            # every host check passes: with no GPU here the call can only fail
            # at its first launch (MOE_ERR_HIP), never with a refusal -- except
            # FP32 weights, which have no grouped path to fall back to, so AUTO
            # names the decode path even for rows it cannot take
            st = lib.moe_layer(ctypes.byref(w), dummy, 0 if fmt == 0 else 1, dummy, dummy, t, k,
                               dummy, 0, DEC, 0, dummy, ws, None, None)
            ok = (moe.ERR_HIP, moe.ERR_UNSUPPORTED) if fmt == 0 else (moe.ERR_HIP,)
            assert st in ok, (fmt, hidden, inter, e, s, k, t, st)
