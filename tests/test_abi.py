"""Host-side checks of the C ABI: the library loads, exports every entry point the header
declares, sizes its buffers as documented and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

from mxfp4_latent_mixture_sigmoid_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(abi.LIB_PATH):
        from mxfp4_latent_mixture_sigmoid_amd import build
        build.build()


def header_functions():
    src = open(os.path.join(ROOT, "include", "mxmoe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_function():
    names = header_functions()
    assert {"moe_query", "moe_create", "moe_route", "moe_forward", "moe_destroy", "moe_strerror"} <= set(names)
    L = ctypes.CDLL(abi.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(abi.SIGNATURES), "binding and header disagree"


def test_kernel_ids_match_header():
    """The binding's kernel names (indexed by the profiling hook's kernel ids) follow the header's
    MOE_KERNEL_* enumeration, and its config struct has the header's fields in order."""
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "mxmoe.h")).read(), flags=re.S)
    ids = {int(v): n.lower() for n, v in re.findall(r"\bMOE_KERNEL_([A-Z0-9_]+)\s*=\s*(\d+)", src)}
    assert sorted(ids) == list(range(len(ids)))
    assert tuple(ids[i] for i in range(len(ids))) == abi.KERNELS
    body = re.search(r"typedef struct \{([^}]*)\}\s*moe_config;", src).group(1)
    fields = re.findall(r"int32_t\s+(\w+);", body)
    assert fields == [f for f, _ in abi.MoeConfig._fields_]


def _cfg(**kw):
    base = dict(hidden=7168, latent=3584, n_experts=896, top_k=16, inter=384, n_shared=2,
                shared_inter=384, has_latent_proj=1)
    base.update(kw)
    return abi.make_config(**base)


def test_packed_size_matches_layout():
    pb, wb = abi.query(_cfg(), 64)
    E, H, Lt, I, S, Is = 896, 7168, 3584, 384, 2, 384
    mx = lambda n, k: (n // 16) * (k // 128) * 1088        # noqa: E731
    # router, x-side, their combined copy (router rows padded to 64), output side, experts
    E_rx = (E + 63) // 64 * 64
    expect = (E * H * 2 + (Lt + 2 * S * Is) * H * 2 + (E_rx + Lt + 2 * S * Is) * H * 2 + H * (Lt + S * Is) * 2
              + E * (mx(2 * I, Lt) + mx(Lt, I)))
    assert expect <= pb < expect + 6 * 256
    # one expert's MXFP4 bytes: three 3584 x 384 matrices at 4.25 bits per value
    assert mx(2 * I, Lt) + mx(Lt, I) == 3 * 3584 * 384 * 17 // 32
    lay = abi.workspace_layout(_cfg(), 64)
    assert lay["total"] == wb and all(lay[k] % 256 == 0 for k in lay)
    assert lay["y"] + 64 * 16 * Lt * 2 <= lay["total"]


@pytest.mark.parametrize("kw", [dict(latent=3500), dict(inter=100), dict(top_k=0), dict(top_k=33),
                                dict(n_experts=1025), dict(top_k=9, n_experts=8),
                                dict(has_latent_proj=0, n_shared=1), dict(hidden=7000),
                                dict(shared_inter=30), dict(n_shared=-1)])
def test_query_rejects_bad_configs(kw):
    c = _cfg(**kw)
    pb = ctypes.c_size_t(0)
    assert abi.lib().moe_query(ctypes.byref(c), 64, ctypes.byref(pb), None) == abi.Status.INVALID_ARG


def test_query_rejects_negative_tokens_and_reports_strings():
    c = _cfg()
    assert abi.lib().moe_query(ctypes.byref(c), -1, None, None) == abi.Status.INVALID_ARG
    for s in abi.Status:
        assert abi.lib().moe_strerror(int(s))
    assert abi.lib().moe_strerror(-99) == b"unknown status"


def test_create_route_forward_reject_null_arguments_without_gpu_work():
    L = abi.lib()
    c = _cfg()
    w = abi.MoeWeights()
    h = ctypes.c_void_p()
    assert L.moe_create(ctypes.byref(c), ctypes.byref(w), None, 0, None, ctypes.byref(h)) == abi.Status.INVALID_ARG
    assert L.moe_create(ctypes.byref(c), ctypes.byref(w), 256, 1 << 40, None, ctypes.byref(h)) == \
        abi.Status.INVALID_ARG
    r = abi.MoeRouting()
    assert L.moe_route(None, None, 4, None, None, None, ctypes.byref(r), None, 0, None) == abi.Status.INVALID_ARG
    assert L.moe_forward(None, None, 4, ctypes.byref(r), None, None, 0, None) == abi.Status.INVALID_ARG
    assert L.moe_unpack_expert(None, 0, 0, None, None) == abi.Status.INVALID_ARG
    L.moe_destroy(None)


def test_graph_entry_points_reject_bad_arguments_without_gpu_work():
    L = abi.lib()
    r = abi.MoeRouting()
    g = ctypes.c_void_p(123)
    assert L.moe_graph_create(None, None, 4, None, None, ctypes.byref(r), None, None, 0, ctypes.byref(g)) == \
        abi.Status.INVALID_ARG
    assert g.value is None                      # cleared before any check that fails
    assert L.moe_graph_create(None, None, 4, None, None, ctypes.byref(r), None, None, 0, None) == \
        abi.Status.INVALID_ARG
    assert L.moe_graph_launch(None, None) == abi.Status.INVALID_ARG
    L.moe_graph_destroy(None)


def test_fp8_second_stage_sizes():
    """MOE_STAGE2_FP8 adds one MX8 copy of the down weights and the FP8 h (codes + scales)."""
    T, E, Lt, I, K = 64, 896, 3584, 384, 16
    pb0, wb0 = abi.query(_cfg(), T)
    pb1, wb1 = abi.query(_cfg(stage2_fp8=True), T)
    mx_down = (Lt // 16) * (I // 128) * 1088
    assert pb1 - pb0 == E * mx_down
    lay0, lay1 = abi.workspace_layout(_cfg(), T), abi.workspace_layout(_cfg(stage2_fp8=True), T)
    assert lay0["partials"] == lay0["h8"]                    # empty region in the BF16 mode
    assert lay1["partials"] - lay1["h8"] == -(-(T * K * I + T * K * I // 32) // 256) * 256
    assert wb1 - wb0 == lay1["partials"] - lay1["h8"]


@pytest.mark.parametrize("kw", [dict(stage2_fp8=True, inter=640)])
def test_fp8_second_stage_rejects_unsupported_shapes(kw):
    c = _cfg(**kw)
    assert abi.lib().moe_query(ctypes.byref(c), 64, None, None) == abi.Status.INVALID_ARG


def test_shared_stream_sizes():
    """MOE_SHARED_STREAM packs the shared gate/up rows once, as a matrix of their own, and leaves them
    out of the x-side and the combined router + x-side matrices; the workspace is unchanged."""
    T, H, S, Is = 64, 7168, 2, 384
    pb0, wb0 = abi.query(_cfg(), T)
    pb1, wb1 = abi.query(_cfg(shared_stream=True), T)
    assert pb0 - pb1 == 2 * S * Is * H * 2   # one BF16 copy of the rows fewer (every region 256-B aligned here)
    assert wb1 == wb0
    none = dict(n_shared=0, shared_inter=0)
    assert abi.query(_cfg(shared_stream=True, **none), T) == abi.query(_cfg(**none), T)


def test_unknown_shared_stream_mode_is_rejected():
    c = _cfg()
    c.shared_stream = 2
    assert abi.lib().moe_query(ctypes.byref(c), 64, None, None) == abi.Status.INVALID_ARG


def test_unknown_second_stage_is_rejected():
    c = _cfg()
    c.stage2 = 2
    assert abi.lib().moe_query(ctypes.byref(c), 64, None, None) == abi.Status.INVALID_ARG


def test_mxfp4_first_stage_sizes():
    """MOE_STAGE1_MXFP4 adds one A4 copy of the gate|up weights and the MX FP4 z (codes + scales)."""
    T, E, Lt, I = 64, 896, 3584, 384
    pb0, wb0 = abi.query(_cfg(), T)
    pb1, wb1 = abi.query(_cfg(stage1_a4=True), T)
    mx_gateup = (2 * I // 16) * (Lt // 128) * 1088
    assert pb1 - pb0 == E * mx_gateup
    lay0, lay1 = abi.workspace_layout(_cfg(), T), abi.workspace_layout(_cfg(stage1_a4=True), T)
    assert lay0["partials"] == lay0["z4"] == lay0["h8"]      # both quantised regions empty
    assert lay1["partials"] - lay1["z4"] == -(-(T * Lt // 2 + T * Lt // 32) // 256) * 256
    assert wb1 - wb0 == lay1["partials"] - lay1["z4"]
    # both modes together: two regions side by side
    lay2 = abi.workspace_layout(_cfg(stage1_a4=True, stage2_fp8=True), T)
    assert lay2["z4"] > lay2["h8"] and lay2["partials"] > lay2["z4"]


def test_unknown_first_stage_is_rejected():
    c = _cfg()
    c.stage1 = 2
    assert abi.lib().moe_query(ctypes.byref(c), 64, None, None) == abi.Status.INVALID_ARG


def _shape_cfg(shape, **kw):
    return abi.make_config(shape.H, shape.Lt, shape.E, shape.K, shape.I, shape.S, shape.Is, shape.has_latent, **kw)


@pytest.mark.parametrize("name", ["tiny", "tp8_decode_t64", "tp8_prefill_t8192", "full_experts_t4096"])
@pytest.mark.parametrize("quant", [{}, dict(stage2_fp8=True, stage1_a4=True)])
def test_query_workspace_serves_every_smaller_batch(name, quant):
    """moe_query(T_max) must cover every call with T <= T_max: the few-token split-K partials exist
    only up to 64 tokens and the tile list shrinks once experts average 32 rows, so the workspace
    of T_max alone can be smaller than that of a smaller T."""
    from workload import SHAPES
    s = SHAPES[name]
    if quant and s.I > 512:
        return   # the FP8 second stage keeps an I-wide h tile in LDS (I <= 512)
    c = _shape_cfg(s, **quant)
    thr = -(-32 * s.E // s.K)                 # first token count on the many-rows expert path
    for T_max in sorted({1, 63, 64, 65, 128, 200, thr - 1, thr, thr + 7, 2 * thr, s.T}):
        _, wb = abi.query(c, T_max)
        for T in sorted({0, 1, 16, 63, 64, 65, T_max // 2, thr - 1, thr, T_max}):
            if 0 <= T <= T_max:
                need = abi.workspace_layout(c, T)["total"]
                assert need <= wb, (name, T_max, T, need, wb)


def test_query_accepts_large_batches_and_rejects_unlaunchable_ones():
    """Token counts past the 65,535 grid.y limit are served (the combine takes a 1-D grid); counts
    whose index products or grids cannot be formed are rejected before anything is enqueued."""
    c = _cfg()
    pb, wb = abi.query(c, 70000)
    assert pb > 0 and wb > 0
    assert abi.lib().moe_query(ctypes.byref(c), 70000, None, None) == abi.Status.OK
    # T x E >= 2^31
    assert abi.lib().moe_query(ctypes.byref(c), 2_400_000, None, None) == abi.Status.INVALID_ARG
    # index products fit, but the combine's grid (T x 7 workgroups) would not
    big = abi.make_config(3584, 3584, 1, 1, 3072, 0, 0, False)
    assert abi.lib().moe_query(ctypes.byref(big), 2_000_000_000, None, None) == abi.Status.INVALID_ARG
    lay = (ctypes.c_size_t * 11)()
    assert abi.lib().moe_query_workspace_layout(ctypes.byref(big), 2_000_000_000, lay) == abi.Status.INVALID_ARG
    r = abi.MoeRouting()
    # route / forward reject such T before touching the handle's GPU state (null handle here)
    assert abi.lib().moe_route(None, None, 2_000_000_000, None, None, None, ctypes.byref(r), None, 0, None) == \
        abi.Status.INVALID_ARG
