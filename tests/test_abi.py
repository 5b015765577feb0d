"""CPU-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

from combine_router_softmax_top_amd import binding as B
from combine_router_softmax_top_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(moe_[a-z0-9_]+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return B.lib()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["moe_route", "moe_dispatch", "moe_expert_mlp", "moe_combine", "moe_forward_dbo"]:
        assert n in names
    assert sorted(B.EXPORTED) == names


def test_library_exports_every_declared_symbol(lib):
    for n in _declared():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert B.status_string(B.MOE_OK) == "ok"
    assert "workspace" in B.status_string(B.MOE_ERR_WORKSPACE_TOO_SMALL)


@pytest.mark.parametrize("field,value,status", [
    ("top_k", 0, B.MOE_ERR_INVALID_ARGUMENT),
    ("top_k", 17, B.MOE_ERR_INVALID_ARGUMENT),
    ("num_experts", 513, B.MOE_ERR_INVALID_ARGUMENT),
    ("num_tokens", 0, B.MOE_ERR_INVALID_ARGUMENT),
    ("expert_end", 257, B.MOE_ERR_INVALID_ARGUMENT),
    ("expert_begin", 32, B.MOE_ERR_INVALID_ARGUMENT),
    ("num_shared", 5, B.MOE_ERR_INVALID_ARGUMENT),
    ("score", 7, B.MOE_ERR_INVALID_ARGUMENT),
    ("dtype", 9, B.MOE_ERR_INVALID_ARGUMENT),
    ("hidden", 7000, B.MOE_ERR_UNSUPPORTED),
    ("intermediate", 100, B.MOE_ERR_UNSUPPORTED),
])
def test_config_validation_on_host(lib, field, value, status):
    cs = B.config_struct(W.CONFIGS["dsv3_prefill_ep"])
    setattr(cs, field, value)
    P = ctypes.c_void_p
    st = lib.moe_route(ctypes.byref(cs), P(16), P(16), None, P(16), P(16), None, P(256), 1 << 30, None)
    assert st == status
    assert lib.moe_workspace_bytes(ctypes.byref(cs), B.MOE_WS_FORWARD) == 0


def test_null_pointers_and_small_workspace_rejected_on_host(lib):
    cs = B.config_struct(W.CONFIGS["dsv3_prefill_ep"])
    P = ctypes.c_void_p
    assert lib.moe_route(ctypes.byref(cs), None, P(16), None, P(16), P(16), None, P(256), 1 << 30, None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_route(ctypes.byref(cs), P(8), P(16), None, P(16), P(16), None, P(256), 1 << 30, None) == \
        B.MOE_ERR_INVALID_ARGUMENT  # misaligned activations
    need = lib.moe_workspace_bytes(ctypes.byref(cs), B.MOE_WS_DISPATCH)
    st = lib.moe_dispatch(ctypes.byref(cs), P(256), P(256), P(256), P(256), P(256), P(256),
                          P(256), P(256), need - 1, None)
    assert st == B.MOE_ERR_WORKSPACE_TOO_SMALL
    # shared-expert pointers must be given iff num_shared > 0
    assert lib.moe_combine(ctypes.byref(cs), P(256), P(256), P(256), P(256), P(256), None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    cs3 = B.config_struct(W.CONFIGS["dsv2lite_decode"])
    assert lib.moe_combine(ctypes.byref(cs3), P(256), P(256), P(256), None, P(256), None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    ws = lib.moe_workspace_bytes(ctypes.byref(cs3), B.MOE_WS_EXPERT_MLP)
    assert lib.moe_expert_mlp(ctypes.byref(cs3), P(256), P(256), P(256), P(256), P(256), P(256),
                              None, None, None, None, None, P(256), ws, None) == \
        B.MOE_ERR_INVALID_ARGUMENT


def test_workspace_sizes_grow_with_tokens(lib):
    cfg = W.CONFIGS["dsv3_prefill_ep"]
    small = B.workspace_bytes(cfg.with_tokens(128), B.MOE_WS_FORWARD)
    big = B.workspace_bytes(cfg, B.MOE_WS_FORWARD)
    assert 0 < small < big
    dbo = B.workspace_bytes(W.CONFIGS["dsv3_dual_microbatch"], B.MOE_WS_FORWARD_DBO)
    assert dbo >= 2 * B.workspace_bytes(cfg, B.MOE_WS_FORWARD) * 0.99


@pytest.mark.parametrize("T,mid", [(8192, 4096), (100, 128), (300, 256), (256, 128), (1, 128)])
def test_dbo_split_point(lib, T, mid):
    assert B.dbo_split_point(T) == mid


def test_graph_entry_points_reject_bad_arguments_on_host(lib):
    cs = B.config_struct(W.CONFIGS["dsv3_prefill_ep"])
    h = ctypes.c_void_p()
    lt = B.LayerTensorsStruct()  # all NULL
    assert lib.moe_graph_launch(None, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_graph_destroy(None) == B.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_graph_capture_forward(ctypes.byref(cs), ctypes.byref(lt), None, 0,
                                         ctypes.byref(h)) == B.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_graph_capture_forward_dbo(ctypes.byref(cs), None, None, 0, 0,
                                             ctypes.byref(h)) == B.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_graph_capture_forward(ctypes.byref(cs), ctypes.byref(lt), None, 0,
                                         None) == B.MOE_ERR_INVALID_ARGUMENT
    bad = B.config_struct(W.CONFIGS["dsv3_prefill_ep"])
    bad.top_k = 0
    assert lib.moe_graph_capture_forward(ctypes.byref(bad), ctypes.byref(lt), None, 0,
                                         ctypes.byref(h)) == B.MOE_ERR_INVALID_ARGUMENT
    assert h.value is None  # nothing written on failure


def test_dbo_plan_split_matches_the_oracle_rule(lib):
    import oracle
    for T in list(range(1, 300, 7)) + [511, 512, 600, 768, 1000, 4096, 8192, 8200]:
        for prefill in (False, True):
            for q in (1, 2, 3, 5, 8, 10, 64, 256):
                for thr in (0, 300, 4096):
                    got = B.dbo_plan_split(T, prefill, thr, thr + 7, q)
                    assert got == oracle.dbo_split(T, prefill, thr, thr + 7, q), (T, prefill, q, thr)


@pytest.mark.parametrize("name", ["tiny_f32", "dsv2lite_decode", "dsv3_prefill_ep",
                                  "dsv2lite_decode+beside"])
def test_dbo_workspace_covers_every_cut(lib, name):
    cfg = W.CONFIGS[name.split("+")[0]]
    if name.endswith("+beside"):
        cfg = cfg.replace(shared_beside_combine=True)
    for T in (2, 3, 97, 256, 700):
        c = cfg.with_tokens(T)
        bound = B.workspace_bytes(c, B.MOE_WS_FORWARD_DBO)
        one = [0] + [B.workspace_bytes(cfg.with_tokens(n), B.MOE_WS_FORWARD) for n in range(1, T)]
        need = max(one[s] + one[T - s] for s in range(1, T))
        assert bound >= need and bound >= B.workspace_bytes(c, B.MOE_WS_FORWARD), (T, bound, need)



def test_quantize_mxfp8_rejects_bad_arguments_on_host(lib):
    P = 0x10000  # never dereferenced: every case below fails before any HIP call
    BF, F32, BAD = B.MOE_BF16, B.MOE_F32, 7
    R, M = B.MOE_MX_ROWS, B.MOE_MX_MFMA
    inv = B.MOE_ERR_INVALID_ARGUMENT
    q = lib.moe_quantize_mxfp8
    assert q(4, 48, BF, P, 48, R, P, P, None) == inv          # cols not a multiple of 32
    assert q(4, 0, BF, P, 0, R, P, P, None) == inv            # no columns
    assert q(-1, 64, BF, P, 64, R, P, P, None) == inv         # negative rows
    assert q(4, 64, BF, P, 32, R, P, P, None) == inv          # pitch below cols
    assert q(4, 64, BAD, P, 64, R, P, P, None) == inv         # unknown element type
    assert q(4, 64, BF, P, 64, 2, P, P, None) == inv          # unknown scale layout
    assert q(4, 992, BF, P, 992, M, P, P, None) == inv        # MFMA layout: cols % 512 != 0
    assert q(4, 64, BF, None, 64, R, P, P, None) == inv       # NULL input
    assert q(4, 64, BF, P, 64, R, None, P, None) == inv       # NULL codes
    assert q(4, 64, BF, P, 64, R, P, None, None) == inv       # NULL scales
    assert q(4, 64, BF, P + 8, 64, R, P, P, None) == inv      # input not 16-byte aligned
    assert q(4, 64, BF, P, 68, R, P, P, None) == inv          # bf16 pitch not 16-byte aligned
    assert q(4, 64, F32, P, 66, R, P, P, None) == inv         # fp32 pitch not 16-byte aligned
    assert q(4, 64, BF, P, 64, R, P + 4, P, None) == inv      # codes not 8-byte aligned
    assert q(4, 64, BF, P, 64, R, P, P + 2, None) == inv      # scales not 4-byte aligned
    assert q(0, 64, BF, None, 64, R, None, None, None) == B.MOE_OK  # nothing to do


def test_expert_mlp_mxfp8_rejects_bad_arguments_on_host(lib):
    P = 0x10000
    f = lib.moe_expert_mlp_mxfp8
    cfg = W.CONFIGS["dsv3_prefill_ep"]
    big = 1 << 30
    # xq, xs, offsets, wq_gate, sg, wq_up, su, w_down, wq_down, sd, y, workspace
    BF16_DOWN = [P] * 8 + [None, None] + [P, P]
    FP8_DOWN = [P] * 7 + [None, P, P] + [P, P]

    def call(c, ptrs=BF16_DOWN, ws=big):
        return f(ctypes.byref(B.config_struct(c)), *ptrs, ws, None)

    inv, uns = B.MOE_ERR_INVALID_ARGUMENT, B.MOE_ERR_UNSUPPORTED
    assert call(cfg.replace(dtype="f32")) == uns
    assert call(cfg.replace(num_shared=1)) == uns
    assert call(cfg.replace(hidden=7168 - 256)) == uns  # d % 512 != 0
    assert call(cfg.replace(intermediate=2048 - 64), FP8_DOWN) == uns  # fp8 down: I % 512 != 0
    for k in (0, 1, 2, 3, 4, 5, 6, 10, 11):  # always required
        for base in (BF16_DOWN, FP8_DOWN):
            p = list(base)
            p[k] = None
            assert call(cfg, p) == inv, k
    assert call(cfg, [P] * 12) == inv  # bf16 and fp8 down weights both given
    assert call(cfg, [P] * 7 + [None, None, None, P, P]) == inv  # neither
    assert call(cfg, [P] * 7 + [None, P, None, P, P]) == inv  # fp8 codes without scales
    p = list(FP8_DOWN)
    p[9] = P + 2  # down scales must be 4-byte aligned
    assert call(cfg, p) == inv
    p = list(BF16_DOWN)
    p[1] = P + 2  # scales must be 4-byte aligned
    assert call(cfg, p) == inv
    p = list(BF16_DOWN)
    p[0] = P + 4  # codes must be 16-byte aligned
    assert call(cfg, p) == inv
    assert call(cfg, ws=1) == B.MOE_ERR_WORKSPACE_TOO_SMALL
    assert call(cfg, FP8_DOWN, ws=1) == B.MOE_ERR_WORKSPACE_TOO_SMALL


def test_block_scaled_forward_and_capture_reject_bad_arguments_on_host(lib):
    cs = B.config_struct(W.CONFIGS["dsv3_prefill_ep"])
    h = ctypes.c_void_p()
    lt = B.LayerTensorsMxfp8Struct()  # all NULL
    inv, uns = B.MOE_ERR_INVALID_ARGUMENT, B.MOE_ERR_UNSUPPORTED
    assert lib.moe_forward_mxfp8(ctypes.byref(cs), ctypes.byref(lt), None, 0, None) == inv
    assert lib.moe_graph_capture_forward_mxfp8(ctypes.byref(cs), ctypes.byref(lt), None, 0,
                                               ctypes.byref(h)) == inv
    assert lib.moe_graph_capture_forward_mxfp8(ctypes.byref(cs), ctypes.byref(lt), None, 0,
                                               None) == inv
    P = 0x10000
    nf = len(B.LayerTensorsMxfp8Struct._fields_)
    SHARED = ("wsq_gate", "wsq_gate_scales", "wsq_up", "wsq_up_scales", "ws_down", "wsq_down",
              "wsq_down_scales")

    def tensors(fp8_down: bool, shared: bool):
        t = B.LayerTensorsMxfp8Struct(*([P] * nf))
        for f in (("w_down", "ws_down") if fp8_down else ("wq_down", "wq_down_scales", "wsq_down",
                                                           "wsq_down_scales")):
            setattr(t, f, None)
        if not shared:
            for f in SHARED:
                setattr(t, f, None)
        return t

    full = tensors(fp8_down=False, shared=False)
    assert lib.moe_forward_mxfp8(ctypes.byref(cs), ctypes.byref(full), P, 1, None) == \
        B.MOE_ERR_WORKSPACE_TOO_SMALL
    # shared-expert weights are given exactly when the layer has shared experts
    assert lib.moe_forward_mxfp8(ctypes.byref(cs), ctypes.byref(tensors(False, True)), P,
                                 1 << 40, None) == inv
    shared = B.config_struct(W.CONFIGS["dsv2lite_decode"])
    for fp8_down in (False, True):
        cfg = B.config_struct(W.CONFIGS["dsv2lite_decode"].replace(intermediate=1536)) \
            if fp8_down else shared
        ok = tensors(fp8_down, shared=True)
        assert lib.moe_forward_mxfp8(ctypes.byref(cfg), ctypes.byref(ok), P, 1, None) == \
            B.MOE_ERR_WORKSPACE_TOO_SMALL
        assert lib.moe_forward_mxfp8(ctypes.byref(cfg), ctypes.byref(tensors(fp8_down, False)),
                                     P, 1 << 40, None) == inv
        for f in SHARED:  # each one missing, or the down weights of the other kind added
            t = tensors(fp8_down, shared=True)
            setattr(t, f, None if getattr(t, f) else P)
            assert lib.moe_forward_mxfp8(ctypes.byref(cfg), ctypes.byref(t), P, 1 << 40,
                                         None) == inv, f
        t = tensors(fp8_down, shared=True)
        t.wsq_up_scales = P + 2  # scales must be 4-byte aligned
        assert lib.moe_forward_mxfp8(ctypes.byref(cfg), ctypes.byref(t), P, 1 << 40, None) == inv
        t = tensors(fp8_down, shared=True)
        t.wsq_gate = P + 4  # codes must be 16-byte aligned
        assert lib.moe_forward_mxfp8(ctypes.byref(cfg), ctypes.byref(t), P, 1 << 40, None) == inv
    # a rejected capture makes no graph
    assert lib.moe_graph_capture_forward_mxfp8(ctypes.byref(shared), ctypes.byref(lt), None, 0,
                                               ctypes.byref(h)) == inv
    assert h.value is None
    both = B.LayerTensorsMxfp8Struct(*([P] * nf))  # bf16 and fp8 down weights both given
    both.wsq_gate = both.wsq_gate_scales = both.wsq_up = both.wsq_up_scales = None
    both.ws_down = both.wsq_down = both.wsq_down_scales = None
    assert lib.moe_forward_mxfp8(ctypes.byref(cs), ctypes.byref(both), P, 1 << 40, None) == inv
    full.wq_gate_scales = P + 2  # scales must be 4-byte aligned
    assert lib.moe_forward_mxfp8(ctypes.byref(cs), ctypes.byref(full), P, 1 << 40, None) == inv


def test_packed_layout_is_validated_on_host(lib):
    P = 0x10000
    inv, uns = B.MOE_ERR_INVALID_ARGUMENT, B.MOE_ERR_UNSUPPORTED
    f = lib.moe_pack_weights
    assert f(-1, 128, 64, P, P * 64, None) == inv
    assert f(1, 0, 64, P, P * 64, None) == inv
    assert f(1, 192, 64, P, P * 64, None) == uns          # rows not a multiple of 128
    assert f(1, 128, 96, P, P * 64, None) == uns          # cols not a multiple of 64
    assert f(1 << 16, 1 << 13, 1 << 14, P, P * 64, None) == uns  # 2^43 elements: grid too large
    assert f(0, 128, 64, None, None, None) == B.MOE_OK    # nothing to do
    assert f(1, 128, 64, None, P * 64, None) == inv
    assert f(1, 128, 64, P + 8, P * 64, None) == inv      # not 16-byte aligned
    assert f(1, 128, 64, P, P + 128 * 64, None) == inv    # overlapping
    cfg = W.CONFIGS["dsv3_prefill_ep"]
    bad = B.config_struct(cfg)
    bad.weight_layout = 2
    assert lib.moe_workspace_bytes(ctypes.byref(bad), B.MOE_WS_FORWARD) == 0
    ok = B.config_struct(cfg.replace(packed_weights=True))
    assert ok.weight_layout == B.MOE_WEIGHTS_PACKED
    assert lib.moe_workspace_bytes(ctypes.byref(ok), B.MOE_WS_FORWARD) == \
        lib.moe_workspace_bytes(ctypes.byref(B.config_struct(cfg)), B.MOE_WS_FORWARD)
    # fp32 layers and widths that are not multiples of 128 have no packed form
    mlp = lib.moe_expert_mlp
    for c in (W.CONFIGS["tiny_f32"].replace(packed_weights=True),
              cfg.replace(intermediate=2048 - 64, packed_weights=True)):
        # x_sorted, offsets, w_gate, w_up, w_down, y_sorted; no shared experts; workspace
        assert mlp(ctypes.byref(B.config_struct(c)), *([P] * 6), *([None] * 5), P, 1 << 40,
                   None) == uns
    # nor does the block-scaled path (its weights are MX-FP8 encoded)
    lt = B.LayerTensorsMxfp8Struct(*([P] * len(B.LayerTensorsMxfp8Struct._fields_)))
    assert lib.moe_forward_mxfp8(ctypes.byref(ok), ctypes.byref(lt), P, 1 << 40, None) == uns


# ------------------------------------------------------------------ launch-size limits

def _route_status(lib, cs):
    P = ctypes.c_void_p
    # a NULL token pointer: INVALID_ARGUMENT once the shape is accepted, so no
    # kernel is ever launched on these fake pointers
    return lib.moe_route(ctypes.byref(cs), None, P(16), None, P(16), P(16), None, P(256),
                         1 << 40, None)


@pytest.mark.parametrize("width,status", [(20, B.MOE_ERR_UNSUPPORTED),   # 4 x odd
                                          (100, B.MOE_ERR_UNSUPPORTED),
                                          (48, B.MOE_ERR_INVALID_ARGUMENT),
                                          (16, B.MOE_ERR_INVALID_ARGUMENT)])
@pytest.mark.parametrize("field", ["hidden", "intermediate"])
def test_fp32_widths_are_multiples_of_16(lib, field, width, status):
    # include/moe.h: fp32 hidden and intermediate must be multiples of 16
    cs = B.config_struct(W.CONFIGS["tiny_f32"])
    setattr(cs, field, width)
    assert _route_status(lib, cs) == status
    assert (lib.moe_workspace_bytes(ctypes.byref(cs), B.MOE_WS_FORWARD) == 0) == \
        (status == B.MOE_ERR_UNSUPPORTED)


def test_token_count_limit(lib):
    # one 64-lane wave per token: T = MOE_MAX_TOKENS would need 2^32 work-items
    cs = B.config_struct(W.CONFIGS["dsv3_prefill_ep"].replace(hidden=64, intermediate=64,
                                                              top_k=1))
    cs.num_tokens = (1 << 26) - 1
    assert _route_status(lib, cs) == B.MOE_ERR_INVALID_ARGUMENT
    cs.num_tokens = 1 << 26
    assert _route_status(lib, cs) == B.MOE_ERR_UNSUPPORTED


def _gemm_workitems(T, K, n_loc, S, d, I):
    """Work-items of the larger bf16 grouped-GEMM launch (256x256 tiles, 512
    threads; gate/up tiles 128 columns wide, down 256), as the launcher sizes
    its grid: 8 XCDs x (column tiles per XCD x (row tiles per XCD + 1))."""
    rt = -(-T * K // 256) + n_loc + S * -(-T // 256)

    def wi(col_tiles):
        rx = 2 if col_tiles >= 4 else 8
        cx = 8 // rx
        return 8 * -(-col_tiles // cx) * (-(-rt // rx) + 1) * 512
    return max(wi(-(-I // 128)), wi(-(-d // 256)))


def test_grouped_gemm_grid_limit(lib):
    # the largest hidden size (a multiple of 64) whose down-projection grid
    # stays under 2^32 work-items is accepted, the next one is not
    T, K = 1 << 20, 8
    cfg = W.CONFIGS["dsv3_prefill_ep"].replace(num_tokens=T, top_k=K, intermediate=64)
    d = 64
    while _gemm_workitems(T, K, cfg.num_local, 0, d + 64, 64) < 0xffffffff:
        d += 64
    for width, status in [(d, B.MOE_ERR_INVALID_ARGUMENT), (d + 64, B.MOE_ERR_UNSUPPORTED)]:
        cs = B.config_struct(cfg.replace(hidden=width))
        assert _route_status(lib, cs) == status, width


def test_pack_and_quantize_launch_limits(lib):
    P = ctypes.c_void_p
    # pack: one work-item per 8 elements; 2^22 stacks of 128 x 64 need 2^32
    assert lib.moe_pack_weights((1 << 22) - 1, 128, 64, None, P(256), None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_pack_weights(1 << 22, 128, 64, P(256), P(4096), None) == B.MOE_ERR_UNSUPPORTED
    # quantize: rows * cols / 8 work-items, rounded up to workgroups of 256
    rows_ok = (1 << 30) - 65
    assert lib.moe_quantize_mxfp8(rows_ok, 32, B.MOE_BF16, None, 32, B.MOE_MX_ROWS, P(256),
                                  P(256), None) == B.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_quantize_mxfp8(rows_ok + 1, 32, B.MOE_BF16, P(256), 32, B.MOE_MX_ROWS,
                                  P(256), P(256), None) == B.MOE_ERR_UNSUPPORTED


def test_probe_header_declares_the_exported_probes(lib):
    src = open(os.path.join(ROOT, "include", "moe_probe.h")).read()
    names = sorted(set(re.findall(r"^\S.*?\b(moe_[a-z0-9_]+)\s*\(", src, flags=re.M)))
    assert names == sorted(B.PROBE_EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    P = ctypes.c_void_p
    # host checks, nothing launched: bad kind, unaligned size, missing pointers
    assert lib.moe_probe_stream(3, P(256), P(256), 1024, None, 8, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_probe_stream(0, P(256), P(256), 1000, None, 8, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_probe_stream(1, None, P(256), 1024, None, 8, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_probe_mfma(2, 1, 1, P(256), None) == B.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_probe_mfma(0, 1, 1, None, None) == B.MOE_ERR_INVALID_ARGUMENT
    # 8 chains x 8 waves x 32x32x16 MFMAs of 32768 flop each
    assert lib.moe_probe_mfma_flops(0, 2, 3) == 2 * 3 * 8 * 8 * 32768
    assert lib.moe_probe_mfma_flops(1, 1, 1) == 8 * 8 * 131072


def test_shared_placement_is_validated_on_host(lib):
    cfg = W.CONFIGS["dsv2lite_decode"]
    cs = B.config_struct(cfg)
    fused = lib.moe_workspace_bytes(ctypes.byref(cs), B.MOE_WS_FORWARD)
    cs.shared_placement = B.MOE_SHARED_BESIDE_COMBINE
    beside = lib.moe_workspace_bytes(ctypes.byref(cs), B.MOE_WS_FORWARD)
    # the combine's fp32 sums [T, d] are kept for the shared rows
    assert beside == fused + cfg.num_tokens * cfg.hidden * 4
    cs.shared_placement = 2
    assert lib.moe_workspace_bytes(ctypes.byref(cs), B.MOE_WS_FORWARD) == 0
    assert _route_status(lib, cs) == B.MOE_ERR_INVALID_ARGUMENT
    # without shared experts the placement changes nothing
    c4 = B.config_struct(W.CONFIGS["dsv3_prefill_ep"])
    a = lib.moe_workspace_bytes(ctypes.byref(c4), B.MOE_WS_FORWARD)
    c4.shared_placement = B.MOE_SHARED_BESIDE_COMBINE
    assert lib.moe_workspace_bytes(ctypes.byref(c4), B.MOE_WS_FORWARD) == a
