"""GPU parity of the block-scaled 8-bit path against the CPU oracle.

MX-FP8 quantization (moe_quantize_mxfp8): codes and scale bytes bit-exact
against the oracle on seeded rows, on hand-built edge blocks (all-zero and
negative-zero blocks, subnormal inputs, ties at every level of E4M3, values that
scale past 448 and into the non-saturating range of the hardware conversion,
values near the top of the input type) and on ragged, strided and full-width
shapes; in the MFMA scale order, the same bytes permuted as the header states.

Block-scaled expert MLP (moe_expert_mlp_mxfp8): against the oracle's fp64 MLP
on the decoded operands (the oracle's own quantization, bit-equal to the GPU's),
rel-L2 <= 1e-2 per output tensor like every bf16 output; the GPU's error comes
only from fp32 accumulation and the bf16 roundings of h and y.  With the down
projection in fp8 too, h is encoded from the kernel's fp32 values and the
oracle's fp64 ones, a decision taken in two precisions; at full size every row
of y is therefore also checked against the oracle's down projection of the
kernel's own h codes and scales (stage-chained), and those codes against the
oracle's encoding of its h (_check_h_encoding).  The block-scaled dispatch at
full size: every row's codes and scales bit-exact.
"""
import math
import sys

import pytest
import torch

import oracle
from combine_router_softmax_top_amd import binding as B
from combine_router_softmax_top_amd import workloads as W
from combine_router_softmax_top_amd.layer import MoELayer

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield


def _seeded_rows(rows: int, cols: int, seed: int, dtype) -> torch.Tensor:
    """Gaussian rows with a per-block magnitude drawn from 2^[-24, 24]."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, cols, generator=g, dtype=torch.float64)
    mag = torch.randint(-24, 25, (rows, cols // 32), generator=g).to(torch.float64)
    x = x * torch.exp2(mag).repeat_interleave(32, dim=1)
    return x.to(dtype)


def _edge_rows(dtype) -> torch.Tensor:
    """One row per edge case, 32 columns each (one block), exactly representable
    in bf16 and fp32."""
    def blk(vals):
        v = list(vals) + [0.0] * (32 - len(vals))
        return v[:32]

    cases = [
        blk([]),                                                    # all zero: scale 2^-127
        blk([-0.0] * 32),                                          # negative zeros
        blk([2.0 ** -130, -3 * 2.0 ** -133, 2.0 ** -127]),         # bf16 subnormals
        blk([1016.0, 944.0, 928.0, 912.0, 896.0, -1016.0, 960.0]),  # scale 2^1: 508, 472, 464 ...
        blk([1.0, 2.0 ** -12, 2.0 ** -17, 3 * 2.0 ** -19, 2.0 ** -19, 2.0 ** -18,
             3 * 2.0 ** -18, -2.0 ** -19, -2.0 ** -17]),            # subnormal E4M3 ties and signs
        blk([300.0, 1.0625, 1.1875, 17.0, 19.0, -17.0, 272.0, 304.0, 0.01171875]),  # normal ties
        blk([3.0e38, -1.0e38, 2.5e37, 1.0]),                       # near the top of the range
        blk([2.0 ** k for k in range(-16, 16)]),                    # one element per binade
        blk([-(2.0 ** 9) + 2.0 ** 1, 2.0 ** 8]),                    # max just under a power of two
        blk([256.0, -255.0, 129.0, 0.5]),                           # scale exactly 2^0
    ]
    return torch.tensor(cases, dtype=torch.float64).to(dtype)


def _gpu_quantize(x: torch.Tensor, layout: int = B.MOE_MX_ROWS):
    rows, cols = x.shape
    codes = torch.full((rows, cols), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows, cols // 32), 0xAB, dtype=torch.uint8, device="cuda")
    B.moe_quantize_mxfp8(x, codes, scales, layout)
    torch.cuda.synchronize()
    return codes.cpu(), scales.cpu()


def _to_mfma_order(nat: torch.Tensor) -> torch.Tensor:
    """Scale bytes in row order [rows, cols/32] -> the MFMA order: block
    q = 16g + m of row r, m = 8d + 4j + 2s + h, to byte 2j + s of 32-bit word
    ((2g + d) rows + r) 2 + h."""
    rows, nb = nat.shape
    out = torch.empty(rows * nb, dtype=torch.uint8)
    r = torch.arange(rows)
    for q in range(nb):
        g, m = divmod(q, 16)
        d, j, s_, h = m >> 3, (m >> 2) & 1, (m >> 1) & 1, m & 1
        out[(((2 * g + d) * rows + r) * 2 + h) * 4 + 2 * j + s_] = nat[:, q]
    return out.view(rows, nb)


def _check(x_cpu: torch.Tensor, x_dev: torch.Tensor):
    want_c, want_s = oracle.mxfp8_quantize(x_cpu)
    got_c, got_s = _gpu_quantize(x_dev)
    bad_s = (got_s != want_s).nonzero()
    assert bad_s.numel() == 0, f"scale mismatch at {bad_s[:8].tolist()}"
    bad_c = (got_c != want_c).nonzero()
    if bad_c.numel():
        r, c = bad_c[0].tolist()
        raise AssertionError(f"{bad_c.shape[0]} code mismatches; first at ({r}, {c}): "
                             f"x={float(x_cpu[r, c])!r} got {int(got_c[r, c]):#04x} "
                             f"want {int(want_c[r, c]):#04x}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_mxfp8_quantize_edge_blocks(dtype):
    x = _edge_rows(dtype)
    # The same blocks again, side by side in one row and in reverse order, so
    # that every block also sits at a non-zero block index.
    wide = torch.cat([x.reshape(1, -1), x.flip(0).reshape(1, -1)], dim=0)
    _check(x, x.cuda())
    _check(wide, wide.cuda())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols", [(1, 32), (37, 96), (300, 512), (5, 7168)])
def test_mxfp8_quantize_seeded(dtype, rows, cols):
    x = _seeded_rows(rows, cols, 11 + rows, dtype)
    _check(x, x.cuda())


def test_mxfp8_quantize_strided_rows():
    """Rows with a pitch beyond cols: only the first cols elements count."""
    full = _seeded_rows(64, 2048 + 64, 5, torch.bfloat16)
    x = full[:, :2048]
    _check(x.contiguous(), full.cuda()[:, :2048])


def test_mxfp8_quantize_full_width_dispatch_payload():
    """A DeepSeek-V3 token payload (d = 7168) for 2048 tokens."""
    x = _seeded_rows(2048, 7168, 3, torch.bfloat16)
    _check(x, x.cuda())


@pytest.mark.parametrize("rows,cols", [(3, 512), (37, 1024), (130, 7168)])
def test_mxfp8_quantize_mfma_scale_order(rows, cols):
    x = _seeded_rows(rows, cols, 7 + rows, torch.bfloat16)
    want_c, want_s = oracle.mxfp8_quantize(x)
    got_c, got_s = _gpu_quantize(x.cuda(), B.MOE_MX_MFMA)
    assert torch.equal(got_c, want_c)
    assert torch.equal(got_s, _to_mfma_order(want_s))


def test_mxfp8_quantize_zero_rows_is_a_no_op():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    codes = torch.empty(0, 64, dtype=torch.uint8, device="cuda")
    scales = torch.empty(0, 2, dtype=torch.uint8, device="cuda")
    B.moe_quantize_mxfp8(x, codes, scales)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- expert MLP

def _mlp_case(n_loc, counts, d, I, seed):
    """Seeded operands of one block-scaled expert-MLP call: x_sorted rows with
    per-block magnitudes 2^[-6, 6], weights N(0, 0.02^2) with per-block
    magnitudes 2^[-3, 3], and expert row counts `counts` (padded with empty
    experts) in a buffer of T*K rows."""
    g = torch.Generator().manual_seed(seed)
    total = int(sum(counts))
    cap = total + 37  # rows past the local count are never read
    def blocky(rows, cols, lo, hi, std):
        v = torch.randn(rows, cols, generator=g, dtype=torch.float64) * std
        mag = torch.randint(lo, hi + 1, (rows, cols // 32), generator=g).to(torch.float64)
        return (v * torch.exp2(mag).repeat_interleave(32, dim=1)).to(torch.bfloat16)
    x = blocky(cap, d, -6, 6, 1.0)
    wg = blocky(n_loc * I, d, -3, 3, 0.02).view(n_loc, I, d)
    wu = blocky(n_loc * I, d, -3, 3, 0.02).view(n_loc, I, d)
    wd = (torch.randn(n_loc, d, I, generator=g) * 0.02).to(torch.bfloat16)
    offsets = torch.zeros(n_loc + 1, dtype=torch.int32)
    offsets[1:len(counts) + 1] = torch.tensor(counts, dtype=torch.int32).cumsum(0)
    offsets[len(counts) + 1:] = total
    return x, wg, wu, wd, offsets, cap


def _encode(w2d: torch.Tensor):
    rows, cols = w2d.shape
    q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    s_ = torch.empty(rows * cols // 32, dtype=torch.uint8, device="cuda")
    B.moe_quantize_mxfp8(w2d.cuda(), q, s_.view(rows, cols // 32), B.MOE_MX_MFMA)
    return q, s_


def _run_mlp_mxfp8(cfg, x, wg, wu, wd, offsets, down=False, keep_workspace=False):
    n_loc, I, d = wg.shape
    rows = x.shape[0]
    xq, xs = _encode(x)
    gq, gs = _encode(wg.reshape(n_loc * I, d))
    uq, us = _encode(wu.reshape(n_loc * I, d))
    y = torch.full((rows, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    work = B.alloc_workspace(cfg, B.MOE_WS_EXPERT_MLP)
    if down:
        dq_, ds_ = _encode(wd.reshape(n_loc * d, I))
        B.moe_expert_mlp_mxfp8(cfg, xq, xs, offsets.cuda(), gq, gs, uq, us, None, y, work,
                               wq_down=dq_, wq_down_scales=ds_)
    else:
        B.moe_expert_mlp_mxfp8(cfg, xq, xs, offsets.cuda(), gq, gs, uq, us, wd.cuda(), y, work)
    torch.cuda.synchronize()
    return (y.cpu(), work.cpu()) if keep_workspace else y.cpu()


def _h_of_workspace(work, rows, I, total):
    """The MX-FP8 h the gate/up kernel left in the expert-MLP workspace:
    codes [T*K, I] first, then the scales in the MFMA layout over T*K rows;
    returned for the first `total` rows, scales in row order."""
    codes = work[:rows * I].view(rows, I)[:total]
    off = (rows * I + 255) // 256 * 256
    sc = work[off:off + rows * I // 32]
    scales = sc[_mfma_positions(rows, I // 32).flatten()].view(rows, I // 32)[:total]
    return codes.contiguous(), scales.contiguous()


def _check_h_encoding(codes_g, scales_g, h_o, delta=1e-4, tau=1e-4):
    """The kernel encodes h from its fp32 values (sums of thousands of fp32
    products: relative errors near 1e-5, absolute ones near 1e-5 of the row's
    largest |h|), the oracle from fp64, so codes near a rounding boundary, the
    tiny elements of a block (whose E4M3 steps, subnormal, are finer than that
    absolute error) and blocks whose largest |h| is on a power of two may be
    encoded differently.  Checked: a scale differs by one binade at most, only
    where the block maximum is within `delta` (relative) plus tau times the
    row's largest |h| of a power of two, in at most 1e-3 of the blocks; every
    code decodes to within one E4M3 step, plus tau times the row's largest
    |h|, of the oracle's value at the kernel's scale (clamped to +-448 as the
    rule clamps); and at most 1 % of the codes differ (a systematic one-step
    error would move most of them)."""
    codes_o, scales_o = oracle.mxfp8_quantize(h_o)
    rows, I = h_o.shape
    sd = scales_g.to(torch.int16) - scales_o.to(torch.int16)
    bad_s = sd != 0
    amax = h_o.abs().view(rows, I // 32, 32).amax(2).clamp_min(1e-300)
    pow2 = torch.exp2(torch.round(torch.log2(amax)))
    near_pow2 = (amax - pow2).abs() <= delta * amax + tau * h_o.abs().amax(1, keepdim=True)
    assert bool((sd[bad_s].abs() == 1).all()), "a scale differs by more than one binade"
    assert bool(near_pow2[bad_s].all()), "a scale differs away from a power-of-two maximum"
    frac_s = float(bad_s.double().mean())
    assert frac_s <= 1e-3, f"{frac_s:.2e} of the h scales differ"
    scale = torch.exp2(scales_g.to(torch.float64) - 127).repeat_interleave(32, dim=1)
    vc = (h_o / scale).clamp(-448.0, 448.0)
    step = torch.exp2(torch.floor(torch.log2(vc.abs().clamp(min=2.0 ** -6))) - 3)  # 2^-9 below 2^-6
    slack = tau * h_o.abs().amax(1, keepdim=True) / scale
    vg = oracle.mxfp8_dequantize(codes_g, scales_g) / scale
    ok = (vg - vc).abs() <= step * (1 + 1e-9) + slack
    bad = (~ok).nonzero()
    assert len(bad) == 0, (f"{len(bad)} codes beyond one E4M3 step of the oracle's value, "
                           f"first at (row, column) {tuple(bad[0].tolist())}")
    mism = codes_g != codes_o
    frac = float(mism.double().mean())
    assert frac <= 1e-2, f"{frac:.2e} of the h codes differ"
    return int(mism.sum()), int(bad_s.sum())


def _oracle_rows(rows, row_expert, x, wg, wu, wd, down=False):
    """The oracle's block-scaled MLP on the given x_sorted rows, with the stacks
    of the experts they use."""
    used = sorted(set(row_expert.tolist()))
    remap = {e: k for k, e in enumerate(used)}
    re = torch.tensor([remap[int(e)] for e in row_expert], dtype=torch.int32)
    pick = lambda w: w[used].contiguous()
    return oracle.expert_mlp_mxfp8(x[rows].contiguous(), re, pick(wg), pick(wu), pick(wd), down)


def _rel_l2(got, want):
    return float((got.double() - want).norm() / want.norm())


MLP_CASES = {
    # name: (n_loc, counts, d, I): ragged groups, empty experts, every short-tile
    # height, several row and column tiles, a partial column tile (I % 128 = 64)
    "ragged_small": (6, [300, 0, 77, 193, 64, 1], 512, 320),
    "deep_k": (3, [257, 130, 511], 2048, 256),
    "one_expert": (1, [700], 1024, 192),
    # I a multiple of 512, so the down projection can run in fp8 too; d = 1536
    # leaves a partial 256-column tile in the fp8 down kernel
    "ragged_i512": (6, [300, 0, 77, 193, 64, 1], 1536, 512),
    "deep_i1024": (3, [257, 130, 511], 1024, 1024),
}
MLP_PARAMS = [(n, False) for n in MLP_CASES] + \
    [(n, True) for n, c in MLP_CASES.items() if c[3] % 512 == 0]


@pytest.mark.parametrize("name,down", MLP_PARAMS)
def test_expert_mlp_mxfp8_matches_oracle(name, down):
    n_loc, counts, d, I = MLP_CASES[name]
    x, wg, wu, wd, offsets, cap = _mlp_case(n_loc, counts, d, I, seed=len(name))
    K = 1
    cfg = W.MoEConfig(name, cap, d, max(n_loc, 1), K, I, 0, n_loc, 0, "softmax", True, "bf16",
                      "normal")
    y = _run_mlp_mxfp8(cfg, x, wg, wu, wd, offsets, down)
    total = int(offsets[-1])
    row_expert = torch.repeat_interleave(torch.arange(n_loc), (offsets[1:] - offsets[:-1]).long())
    want = _oracle_rows(torch.arange(total), row_expert, x, wg, wu, wd, down)
    err = _rel_l2(y[:total], want)
    print(f"{name} (fp8 down: {down}): rel-L2 {err:.2e}", file=sys.stderr)
    assert torch.isfinite(y[:total].float()).all()
    assert err <= 1e-2
    assert torch.isnan(y[total:].float()).all()  # rows past the local count untouched


# Per-row bound at full size, on top of the whole-output rel-L2: one column
# off by the size of the values moves a row of width 7168 by about 0.017.
ROW_REL_L2 = 1e-2


@pytest.mark.parametrize("down", [False, True])
def test_expert_mlp_mxfp8_full_size_every_row(down):
    """The DeepSeek-V3 expert share at full size (T=4096, d=7168, 32 local
    experts, I=2048) with the routing of its seeded workload, every row of
    y_sorted.  bf16 down projection: each row against the oracle's
    block-scaled MLP within ROW_REL_L2.  fp8 down projection: the kernel
    encodes h from fp32 and the oracle from fp64, so the encoding decision is
    taken from the kernel (stage-chained): each row of y within ROW_REL_L2 of
    the oracle's decoded h (the kernel's codes and scales) times the decoded
    down weights, and the codes themselves valid encodings of the oracle's h
    (_check_h_encoding).  Both: the whole output within 1e-2 of the oracle."""
    cfg = W.CONFIGS["dsv3_prefill_ep"]
    T, K, d, I, n_loc = cfg.num_tokens, cfg.top_k, cfg.hidden, cfg.intermediate, cfg.num_local
    inp = W.make_inputs(cfg, 0, with_experts=False)
    ids, _, _ = oracle.route(inp["x"], inp["w_router"], inp["bias"], K, cfg.score,
                            cfg.renormalize)
    counts = torch.bincount(ids.flatten().long(), minlength=cfg.num_experts)[:n_loc]
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(T * K, d, generator=g) * 0.5).to(torch.bfloat16)
    wg = (torch.randn(n_loc, I, d, generator=g) * 0.02).to(torch.bfloat16)
    wu = (torch.randn(n_loc, I, d, generator=g) * 0.02).to(torch.bfloat16)
    wd = (torch.randn(n_loc, d, I, generator=g) * 0.02).to(torch.bfloat16)
    offsets = torch.zeros(n_loc + 1, dtype=torch.int32)
    offsets[1:] = counts.cumsum(0).to(torch.int32)
    y, work = _run_mlp_mxfp8(cfg, x, wg, wu, wd, offsets, down, keep_workspace=True)
    total = int(offsets[-1])
    assert torch.isfinite(y[:total].float()).all()
    row_expert = torch.repeat_interleave(torch.arange(n_loc, dtype=torch.int32), counts)

    def rows_against(ref_fn, what, bound):
        worst, worst_row, num, den = 0.0, -1, 0.0, 0.0
        for r0 in range(0, total, 1024):
            r1 = min(total, r0 + 1024)
            want = ref_fn(r0, r1)
            diff = y[r0:r1].double() - want
            nr, dr = diff.pow(2).sum(1), want.pow(2).sum(1)
            e = nr.sqrt() / dr.sqrt().clamp_min(1e-300)
            i = int(e.argmax())
            if float(e[i]) > worst:
                worst, worst_row = float(e[i]), r0 + i
            num, den = num + float(nr.sum()), den + float(dr.sum())
            print(f"[{what}] rows {r1}/{total}: worst {worst:.3g} at row {worst_row}",
                  file=sys.stderr, flush=True)
        if bound is not None:
            assert worst <= bound, f"{what}: row {worst_row}: rel-L2 {worst:.3g}"
        return (num / den) ** 0.5

    # end to end against the oracle's block-scaled MLP
    tot = rows_against(lambda a, b: _oracle_rows(torch.arange(a, b), row_expert[a:b], x, wg, wu,
                                                 wd, down),
                       f"fp8 MLP vs oracle, fp8 down: {down}", None if down else ROW_REL_L2)
    assert tot <= 1e-2, f"rel-L2 {tot:.3g}"
    if not down:
        return
    # stage-chained: the kernel's h (codes, scales) times the decoded down weights
    codes_g, scales_g = _h_of_workspace(work, T * K, I, total)
    h_dec = oracle.mxfp8_dequantize(codes_g, scales_g)
    wdq = oracle.mxfp8_quantize(wd.reshape(n_loc * d, I))
    wd_dec = oracle.mxfp8_dequantize(*wdq).view(n_loc, d, I)
    ends = offsets.tolist()

    def chained(a, b):
        out = torch.empty(b - a, d, dtype=torch.float64)
        for e in range(n_loc):
            lo, hi = max(a, ends[e]), min(b, ends[e + 1])
            if hi > lo:
                out[lo - a:hi - a] = h_dec[lo:hi] @ wd_dec[e].T
        return out

    rows_against(chained, "fp8 down, stage-chained on the kernel's h", ROW_REL_L2)
    # the kernel's h codes are valid encodings of the oracle's h: the oracle's
    # fp64 h is its MLP with a down projection that selects the first I columns
    sel = torch.zeros(n_loc, d, I, dtype=torch.bfloat16)
    sel[:, torch.arange(I), torch.arange(I)] = 1
    h_o = torch.empty(total, I, dtype=torch.float64)
    for r0 in range(0, total, 2048):
        r1 = min(total, r0 + 2048)
        h_o[r0:r1] = _oracle_rows(torch.arange(r0, r1), row_expert[r0:r1], x, wg, wu, sel,
                                  False)[:, :I]
    n_codes, n_scales = _check_h_encoding(codes_g, scales_g, h_o)
    print(f"[fp8 down] h encodings differing from the oracle's: {n_codes} codes, "
          f"{n_scales} scales (of {total * I} and {total * I // 32})", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- dispatch and layer

MX_LAYERS = {
    # reduced widths with the real routing structure; hidden a multiple of 512
    "dsv3_mx_small": W.CONFIGS["dsv3_prefill_ep"].replace(num_tokens=300, hidden=512,
                                                          intermediate=256),
    "mixtral_mx_small": W.CONFIGS["mixtral_bf16"].replace(num_tokens=257, hidden=1024,
                                                          intermediate=384),
    "dsv2lite_mx_decode": W.CONFIGS["dsv2lite_decode"].replace(num_shared=0),
}

MX_SHARED_LAYERS = {
    # the block-scaled layer with shared experts: DeepSeek-V2-Lite as it is
    # (two shared experts, I = 1408, so the down projection stays bf16) and a
    # reduced DeepSeek-V3 share with one shared expert
    "dsv2lite_mx_decode_shared": W.CONFIGS["dsv2lite_decode"],
    "dsv3_mx_small_shared": W.CONFIGS["dsv3_prefill_ep"].replace(num_tokens=300, hidden=512,
                                                                 intermediate=256, num_shared=1),
}


def _mfma_positions(R: int, nb: int) -> torch.Tensor:
    """Byte position of (row r, block q) in the MFMA scale layout over R rows."""
    r = torch.arange(R).unsqueeze(1)
    q = torch.arange(nb).unsqueeze(0)
    g, m = q // 16, q % 16
    d, j, s_, h = m >> 3, (m >> 2) & 1, (m >> 1) & 1, m & 1
    return (((2 * g + d) * R + r) * 2 + h) * 4 + 2 * j + s_


def _dispatch_mx(cfg, L):
    T, K, d, E = cfg.num_tokens, cfg.top_k, cfg.hidden, cfg.num_experts
    xq = torch.full((T * K, d), 0xAB, dtype=torch.uint8, device="cuda")
    xs = torch.full((T * K * d // 32,), 0xAB, dtype=torch.uint8, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(cfg.num_local + 1, dtype=torch.int32, device="cuda")
    src = torch.full((T * K,), -7, dtype=torch.int32, device="cuda")
    row_of = torch.empty(T * K, dtype=torch.int32, device="cuda")
    B.moe_dispatch_mxfp8(cfg, L.x, L.topk_ids, counts, offsets, xq, xs, src, row_of,
                         L.ws_dispatch)
    torch.cuda.synchronize()
    return xq.cpu(), xs.cpu(), counts.cpu(), offsets.cpu(), src.cpu(), row_of.cpu()


def _check_dispatch_mx(cfg, inp, L, rows=None):
    T, K, d = cfg.num_tokens, cfg.top_k, cfg.hidden
    L.route()
    torch.cuda.synchronize()
    ids = L.topk_ids.cpu()
    xq, xs, counts, offsets, src, row_of = _dispatch_mx(cfg, L)
    r = oracle.dispatch(ids, cfg.num_experts, cfg.expert_begin, cfg.expert_end)
    n = r["n_rows"]
    assert torch.equal(counts, r["counts"]) and torch.equal(offsets, r["offsets"])
    assert torch.equal(row_of, r["row_of"]) and torch.equal(src[:n], r["src_index"])
    assert bool((src[n:] == -7).all())
    rows = torch.arange(n) if rows is None else rows
    x_rows = inp["x"][src[rows].long() // K].contiguous()  # the oracle's x_sorted rows
    want_c, want_s = oracle.mxfp8_quantize(x_rows)
    assert torch.equal(xq[rows], want_c), "codes differ from the oracle's encoding"
    pos = _mfma_positions(T * K, d // 32)
    assert torch.equal(xs[pos[rows]], want_s), "scales differ from the oracle's encoding"
    if n < T * K:  # rows past the local count untouched
        assert bool((xq[n:] == 0xAB).all()) and bool((xs[pos[n:]] == 0xAB).all())
    return n


@pytest.mark.parametrize("name", list(MX_LAYERS))
def test_dispatch_mxfp8_matches_oracle(name):
    cfg = MX_LAYERS[name]
    inp = W.make_inputs(cfg, 0, with_experts=False)
    _check_dispatch_mx(cfg, inp, MoELayer(cfg, inp))


def test_dispatch_mxfp8_full_size_every_row():
    """The DeepSeek-V3 expert share at full size: every map exact, and the
    codes and scales of every dispatched row equal to the oracle's encoding."""
    cfg = W.CONFIGS["dsv3_prefill_ep"]
    inp = W.make_inputs(cfg, 0, with_experts=False)
    L = MoELayer(cfg, inp)
    n = _check_dispatch_mx(cfg, inp, L)
    print(f"[fp8 dispatch] {n} rows checked", file=sys.stderr, flush=True)


def _check_forward_mx(name, cfg, down: bool):
    """The block-scaled layer against the oracle: routing equal up to the
    router's near-ties, output within the bf16 bar, a second call and a graph
    replay bit-equal to the first call."""
    inp = W.make_inputs(cfg, 0)
    L = MoELayer(cfg, inp)
    L.quantize_weights(down=down)
    L.forward_mxfp8()
    torch.cuda.synchronize()
    out_o, ids_o, _, _ = oracle.forward_mxfp8(cfg, inp, down=down)
    ids_g = L.topk_ids.cpu()
    bad = (ids_g != ids_o).any(1).nonzero().flatten().tolist()
    if bad:  # near-ties of the router: allowed only within the measured logit error
        z_or = oracle.router_logits(inp["x"], inp["w_router"], inp["bias"])
        L.route()
        torch.cuda.synchronize()
        eps = float((L.logits.cpu().double() - z_or).abs().max())
        for t in bad:
            zs = torch.sort(z_or[t], descending=True).values
            assert float(zs[cfg.top_k - 1] - zs[cfg.top_k]) <= 2 * eps, f"token {t}"
    keep = torch.tensor([t for t in range(cfg.num_tokens) if t not in set(bad)])
    err = _rel_l2(L.out.cpu()[keep], out_o[keep])
    print(f"{name} (fp8 down: {down}): rel-L2 {err:.2e}, near-tie tokens {bad}",
          file=sys.stderr)
    assert err <= 1e-2
    first = L.out.clone()
    L.forward_mxfp8()  # the same layer twice gives the same bits
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), L.out.view(torch.int16))
    g = L.capture_forward_mxfp8()  # and a graph of it replays them
    L.out.zero_()
    g.launch()
    torch.cuda.synchronize()
    assert torch.equal(L.out.view(torch.int16), first.view(torch.int16))
    g.destroy()


@pytest.mark.parametrize("name", list(MX_LAYERS))
def test_forward_mxfp8_matches_oracle(name):
    _check_forward_mx(name, MX_LAYERS[name], down=False)


def test_graph_replay_of_the_block_scaled_layer():
    """The captured block-scaled layer replays bit-equal to the eager call, three
    times with eager work between, and follows a change of the token buffer."""
    cfg = MX_LAYERS["dsv3_mx_small"]
    inp = W.make_inputs(cfg, 0)
    L = MoELayer(cfg, inp)
    L.forward_mxfp8()
    torch.cuda.synchronize()
    ref = L.out.clone()
    out = torch.empty_like(L.out)
    g = L.capture_forward_mxfp8(out=out)
    for _ in range(3):
        out.zero_()
        g.launch()
        L.forward_mxfp8(out=torch.empty_like(ref))  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    L.x.copy_(torch.flip(L.x, dims=[0]))
    L.forward_mxfp8()
    torch.cuda.synchronize()
    ref2 = L.out.clone()
    g.launch()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref2.view(torch.int16))
    g.destroy()


MX_DOWN_LAYERS = {
    # the block-scaled layer with the down projection in fp8 too (I % 512 == 0)
    "dsv3_mxd_small": W.CONFIGS["dsv3_prefill_ep"].replace(num_tokens=300, hidden=512,
                                                           intermediate=512),
    "mixtral_mxd_small": W.CONFIGS["mixtral_bf16"].replace(num_tokens=257, hidden=1024,
                                                           intermediate=1536),
}


@pytest.mark.parametrize("name", list(MX_DOWN_LAYERS))
def test_forward_mxfp8_with_fp8_down_matches_oracle(name):
    _check_forward_mx(name, MX_DOWN_LAYERS[name], down=True)


MX_SHARED_DOWN_LAYERS = {
    # shared experts with both projections in fp8 (I % 512 == 0): two shared
    # experts on a DeepSeek-V2-Lite-shaped decode, one on a DeepSeek-V3 share
    "dsv2lite_mxd_decode_shared": W.CONFIGS["dsv2lite_decode"].replace(intermediate=1536),
    "dsv3_mxd_small_shared": W.CONFIGS["dsv3_prefill_ep"].replace(num_tokens=300, hidden=512,
                                                                  intermediate=512, num_shared=1),
}


MX_EDGE = [
    # (name, config, fp8 down)
    ("mx_one_token", W.CONFIGS["dsv3_prefill_ep"].replace(num_tokens=1, hidden=512,
                                                          intermediate=256), False),
    ("mxd_one_token_shared", W.CONFIGS["dsv3_prefill_ep"].replace(
        num_tokens=1, hidden=512, intermediate=512, num_shared=1), True),
    # no token reaches the least popular experts: the output is the shared
    # experts' alone, the routed groups all empty
    ("mx_no_local_rows_shared", W.CONFIGS["dsv3_prefill_ep"].replace(
        num_tokens=64, hidden=512, intermediate=256, expert_begin=248, expert_end=256,
        num_shared=2), False),
    ("mxd_max_shared", W.CONFIGS["dsv2lite_decode"].replace(num_tokens=77, hidden=512,
                                                            intermediate=512, num_shared=4), True),
]


@pytest.mark.parametrize("name,cfg,down", MX_EDGE, ids=[e[0] for e in MX_EDGE])
def test_forward_mxfp8_edge_cases(name, cfg, down):
    _check_forward_mx(name, cfg, down)


@pytest.mark.parametrize("name", list(MX_SHARED_LAYERS))
def test_forward_mxfp8_with_shared_experts_matches_oracle(name):
    _check_forward_mx(name, MX_SHARED_LAYERS[name], down=False)


@pytest.mark.parametrize("name", list(MX_SHARED_DOWN_LAYERS))
def test_forward_mxfp8_with_shared_experts_and_fp8_down_matches_oracle(name):
    _check_forward_mx(name, MX_SHARED_DOWN_LAYERS[name], down=True)
