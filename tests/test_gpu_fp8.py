"""GPU parity of the block-scaled 8-bit path against the CPU oracle.

MX-FP8 quantization (moe_quantize_mxfp8): codes and scale bytes bit-exact
against the oracle on seeded rows, on hand-built edge blocks (all-zero and
negative-zero blocks, subnormal inputs, ties at every level of E4M3, values that
scale past 448 and into the non-saturating range of the hardware conversion,
values near the top of the input type) and on ragged, strided and full-width
shapes.
"""
import sys

import pytest
import torch

import oracle
from combine_router_softmax_top_amd import binding as B

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


def _gpu_quantize(x: torch.Tensor):
    rows, cols = x.shape
    codes = torch.full((rows, cols), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows, cols // 32), 0xAB, dtype=torch.uint8, device="cuda")
    B.moe_quantize_mxfp8(x, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu(), scales.cpu()


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


def test_mxfp8_quantize_zero_rows_is_a_no_op():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    codes = torch.empty(0, 64, dtype=torch.uint8, device="cuda")
    scales = torch.empty(0, 2, dtype=torch.uint8, device="cuda")
    B.moe_quantize_mxfp8(x, codes, scales)
    torch.cuda.synchronize()
