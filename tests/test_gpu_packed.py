"""The packed weight layout (moe_pack_weights, MOE_WEIGHTS_PACKED): the packing
is the documented permutation, bit for bit, and a layer given packed weights
computes the same products in the same order as with row-major weights, so
its output is bit-identical; it is also checked against the oracle."""
import sys

import pytest
import torch

import oracle
from combine_router_softmax_top_amd import binding as B
from combine_router_softmax_top_amd import workloads as W
from combine_router_softmax_top_amd.layer import MoELayer

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_pack_weights_is_the_documented_permutation():
    g = torch.Generator().manual_seed(3)
    for n, rows, cols in ((3, 256, 192), (1, 128, 64), (2, 384, 1024)):
        w = torch.randn(n, rows, cols, generator=g).to(torch.bfloat16)
        p = torch.full_like(w, 7.0).cuda()
        B.moe_pack_weights(w.cuda(), p)
        torch.cuda.synchronize()
        want = w.view(n, rows // 128, 128, cols // 64, 64).permute(0, 1, 3, 2, 4).contiguous()
        assert torch.equal(bits(p.cpu()).flatten(), bits(want).flatten()), (n, rows, cols)


PACKED = {
    # hidden and intermediate multiples of 128
    "mixtral_small": W.CONFIGS["mixtral_bf16"].replace(num_tokens=300, hidden=512,
                                                        intermediate=384),
    "dsv3_small": W.CONFIGS["dsv3_prefill_ep"].replace(num_tokens=300, hidden=512,
                                                       intermediate=256),
    # two shared experts; 12 rows per expert, so 64-row tiles (the deep ring)
    "dsv2lite_small_shared": W.CONFIGS["dsv2lite_decode"].replace(hidden=512, intermediate=384),
    "dsv3_dbo_small": W.CONFIGS["dsv3_dual_microbatch"].replace(num_tokens=600, hidden=512,
                                                               intermediate=256),
    # down-projection column tiles past the last 128-row block of a 256-row tile
    "odd_row_blocks": W.CONFIGS["dsv3_prefill_ep"].replace(num_tokens=77, hidden=384,
                                                           intermediate=640, num_shared=1),
}


@pytest.mark.parametrize("name", list(PACKED))
def test_packed_layer_equals_row_major_and_oracle(name):
    cfg = PACKED[name]
    inp = W.make_inputs(cfg, 0)
    R = MoELayer(cfg, inp)
    R.forward()
    P = MoELayer(cfg.replace(packed_weights=True), inp)
    P.forward()
    torch.cuda.synchronize()
    assert torch.equal(R.topk_ids, P.topk_ids)
    assert torch.equal(bits(R.out), bits(P.out)), "packed layer differs from the row-major one"
    if cfg.dual_microbatch:
        o = torch.empty_like(P.out)
        P.forward_dbo(comm=torch.cuda.Stream(), out=o)
        torch.cuda.synchronize()
        assert torch.equal(bits(o), bits(R.out))
    g = P.capture_forward()  # a graph of the packed layer replays the same bits
    P.out.zero_()
    g.launch()
    torch.cuda.synchronize()
    assert torch.equal(bits(P.out), bits(R.out))
    g.destroy()
    out_o, ids_o, _, _ = oracle.forward(cfg, inp)
    same = (P.topk_ids.cpu() == ids_o).all(1)
    assert int(same.sum()) >= cfg.num_tokens - 1, "more than one near-tie swap"
    got = P.out.cpu().double()[same]
    err = float((got - out_o[same]).norm() / out_o[same].norm())
    print(f"{name}: packed rel-L2 vs oracle {err:.2e}", file=sys.stderr)
    assert err <= 1e-2


@pytest.mark.parametrize("name", ["dsv2lite_decode", "dsv3_prefill_ep"])
def test_packed_full_size_equals_row_major(name):
    cfg = W.CONFIGS[name]
    inp = W.make_inputs(cfg, 0)
    # The row-major layer is checked row by row against the oracle at these
    # sizes (test_gpu_parity.test_full_size); here every row of the packed
    # layer's expert output and every token of its output must equal it bit for
    # bit.
    R = MoELayer(cfg, inp)
    R.route()
    R.dispatch()
    R.expert_mlp()
    R.combine()
    torch.cuda.synchronize()
    n = R.n_rows()
    ref, ref_y = R.out.cpu(), R.y_sorted[:n].cpu()
    del R
    torch.cuda.empty_cache()
    P = MoELayer(cfg.replace(packed_weights=True), inp)
    P.route()
    P.dispatch()
    P.expert_mlp()
    P.combine()
    torch.cuda.synchronize()
    assert P.n_rows() == n
    assert torch.equal(bits(P.y_sorted[:n].cpu()), bits(ref_y))
    assert torch.equal(bits(P.out.cpu()), bits(ref))
    o = torch.empty_like(P.out)
    P.forward(out=o)
    torch.cuda.synchronize()
    assert torch.equal(bits(o.cpu()), bits(ref))
