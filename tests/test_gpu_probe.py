"""The achievable-peak probes (include/moe_probe.h) do what they say: the copy
copies, the write writes its pattern, the read's sink is the xor of the data,
and the MFMA loops return finite sums."""
import sys

import pytest
import torch

from combine_router_softmax_top_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [(1 << 20) + 48, 4112])
def test_stream_probes(n):
    # (1 << 20) + 48: whole blocks and a ragged tail; 4112: less than one block
    print(f"[gpu-case] stream probes n={n}", file=sys.stderr, flush=True)
    g = torch.Generator().manual_seed(3)
    a = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).cuda()
    b = torch.zeros_like(a)
    B.probe_stream(B.PROBE_COPY, n, dst=b, src=a, workgroups=64)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    B.probe_stream(B.PROBE_WRITE, n, dst=b, workgroups=64)
    torch.cuda.synchronize()
    w = b.view(torch.int32).view(-1, 4).cpu()
    assert bool((w[:, 1:] == torch.tensor([1, 2, 3], dtype=torch.int32)).all())
    sink = torch.zeros(64 * 256, dtype=torch.int32, device="cuda")
    B.probe_stream(B.PROBE_READ, n, src=a, sink=sink, workgroups=64)
    torch.cuda.synchronize()
    words = a.view(torch.int32).cpu()
    ref = 0
    for v in words.tolist():
        ref ^= v
    got = 0
    for v in sink.cpu().tolist():
        got ^= v
    assert got == ref


@pytest.mark.parametrize("kind", [B.PROBE_MFMA_BF16, B.PROBE_MFMA_FP8])
def test_mfma_probes(kind):
    print(f"[gpu-case] mfma probe {kind}", file=sys.stderr, flush=True)
    out = torch.full((4 * 512,), float("nan"), device="cuda")
    B.probe_mfma(kind, 4, 16, out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool((out > 0).any())
