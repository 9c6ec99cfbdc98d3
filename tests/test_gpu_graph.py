"""The kernels under HIP graph capture and replay.

Calls that keep state between launches in device memory -- the RaBiT split-k
words (reset by the last arriving split), the HGF down-projection words
(reset by the last arriving workgroup) -- must leave it ready for the next
replay, and no library call may record anything that misbehaves on replay.
One graph holds a RaBiT GEMV with split-k, a fused-quantizer W2A8 GEMV, an
activation quantizer + W2A8 GEMV and an HGF activation step + GEMV; it is
replayed several times with other device work and synchronizations in
between, and every replay must reproduce the eager results bit for bit.
"""
import numpy as np
import pytest

import bit_plane_gemv_amd as bq
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_graph_replays_match_eager():
    import torch
    from gpuhelp import say
    dev = torch.device("cuda:0")
    N, K = 1000, 4096
    say("graph replay", N, K)
    rng = np.random.default_rng(77)
    W = synth.gaussian_f32(rng, (N, K), 0.02)
    xs, _ = synth.random_bf16(rng, (1, K))
    x = torch.from_numpy(xs[0].view(np.int16)).to(dev)

    dr = bq.wdesc(bq.RABIT, N, K)
    wr = torch.from_numpy(bq.quantize_weights(dr, W)).to(dev)
    wsr = torch.zeros(bq.workspace_size(dr, 1), dtype=torch.uint8, device=dev)
    assert wsr.numel() > 0                       # several k splits meet in the workspace

    dw = bq.wdesc(bq.W2A8, N, K)
    ww = torch.from_numpy(bq.quantize_weights(dw, W)).to(dev)
    act = torch.zeros(bq.act_size(1, K), dtype=torch.uint8, device=dev)

    dh = bq.wdesc(bq.HGF, N, K, rank=32)
    Ab, Bb, alpha = synth.lora_params(3, N, K, 32)
    wh = torch.from_numpy(bq.quantize_weights_hgf(dh, W, Ab, Bb, alpha)).to(dev)
    ab, wb = bq.hgf_act_size(dh, 1)
    acth = torch.zeros(ab, dtype=torch.uint8, device=dev)
    wsh = torch.zeros(wb, dtype=torch.uint8, device=dev)

    outs = [torch.empty(N, dtype=torch.float32, device=dev) for _ in range(4)]

    def work():
        bq.gemv(dr, wr, x, bq.DT_BF16, outs[0], wsr)
        bq.gemv(dw, ww, x, bq.DT_BF16, outs[1], None, flags=bq.F_FUSE_QUANT)
        bq.quantize_act(x, bq.DT_BF16, 1, K, act)
        bq.gemv(dw, ww, act, bq.DT_ACT, outs[2], None)
        bq.quantize_act_hgf(dh, wh, x, bq.DT_BF16, 1, acth, wsh)
        bq.gemv(dh, wh, acth, bq.DT_ACT, outs[3], None)

    work()
    torch.cuda.synchronize()
    eager = [o.cpu().numpy().view(np.uint32).copy() for o in outs]
    assert np.array_equal(eager[1], eager[2]), "fused and two-launch W2A8 differ"

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    filler = torch.randn(1 << 20, device=dev)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        s = float((filler * (rep + 1)).sum())     # other device work between replays
        assert np.isfinite(s)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            got = o.cpu().numpy().view(np.uint32)
            assert np.array_equal(got, eager[i]), f"replay {rep}: output {i} differs from the eager result"
    # the split-k and HGF words are back at zero after the replays
    assert int(wsr.count_nonzero()) == 0
    assert int(wsh.count_nonzero()) == 0
