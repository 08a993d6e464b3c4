"""The library's calls under HIP graph capture and on concurrent streams: a
captured layer (route prep without a workspace included) replays to the
eager result, bit for bit, on every replay.  The library allocates nothing,
copies nothing and records no memset, and the NVFP4 work queue zeroes itself
at the end of each launch, so a replay needs no reset; two launches running
at once on two streams with separate queues each give the lone result."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

mq = pytest.importorskip("quantized_moe_grouped_route_amd")


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mq.lib()


def _capture_and_replay(step, outputs, replays=3):
    """Run `step` eagerly, capture it, then replay it `replays` times with
    the outputs scrambled and other eager work in between; every replay must
    reproduce the eager outputs exactly."""
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the side stream, as torch's capture expects
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(replays):
        for o in outputs:
            o.fill_(7)
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outputs, ref):
            assert torch.equal(o, r), f"replay {i} differs"
        del junk


def test_int4_decode_layer_replays():
    # route -> int4 of x -> FC1 (SiLU, streaming) -> int4 of h -> FC2 -> combine
    T, E, k, H, I = 8, 8, 2, 1024, 2048
    d = synth.int4_chain(61, T, E, k, H, I)
    ids, tw = dev(d["topk_ids"]), dev(d["topk_weights"])
    x, w, sw, w2, sw2 = dev(d["x"]), dev(d["w"]), dev(d["w_scale"]), dev(d["w2"]), dev(d["w2_scale"])
    P = T * k
    i32 = dict(dtype=torch.int32, device="cuda")
    route = (torch.empty(E + 1, **i32), torch.empty(P, **i32), torch.empty(P, **i32), torch.empty(1, **i32))
    qx = torch.empty(T, H // 2, dtype=torch.uint8, device="cuda")
    sx = torch.empty(T, dtype=torch.float32, device="cuda")
    h = torch.empty(P, I, dtype=torch.float16, device="cuda")
    qh = torch.empty(P, I // 2, dtype=torch.uint8, device="cuda")
    sh = torch.empty(P, dtype=torch.float32, device="cuda")
    y = torch.empty(P, H, dtype=torch.float16, device="cuda")
    out = torch.empty(T, H, dtype=torch.float16, device="cuda")

    def step():
        offs, srt, p2s, _ = mq.moe_route_prep_noalloc(ids, E, out=route)  # no caller workspace
        mq.quantize_int4_rows(x, q=qx, scale=sx)
        mq.grouped_gemm_qint4(qx, sx, w, sw, offs, srt, k, act="silu_mul", out=h)
        mq.quantize_int4_rows(h, q=qh, scale=sh)
        mq.grouped_gemm_qint4(qh, sh, w2, sw2, offs, srt, k, a_row="sorted", out=y)
        mq.moe_scatter_combine(y, p2s, tw, out=out)

    _capture_and_replay(step, [h, qh, sh, y, out])


@pytest.mark.parametrize("pair", [False, True])
def test_nvfp4_prefill_layer_with_work_queue_replays(pair):
    # Zipf routing over more tiles than workgroups, both GEMMs on the tiled
    # schedule with one work queue; the multi-chunk route prep uses its
    # caller workspace
    T, E, k, H, I = 600, 40, 4, 1024, 512
    d = synth.nvfp4_moe(62, T, E, k, H, I, routing="zipf")
    ids = dev(d["topk_ids"])
    tw = dev(d["topk_weights"])
    tw_flat = tw.reshape(-1)
    x, w1, s1, g1 = dev(d["x"]), dev(d["w1"]), dev(d["s1"]), dev(d["g1"])
    w2, s2, g2 = dev(d["w2"]), dev(d["s2"]), dev(d["g2"])
    P = T * k
    i32 = dict(dtype=torch.int32, device="cuda")
    route = (torch.empty(E + 1, **i32), torch.empty(P, **i32), torch.empty(P, **i32), torch.empty(1, **i32))
    ws = torch.empty(max(mq.route_workspace_bytes(T, k, E), 1), dtype=torch.uint8, device="cuda")
    wq = mq.work_queue()
    h = torch.empty(P, I, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(P, H, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")

    def step():
        offs, srt, p2s, _ = mq.moe_route_prep(ids, E, out=route, workspace=ws)
        mq.grouped_gemm_qnvfp4(x, w1, s1, g1, offs, srt, k, act="silu_mul", out=h, sched="prefill",
                               work_queue=wq)
        if pair:
            mq.grouped_gemm_qnvfp4(h, w2, s2, g2, offs, srt, k, a_row="sorted", pair_weights=tw_flat, out=y,
                                   sched="prefill", work_queue=wq)
            mq.moe_sum_pairs(y, p2s, T, k, out=out)
        else:
            mq.grouped_gemm_qnvfp4(h, w2, s2, g2, offs, srt, k, a_row="sorted", out=y, sched="prefill",
                                   work_queue=wq)
            mq.moe_scatter_combine(y, p2s, tw, out=out)

    outputs = [h, out] if pair else [h, y, out]
    _capture_and_replay(step, outputs)
    assert torch.all(wq == 0)


def test_nvfp4_prefill_on_two_streams_with_separate_queues():
    # two tiled-schedule GEMMs running at the same time on two streams, each
    # with its own work queue, give the outputs each gives alone
    T, E, k, H, I = 600, 40, 4, 1024, 512
    d = synth.nvfp4_moe(63, T, E, k, H, I, routing="zipf")
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    x, w1, s1, g1 = dev(d["x"]), dev(d["w1"]), dev(d["s1"]), dev(d["g1"])
    ref = mq.grouped_gemm_qnvfp4(x, w1, s1, g1, offs, srt, k, act="silu_mul", sched="prefill")
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    queues = [mq.work_queue(), mq.work_queue()]
    outs = [torch.empty_like(ref), torch.empty_like(ref)]
    for rep in range(3):
        for o in outs:
            o.fill_(5)
        torch.cuda.synchronize()
        for s, q, o in zip(streams, queues, outs):
            with torch.cuda.stream(s):
                mq.grouped_gemm_qnvfp4(x, w1, s1, g1, offs, srt, k, act="silu_mul", sched="prefill", out=o,
                                       work_queue=q)
        torch.cuda.synchronize()
        n = int(offs[-1].item())
        for o in outs:
            assert torch.equal(o[:n], ref[:n]), f"repeat {rep}"
        assert all(torch.all(q == 0) for q in queues)
