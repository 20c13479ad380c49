"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) give,
on every replay, the bits of the same calls issued eagerly.  The split
combines keep their arrival counters in the caller's workspace and return
them to zero themselves, so a replay needs no reset; no call records a
memset.  Replays alternate with eager calls on the same buffers and
workspaces, and every replay is checked."""
import numpy as np
import pytest
import torch

from helpers import dev_bf16
from invariant_reduction_amd import detred, inputs

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int32).clone()


def test_graph_replays_match_eager(dev):
    X1, A1, _ = inputs.lora_inputs(200, 4096, 64, seed=11)
    X2, W2 = inputs.dense_inputs(200, 4096, 1024, seed=12)
    X3, W3 = inputs.dense_inputs(96, 2048, 640, seed=13)
    x4, g4 = inputs.rmsnorm_inputs(33, 4096, seed=14)
    lg = torch.from_numpy(inputs.logits_inputs(8, 151936, seed=15)).to(dev)
    q, k, v = inputs.attention_inputs(2, 8, 2, 700, 128, seed=16)
    d = [dev_bf16(t, dev) for t in (X1, A1, X2, W2, X3, W3, x4, g4, q, k, v)]
    lens = torch.tensor([700, 333], dtype=torch.int32, device=dev)

    y_shr = torch.empty((200, 64), dtype=torch.float32, device=dev)
    y_dns = torch.empty((200, 1024), dtype=torch.float32, device=dev)
    y_tp = torch.empty((96, 640), dtype=torch.float32, device=dev)
    y_rms = torch.empty((33, 4096), dtype=torch.float32, device=dev)
    y_lsm = torch.empty_like(lg)
    y_mean = torch.empty((8,), dtype=torch.float32, device=dev)
    y_att = torch.empty((2, 8, 128), dtype=torch.float32, device=dev)
    outs = (y_shr, y_dns, y_tp, y_rms, y_lsm, y_mean, y_att)

    ws_shr = detred.workspace(200, 64, 4096, 8, dev)
    ws_dns = detred.workspace(200, 1024, 4096, 4, dev)
    ws_tp = detred.workspace(96, 640, 2048, 4, dev)
    ws_att = detred.attention_workspace(2, 8, 128, 700, dev)

    def calls():
        detred.det_splitk_gemm(d[0], d[1], y_shr, 8, ws_shr)
        detred.det_splitk_gemm(d[2], d[3], y_dns, 4, ws_dns)
        detred.tree_tp_gemm(d[4], d[5], y_tp, 4, ws_tp)
        detred.inv_rmsnorm(d[6], d[7], y_rms, 1e-6)
        detred.inv_log_softmax(lg, y_lsm)
        detred.inv_mean(lg, y_mean)
        detred.inv_decode_attention(d[8], d[9], d[10], lens, y_att, 128 ** -0.5, ws_att)

    side = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(side):
        calls()
    torch.cuda.synchronize()
    ref = [_bits(t) for t in outs]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        calls()
    torch.cuda.synchronize()

    for replay in range(4):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("shrink", "dense", "tree_tp", "rmsnorm", "log_softmax", "mean",
                               "attention"), outs, ref):
            assert torch.equal(_bits(t), r), "replay %d: %s differs from the eager bits" % (
                replay, name)
        # eager calls on the same buffers and workspaces between replays
        with torch.cuda.stream(side):
            calls()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            assert torch.equal(_bits(t), r)
