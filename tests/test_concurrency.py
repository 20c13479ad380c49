"""Deterministic calls running at the same time on several streams give the
bits they give alone: the last-arriver combine (device-coherent partial
stores, arrival counters in each call's own workspace) and the row kernels
keep no state outside their arguments."""
import numpy as np
import pytest
import torch

from helpers import dev_bf16
from invariant_reduction_amd import detred, inputs

pytestmark = pytest.mark.gpu


def test_concurrent_streams_match_serial(dev):
    X1, A1, _ = inputs.lora_inputs(256, 4096, 64, seed=1)
    X2, W2 = inputs.dense_inputs(256, 4096, 4096, seed=2)
    X3, W3 = inputs.dense_inputs(512, 2048, 2048, seed=3)
    lg = torch.from_numpy(inputs.logits_inputs(64, 20000, seed=4)).to(dev)
    d = [dev_bf16(t, dev) for t in (X1, A1, X2, W2, X3, W3)]
    ys = [torch.empty((256, 64), dtype=torch.float32, device=dev),
          torch.empty((256, 4096), dtype=torch.float32, device=dev),
          torch.empty((512, 2048), dtype=torch.float32, device=dev),
          torch.empty((64, 20000), dtype=torch.float32, device=dev)]
    streams = [torch.cuda.Stream(device=dev) for _ in range(3)]
    ws = [detred.workspace(256, 64, 4096, 8, dev), detred.workspace(256, 4096, 4096, 4, dev),
          detred.workspace(512, 2048, 2048, 8, dev)]

    def calls(sts):
        return [
            detred.prepare(detred.det_splitk_gemm, d[0], d[1], ys[0], 8, ws[0], stream=sts[0]),
            detred.prepare(detred.det_splitk_gemm, d[2], d[3], ys[1], 4, ws[1], stream=sts[1]),
            detred.prepare(detred.tree_tp_gemm, d[4], d[5], ys[2], 8, ws[2], stream=sts[2]),
            detred.prepare(detred.inv_log_softmax, lg, ys[3], stream=sts[0]),
        ]

    main = torch.cuda.current_stream()
    for fn in calls([main] * 3):
        fn()
    torch.cuda.synchronize()
    ref = [y.clone() for y in ys]
    conc = calls(streams)
    for _ in range(10):
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        for _ in range(3):                 # back-to-back calls on every stream
            for fn in conc:
                fn()
        torch.cuda.synchronize()
        for y, r in zip(ys, ref):
            assert torch.equal(y.view(torch.int32), r.view(torch.int32))
