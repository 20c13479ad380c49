"""100 identical-input replays over the whole configuration set.

Every deterministic call is launched 100 times on the same inputs and its
output compared bit for bit with the first replay: it must give one output.
The atomic control of the same product is replayed beside it and its
divergence printed with the three measures of the reading of the 97.61 %
figure ("Reproducible LoRA Inference Through Deterministic Split-K
Reduction", Highlights and Q&A): the share of replays 1..99 that differ
anywhere from replay 0, the number of distinct outputs among the 100, and
the mean share of elements that differ from replay 0.

Outputs stay on the GPU: each replay is compared with replay 0 there, and
distinct outputs are counted by a 64-bit fingerprint of the bit patterns
(a fixed random weighting, wrapping), so that full-size outputs need no
host copies."""
import pytest
import torch

from helpers import dev_bf16
from invariant_reduction_amd import detred, inputs

pytestmark = pytest.mark.gpu

REPLAYS = 100
H, F, V = 4096, 14336, 151936


def _weights(n, dev):
    g = torch.Generator(device=dev)
    g.manual_seed(12345)
    return torch.randint(1, 2 ** 62, (n,), generator=g, dtype=torch.int64, device=dev)


def replay_stats(launch, out):
    """Launch 100 times; compare every replay's bits with replay 0.
    Returns (replays differing, distinct outputs, mean share of elements
    differing) over replays 1..99."""
    flat = out.view(-1)
    bits = flat.view(torch.int32) if flat.dtype == torch.float32 else flat.view(torch.int16)
    w = _weights(bits.numel(), out.device)
    launch()
    ref = bits.clone()
    prints = [int((ref.to(torch.int64) * w).sum())]
    differing = []
    for _ in range(REPLAYS - 1):
        launch()
        differing.append(int((bits != ref).sum()))
        prints.append(int((bits.to(torch.int64) * w).sum()))
    torch.cuda.synchronize()
    n_diff = sum(d > 0 for d in differing)
    distinct = len(set(prints))
    mean_frac = sum(differing) / len(differing) / bits.numel()
    return n_diff, distinct, mean_frac


def report(name, det_stats, atom_stats=None):
    d = det_stats
    line = "replays %-34s det: %d/99 differ, %d distinct" % (name, d[0], d[1])
    if atom_stats is not None:
        a = atom_stats
        line += " | atomic: %d/99 differ, %d distinct, %.2f%% of elements" % (
            a[0], a[1], 100.0 * a[2])
    print(line, flush=True)


def assert_one_output(name, stats):
    assert stats[0] == 0 and stats[1] == 1, "%s: %d of 99 replays differ (%d distinct)" % (
        name, stats[0], stats[1])


@pytest.mark.parametrize("r", [16, 64])
@pytest.mark.parametrize("M", [1, 8, 64, 256])
def test_lora_shrink_expand_replays(M, r, dev):
    """LoRA shrink X[M,4096] A[4096,r] at split 1, 4 and 8, its bf16 cast
    and the expand [M,r] B[r,4096]: one output each over 100 replays, the
    same bits for every split; the atomic shrink at the same split is
    replayed beside it."""
    X, A, Bm = inputs.lora_inputs(M, H, r, seed=0)
    Xd, Ad, Bd = dev_bf16(X, dev), dev_bf16(A, dev), dev_bf16(Bm, dev)
    ys = torch.empty((M, r), dtype=torch.float32, device=dev)
    ya = torch.empty((M, r), dtype=torch.float32, device=dev)
    yb = torch.empty((M, r), dtype=torch.int16, device=dev)
    z = torch.empty((M, H), dtype=torch.float32, device=dev)
    first = None
    for S in (1, 4, 8):
        print("case M=%d r=%d S=%d" % (M, r, S), flush=True)
        ws = detred.workspace(M, r, H, S, dev)
        shrink = detred.prepare(detred.det_splitk_gemm, Xd, Ad, ys, S, ws)
        cast = detred.prepare(detred.detred_f32_to_bf16, ys, yb)
        expand = detred.prepare(detred.det_splitk_gemm, yb, Bd, z, 0)
        det = replay_stats(shrink, ys)
        atom = replay_stats(detred.prepare(detred.atomic_splitk_gemm, Xd, Ad, ya, S), ya)
        report("shrink %dx%dx%d S=%d" % (M, r, H, S), det, atom)
        assert_one_output("shrink S=%d" % S, det)

        def chain():
            shrink()
            cast()
            expand()
        chain_stats = replay_stats(chain, z)
        report("shrink+cast+expand %dx%dx%d S=%d" % (M, H, r, S), chain_stats)
        assert_one_output("shrink+cast+expand S=%d" % S, chain_stats)
        if first is None:
            first = (ys.clone(), z.clone())
        else:
            assert torch.equal(ys.view(torch.int32), first[0].view(torch.int32)), \
                "shrink bits differ between splits"
            assert torch.equal(z.view(torch.int32), first[1].view(torch.int32)), \
                "expand bits differ between splits"


@pytest.mark.parametrize("M", [1, 1024, 4096])
def test_dense_replays(M, dev):
    """Dense X[M,4096] W[4096,14336] at the automatic split: one output over
    100 replays; the atomic control at 4 slices replayed beside it."""
    print("case dense M=%d" % M, flush=True)
    X, W = inputs.dense_inputs(M, H, F, seed=0)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    y = torch.empty((M, F), dtype=torch.float32, device=dev)
    ws = detred.workspace(M, F, H, 0, dev)
    det = replay_stats(detred.prepare(detred.det_splitk_gemm, Xd, Wd, y, 0, ws), y)
    ya = torch.empty_like(y)
    atom = replay_stats(detred.prepare(detred.atomic_splitk_gemm, Xd, Wd, ya, 4), ya)
    report("dense %dx%dx%d auto split" % (M, F, H), det, atom)
    assert_one_output("dense M=%d" % M, det)


@pytest.mark.parametrize("T", [1, 8])
def test_tree_tp_replays(T, dev):
    """Tree-TP X[512,8192] W[8192,8192] with T virtual shards: one output
    over 100 replays, equal for T = 1 and 8."""
    print("case tree_tp T=%d" % T, flush=True)
    X, W = inputs.dense_inputs(512, 8192, 8192, seed=0)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    y = torch.empty((512, 8192), dtype=torch.float32, device=dev)
    ws = detred.workspace(512, 8192, 8192, T, dev)
    det = replay_stats(detred.prepare(detred.tree_tp_gemm, Xd, Wd, y, T, ws), y)
    atom = None
    if T == 8:
        ya = torch.empty_like(y)
        atom = replay_stats(detred.prepare(detred.atomic_splitk_gemm, Xd, Wd, ya, 8), ya)
    report("tree_tp 512x8192x8192 T=%d" % T, det, atom)
    assert_one_output("tree_tp T=%d" % T, det)
    y1 = torch.empty_like(y)
    detred.tree_tp_gemm(Xd, Wd, y1, 1)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y1.view(torch.int32))


def test_row_op_replays(dev):
    """RMSNorm over [4096, 4096] and log_softmax + mean over [4096, 151936]:
    one output each over 100 replays."""
    x, g = inputs.rmsnorm_inputs(4096, H, seed=0)
    y = torch.empty((4096, H), dtype=torch.float32, device=dev)
    st = replay_stats(detred.prepare(detred.inv_rmsnorm, dev_bf16(x, dev), dev_bf16(g, dev), y,
                                     1e-6), y)
    report("rmsnorm 4096x4096", st)
    assert_one_output("rmsnorm", st)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    lg = torch.randn((4096, V), device=dev, generator=gen) * 3.0
    ls = torch.empty_like(lg)
    mu = torch.empty((4096,), dtype=torch.float32, device=dev)
    fused = detred.prepare(detred.inv_log_softmax_mean, lg, ls, mu)
    st = replay_stats(fused, ls)
    report("log_softmax (fused) 4096x151936", st)
    assert_one_output("log_softmax", st)
    st = replay_stats(fused, mu)
    report("mean (fused) 4096x151936", st)
    assert_one_output("mean", st)
    del ls, lg
