"""The C-ABI library: it loads, exports every entry point include/detred.h
declares, and rejects bad arguments before any GPU work.  CPU only: no
call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

from invariant_reduction_amd import detred

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "detred.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "defined")))


def test_header_declares_the_entry_points():
    names = header_functions()
    for must in ["det_splitk_gemm", "atomic_splitk_gemm", "tree_tp_gemm", "inv_rmsnorm",
                 "inv_log_softmax", "inv_mean"]:
        assert must in names


def test_library_exports_every_declared_symbol():
    L = detred.lib()
    missing = [n for n in header_functions() if not hasattr(L, n)]
    assert not missing, missing
    assert set(header_functions()) == set(detred.SIGNATURES), \
        "binding signatures out of sync with the header"


def test_status_strings_and_version():
    assert detred.status_string(0) == "DETRED_OK"
    for s in range(1, 5):
        assert detred.status_string(s).startswith("DETRED_E")
    assert detred.lib().detred_version() >= 100


def test_policy_is_locked_by_n_and_k():
    p = detred.policy(16, 512)
    assert p["chunks"] == 8 and p["chunk_k"] == 64 and p["default_split"] == 8
    p = detred.policy(14336, 4096)
    assert p["chunks"] == 8 and p["chunk_k"] == 512 and p["default_split"] == 1
    assert (p["tile_m"], p["tile_n"]) == (128, 128)
    p = detred.policy(4096, 64)  # LoRA expand: K = r < 256 -> one chunk
    assert p["chunks"] == 1 and p["chunk_k"] == 64 and p["default_split"] == 1
    p = detred.policy(64, 264)   # K not a multiple of 256 -> one chunk
    assert p["chunks"] == 1
    assert detred.lib().detred_policy(-1, 4, None, None, None, None, None) == detred.EINVAL


def test_auto_split():
    # wide outputs: the most slices that keep the grid at <= 256 workgroups
    # below 129 tiles, unsplit above 192 tiles, 4 slices between with long
    # chunks and for 257..447 tiles with long chunks (unless one round of
    # 192x128 tiles holds the product)
    assert detred.auto_split(256, 14336, 4096) == 1      # 224 tiles
    assert detred.auto_split(1, 14336, 4096) == 4        # 112 tiles, at most 16 rows
    assert detred.auto_split(32, 14336, 4096) == 2       # 112 tiles
    assert detred.auto_split(128, 14336, 4096) == 2      # 112 tiles
    assert detred.auto_split(256, 4096, 4096) == 4       # 64 tiles
    assert detred.auto_split(512, 4096, 4096) == 2       # 128 tiles
    assert detred.auto_split(768, 1024, 4096) == 4       # 48 tiles
    assert detred.auto_split(1, 1024, 4096) == 8         # 8 tiles, capped at P
    assert detred.auto_split(640, 4096, 4096) == 1       # 160 tiles, chunks of 512
    assert detred.auto_split(640, 4096, 8192) == 4       # 160 tiles, chunks of 1024
    assert detred.auto_split(320, 8192, 8192) == 4       # 192 tiles, chunks of 1024
    assert detred.auto_split(768, 4096, 4096) == 1       # 192 tiles, chunks of 512
    assert detred.auto_split(384, 14336, 8192) == 1      # 336 tiles, one round of 192x128
    assert detred.auto_split(384, 14336, 4096) == 1      # 336 tiles, one round of 192x128
    assert detred.auto_split(1280, 4096, 4096) == 1      # 320 tiles, one round of 192x128
    assert detred.auto_split(1664, 4096, 4096) == 2      # 416 tiles, 288 of 192x128
    assert detred.auto_split(384, 14336, 14336) == 1     # 336 tiles, one round of 192x128
    assert detred.auto_split(256, 14336, 14336) == 8     # 224 tiles, chunks of 1792
    assert detred.auto_split(384, 8192, 14336) == 8      # chunks of 1792, 256+ rows
    assert detred.auto_split(128, 14336, 14336) == 2     # chunks of 1792, 128 rows
    assert detred.auto_split(512, 14336, 8192) == 1      # 448 tiles
    assert detred.auto_split(1024, 4096, 4096) == 1      # 256 tiles
    assert detred.auto_split(1, 4096, 64) == 1           # one chunk
    assert detred.auto_split(4096, 64, 4096) == 8        # narrow: one slice per chunk
    assert detred.auto_split(-1, 64, 4096) == 0
    assert detred.detred_gemm_workspace_bytes(256, 4096, 4096, 0) == \
        detred.detred_gemm_workspace_bytes(256, 4096, 4096, 4)
    assert detred.detred_gemm_workspace_bytes(256, 14336, 4096, 0) == 0
    # split 0 also covers an addmm that cannot take the 192x128 tile (bf16
    # output), which keeps the 2 slices of 336 tiles with chunks of 512
    assert detred.detred_gemm_workspace_bytes(384, 14336, 4096, 0) == \
        detred.detred_gemm_workspace_bytes(384, 14336, 4096, 2) > 0


def test_workspace_bytes():
    assert detred.detred_gemm_workspace_bytes(16, 16, 512, 1) == 0
    n = detred.detred_gemm_workspace_bytes(16, 16, 512, 8)
    assert n >= 8 * 16 * 16 * 4 + 4 and n % 256 == 0
    assert detred.detred_gemm_workspace_bytes(16, 16, 512, 3) == 0
    # a split the products reject needs no workspace either (one chunk: P = 1)
    assert detred.detred_gemm_workspace_bytes(16, 16, 264, 2) == 0
    assert detred.detred_gemm_workspace_bytes(16, 4096, 64, 8) == 0


A16 = 0x10000          # fake, 16-byte aligned addresses: never dereferenced
A16b = 0x20000
A16c = 0x30000
MIS = 0x10002          # misaligned


def call_det(X=A16, ldx=512, W=A16b, ldw=16, Y=A16c, ldy=16, M=16, N=16, K=512, S=8,
             ws=None, nws=0):
    return detred.lib().det_splitk_gemm(X, ldx, W, ldw, Y, ldy, M, N, K, S, ws, nws, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), detred.EINVAL),
    (dict(K=-8), detred.EINVAL),
    (dict(ldx=100), detred.EINVAL),              # ldx < K
    (dict(ldw=8), detred.EINVAL),                # ldw < N
    (dict(ldy=8), detred.EINVAL),                # ldy < N
    (dict(X=None), detred.EINVAL),
    (dict(W=None), detred.EINVAL),
    (dict(Y=None), detred.EINVAL),
    (dict(X=MIS), detred.EINVAL),
    (dict(Y=MIS), detred.EINVAL),
    (dict(ldx=516), detred.EINVAL),              # row stride not 16-byte aligned
    (dict(K=500, ldx=504), detred.EUNSUPPORTED),  # K % 8 != 0
    (dict(N=12, ldw=16, ldy=16), detred.EUNSUPPORTED),  # N % 8 != 0
    (dict(S=3), detred.EUNSUPPORTED),
    (dict(S=16), detred.EUNSUPPORTED),
    (dict(K=264, ldx=264, S=2), detred.EUNSUPPORTED),  # one chunk only
    (dict(S=8, ws=None), detred.EWORKSPACE),
    (dict(S=8, ws=0x100000, nws=64), detred.EWORKSPACE),
    (dict(S=8, ws=0x100010, nws=1 << 20), detred.EWORKSPACE),  # not 256-aligned
])
def test_det_splitk_rejects(kw, status):
    assert call_det(**kw) == status


def test_noalloc_entry_point_rejects_before_any_gpu_work():
    L = detred.lib()

    def na(**kw):
        a = dict(X=A16, ldx=512, W=A16b, ldw=16, Y=A16c, ldy=16, M=16, N=16, K=512, S=8)
        a.update(kw)
        return L.det_splitk_gemm_noalloc(a["X"], a["ldx"], a["W"], a["ldw"], a["Y"], a["ldy"],
                                         a["M"], a["N"], a["K"], a["S"], None)
    assert na(M=-1) == detred.EINVAL
    assert na(X=MIS) == detred.EINVAL
    assert na(ldy=8) == detred.EINVAL
    assert na(S=3) == detred.EUNSUPPORTED
    assert na(K=264, ldx=264, S=2) == detred.EUNSUPPORTED
    assert na(M=0, X=None, W=None, Y=None) == detred.OK
    # partials beyond the scratch: 8 x 4096 x 4096 fp32 = 512 MiB, and the
    # first size past the limit (8 planes of 1024 x 1024 = 32 MiB)
    big = dict(ldx=4096, ldw=4096, ldy=4096, M=4096, N=4096, K=4096, S=8)
    assert na(**big) == detred.EWORKSPACE
    assert na(**dict(big, M=1024, N=1024, ldw=1024, ldy=1024)) == detred.EWORKSPACE
    assert 8 * 1024 * 1016 * 4 <= 33488896 < 8 * 1024 * 1024 * 4


def test_transposed_weight_entry_points_reject():
    L = detred.lib()
    f = ctypes.c_float
    # det_splitk_gemm_wt(X, ldx, Wt, ldwt, Y, ldy, M, N, K, S, ws, ws_bytes, s): Wt is [N, K]
    g = lambda **kw: [kw.get("X", A16), 512, kw.get("W", A16b), kw.get("ldw", 512), A16c,
                      kw.get("ldy", 16), 16, kw.get("N", 16), 512, kw.get("S", 1), None, 0, None]
    assert L.det_splitk_gemm_wt(*g(ldw=16)) == detred.EINVAL       # ldwt < K (ldw >= N is not enough)
    assert L.det_splitk_gemm_wt(*g(ldw=500)) == detred.EINVAL      # ldwt < K
    assert L.det_splitk_gemm_wt(*g(ldw=516)) == detred.EINVAL      # ldwt % 8 != 0
    assert L.det_splitk_gemm_wt(*g(W=MIS)) == detred.EINVAL
    assert L.det_splitk_gemm_wt(*g(W=None)) == detred.EINVAL
    assert L.det_splitk_gemm_wt(*g(S=3)) == detred.EUNSUPPORTED
    assert L.det_splitk_gemm_wt(*g(S=8)) == detred.EWORKSPACE
    assert L.det_splitk_gemm_wt(*g(N=12, ldy=16)) == detred.EUNSUPPORTED
    a = g(X=None, W=None)
    a[6] = 0                                                      # M == 0
    assert L.det_splitk_gemm_wt(*a) == detred.OK
    # tree_tp_gemm_wt(X, ldx, Wt, ldwt, Y, ldy, M, N, K, T, ws, ws_bytes, s)
    assert L.tree_tp_gemm_wt(*g(ldw=16)) == detred.EINVAL          # ldwt < K
    assert L.tree_tp_gemm_wt(*g(ldw=516)) == detred.EINVAL         # ldwt % 8 != 0
    assert L.tree_tp_gemm_wt(*g(S=3)) == detred.EUNSUPPORTED
    assert L.tree_tp_gemm_wt(*g(S=8)) == detred.EWORKSPACE
    # tree_tp_shards_gemm_wt(X, ldx, Wt, ldwt, P, M, N, K, T, s)
    assert L.tree_tp_shards_gemm_wt(A16, 512, A16b, 16, A16c, 16, 16, 512, 8, None) == detred.EINVAL
    assert L.tree_tp_shards_gemm_wt(A16, 512, A16b, 512, A16c, 16, 16, 512, 3, None) == \
        detred.EUNSUPPORTED
    # tree_tp_shard_gemm_wt(Xt, ldx, Wt, ldwt, Pt, ldp, M, N, Kt, T, s): ldwt >= Kt
    assert L.tree_tp_shard_gemm_wt(A16, 64, A16b, 32, A16c, 16, 16, 16, 64, 8, None) == detred.EINVAL
    assert L.tree_tp_shard_gemm_wt(A16, 64, A16b, 64, A16c, 16, 16, 16, 64, 3, None) == \
        detred.EINVAL
    # det_splitk_addmm_wt(X, ldx, Wt, ldwt, C, ldc, alpha, beta, Y, ldy, y_dtype, M, N, K, S, ws, ws_bytes, s)
    am = lambda **kw: [A16, 512, A16b, kw.get("ldw", 512), A16c, kw.get("ldc", 16), f(1.0), f(1.0),
                       A16, 16, kw.get("dt", detred.F32), 16, 16, 512, 1, None, 0, None]
    assert L.det_splitk_addmm_wt(*am(ldw=16)) == detred.EINVAL
    assert L.det_splitk_addmm_wt(*am(dt=2)) == detred.EINVAL
    assert L.det_splitk_addmm_wt(*am(ldc=8)) == detred.EINVAL


def test_empty_problem_launches_nothing():
    # M == 0 or N == 0: OK without touching the (null) pointers
    assert call_det(X=None, W=None, Y=None, M=0) == detred.OK
    assert detred.lib().atomic_splitk_gemm(None, 512, None, 0, None, 0, 16, 0, 512, 8, None) == detred.OK
    assert detred.lib().tree_tp_gemm(None, 8, None, 8, None, 8, 0, 8, 8, 1, None, 0, None) == detred.OK


def test_other_entry_points_reject():
    L = detred.lib()
    assert L.atomic_splitk_gemm(A16, 512, A16b, 16, A16c, 16, 16, 16, 512, 5, None) == detred.EUNSUPPORTED
    assert L.tree_tp_gemm(A16, 512, A16b, 16, A16c, 16, 16, 16, 512, 3, None, 0, None) == detred.EUNSUPPORTED
    assert L.tree_tp_gemm(A16, 512, A16b, 16, A16c, 16, 16, 16, 512, 4, None, 0, None) == detred.EWORKSPACE
    assert L.tree_tp_shards_gemm(A16, 512, A16b, 16, A16c, 16, 16, 512, 3, None) == detred.EUNSUPPORTED
    assert L.tree_tp_shards_gemm(None, 512, A16b, 16, A16c, 16, 16, 512, 2, None) == detred.EINVAL
    assert L.tree_tp_shard_gemm(A16, 64, A16b, 16, A16c, 16, 16, 16, 64, 6, None) == detred.EINVAL
    assert L.tree_tp_shard_gemm(A16, 40, A16b, 16, A16c, 16, 16, 16, 40, 2, None) == detred.EUNSUPPORTED
    assert L.tree_combine_f32(A16, 16, 3, A16b, 16, None) == detred.EUNSUPPORTED
    assert L.tree_combine_f32(A16, 8, 2, A16b, 16, None) == detred.EINVAL   # stride < n
    assert L.tree_combine_f32(MIS, 16, 2, A16b, 16, None) == detred.EINVAL
    assert L.detred_f32_to_bf16(A16, A16b, 12, None) == detred.EUNSUPPORTED
    assert L.detred_f32_to_bf16(None, A16b, 16, None) == detred.EINVAL
    assert L.inv_rmsnorm(A16, A16b, A16c, 4, 4100, ctypes.c_float(1e-6), None) == detred.EUNSUPPORTED
    assert L.inv_rmsnorm(A16, None, A16c, 4, 4096, ctypes.c_float(1e-6), None) == detred.EINVAL
    assert L.inv_rmsnorm(A16, A16b, A16c, -1, 4096, ctypes.c_float(1e-6), None) == detred.EINVAL
    assert L.inv_rmsnorm(None, None, None, 0, 4096, ctypes.c_float(1e-6), None) == detred.OK
    assert L.inv_log_softmax(A16, A16b, 4, 6, None) == detred.EUNSUPPORTED
    assert L.inv_log_softmax(MIS, A16b, 4, 8, None) == detred.EINVAL
    assert L.inv_mean(A16, A16b, 4, 0, None) == detred.EUNSUPPORTED
    assert L.inv_mean(None, A16b, 4, 8, None) == detred.EINVAL
    assert L.inv_log_softmax_mean(A16, A16b, A16c, 4, 6, None) == detred.EUNSUPPORTED
    assert L.inv_log_softmax_mean(A16, A16b, None, 4, 8, None) == detred.EINVAL
    assert L.inv_log_softmax_mean(A16, MIS, A16c, 4, 8, None) == detred.EINVAL
    assert L.inv_log_softmax_mean(A16, A16b, A16c + 2, 4, 8, None) == detred.EINVAL
    assert L.inv_log_softmax_mean(None, None, None, 0, 8, None) == detred.OK
    assert L.detred_workspace_init(None, 16, None) == detred.EINVAL


def test_addmm_lora_and_bf16_rmsnorm_reject():
    L = detred.lib()
    f = ctypes.c_float
    # det_splitk_addmm(X, ldx, W, ldw, C, ldc, alpha, beta, Y, ldy, y_dtype, M, N, K, S, ws, ws_bytes, s)
    args = lambda **kw: [kw.get("X", A16), 512, A16b, 16, kw.get("C", A16c), kw.get("ldc", 16),
                         f(1.0), f(1.0), kw.get("Y", A16), 16, kw.get("dt", detred.F32),
                         16, 16, 512, kw.get("S", 1), None, 0, None]
    assert L.det_splitk_addmm(*args(dt=2)) == detred.EINVAL
    assert L.det_splitk_addmm(*args(C=MIS)) == detred.EINVAL
    assert L.det_splitk_addmm(*args(ldc=8)) == detred.EINVAL      # ldc < N
    assert L.det_splitk_addmm(*args(ldc=18)) == detred.EINVAL     # ldc % 4 != 0
    assert L.det_splitk_addmm(*args(ldc=-4)) == detred.EINVAL
    assert L.det_splitk_addmm(*args(X=MIS)) == detred.EINVAL
    assert L.det_splitk_addmm(*args(S=3)) == detred.EUNSUPPORTED
    assert L.det_splitk_addmm(*args(S=4)) == detred.EWORKSPACE
    # M == 0 launches nothing
    a = args()
    a[11] = 0
    assert L.det_splitk_addmm(*a) == detred.OK
    # det_lora_forward(X, ldx, W, ldw, A, lda, B, ldb, scale, Y, ldy, M, N, K, r, ws, ws_bytes, s)
    WS = 0x100000                     # fake, 256-byte aligned
    big = 1 << 40
    lora = lambda **kw: [kw.get("X", A16), 512, A16b, 64, A16c, kw.get("r", 16), A16b,
                         64, f(1.0), A16c, 64, 16, 64, 512, kw.get("r", 16),
                         kw.get("ws", WS), kw.get("nws", big), None]
    assert L.det_lora_forward(*lora(r=0)) == detred.EINVAL
    assert L.det_lora_forward(*lora(r=12)) == detred.EUNSUPPORTED
    assert L.det_lora_forward(*lora(ws=None)) == detred.EWORKSPACE
    assert L.det_lora_forward(*lora(ws=WS + 16)) == detred.EWORKSPACE
    assert L.det_lora_forward(*lora(nws=16)) == detred.EWORKSPACE
    assert L.det_lora_forward(*lora(X=MIS)) == detred.EINVAL
    assert L.det_lora_workspace_bytes(16, 64, 512, 0) == 0
    need = L.det_lora_workspace_bytes(16, 64, 512, 16)
    # base [16,64] fp32 + the bf16 shrink [16,16] + the split-K workspaces of
    # the base product and the shrink (both split 8 by the policy: N <= 64)
    assert need == 4096 + 512 + L.detred_gemm_workspace_bytes(16, 64, 512, 8) + \
        L.detred_gemm_workspace_bytes(16, 16, 512, 8)
    assert L.inv_rmsnorm_bf16(A16, A16b, A16c, 4, 4100, f(1e-6), None) == detred.EUNSUPPORTED
    assert L.inv_rmsnorm_bf16(A16, None, A16c, 4, 4096, f(1e-6), None) == detred.EINVAL
    assert L.inv_rmsnorm_bf16(A16, A16b, MIS, 4, 4096, f(1e-6), None) == detred.EINVAL


def test_decode_attention_rejects():
    L = detred.lib()
    f = ctypes.c_float
    WS = 0x100000
    big = 1 << 40
    # (q, k, v, sb, sh, st, lens, out, B, Hq, Hkv, D, max_len, scale, ws, nws, s)
    base = dict(q=A16, k=A16b, v=A16c, sb=8 * 1024 * 128, sh=1024 * 128, st=128, lens=A16,
                out=A16b, B=2, Hq=8, Hkv=2, D=128, L=1024, ws=WS, nws=big)

    def call(**kw):
        a = dict(base, **kw)
        return L.inv_decode_attention(a["q"], a["k"], a["v"], a["sb"], a["sh"], a["st"], a["lens"],
                                      a["out"], a["B"], a["Hq"], a["Hkv"], a["D"], a["L"], f(0.1),
                                      a["ws"], a["nws"], None)
    assert call(Hq=6, Hkv=4) == detred.EINVAL          # Hq % Hkv
    assert call(Hkv=0) == detred.EINVAL
    assert call(B=-1) == detred.EINVAL
    assert call(L=-1) == detred.EINVAL
    assert call(D=96) == detred.EUNSUPPORTED
    assert call(Hq=34, Hkv=2) == detred.EUNSUPPORTED    # group of 17
    assert call(k=MIS) == detred.EINVAL
    assert call(lens=None) == detred.EINVAL
    assert call(st=100) == detred.EINVAL                 # row stride not 16-byte aligned
    assert call(sh=-8) == detred.EINVAL
    assert call(ws=None) == detred.EWORKSPACE
    assert call(ws=WS + 16) == detred.EWORKSPACE
    assert call(nws=16) == detred.EWORKSPACE
    assert call(B=0, q=None, k=None, v=None, lens=None, out=None) == detred.OK
    # per-chunk results: B*Hq rows x 4 chunks x (D floats + 2 floats)
    assert L.inv_decode_attention_workspace_bytes(2, 8, 128, 1024) == 16 * 4 * 128 * 4 + 512
    assert L.inv_decode_attention_workspace_bytes(2, 8, 128, 1025) == 16 * 5 * 128 * 4 + 768
    assert L.inv_decode_attention_workspace_bytes(2, 0, 128, 1024) == 0


def test_torch_mode_registers_and_restores():
    # registration only (CPU): entering and leaving the mode; CPU operators
    # are not affected by the GPU-key replacements
    import torch
    from invariant_reduction_amd import torch_ops
    a = torch.ones(4, 8, dtype=torch.bfloat16)
    with torch_ops.batch_invariant_mode():
        assert torch_ops.is_enabled()
        assert torch.equal(torch.mm(a, a.t()), torch.full((4, 4), 8.0, dtype=torch.bfloat16))
    assert not torch_ops.is_enabled()


def _documented_split(M, N, K, wide=True):
    """The automatic split as include/detred.h states it, written out here
    independently of the library (wide: the call may take the 192 x 128
    tile, as det_splitk_gemm always may)."""
    P = 8 if (K >= 256 and K % 256 == 0) else 1
    if N <= 64 or P == 1:
        return None  # narrow outputs and one-chunk K keep the policy's split
    Kc = K // P
    t = ((M + 127) // 128) * ((N + 127) // 128)
    one_wide_round = Kc % 64 == 0 and ((M + 191) // 192) * ((N + 127) // 128) <= 256
    if wide and 257 <= t <= 447 and one_wide_round:
        S = 1
    elif Kc >= 1536 and M >= 256 and t >= 96:
        S = 8
    elif t <= 128:
        S = 1
        while S < P and t * S * 2 <= 256:
            S *= 2
        if S == 2 and M <= 16:
            S = 4
    elif t <= 192:
        S = 4 if Kc >= 1024 else 1
    else:
        S = (4 if Kc >= 1024 else 2) if 257 <= t <= 447 else 1
    return min(S, P)


def test_auto_split_follows_the_documented_rule():
    for K in (256, 1024, 4096, 8192, 12288, 14336, 16384):
        for N in (72, 128, 1000, 1024, 4096, 8192, 14336, 28672):
            for M in (1, 2, 16, 17, 63, 64, 65, 128, 192, 255, 256, 257, 384, 512, 640, 768, 1024,
                      1536, 2048, 2560, 3000, 4096, 8192):
                want = _documented_split(M, N, K)
                if want is not None:
                    assert detred.auto_split(M, N, K) == want, (M, N, K)


def test_workspace_sizes_cover_the_partial_planes():
    """For every split the library may pick, detred_gemm_workspace_bytes
    covers S fp32 [M][N] planes (the slice roots) plus one counter per
    output tile, rounded to 256 bytes; S = 1 needs none."""
    L = detred.lib()
    for K in (64, 512, 4096, 14336):
        for N in (8, 16, 64, 72, 1024, 14336):
            for M in (1, 7, 64, 255, 256, 1000, 4096):
                for S in (0, 1, 2, 4, 8):
                    got = L.detred_gemm_workspace_bytes(M, N, K, S)
                    s = S if S else detred.auto_split(M, N, K)
                    if S == 0:
                        # also the split of a call that cannot take the 192x128 tile
                        s = max(s, _documented_split(M, N, K, wide=False) or 0)
                    P = 8 if (K >= 256 and K % 256 == 0) else 1
                    if s <= 1 or s > P:
                        if s <= 1:
                            assert got == 0, (M, N, K, S)
                        continue
                    assert got % 256 == 0, (M, N, K, S)
                    assert got >= s * M * N * 4 + 4, (M, N, K, S)  # planes + at least one counter
