"""The entry points under HIP graph capture: they enqueue kernel launches only
(no allocation, copy or memset), so a captured GEMM replays.  Each replay
follows eager work that overwrites the output with a sentinel, and must give
the eager result bit for bit; the integer results are also checked against
the oracle.  Every case prints its name before it touches the GPU."""
from __future__ import annotations

import pytest

import oracle
import synth
from tests import gpu_util as gu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_dense_gemm_amd as pd
    return pd


@pytest.fixture(scope="module")
def dev(pd):
    return torch.device("cuda:0")


@pytest.mark.parametrize("prec", ["f16", "i8", "i4"])
@pytest.mark.parametrize("shape", [(520, 600, 1024), (16, 2048, 4096)], ids=["multi-tile", "k-split"])
def test_captured_gemm_replays(pd, dev, prec, shape):
    M, N, K = shape
    gu.note(f"[case] graph {prec} {M}x{N}x{K}")
    A, Bt = synth.operands(prec, M, N, K, 91, 92)
    Ad, Bd = torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev)
    out_dtype = torch.float32 if prec == "f16" else torch.int32
    out = torch.empty((M, N), dtype=out_dtype, device=dev)

    def call():
        if prec == "f16":
            pd.gemm_f16(Ad, Bd, out=out)
        elif prec == "i8":
            pd.gemm_i8(Ad, Bd, out=out)
        else:
            pd.gemm_i4(Ad, Bd, K, out=out)

    call()
    torch.cuda.synchronize()
    eager = out.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on the capture stream, as torch recommends
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for replay in range(3):
        out.view(torch.int32).fill_(gu.C_SENTINEL_BITS)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32)), f"replay {replay}"
    if prec != "f16":
        ref = oracle.gemm_i8(A, Bt) if prec == "i8" else oracle.gemm_i4(A, Bt, K)
        gu.assert_int_equal(eager.cpu().numpy(), ref, f"graph {prec}")
    else:
        R, S = oracle.gemm_f16(A, Bt)
        gu.assert_f16_close(eager.cpu().numpy(), R, S, "graph f16")
    del g


@pytest.mark.parametrize("prec", ["f16", "i8", "i4"])
def test_prepared_launches_captured_in_a_graph(pd, dev, prec):
    # prepare() inside a capture: its first launch and the callable's later ones
    # are all recorded on the capture stream, as the back-to-back timing uses them
    M, N, K = 300, 200, 512
    gu.note(f"[case] graph prepare {prec} {M}x{N}x{K}")
    A, Bt = synth.operands(prec, M, N, K, 93, 94)
    Ad, Bd = torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev)
    out = torch.empty((M, N), dtype=torch.float32 if prec == "f16" else torch.int32, device=dev)
    pd.prepare(prec, Ad, Bd, out, K=K)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        go = pd.prepare(prec, Ad, Bd, out, K=K)
        go()
        go()
    for replay in range(3):
        out.view(torch.int32).fill_(gu.C_SENTINEL_BITS)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32)), f"replay {replay}"
    if prec != "f16":
        ref = oracle.gemm_i8(A, Bt) if prec == "i8" else oracle.gemm_i4(A, Bt, K)
        gu.assert_int_equal(eager.cpu().numpy(), ref, f"graph prepare {prec}")
    del g


@pytest.mark.parametrize("route", ["workspace", "noalloc", "packed_b"])
def test_captured_fp6_routes_replay(pd, dev, route):
    """INT4 on the FP6 cores under capture: the pre-pass and the GEMM (two
    kernels) recorded together, with the caller's workspace, the library's
    static one, or a B image made beforehand; each replay follows eager work
    that overwrites the output, and must give the oracle's result."""
    M, N, K = 4096, 3072, 1056   # 192 tiles of 256 x 256: the FP6 route is taken
    gu.note(f"[case] graph fp6 {route} {M}x{N}x{K}")
    A, Bt = synth.operands("i4", M, N, K, 95, 96)
    Ad, Bd = torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev)
    out = torch.empty((M, N), dtype=torch.int32, device=dev)
    ws = pd.i4_workspace(M, N, K, dev, f6=True)
    img = pd.i4_f6_pack(Bd, K) if route == "packed_b" else None
    torch.cuda.synchronize()

    def call():
        if route == "workspace":
            pd.gemm_i4(Ad, Bd, K, out=out, workspace=ws, f6cfg=1)
        elif route == "noalloc":
            pd.gemm_i4_noalloc(Ad, Bd, K, out=out)
        else:
            pd.gemm_i4_packed_b(Ad, img, K, N, out=out, workspace=ws)

    call()
    torch.cuda.synchronize()
    assert pd.i4_f6_pick(M, N, K) >= 0
    ref = gu.oracle_whole("i4", A, Bt, K)
    gu.assert_int_equal(out.cpu().numpy(), ref, f"graph fp6 {route} eager")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for replay in range(3):
        out.view(torch.int32).fill_(gu.C_SENTINEL_BITS)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        gu.assert_int_equal(out.cpu().numpy(), ref, f"graph fp6 {route} replay {replay}")
    del g
