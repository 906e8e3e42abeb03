"""The allocation-free INT4 entry point (gemm_i4_noalloc) against the workspace
entry point it stands for (gemm_i4_ws), through the C ABI: bit-exact int32
results on two calls in a row, the second with a smaller input, then a shape
that runs without the fixed workspace, and a shape too large for it."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

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


def operands(M, N, K, seed, dev):
    A, Bt = synth.operands("i4", M, N, K, seed, seed + 1)
    ld = gu.round_up(K // 2, 16) + 16
    return A, Bt, gu.to_device_padded(torch, A, ld, gu.POISON["i4"], dev), \
        gu.to_device_padded(torch, Bt, ld, gu.POISON["i4"], dev)


def noalloc_call(pd, Ad, Bd, K, out):
    """gemm_i4_noalloc called through the C ABI directly (ctypes)."""
    M, N = out.shape
    rc = pd.lib.gemm_i4_noalloc(M, N, K, Ad.data_ptr(), 2 * Ad.stride(0), Bd.data_ptr(), 2 * Bd.stride(0),
                                out.data_ptr(), out.stride(0),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, pd.strerror(rc)


def test_noalloc_matches_workspace_entry_on_two_calls(pd):
    dev = torch.device("cuda:0")
    # the FP6 path with the fixed workspace, then a smaller product on it, then
    # one that the INT8-MFMA kernels take (no workspace)
    for (M, N, K), seed in (((4096, 4096, 4096), 11), ((3584, 3840, 2050), 12), ((300, 260, 1030), 13)):
        gu.note(f"[case] noalloc i4 {M}x{N}x{K} seed={seed} pick={pd.i4_f6_pick(M, N, K)}")
        A, Bt, Ad, Bd = operands(M, N, K, seed, dev)
        ref = torch.empty((M, N), dtype=torch.int32, device=dev)
        ws = pd.i4_workspace(M, N, K, dev)
        pd.gemm_i4(Ad, Bd, K, out=ref, workspace=ws)
        out = torch.full((M, N), -1, dtype=torch.int32, device=dev)
        noalloc_call(pd, Ad, Bd, K, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"gemm_i4_noalloc differs from gemm_i4_ws at {M}x{N}x{K}"
        if M * N <= 4096 * 4096:
            gu.check_whole("i4", A, Bt, K, out.cpu().numpy(), f"noalloc {M}x{N}x{K}")
        del Ad, Bd, ref, out, ws


def test_noalloc_rejects_a_shape_beyond_its_workspace(pd):
    dev = torch.device("cuda:0")
    M, N, K = 8192, 8192, 16384
    assert pd.i4_f6_workspace_bytes(M, N, K) > pd.lib.pdgemm_i4_noalloc_max_bytes()
    gu.note(f"[case] noalloc beyond the fixed workspace {M}x{N}x{K}")
    A = torch.zeros((M, K // 2), dtype=torch.uint8, device=dev)
    with pytest.raises(pd.PdgemmError) as e:
        pd.gemm_i4_noalloc(A, A, K)
    assert e.value.code == -7
