"""Python binding of libpdgemm: multi-precision dense GEMM on MI355X (gfx950).

Argument marshalling only.  Every GEMM runs in the HIP kernels of
libpdgemm.so, called through its C ABI (include/pdgemm.h) on the current
torch stream.  torch is used for device memory and streams; nothing here
computes.  If the library has not been built, importing this package fails.

Operands are torch tensors on the GPU whose rows are contiguous in K:

    A    (M, K) row-major; a column slice of a wider buffer is fine
         (lda = A.stride(0))
    Bt   (N, K): the column-major B of C = A*B, stored as the rows of its
         transpose (ldb = Bt.stride(0))
    out  (M, N) row-major (ldc = out.stride(0)); allocated when omitted

With the *_rowb functions B is instead a (K, N) row-major tensor
(ldb = B.stride(0)); INT4 packs it along N, (K, N/2) bytes.

INT4 operands are uint8 tensors of packed bytes, (rows, K/2), two signed
4-bit values per byte with the even k in the low nibble; K is passed
explicitly and the leading dimensions are counted in 4-bit elements.

The dequantizing variants of the integer GEMMs take float32 scale vectors
scale_a (M,) and scale_b (N,) and write ((float)sum * scale_a[i]) *
scale_b[j] as float32, or rounded to float16.
"""
from __future__ import annotations

import ctypes
import os

# torch first: in a process that opened a HIP library before importing torch,
# torch's later device set-up failed (every GPU call returned hipErrorNoDevice)
import torch  # noqa: E402

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libpdgemm.so")

PREC_F16, PREC_I8, PREC_I4 = 0, 1, 2
I4_MAX_K = 131071

if not os.path.exists(LIBRARY):
    raise ImportError(
        f"{LIBRARY} is missing: build the HIP library first "
        "(python precision_dense_gemm_amd/build.py, or __graft_entry__.build())")

lib = ctypes.CDLL(LIBRARY)
_i64, _p, _i = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
for _name in ("gemm_f16", "gemm_i8", "gemm_i4"):
    getattr(lib, _name).argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
    getattr(lib, _name).restype = _i
for _name in ("gemm_i8_dequant", "gemm_i4_dequant"):
    getattr(lib, _name).argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _p, _p, _i64, _i, _p]
    getattr(lib, _name).restype = _i
for _name in ("gemm_f16_rowb", "gemm_i8_rowb", "gemm_i4_rowb"):
    getattr(lib, _name).argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
    getattr(lib, _name).restype = _i
lib.pdgemm_gemm_rowb_cfg.argtypes = [_i, _i, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
lib.pdgemm_gemm_rowb_cfg.restype = _i
lib.pdgemm_dequant_cfg.argtypes = [_i, _i, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _p, _p, _i64,
                                   _i, _p]
lib.pdgemm_dequant_cfg.restype = _i
lib.pdgemm_gemm_cfg.argtypes = [_i, _i, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
lib.pdgemm_gemm_cfg.restype = _i
lib.pdgemm_gemm_splitk_cfg.argtypes = [_i, _i, _i, _i, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
lib.pdgemm_gemm_splitk_cfg.restype = _i
lib.pdgemm_pick_splits.argtypes = [_i, _i, _i64, _i64, _i64, ctypes.POINTER(_i)]
lib.pdgemm_pick_splits.restype = _i
lib.pdgemm_num_configs.argtypes = []
lib.pdgemm_num_configs.restype = _i
lib.pdgemm_pick_config.argtypes = [_i, _i64, _i64, _i64]
lib.pdgemm_pick_config.restype = _i
lib.pdgemm_config_info.argtypes = [_i] + [ctypes.POINTER(_i)] * 5
lib.pdgemm_config_info.restype = _i
lib.pdgemm_i4_workspace_size.argtypes = [_i64, _i64, _i64]
lib.pdgemm_i4_workspace_size.restype = _i64
lib.pdgemm_i4_f6_workspace_bytes.argtypes = [_i64, _i64, _i64]
lib.pdgemm_i4_f6_workspace_bytes.restype = _i64
lib.pdgemm_i4_f6_pick.argtypes = [_i64, _i64, _i64]
lib.pdgemm_i4_f6_pick.restype = _i
lib.pdgemm_i4_f6_num_configs.argtypes = []
lib.pdgemm_i4_f6_num_configs.restype = _i
for _name in ("gemm_i4_ws", "gemm_i4_rowb_ws"):
    getattr(lib, _name).argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
    getattr(lib, _name).restype = _i
lib.gemm_i4_dequant_ws.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _p, _p, _i64, _i, _p, _i64,
                                   _p]
lib.gemm_i4_dequant_ws.restype = _i
lib.pdgemm_i4_f6_cfg.argtypes = [_i, _i, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _p, _p, _i64, _i, _p,
                                 _i64, _p]
lib.pdgemm_i4_f6_cfg.restype = _i
lib.pdgemm_i4_f6_image_bytes.argtypes = [_i64, _i64]
lib.pdgemm_i4_f6_image_bytes.restype = _i64
lib.pdgemm_i4_f6_pack.argtypes = [_i64, _i64, _p, _i64, _i, _p, _i64, _p]
lib.pdgemm_i4_f6_pack.restype = _i
lib.gemm_i4_packed_b.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
lib.gemm_i4_packed_b.restype = _i
lib.gemm_i4_dequant_packed_b.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _p, _p, _i64, _i, _p,
                                         _i64, _p]
lib.gemm_i4_dequant_packed_b.restype = _i
lib.pdgemm_i4_packed_b_cfg.argtypes = [_i, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _p, _p, _i64, _i, _p,
                                       _i64, _p]
lib.pdgemm_i4_packed_b_cfg.restype = _i
lib.gemm_i4_noalloc.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
lib.gemm_i4_noalloc.restype = _i
lib.pdgemm_i4_noalloc_max_bytes.argtypes = []
lib.pdgemm_i4_noalloc_max_bytes.restype = _i64
lib.pdgemm_strerror.argtypes = [_i]
lib.pdgemm_strerror.restype = ctypes.c_char_p
lib.pdgemm_version.argtypes = []
lib.pdgemm_version.restype = _i


class PdgemmError(RuntimeError):
    def __init__(self, code: int):
        self.code = code
        super().__init__(f"pdgemm error {code}: {strerror(code)}")


def strerror(code: int) -> str:
    return lib.pdgemm_strerror(code).decode()


def version() -> int:
    return lib.pdgemm_version()


def num_configs() -> int:
    return lib.pdgemm_num_configs()


def pick_config(prec: int, M: int, N: int, K: int) -> int:
    return lib.pdgemm_pick_config(prec, M, N, K)


def pick_splits(prec: int, M: int, N: int, K: int, rowb: bool = False) -> tuple[int, int]:
    """(ranges of K, tile configuration) the raw-sum entry points use for a shape;
    ranges == 1: no K split across workgroups."""
    cfg = _i()
    s = lib.pdgemm_pick_splits(prec, 1 if rowb else 0, M, N, K, ctypes.byref(cfg))
    return s, cfg.value


def config_info(cfg: int) -> dict:
    vals = [_i() for _ in range(5)]
    rc = lib.pdgemm_config_info(cfg, *[ctypes.byref(v) for v in vals])
    if rc:
        raise PdgemmError(rc)
    keys = ("block_m", "block_n", "wave_m", "wave_n", "threads")
    return {k: v.value for k, v in zip(keys, vals)}


def i4_workspace_size(M: int, N: int, K: int) -> int:
    """Bytes of workspace the INT4 workspace entry points need for this shape
    (0 where they run the INT8-MFMA kernels)."""
    return lib.pdgemm_i4_workspace_size(M, N, K)


def i4_f6_workspace_bytes(M: int, N: int, K: int) -> int:
    """Bytes of workspace of the FP6 path for this shape, whichever tile it takes."""
    return lib.pdgemm_i4_f6_workspace_bytes(M, N, K)


def i4_f6_pick(M: int, N: int, K: int) -> int:
    """The FP6 tile the workspace entry points take for this shape (-1: INT8-MFMA kernels)."""
    return lib.pdgemm_i4_f6_pick(M, N, K)


def i4_f6_num_configs() -> int:
    return lib.pdgemm_i4_f6_num_configs()


def i4_workspace(M: int, N: int, K: int, device=None, f6: bool = False) -> torch.Tensor:
    """A workspace tensor for an INT4 GEMM of this shape (at least 256 bytes; with f6,
    sized for the FP6 path whatever the library would pick)."""
    n = i4_f6_workspace_bytes(M, N, K) if f6 else i4_workspace_size(M, N, K)
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _row_major_2d(t: torch.Tensor, name: str):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have contiguous rows (stride(1) == 1)")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _scale(t: torch.Tensor, n: int, name: str) -> int:
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.dim() != 1:
        raise TypeError(f"{name} must be a 1-D float32 tensor")
    if t.shape[0] != n:
        raise ValueError(f"{name} must hold {n} values")
    if n > 1 and t.stride(0) != 1:
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t.data_ptr()


def _workspace(ws, device):
    """(pointer, bytes) of a workspace tensor (or (None, 0))."""
    if ws is None:
        return None, 0
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise TypeError("workspace must be a contiguous GPU tensor")
    if ws.device != device:
        raise ValueError("workspace must be on the operands' GPU")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _marshal(prec, A, Bt, out, K, lda, ldb, stream, cfg, scales=None, N=None, rowb=False,
             workspace=None, f6cfg=None, splits=None):
    """The C function and its argument tuple for one GEMM (dequantizing when
    scales = (scale_a, scale_b) is given; B row-major when rowb, with N given;
    INT4 on the FP6 cores with a workspace, by the library's choice or with
    the FP6 tile f6cfg; K split over `splits` ranges across workgroups on the
    tile cfg)."""
    M = A.shape[0]
    N = Bt.shape[0] if N is None else N
    ldc = _row_major_2d(out, "out")
    tensors = [A, Bt, out] + ([] if scales is None else list(scales))
    if any(isinstance(t, torch.Tensor) and t.device != out.device for t in tensors):
        raise ValueError("operands, scales and out must be on the same GPU")
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must have shape {(M, N)}")
    if splits is not None:
        if cfg is None or scales is not None or workspace is not None or f6cfg is not None:
            raise ValueError("a K split across workgroups takes a tile cfg and no scales or workspace")
        return lib.pdgemm_gemm_splitk_cfg, (prec, cfg, 1 if rowb else 0, splits, M, N, K, A.data_ptr(), lda,
                                            Bt.data_ptr(), ldb, out.data_ptr(), ldc, _stream(stream))
    if workspace is not None or f6cfg is not None:
        if prec != PREC_I4:
            raise ValueError("a workspace serves the INT4 GEMM on the FP6 cores only")
        if cfg is not None:
            raise ValueError("cfg selects an INT8-MFMA tile; the FP6 tile is f6cfg")
        ws, ws_bytes = _workspace(workspace, out.device)
        sa = sb = None
        if scales is not None:
            if out.dtype not in (torch.float32, torch.float16):
                raise TypeError("a dequantizing GEMM writes float32 or float16")
            sa, sb = _scale(scales[0], M, "scale_a"), _scale(scales[1], N, "scale_b")
        half = 1 if out.dtype == torch.float16 else 0
        if f6cfg is not None:
            return lib.pdgemm_i4_f6_cfg, (f6cfg, 1 if rowb else 0, M, N, K, A.data_ptr(), lda,
                                          Bt.data_ptr(), ldb, sa, sb, out.data_ptr(), ldc, half, ws,
                                          ws_bytes, _stream(stream))
        if scales is not None:
            if rowb:
                raise ValueError("the dequantizing epilogue takes a column-major B")
            return lib.gemm_i4_dequant_ws, (M, N, K, A.data_ptr(), lda, Bt.data_ptr(), ldb, sa, sb,
                                            out.data_ptr(), ldc, half, ws, ws_bytes, _stream(stream))
        fn = lib.gemm_i4_rowb_ws if rowb else lib.gemm_i4_ws
        return fn, (M, N, K, A.data_ptr(), lda, Bt.data_ptr(), ldb, out.data_ptr(), ldc, ws, ws_bytes,
                    _stream(stream))
    if rowb:
        if scales is not None:
            raise ValueError("the dequantizing epilogue takes a column-major B")
        args = (M, N, K, A.data_ptr(), lda, Bt.data_ptr(), ldb, out.data_ptr(), ldc,
                _stream(stream))
        if cfg is None:
            return (lib.gemm_f16_rowb, lib.gemm_i8_rowb, lib.gemm_i4_rowb)[prec], args
        return lib.pdgemm_gemm_rowb_cfg, (prec, cfg) + args
    if scales is None:
        args = (M, N, K, A.data_ptr(), lda, Bt.data_ptr(), ldb, out.data_ptr(), ldc,
                _stream(stream))
        if cfg is None:
            return (lib.gemm_f16, lib.gemm_i8, lib.gemm_i4)[prec], args
        return lib.pdgemm_gemm_cfg, (prec, cfg) + args
    if prec == PREC_F16:
        raise ValueError("the dequantizing epilogue is for INT8 and INT4")
    if out.dtype not in (torch.float32, torch.float16):
        raise TypeError("a dequantizing GEMM writes float32 or float16")
    args = (M, N, K, A.data_ptr(), lda, Bt.data_ptr(), ldb, _scale(scales[0], M, "scale_a"),
            _scale(scales[1], N, "scale_b"), out.data_ptr(), ldc,
            1 if out.dtype == torch.float16 else 0, _stream(stream))
    if cfg is None:
        return (None, lib.gemm_i8_dequant, lib.gemm_i4_dequant)[prec], args
    return lib.pdgemm_dequant_cfg, (prec, cfg) + args


def _call(prec, A, Bt, out, K, lda, ldb, stream, cfg, scales=None, N=None, rowb=False, workspace=None,
          f6cfg=None, splits=None):
    fn, args = _marshal(prec, A, Bt, out, K, lda, ldb, stream, cfg, scales, N, rowb, workspace, f6cfg, splits)
    rc = fn(*args)
    if rc != 0:
        raise PdgemmError(rc)
    return out


def gemm_f16(A: torch.Tensor, Bt: torch.Tensor, out: torch.Tensor | None = None,
             stream=None, cfg: int | None = None, splits: int | None = None) -> torch.Tensor:
    """C = A * B for binary16 A (M, K) and Bt (N, K); fp32 accumulate, fp32 C (M, N)."""
    if A.dtype != torch.float16 or Bt.dtype != torch.float16:
        raise TypeError("gemm_f16 takes float16 operands")
    K = A.shape[1]
    if Bt.shape[1] != K:
        raise ValueError("A and Bt disagree on K")
    lda, ldb = _row_major_2d(A, "A"), _row_major_2d(Bt, "Bt")
    if out is None:
        out = torch.empty((A.shape[0], Bt.shape[0]), dtype=torch.float32, device=A.device)
    elif out.dtype != torch.float32:
        raise TypeError("gemm_f16 writes a float32 output")
    return _call(PREC_F16, A, Bt, out, K, lda, ldb, stream, cfg, splits=splits)


def gemm_i8(A: torch.Tensor, Bt: torch.Tensor, out: torch.Tensor | None = None,
            stream=None, cfg: int | None = None, splits: int | None = None) -> torch.Tensor:
    """C = A * B for int8 A (M, K) and Bt (N, K); int32 accumulate, int32 C (M, N)."""
    if A.dtype != torch.int8 or Bt.dtype != torch.int8:
        raise TypeError("gemm_i8 takes int8 operands")
    K = A.shape[1]
    if Bt.shape[1] != K:
        raise ValueError("A and Bt disagree on K")
    lda, ldb = _row_major_2d(A, "A"), _row_major_2d(Bt, "Bt")
    if out is None:
        out = torch.empty((A.shape[0], Bt.shape[0]), dtype=torch.int32, device=A.device)
    elif out.dtype != torch.int32:
        raise TypeError("gemm_i8 writes an int32 output")
    return _call(PREC_I8, A, Bt, out, K, lda, ldb, stream, cfg, splits=splits)


def gemm_i4(A: torch.Tensor, Bt: torch.Tensor, K: int | None = None,
            out: torch.Tensor | None = None, stream=None, cfg: int | None = None,
            workspace: torch.Tensor | None = None, f6cfg: int | None = None,
            splits: int | None = None) -> torch.Tensor:
    """C = A * B for packed INT4 A (M, K/2) and Bt (N, K/2) bytes; int32 C (M, N).
    With a workspace (see i4_workspace) the library may run it on the FP6 cores."""
    if A.dtype != torch.uint8 or Bt.dtype != torch.uint8:
        raise TypeError("gemm_i4 takes uint8 tensors of packed 4-bit values")
    if K is None:
        K = 2 * A.shape[1]
    if A.shape[1] * 2 < K or Bt.shape[1] * 2 < K:
        raise ValueError("packed operands hold fewer than K values per row")
    lda, ldb = 2 * _row_major_2d(A, "A"), 2 * _row_major_2d(Bt, "Bt")
    if out is None:
        out = torch.empty((A.shape[0], Bt.shape[0]), dtype=torch.int32, device=A.device)
    elif out.dtype != torch.int32:
        raise TypeError("gemm_i4 writes an int32 output")
    return _call(PREC_I4, A, Bt, out, K, lda, ldb, stream, cfg, workspace=workspace, f6cfg=f6cfg,
                 splits=splits)


def gemm_i4_noalloc(A: torch.Tensor, Bt: torch.Tensor, K: int | None = None,
                    out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """gemm_i4 through the allocation-free entry point (the library's own fixed
    workspace; calls that overlap on one GPU race)."""
    if A.dtype != torch.uint8 or Bt.dtype != torch.uint8:
        raise TypeError("gemm_i4_noalloc takes uint8 tensors of packed 4-bit values")
    if K is None:
        K = 2 * A.shape[1]
    if A.shape[1] * 2 < K or Bt.shape[1] * 2 < K:
        raise ValueError("packed operands hold fewer than K values per row")
    lda, ldb = 2 * _row_major_2d(A, "A"), 2 * _row_major_2d(Bt, "Bt")
    if out is None:
        out = torch.empty((A.shape[0], Bt.shape[0]), dtype=torch.int32, device=A.device)
    elif out.dtype != torch.int32:
        raise TypeError("gemm_i4_noalloc writes an int32 output")
    M, N = A.shape[0], Bt.shape[0]
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must have shape {(M, N)}")
    if A.device != out.device or Bt.device != out.device:
        raise ValueError("operands and out must be on the same GPU")
    rc = lib.gemm_i4_noalloc(M, N, K, A.data_ptr(), lda, Bt.data_ptr(), ldb, out.data_ptr(),
                             _row_major_2d(out, "out"), _stream(stream))
    if rc != 0:
        raise PdgemmError(rc)
    return out


def i4_f6_image_bytes(rows: int, K: int) -> int:
    """Bytes of the FP6 image of an INT4 operand of `rows` rows of K values."""
    return int(lib.pdgemm_i4_f6_image_bytes(rows, K))


def i4_f6_pack(src: torch.Tensor, K: int | None = None, rowmajor: bool = False, N: int | None = None,
               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The FP6 image (a uint8 tensor) of an INT4 operand, for gemm_i4_packed_b:
    src (rows, K/2) packed along K (A, or a column-major B as Bt), or with
    rowmajor a row-major B (K, N/2) packed along N (N defaults to 2 * src.shape[1])."""
    if src.dtype != torch.uint8:
        raise TypeError("i4_f6_pack takes a uint8 tensor of packed 4-bit values")
    ld = 2 * _row_major_2d(src, "src")
    if rowmajor:
        K = src.shape[0] if K is None else K
        rows = 2 * src.shape[1] if N is None else N
        if src.shape[0] < K or 2 * src.shape[1] < rows:
            raise ValueError("src holds fewer than K rows of N values")
    else:
        K = 2 * src.shape[1] if K is None else K
        rows = src.shape[0]
        if 2 * src.shape[1] < K:
            raise ValueError("src holds fewer than K values per row")
    need = i4_f6_image_bytes(rows, K)
    if out is None:
        out = torch.empty(max(need, 16), dtype=torch.uint8, device=src.device)
    ptr, nbytes = _workspace(out, src.device)
    rc = lib.pdgemm_i4_f6_pack(rows, K, src.data_ptr(), ld, 1 if rowmajor else 0, ptr, nbytes, _stream(stream))
    if rc != 0:
        raise PdgemmError(rc)
    return out


def gemm_i4_packed_b(A: torch.Tensor, image_b: torch.Tensor, K: int, N: int, out: torch.Tensor | None = None,
                     scales=None, workspace: torch.Tensor | None = None, f6cfg: int | None = None,
                     stream=None) -> torch.Tensor:
    """C = A * B with B given as its FP6 image (i4_f6_pack of N rows, same K): int32 C,
    or with scales = (scale_a, scale_b) the dequantized float32 / float16 C."""
    if A.dtype != torch.uint8:
        raise TypeError("gemm_i4_packed_b takes a uint8 A of packed 4-bit values")
    if 2 * A.shape[1] < K:
        raise ValueError("A holds fewer than K values per row")
    M = A.shape[0]
    lda = 2 * _row_major_2d(A, "A")
    if out is None:
        out = torch.empty((M, N), dtype=torch.int32 if scales is None else torch.float32, device=A.device)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must have shape {(M, N)}")
    if scales is None and out.dtype != torch.int32:
        raise TypeError("gemm_i4_packed_b writes an int32 output")
    if scales is not None and out.dtype not in (torch.float32, torch.float16):
        raise TypeError("a dequantizing GEMM writes float32 or float16")
    if A.device != out.device:
        raise ValueError("A and out must be on the same GPU")
    if workspace is None:
        workspace = torch.empty(max(i4_f6_image_bytes(M, K), 16), dtype=torch.uint8, device=A.device)
    ws, ws_bytes = _workspace(workspace, out.device)
    img, img_bytes = _workspace(image_b, out.device)
    ldc = _row_major_2d(out, "out")
    sa = sb = None
    if scales is not None:
        sa, sb = _scale(scales[0], M, "scale_a"), _scale(scales[1], N, "scale_b")
    half = 1 if out.dtype == torch.float16 else 0
    if f6cfg is not None:
        rc = lib.pdgemm_i4_packed_b_cfg(f6cfg, M, N, K, A.data_ptr(), lda, img, img_bytes, sa, sb,
                                        out.data_ptr(), ldc, half, ws, ws_bytes, _stream(stream))
    elif scales is not None:
        rc = lib.gemm_i4_dequant_packed_b(M, N, K, A.data_ptr(), lda, img, img_bytes, sa, sb, out.data_ptr(),
                                          ldc, half, ws, ws_bytes, _stream(stream))
    else:
        rc = lib.gemm_i4_packed_b(M, N, K, A.data_ptr(), lda, img, img_bytes, out.data_ptr(), ldc, ws,
                                  ws_bytes, _stream(stream))
    if rc != 0:
        raise PdgemmError(rc)
    return out


_DTYPES = {"f16": (torch.float16, torch.float32, PREC_F16), "i8": (torch.int8, torch.int32, PREC_I8),
           "i4": (torch.uint8, torch.int32, PREC_I4)}


def _gemm_rowb(prec, A, B, K, N, out, stream, cfg, workspace=None, f6cfg=None, splits=None):
    in_t, out_t, p = _DTYPES[prec]
    if A.dtype != in_t or B.dtype != in_t:
        raise TypeError(f"{prec} with row-major B takes {in_t} operands")
    per = 2 if prec == "i4" else 1
    K = per * A.shape[1] if K is None else K
    N = per * B.shape[1] if N is None else N
    if per * A.shape[1] < K or B.shape[0] < K or per * B.shape[1] < N:
        raise ValueError("operands hold fewer than K values per row of A, K rows of B or N columns")
    lda, ldb = per * _row_major_2d(A, "A"), per * _row_major_2d(B, "B")
    if out is None:
        out = torch.empty((A.shape[0], N), dtype=out_t, device=A.device)
    elif out.dtype != out_t:
        raise TypeError(f"{prec} writes a {out_t} output")
    return _call(p, A, B, out, K, lda, ldb, stream, cfg, N=N, rowb=True, workspace=workspace,
                 f6cfg=f6cfg, splits=splits)


def gemm_f16_rowb(A: torch.Tensor, B: torch.Tensor, out: torch.Tensor | None = None,
                  stream=None, cfg: int | None = None, splits: int | None = None) -> torch.Tensor:
    """C = A * B for binary16 A (M, K) and row-major B (K, N); fp32 C (M, N)."""
    return _gemm_rowb("f16", A, B, None, None, out, stream, cfg, splits=splits)


def gemm_i8_rowb(A: torch.Tensor, B: torch.Tensor, out: torch.Tensor | None = None,
                 stream=None, cfg: int | None = None, splits: int | None = None) -> torch.Tensor:
    """C = A * B for int8 A (M, K) and row-major B (K, N); int32 C (M, N)."""
    return _gemm_rowb("i8", A, B, None, None, out, stream, cfg, splits=splits)


def gemm_i4_rowb(A: torch.Tensor, B: torch.Tensor, K: int | None = None, N: int | None = None,
                 out: torch.Tensor | None = None, stream=None, cfg: int | None = None,
                 workspace: torch.Tensor | None = None, f6cfg: int | None = None,
                 splits: int | None = None) -> torch.Tensor:
    """C = A * B for packed INT4 A (M, K/2) and row-major B (K, N/2 bytes, packed along N)."""
    return _gemm_rowb("i4", A, B, K, N, out, stream, cfg, workspace, f6cfg, splits)


def gemm_i8_dequant(A: torch.Tensor, Bt: torch.Tensor, scale_a: torch.Tensor,
                    scale_b: torch.Tensor, out: torch.Tensor | None = None,
                    out_dtype: torch.dtype = torch.float32, stream=None,
                    cfg: int | None = None) -> torch.Tensor:
    """INT8 GEMM, then C[i][j] = ((float)sum * scale_a[i]) * scale_b[j] in binary32,
    stored as float32 or rounded to float16 (out's dtype, else out_dtype)."""
    if A.dtype != torch.int8 or Bt.dtype != torch.int8:
        raise TypeError("gemm_i8_dequant takes int8 operands")
    K = A.shape[1]
    if Bt.shape[1] != K:
        raise ValueError("A and Bt disagree on K")
    lda, ldb = _row_major_2d(A, "A"), _row_major_2d(Bt, "Bt")
    if out is None:
        out = torch.empty((A.shape[0], Bt.shape[0]), dtype=out_dtype, device=A.device)
    return _call(PREC_I8, A, Bt, out, K, lda, ldb, stream, cfg, (scale_a, scale_b))


def gemm_i4_dequant(A: torch.Tensor, Bt: torch.Tensor, scale_a: torch.Tensor,
                    scale_b: torch.Tensor, K: int | None = None,
                    out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32,
                    stream=None, cfg: int | None = None, workspace: torch.Tensor | None = None,
                    f6cfg: int | None = None) -> torch.Tensor:
    """Packed INT4 GEMM with the dequantizing epilogue of gemm_i8_dequant."""
    if A.dtype != torch.uint8 or Bt.dtype != torch.uint8:
        raise TypeError("gemm_i4_dequant takes uint8 tensors of packed 4-bit values")
    if K is None:
        K = 2 * A.shape[1]
    if A.shape[1] * 2 < K or Bt.shape[1] * 2 < K:
        raise ValueError("packed operands hold fewer than K values per row")
    lda, ldb = 2 * _row_major_2d(A, "A"), 2 * _row_major_2d(Bt, "Bt")
    if out is None:
        out = torch.empty((A.shape[0], Bt.shape[0]), dtype=out_dtype, device=A.device)
    return _call(PREC_I4, A, Bt, out, K, lda, ldb, stream, cfg, (scale_a, scale_b), workspace=workspace,
                 f6cfg=f6cfg)


def prepare(prec: str, A: torch.Tensor, Bt: torch.Tensor, out: torch.Tensor, K: int | None = None,
            stream=None, cfg: int | None = None, scales=None, rowb: bool = False,
            workspace: torch.Tensor | None = None, f6cfg: int | None = None):
    """Check and marshal one GEMM once; return a no-argument callable that
    enqueues it again (on the stream current now) through the C ABI.

    For repeated launches of the same operands, e.g. timing loops: the
    callable skips the per-call Python checks, so host time stays far below
    the kernel time even for small shapes.  The tensors must stay alive.
    With scales = (scale_a, scale_b) an INT8 / INT4 GEMM is the dequantizing
    one, and out is float32 or float16.  With rowb, Bt is a row-major B
    (K, N) instead (INT4: packed along N) and N is out's column count.  An
    INT4 GEMM with a workspace runs through the workspace entry points.
    """
    integer_out = (torch.int32,) if scales is None else (torch.float32, torch.float16)
    if prec == "f16":
        if A.dtype != torch.float16 or Bt.dtype != torch.float16 or out.dtype != torch.float32:
            raise TypeError("f16 takes float16 operands and a float32 output")
        K = A.shape[1] if K is None else K
        lda, ldb, p = _row_major_2d(A, "A"), _row_major_2d(Bt, "Bt"), PREC_F16
    elif prec == "i8":
        if A.dtype != torch.int8 or Bt.dtype != torch.int8 or out.dtype not in integer_out:
            raise TypeError("i8 takes int8 operands and an int32 (dequantizing: float) output")
        K = A.shape[1] if K is None else K
        lda, ldb, p = _row_major_2d(A, "A"), _row_major_2d(Bt, "Bt"), PREC_I8
    elif prec == "i4":
        if A.dtype != torch.uint8 or Bt.dtype != torch.uint8 or out.dtype not in integer_out:
            raise TypeError("i4 takes uint8 packed operands and an int32 (dequantizing: float) output")
        K = 2 * A.shape[1] if K is None else K
        lda, ldb, p = 2 * _row_major_2d(A, "A"), 2 * _row_major_2d(Bt, "Bt"), PREC_I4
    else:
        raise ValueError(f"unknown precision {prec!r}")
    per = 2 if prec == "i4" else 1
    N = out.shape[1]
    if rowb:
        if A.shape[1] * per < K or Bt.shape[0] < K or Bt.shape[1] * per < N:
            raise ValueError("operands hold fewer than K values per row of A, K rows of B or N columns")
    elif A.shape[1] * per < K or Bt.shape[1] * per < K:
        raise ValueError("operands hold fewer than K values per row")
    fn, args = _marshal(p, A, Bt, out, K, lda, ldb, stream, cfg, scales, N=N if rowb else None,
                        rowb=rowb, workspace=workspace, f6cfg=f6cfg)
    rc = fn(*args)  # validates the arguments once, and is a first launch
    if rc != 0:
        raise PdgemmError(rc)

    # the callable holds the tensors, so their memory outlives it
    keep = (A, Bt, out) + (tuple(scales) if scales is not None else ()) + (
        (workspace,) if workspace is not None else ())

    def launch():
        rc = fn(*args)
        if rc != 0:
            raise PdgemmError(rc)

    launch.tensors = keep
    return launch
