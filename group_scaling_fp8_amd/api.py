"""Torch-tensor front end of the C entry points (argument marshalling only).

PyTorch supplies device memory and the current HIP stream. Inputs must
already be on the GPU; bf16 tensors may be torch.bfloat16, int16 or
uint16 (the raw bit patterns are used). Outputs come back as torch.uint8
(E4M3 bytes; ``.view(torch.float8_e4m3fn)`` reinterprets them), float32
scales, and uint8 E8M0 scales.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from ._lib import MGS_FLAG_POW2_SCALE, MGS_FLAG_VALIDATE, MGS_MX_FLOOR, MGS_MX_RCEIL, check, lib

_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


try:
    _raw_stream = torch._C._cuda_getCurrentRawStream     # the current stream of a device, as an int
except AttributeError:  # pragma: no cover - other torch builds
    _raw_stream = None


def _stream_handle(stream, t: Optional[torch.Tensor] = None) -> int:
    """The hipStream_t to launch on: `stream` if given, else torch's current
    stream on t's device."""
    if stream is None:
        if _raw_stream is not None and t is not None:
            return _raw_stream(t.get_device())
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, name: str, dtypes, ndim: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU (got %s)" % (name, t.device))
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims" % (name, ndim))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


_U8_LIKE = (torch.uint8, torch.float8_e4m3fn)


def _out(t, shape, dtype, device, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(t, name, (dtype,) if dtype != torch.uint8 else _U8_LIKE)
    if t.shape != shape:
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.get_device() != device.index:
        raise ValueError("%s is on %s, the input on %s" % (name, t.device, device))
    return t


def _flags(pow2: bool, validate: bool) -> int:
    # validate: the library copies the offsets to the host and rejects bad ones
    return (MGS_FLAG_POW2_SCALE if pow2 else 0) | (MGS_FLAG_VALIDATE if validate else 0)


def mgs_dim0_workspace_bytes(M: int, K: int) -> int:
    """Bytes of workspace the dim0-family calls need for an (M, K) input
    (0 when no group can be cut into chunks)."""
    import ctypes
    n = ctypes.c_int64(0)
    check("mgs_dim0_workspace_bytes", lib().mgs_dim0_workspace_bytes(int(M), int(K), ctypes.byref(n)))
    return int(n.value)


def dim0_workspace(M: int, K: int, device=None) -> torch.Tensor:
    """A zero-filled workspace for dim0-family calls on (M, K) inputs (any
    smaller shape fits too). Keep it for reuse: calls leave it valid."""
    n = mgs_dim0_workspace_bytes(M, K)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device or "cuda")


def _ws_args(workspace: Optional[torch.Tensor]):
    if workspace is None:
        return None, 0
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" \
            or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def mgs_quant_groups_dim0(x: torch.Tensor, offsets: torch.Tensor, pow2: bool = False,
                          q: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                          stream=None, validate: bool = False,
                          workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-group scaling along dim0: x (M, K) bf16, int32 end offsets over M.
    Returns q (M, K) uint8 E4M3 and scales (G, K) float32. With `workspace`
    (from dim0_workspace) it calls mgs_quant_groups_dim0_ws, else
    mgs_quant_groups_dim0 (the library's own workspace)."""
    _need(x, "x", _BF16_LIKE, 2)
    _need(offsets, "offsets", (torch.int32,), 1)
    M, K = x.shape
    G = offsets.shape[0]
    q = _out(q, (M, K), torch.uint8, x.device, "q")
    scales = _out(scales, (G, K), torch.float32, x.device, "scales")
    if workspace is None:
        st = lib().mgs_quant_groups_dim0(x.data_ptr(), M, K, offsets.data_ptr(), G,
                                         _flags(pow2, validate), q.data_ptr(),
                                         scales.data_ptr(), _stream_handle(stream, x))
        check("mgs_quant_groups_dim0", st)
    else:
        wp, wb = _ws_args(workspace)
        st = lib().mgs_quant_groups_dim0_ws(x.data_ptr(), M, K, offsets.data_ptr(), G,
                                            _flags(pow2, validate), q.data_ptr(),
                                            scales.data_ptr(), wp, wb, _stream_handle(stream, x))
        check("mgs_quant_groups_dim0_ws", st)
    return q, scales


def mgs_quant_groups_dim0_noalloc(x: torch.Tensor, offsets: torch.Tensor, pow2: bool = False,
                                  q: Optional[torch.Tensor] = None,
                                  scales: Optional[torch.Tensor] = None, stream=None,
                                  validate: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """mgs_quant_groups_dim0 on the library's fixed per-device scratch array:
    no device memory is allocated (pass q and scales to allocate nothing on
    the Python side either)."""
    _need(x, "x", _BF16_LIKE, 2)
    _need(offsets, "offsets", (torch.int32,), 1)
    M, K = x.shape
    G = offsets.shape[0]
    q = _out(q, (M, K), torch.uint8, x.device, "q")
    scales = _out(scales, (G, K), torch.float32, x.device, "scales")
    st = lib().mgs_quant_groups_dim0_noalloc(x.data_ptr(), M, K, offsets.data_ptr(), G,
                                             _flags(pow2, validate), q.data_ptr(),
                                             scales.data_ptr(), _stream_handle(stream, x))
    check("mgs_quant_groups_dim0_noalloc", st)
    return q, scales


def mgs_quant_groups_dim0_t(x: torch.Tensor, offsets: torch.Tensor, pow2: bool = False,
                            q_t: Optional[torch.Tensor] = None,
                            scales_t: Optional[torch.Tensor] = None, stream=None,
                            validate: bool = False,
                            workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-group scaling along dim0 with transposed outputs: x (M, K) bf16,
    int32 end offsets over M (multiples of 16). Returns q_t (K, M) uint8
    E4M3 and scales_t (K, G) float32, the transposes of dim0's outputs."""
    _need(x, "x", _BF16_LIKE, 2)
    _need(offsets, "offsets", (torch.int32,), 1)
    M, K = x.shape
    G = offsets.shape[0]
    q_t = _out(q_t, (K, M), torch.uint8, x.device, "q_t")
    scales_t = _out(scales_t, (K, G), torch.float32, x.device, "scales_t")
    wp, wb = _ws_args(workspace)
    st = lib().mgs_quant_groups_dim0_t(x.data_ptr(), M, K, offsets.data_ptr(), G,
                                       _flags(pow2, validate), q_t.data_ptr(),
                                       scales_t.data_ptr(), wp, wb, _stream_handle(stream, x))
    check("mgs_quant_groups_dim0_t", st)
    return q_t, scales_t


def mgs_quant_experts_dim1(w: torch.Tensor, pow2: bool = False, q: Optional[torch.Tensor] = None,
                           scales: Optional[torch.Tensor] = None, stream=None,
                           workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-expert scaling of a 3D weight w (E, D1, D2) bf16 along dim 1.
    Returns q (E, D1, D2) uint8 E4M3 and scales (E, D2) float32."""
    _need(w, "w", _BF16_LIKE, 3)
    E, D1, D2 = w.shape
    q = _out(q, (E, D1, D2), torch.uint8, w.device, "q")
    scales = _out(scales, (E, D2), torch.float32, w.device, "scales")
    wp, wb = _ws_args(workspace)
    st = lib().mgs_quant_experts_dim1(w.data_ptr(), E, D1, D2, MGS_FLAG_POW2_SCALE if pow2 else 0,
                                      q.data_ptr(), scales.data_ptr(), wp, wb, _stream_handle(stream, w))
    check("mgs_quant_experts_dim1", st)
    return q, scales


def mgs_quant_groups_dim1(x: torch.Tensor, offsets: torch.Tensor, pow2: bool = False,
                          q: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                          stream=None, validate: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-group rowwise scaling: x (M, K) bf16, int32 end offsets over K
    (multiples of 16). Returns q (M, K) uint8 E4M3 and scales (M, G) float32."""
    _need(x, "x", _BF16_LIKE, 2)
    _need(offsets, "offsets", (torch.int32,), 1)
    M, K = x.shape
    G = offsets.shape[0]
    q = _out(q, (M, K), torch.uint8, x.device, "q")
    scales = _out(scales, (M, G), torch.float32, x.device, "scales")
    st = lib().mgs_quant_groups_dim1(x.data_ptr(), M, K, offsets.data_ptr(), G,
                                     _flags(pow2, validate), q.data_ptr(),
                                     scales.data_ptr(), _stream_handle(stream, x))
    check("mgs_quant_groups_dim1", st)
    return q, scales


def mgs_mx_quant_dim0(x: torch.Tensor, mode: int = MGS_MX_FLOOR,
                      q: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                      offsets: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """MX block-32 cast along the last dim: x (M, K) bf16, K % 32 == 0.
    mode MGS_MX_FLOOR (0) or MGS_MX_RCEIL (1). Returns q (M, K) uint8 E4M3
    and scales (M, K/32) uint8 E8M0."""
    _need(x, "x", _BF16_LIKE, 2)
    if mode not in (MGS_MX_FLOOR, MGS_MX_RCEIL):
        raise ValueError("mode must be MGS_MX_FLOOR or MGS_MX_RCEIL")
    M, K = x.shape
    q = _out(q, (M, K), torch.uint8, x.device, "q")
    scales = _out(scales, (M, K // 32), torch.uint8, x.device, "scales")
    off_ptr, G = (None, 0)
    if offsets is not None:
        _need(offsets, "offsets", (torch.int32,), 1)
        off_ptr, G = offsets.data_ptr(), offsets.shape[0]
    st = lib().mgs_mx_quant_dim0(x.data_ptr(), M, K, off_ptr, G, int(mode), q.data_ptr(),
                                 scales.data_ptr(), _stream_handle(stream, x))
    check("mgs_mx_quant_dim0", st)
    return q, scales


def mgs_mx_quant_dim1(x: torch.Tensor, mode: int = MGS_MX_FLOOR, q_t: Optional[torch.Tensor] = None,
                      scales_t: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """MX block-32 cast along dim0 with transposed outputs: x (M, K) bf16,
    M % 32 == 0. Returns q_t (K, M) uint8 E4M3 and scales_t (K, M/32) uint8
    E8M0 -- mgs_mx_quant_dim0 of x^T."""
    _need(x, "x", _BF16_LIKE, 2)
    M, K = x.shape
    q_t = _out(q_t, (K, M), torch.uint8, x.device, "q_t")
    scales_t = _out(scales_t, (K, M // 32), torch.uint8, x.device, "scales_t")
    st = lib().mgs_mx_quant_dim1(x.data_ptr(), M, K, int(mode), q_t.data_ptr(), scales_t.data_ptr(),
                                 _stream_handle(stream, x))
    check("mgs_mx_quant_dim1", st)
    return q_t, scales_t


def mgs_mx_dequant_dim0(q: torch.Tensor, scales: torch.Tensor, y: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """MX dequantisation: q (M, K) E4M3 bytes (uint8 or float8_e4m3fn),
    scales (M, K/32) E8M0 bytes. Returns y (M, K) bf16 (torch.bfloat16),
    y = E4M3(q) * 2^(byte - 127) rounded to nearest even."""
    _need(q, "q", (torch.uint8, torch.float8_e4m3fn), 2)
    _need(scales, "scales", (torch.uint8,), 2)
    M, K = q.shape
    if tuple(scales.shape) != (M, K // 32):
        raise ValueError("scales has shape %s, expected %s" % (tuple(scales.shape), (M, K // 32)))
    if y is None:
        y = torch.empty((M, K), dtype=torch.bfloat16, device=q.device)
    else:
        _need(y, "y", _BF16_LIKE, 2)
        if tuple(y.shape) != (M, K):
            raise ValueError("y has shape %s, expected %s" % (tuple(y.shape), (M, K)))
    st = lib().mgs_mx_dequant_dim0(q.data_ptr(), scales.data_ptr(), M, K, y.data_ptr(),
                                   _stream_handle(stream, q))
    check("mgs_mx_dequant_dim0", st)
    return y


def mgs_cast_e4m3(x: torch.Tensor, out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """E4M3 cast of a float32 tensor (numel % 4 == 0) with the library's cast."""
    _need(x, "x", (torch.float32,))
    out = _out(out, tuple(x.shape), torch.uint8, x.device, "out")
    st = lib().mgs_cast_e4m3(x.data_ptr(), x.numel(), out.data_ptr(), _stream_handle(stream, x))
    check("mgs_cast_e4m3", st)
    return out


def mgs_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> torch.Tensor:
    """Plain copy kernel (byte size % 16 == 0), for traffic calibration."""
    if src.device.type != "cuda" or dst.device.type != "cuda":
        raise ValueError("mgs_copy needs GPU tensors")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("mgs_copy needs contiguous tensors of equal byte size")
    st = lib().mgs_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream_handle(stream, src))
    check("mgs_copy", st)
    return dst


# Default wait bound and team limit for _test_quant_dim0 (below -1 and 0).
TEST_DEFAULT_SPIN = -2
TEST_DEFAULT_TEAM = 0


def _test_quant_dim0(x: torch.Tensor, offsets: Optional[torch.Tensor], q: torch.Tensor,
                     scales: torch.Tensor, pow2: bool = False, transposed: bool = False,
                     uniform_rows: int = -1, n_groups: Optional[int] = None,
                     spin_ticks: int = TEST_DEFAULT_SPIN, team_max: int = TEST_DEFAULT_TEAM,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Test-only: mgs_test_quant_dim0 (the dim0-family call with the wait
    bound and the team limit overridden). x is 2D (M, K); for equal groups
    pass offsets=None, uniform_rows and n_groups."""
    _need(x, "x", _BF16_LIKE, 2)
    M, K = x.shape
    if offsets is not None:
        _need(offsets, "offsets", (torch.int32,), 1)
        off_ptr, G = offsets.data_ptr(), offsets.shape[0]
    else:
        off_ptr, G = None, int(n_groups)
    wp, wb = _ws_args(workspace)
    st = lib().mgs_test_quant_dim0(x.data_ptr(), M, K, off_ptr, G, int(uniform_rows),
                                   MGS_FLAG_POW2_SCALE if pow2 else 0, 1 if transposed else 0,
                                   q.data_ptr(), scales.data_ptr(), wp, wb, int(spin_ticks),
                                   int(team_max), _stream_handle(stream, x))
    check("mgs_test_quant_dim0", st)
