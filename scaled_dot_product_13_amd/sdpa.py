"""Thin ctypes binding of libsdpa.so (include/sdpa.h), same entry-point names.

Argument marshalling only: torch tensors supply device memory, strides and
the current HIP stream; every step of the computation runs in the library's
HIP kernels.  There is no fallback: if libsdpa.so is missing this module
raises on import.

Output allocation follows PyTorch's cuDNN attention glue ("MHA.cpp",
alloc_with_matching_layout): outputs take the stride order of the
corresponding input; dO is made unit-stride in its last dimension
(permute_to_matching_layout / the bprop stride fix).
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsdpa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} not found: build it first (python -m scaled_dot_product_13_amd.build "
        "or __graft_entry__.build()); there is no fallback implementation")

SDPA_OK, SDPA_ERR_INVALID_ARG, SDPA_ERR_UNSUPPORTED, SDPA_ERR_WORKSPACE, SDPA_ERR_HIP = range(5)
SDPA_F32, SDPA_F16, SDPA_BF16 = 0, 1, 2
_DTYPES = {torch.float32: SDPA_F32, torch.float16: SDPA_F16, torch.bfloat16: SDPA_BF16}


class Strides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("seq", ctypes.c_int64)]


class Problem(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("dtype", ctypes.c_int),
        ("b", ctypes.c_int64), ("h", ctypes.c_int64),
        ("s_q", ctypes.c_int64), ("s_kv", ctypes.c_int64),
        ("d_qk", ctypes.c_int64), ("d_v", ctypes.c_int64),
        ("scaling_factor", ctypes.c_float), ("is_causal", ctypes.c_int32),
        ("dropout_probability", ctypes.c_float),
        ("dropout_seed", ctypes.c_uint64), ("dropout_offset", ctypes.c_uint64),
        ("dropout_seed_offset_dev", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_kv", ctypes.c_void_p),
        ("h_kv", ctypes.c_int64),
        ("mask_flags", ctypes.c_uint32), ("window_left", ctypes.c_int64),
        ("window_right", ctypes.c_int64),
        ("alibi_slopes", ctypes.c_void_p), ("alibi_batch_stride", ctypes.c_int64),
        ("kv_quant", ctypes.c_int32), ("kv_group_size", ctypes.c_int32),
        ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
        ("k_zero_points", ctypes.c_void_p), ("v_zero_points", ctypes.c_void_p),
        ("kv_scale_strides", Strides),
        ("total_q", ctypes.c_int64),
    ]


MASK_BOTTOM_RIGHT = 1
MASK_WINDOW = 2


_lib = ctypes.CDLL(LIB_PATH)
_vp, _sz = ctypes.c_void_p, ctypes.c_size_t
_P = ctypes.POINTER(Problem)
_lib.sdpa_fwd_workspace_size.argtypes = [_P]
_lib.sdpa_fwd_workspace_size.restype = _sz
_lib.sdpa_bwd_workspace_size.argtypes = [_P]
_lib.sdpa_bwd_workspace_size.restype = _sz
_lib.sdpa_fwd.argtypes = [_P, _vp, Strides, _vp, Strides, _vp, Strides, _vp, Strides,
                          _vp, Strides, _vp, _vp, _vp, _sz, _vp]
_lib.sdpa_fwd.restype = ctypes.c_int
_lib.sdpa_bwd.argtypes = [_P, _vp, Strides, _vp, Strides, _vp, Strides, _vp, Strides,
                          _vp, Strides, _vp, Strides, _vp, _vp, Strides, _vp, Strides,
                          _vp, Strides, _vp, Strides, _vp, _sz, _vp]
_lib.sdpa_bwd.restype = ctypes.c_int
_lib.sdpa_bwd_noalloc.argtypes = [_P, _vp, Strides, _vp, Strides, _vp, Strides, _vp, Strides,
                                  _vp, Strides, _vp, Strides, _vp, _vp, Strides, _vp, Strides,
                                  _vp, Strides, _vp, Strides, _vp]
_lib.sdpa_bwd_noalloc.restype = ctypes.c_int
_lib.sdpa_bwd_preprocess.argtypes = [_P, _vp, Strides, _vp, Strides, _vp, _vp, _vp]
_lib.sdpa_bwd_preprocess.restype = ctypes.c_int
_lib.sdpa_bwd_dkdv.argtypes = [_P, _vp, Strides, _vp, Strides, _vp, Strides, _vp, Strides,
                               _vp, Strides, _vp, _vp, Strides, _vp, Strides, _vp, Strides, _vp]
_lib.sdpa_bwd_dkdv.restype = ctypes.c_int
_lib.sdpa_bwd_dq.argtypes = [_P, _vp, Strides, _vp, Strides, _vp, Strides, _vp, Strides,
                             _vp, Strides, _vp, _vp, Strides, _vp]
_lib.sdpa_bwd_dq.restype = ctypes.c_int
_lib.sdpa_bwd_dq_preprocess.argtypes = [_P, _vp, Strides, _vp, Strides, _vp, Strides, _vp, Strides,
                                        _vp, Strides, _vp, Strides, _vp, _vp, _vp, Strides, _vp]
_lib.sdpa_bwd_dq_preprocess.restype = ctypes.c_int
_lib.sdpa_status_string.argtypes = [ctypes.c_int]
_lib.sdpa_status_string.restype = ctypes.c_char_p
_lib.sdpa_last_error_message.restype = ctypes.c_char_p
_lib.sdpa_version.restype = ctypes.c_char_p


class SdpaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_lib.sdpa_status_string(status).decode()}: {message}")
        self.status = status


def _check(status):
    if status != SDPA_OK:
        raise SdpaError(status, _lib.sdpa_last_error_message().decode())


def version() -> str:
    return _lib.sdpa_version().decode()


def lib():
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides(t, group):
    if t is None:
        return Strides(0, 0, 0)
    s = t.stride()
    if group:  # [T, H, D]
        return Strides(0, s[1], s[0])
    return Strides(s[0], s[1], s[2])


def _alloc_like(ref, shape, dtype=None):
    """Allocate `shape` with the stride order of `ref` (same rank)."""
    order = sorted(range(ref.dim()), key=lambda i: -ref.stride(i))
    perm_shape = [shape[i] for i in order]
    out = torch.empty(perm_shape, dtype=dtype or ref.dtype, device=ref.device)
    inv = [0] * len(order)
    for pos, i in enumerate(order):
        inv[i] = pos
    return out.permute(inv)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


KV_QUANT = {"s8": 1, "s4": 2, "u4": 3}  # SDPA_KV_QUANT_S8 / _S4 / _U4


def _check_operands(q, k=None, v=None, *, quant_kv=None, cu=(), same=()):
    """Raise TypeError unless every operand is on q's device with q's dtype
    (k, v: int8 codes for quant_kv "s8", uint8 bytes of two 4-bit codes for
    "s4" / "u4") and every cu_seqlens array is a contiguous int32 tensor
    there: the library reads raw bytes, so a wrong dtype would otherwise give
    wrong results with no error."""
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("k", k), ("v", v)):
        if t is None:
            continue
        want = (q.dtype if quant_kv is None else torch.int8 if quant_kv == "s8" else torch.uint8)
        if t.dtype != want or t.device != q.device:
            raise TypeError(f"{name} must be {want} on {q.device}, got {t.dtype} on {t.device}")
    for name, t in same:
        if t is not None and (t.dtype != q.dtype or t.device != q.device):
            raise TypeError(f"{name} must be {q.dtype} on {q.device}, got {t.dtype} on {t.device}")
    for name, t in cu:
        if t is not None and (t.dtype != torch.int32 or t.device != q.device or not t.is_contiguous()):
            raise TypeError(f"{name} must be a contiguous int32 tensor on {q.device}")


def make_problem(q, k, v, *, scale=None, causal=False, dropout_p=0.0, seed=0, offset=0,
                 seed_offset=None, cu_seqlens_q=None, cu_seqlens_kv=None, max_seqlen_q=None,
                 max_seqlen_kv=None, bottom_right=False, window_left=None, window_right=None,
                 alibi_slopes=None, kv_scales=None, kv_zero_points=None, kv_group_size=None,
                 kv_format=None):
    """Fill the C problem struct from tensor shapes (batch [B,H,S,D] or group
    [T,H,D]); k and v may have fewer heads than q (grouped-query attention).

    Mask: row i sees key j iff -window_left <= j - i - off <= window_right
    (a window side that is None is unbounded; causal caps window_right at 0),
    off = s_kv - s_q per sequence with bottom_right, else 0.

    alibi_slopes: fp32 device tensor [B, H] (or [H], shared by the batch);
    adds -slope |j - i - off'| to the scores, off' the mask's alignment
    (bottom-right without a mask).  The tensor must outlive the call.

    Quantized K/V: kv_scales = (k_scales, v_scales), fp32 [.., tokens,
    d / kv_group_size] laid out like k without its last dimension (batch
    [B, Hkv, S, G] or group [T, Hkv, G]); kv_zero_points likewise int8, or
    None.  k and v are int8 codes (kv_format "s8", the default for int8
    tensors) or uint8 tensors of packed 4-bit codes, two per byte with the
    low nibble first (kv_format "s4" signed or "u4" unsigned; the last
    dimension is then d / 2)."""
    fmt = None
    if kv_scales is not None:
        fmt = kv_format or ("s8" if k.dtype == torch.int8 else None)
        if fmt not in KV_QUANT:
            raise TypeError("kv_format must be 's8', 's4' or 'u4' (uint8 K/V need 's4' or 'u4')")
    _check_operands(q, k, v, quant_kv=fmt,
                    cu=(("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_kv", cu_seqlens_kv)))
    if seed_offset is not None and (seed_offset.dtype not in (torch.int64, torch.uint64)
                                    or seed_offset.numel() < 2 or seed_offset.device != q.device):
        raise TypeError("seed_offset must hold two 64-bit integers on q's device")
    group = cu_seqlens_q is not None
    p = Problem()
    p.struct_size = ctypes.sizeof(Problem)
    p.dtype = _DTYPES[q.dtype]
    if group:
        p.b = cu_seqlens_q.numel() - 1
        p.h = q.shape[1]
        p.s_q = int(max_seqlen_q)
        p.s_kv = int(max_seqlen_kv)
        p.d_qk, p.d_v = q.shape[2], v.shape[2]
        p.cu_seqlens_q = cu_seqlens_q.data_ptr()
        p.cu_seqlens_kv = cu_seqlens_kv.data_ptr()
        p.total_q = q.shape[0]  # the LSE is [H, q.shape[0]]
    else:
        p.b, p.h, p.s_q, p.d_qk = q.shape
        p.s_kv, p.d_v = k.shape[2], v.shape[3]
    p.h_kv = k.shape[1]
    p.scaling_factor = float(scale if scale is not None else 1.0 / math.sqrt(p.d_qk))
    p.is_causal = 1 if causal else 0
    windowed = window_left is not None or window_right is not None
    p.mask_flags = (MASK_BOTTOM_RIGHT if bottom_right else 0) | (MASK_WINDOW if windowed else 0)
    p.window_left = -1 if window_left is None else int(window_left)
    p.window_right = -1 if window_right is None else int(window_right)
    if alibi_slopes is not None:
        if (alibi_slopes.dtype != torch.float32 or alibi_slopes.stride(-1) != 1
                or alibi_slopes.device != q.device):
            raise TypeError("alibi_slopes must be a float32 tensor on q's device with unit "
                            "stride along heads")
        p.alibi_slopes = alibi_slopes.data_ptr()
        p.alibi_batch_stride = alibi_slopes.stride(0) if alibi_slopes.dim() == 2 else 0
    if kv_scales is not None:
        ks, vs = kv_scales
        if (ks.dtype != torch.float32 or vs.dtype != torch.float32 or ks.stride() != vs.stride()
                or ks.device != q.device or vs.device != q.device):
            raise TypeError("kv_scales: two float32 tensors on q's device with equal strides")
        p.kv_quant = KV_QUANT[fmt]
        if fmt != "s8":
            p.d_v = 2 * v.shape[-1]  # two codes per byte
        p.kv_group_size = int(kv_group_size)
        p.k_scales, p.v_scales = ks.data_ptr(), vs.data_ptr()
        p.kv_scale_strides = _strides(ks, group)
        if kv_zero_points is not None:
            kz, vz = kv_zero_points
            if (kz.stride() != ks.stride() or vz.stride() != ks.stride()
                    or kz.dtype != torch.int8 or vz.dtype != torch.int8
                    or kz.device != q.device or vz.device != q.device):
                raise TypeError("kv_zero_points must be int8 on q's device with the strides of "
                                "kv_scales")
            p.k_zero_points, p.v_zero_points = kz.data_ptr(), vz.data_ptr()
    p.dropout_probability = float(dropout_p)
    p.dropout_seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    p.dropout_offset = int(offset) & 0xFFFFFFFFFFFFFFFF
    p.dropout_seed_offset_dev = seed_offset.data_ptr() if seed_offset is not None else None
    return p


def sdpa_fwd(q, k, v, *, bias=None, scale=None, causal=False, dropout_p=0.0, seed=0, offset=0,
             seed_offset=None, cu_seqlens_q=None, cu_seqlens_kv=None, max_seqlen_q=None,
             max_seqlen_kv=None, return_lse=True, return_keep=False, out=None, lse=None,
             bottom_right=False, window_left=None, window_right=None, split_kv=True,
             workspace=None, alibi_slopes=None, kv_scales=None, kv_zero_points=None,
             kv_group_size=None, kv_format=None):
    """Forward.  Returns (o, lse or None, keep or None).  split_kv=False
    passes no workspace, so a thin-query problem runs unsplit; `workspace`
    (uint8, at least fwd_workspace_size bytes) avoids an allocation."""
    group = cu_seqlens_q is not None
    p = make_problem(q, k, v, scale=scale, causal=causal, dropout_p=dropout_p, seed=seed,
                     offset=offset, seed_offset=seed_offset, cu_seqlens_q=cu_seqlens_q,
                     cu_seqlens_kv=cu_seqlens_kv, max_seqlen_q=max_seqlen_q,
                     max_seqlen_kv=max_seqlen_kv, bottom_right=bottom_right,
                     window_left=window_left, window_right=window_right,
                     alibi_slopes=alibi_slopes, kv_scales=kv_scales,
                     kv_zero_points=kv_zero_points, kv_group_size=kv_group_size,
                     kv_format=kv_format)
    _check_operands(q, same=(("bias", bias), ("out", out)))
    if lse is not None and (lse.dtype != torch.float32 or lse.device != q.device):
        raise TypeError("lse must be float32 on q's device")
    if out is None:
        oshape = list(q.shape)
        oshape[-1] = p.d_v
        out = _alloc_like(q, oshape)
    if return_lse and lse is None:
        lse = (torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device) if group
               else torch.empty((p.b, p.h, p.s_q), dtype=torch.float32, device=q.device))
    keep = None
    if return_keep:
        keep = torch.zeros((p.b, p.h, p.s_q, p.s_kv), dtype=torch.uint8, device=q.device)
    ws_n = _lib.sdpa_fwd_workspace_size(ctypes.byref(p)) if split_kv else 0
    if workspace is not None and workspace.numel() >= ws_n:
        ws = workspace
    else:
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device) if ws_n else None
    _check(_lib.sdpa_fwd(ctypes.byref(p), _ptr(q), _strides(q, group), _ptr(k), _strides(k, group),
                         _ptr(v), _strides(v, group), _ptr(bias), _strides(bias, False),
                         _ptr(out), _strides(out, group), _ptr(lse if return_lse else None),
                         _ptr(keep), _ptr(ws), ws_n, _stream()))
    return out, (lse if return_lse else None), keep


def sdpa_bwd(q, k, v, o, dout, lse, *, bias=None, scale=None, causal=False, dropout_p=0.0,
             seed=0, offset=0, seed_offset=None, cu_seqlens_q=None, cu_seqlens_kv=None,
             max_seqlen_q=None, max_seqlen_kv=None, want_dbias=False, workspace=None,
             bottom_right=False, window_left=None, window_right=None, alibi_slopes=None):
    """Backward.  Returns (dq, dk, dv, dbias or None)."""
    group = cu_seqlens_q is not None
    p = make_problem(q, k, v, scale=scale, causal=causal, dropout_p=dropout_p, seed=seed,
                     offset=offset, seed_offset=seed_offset, cu_seqlens_q=cu_seqlens_q,
                     cu_seqlens_kv=cu_seqlens_kv, max_seqlen_q=max_seqlen_q,
                     max_seqlen_kv=max_seqlen_kv, bottom_right=bottom_right,
                     window_left=window_left, window_right=window_right,
                     alibi_slopes=alibi_slopes)
    _check_operands(q, same=(("o", o), ("dout", dout), ("bias", bias)))
    if lse.dtype != torch.float32 or lse.device != q.device:
        raise TypeError("lse must be float32 on q's device")
    if dout.stride(-1) != 1:
        dout = dout.contiguous()
    dq, dk, dv = _alloc_like(q, q.shape), _alloc_like(k, k.shape), _alloc_like(v, v.shape)
    dbias = _alloc_like(bias, bias.shape) if (want_dbias and bias is not None) else None
    ws_n = _lib.sdpa_bwd_workspace_size(ctypes.byref(p))
    if workspace is None or workspace.numel() < ws_n:
        workspace = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
    _check(_lib.sdpa_bwd(ctypes.byref(p), _ptr(q), _strides(q, group), _ptr(k), _strides(k, group),
                         _ptr(v), _strides(v, group), _ptr(bias), _strides(bias, False),
                         _ptr(o), _strides(o, group), _ptr(dout), _strides(dout, group), _ptr(lse),
                         _ptr(dq), _strides(dq, group), _ptr(dk), _strides(dk, group),
                         _ptr(dv), _strides(dv, group), _ptr(dbias), _strides(dbias, False),
                         _ptr(workspace), workspace.numel(), _stream()))
    return dq, dk, dv, dbias


NOALLOC_MAX_ROWS = 1 << 20  # SDPA_NOALLOC_MAX_ROWS


def sdpa_bwd_noalloc(q, k, v, o, dout, lse, *, bias=None, dq=None, dk=None, dv=None, dbias=None,
                     want_dbias=False, **kw):
    """Backward through sdpa_bwd_noalloc: no workspace, the library's own
    per-GPU stats array instead (b*h*s_q <= NOALLOC_MAX_ROWS; calls on one
    GPU must not overlap).  Pass preallocated dq, dk, dv (and dbias) for a
    call that allocates nothing.  Returns (dq, dk, dv, dbias or None)."""
    group = kw.get("cu_seqlens_q") is not None
    p = make_problem(q, k, v, **kw)
    _check_operands(q, same=(("o", o), ("dout", dout), ("bias", bias), ("dq", dq), ("dk", dk),
                             ("dv", dv), ("dbias", dbias)))
    if lse.dtype != torch.float32 or lse.device != q.device:
        raise TypeError("lse must be float32 on q's device")
    if dout.stride(-1) != 1:
        raise TypeError("dout must have unit stride in its last dimension")
    dq = _alloc_like(q, q.shape) if dq is None else dq
    dk = _alloc_like(k, k.shape) if dk is None else dk
    dv = _alloc_like(v, v.shape) if dv is None else dv
    if want_dbias and bias is not None and dbias is None:
        dbias = _alloc_like(bias, bias.shape)
    _check(_lib.sdpa_bwd_noalloc(ctypes.byref(p), _ptr(q), _strides(q, group), _ptr(k),
                                 _strides(k, group), _ptr(v), _strides(v, group), _ptr(bias),
                                 _strides(bias, False), _ptr(o), _strides(o, group), _ptr(dout),
                                 _strides(dout, group), _ptr(lse), _ptr(dq), _strides(dq, group),
                                 _ptr(dk), _strides(dk, group), _ptr(dv), _strides(dv, group),
                                 _ptr(dbias), _strides(dbias, False), _stream()))
    return dq, dk, dv, dbias


def fwd_workspace_size(q, k, v, **kw):
    """Bytes of forward workspace for these tensors and options (see
    make_problem); nonzero only for split-KV thin-query problems."""
    return _lib.sdpa_fwd_workspace_size(ctypes.byref(make_problem(q, k, v, **kw)))


def bwd_workspace_size(q, k, v, **kw):
    """Bytes of backward workspace for these tensors and options (see
    make_problem)."""
    return _lib.sdpa_bwd_workspace_size(ctypes.byref(make_problem(q, k, v, **kw)))


def stats_layout(b, h, s_q):
    """(n, offset) of the backward stats: D at [0, n), LSE*log2(e) at
    [offset, offset + n) floats (offset = n rounded up to 64 floats)."""
    n = b * h * s_q
    return n, (n + 63) // 64 * 64


def sdpa_bwd_preprocess(o, dout, lse, *, cu_seqlens_q=None, max_seqlen_q=None, out=None):
    """Backward stats: a flat fp32 tensor holding D = rowsum(dO o O) and
    LSE*log2(e) (see stats_layout); returns it.  D alone is
    stats[:n] viewed as [B,H,S_q] (group mode [H, B*max_seqlen_q])."""
    _check_operands(o, same=(("dout", dout),), cu=(("cu_seqlens_q", cu_seqlens_q),))
    group = cu_seqlens_q is not None
    p = Problem()
    p.struct_size = ctypes.sizeof(Problem)
    p.dtype = _DTYPES[o.dtype]
    if group:
        p.b = cu_seqlens_q.numel() - 1
        p.h, p.d_v = o.shape[1], o.shape[2]
        p.s_q = p.s_kv = int(max_seqlen_q)
        p.cu_seqlens_q = p.cu_seqlens_kv = cu_seqlens_q.data_ptr()
        p.total_q = o.shape[0]
    else:
        p.b, p.h, p.s_q, p.d_v = o.shape
        p.s_kv = 1
    p.d_qk = p.d_v
    p.scaling_factor = 1.0
    n, off = stats_layout(p.b, p.h, p.s_q)
    d = out if out is not None else torch.empty(off + n, dtype=torch.float32, device=o.device)
    assert d.numel() >= off + n and d.dtype == torch.float32 and d.is_contiguous()
    _check(_lib.sdpa_bwd_preprocess(ctypes.byref(p), _ptr(o), _strides(o, group), _ptr(dout),
                                    _strides(dout, group), _ptr(lse), _ptr(d), _stream()))
    return d


def sdpa_bwd_dkdv(q, k, v, dout, stats, *, bias=None, dk=None, dv=None, dbias=None,
                  want_dbias=False, **kw):
    """dK, dV (and dBias) from the backward stats.  Returns (dk, dv, dbias)."""
    group = kw.get("cu_seqlens_q") is not None
    p = make_problem(q, k, v, **kw)
    _check_operands(q, same=(("dout", dout), ("bias", bias), ("dbias", dbias)))
    dk = _alloc_like(k, k.shape) if dk is None else dk
    dv = _alloc_like(v, v.shape) if dv is None else dv
    if want_dbias and bias is not None and dbias is None:
        dbias = _alloc_like(bias, bias.shape)
    _check(_lib.sdpa_bwd_dkdv(ctypes.byref(p), _ptr(q), _strides(q, group), _ptr(k), _strides(k, group),
                              _ptr(v), _strides(v, group), _ptr(bias), _strides(bias, False),
                              _ptr(dout), _strides(dout, group), _ptr(stats),
                              _ptr(dk), _strides(dk, group), _ptr(dv), _strides(dv, group),
                              _ptr(dbias), _strides(dbias, False), _stream()))
    return dk, dv, dbias


def sdpa_bwd_dq_preprocess(q, k, v, o, dout, lse, *, bias=None, dq=None, stats=None, **kw):
    """dQ and, for the same rows, the backward stats in one kernel (16-bit io).
    Returns (dq, stats); run sdpa_bwd_dkdv on the stats afterwards."""
    group = kw.get("cu_seqlens_q") is not None
    p = make_problem(q, k, v, **kw)
    _check_operands(q, same=(("o", o), ("dout", dout), ("bias", bias), ("dq", dq)))
    dq = _alloc_like(q, q.shape) if dq is None else dq
    n, off = stats_layout(p.b, p.h, p.s_q)
    if stats is None:
        stats = torch.empty(off + n, dtype=torch.float32, device=q.device)
    assert stats.numel() >= off + n and stats.dtype == torch.float32 and stats.is_contiguous()
    _check(_lib.sdpa_bwd_dq_preprocess(ctypes.byref(p), _ptr(q), _strides(q, group), _ptr(k),
                                       _strides(k, group), _ptr(v), _strides(v, group), _ptr(bias),
                                       _strides(bias, False), _ptr(o), _strides(o, group),
                                       _ptr(dout), _strides(dout, group), _ptr(lse), _ptr(stats),
                                       _ptr(dq), _strides(dq, group), _stream()))
    return dq, stats


def sdpa_bwd_dq(q, k, v, dout, stats, *, bias=None, dq=None, **kw):
    """dQ from the backward stats.  Returns dq."""
    group = kw.get("cu_seqlens_q") is not None
    p = make_problem(q, k, v, **kw)
    _check_operands(q, same=(("dout", dout), ("bias", bias), ("dq", dq)))
    dq = _alloc_like(q, q.shape) if dq is None else dq
    _check(_lib.sdpa_bwd_dq(ctypes.byref(p), _ptr(q), _strides(q, group), _ptr(k), _strides(k, group),
                            _ptr(v), _strides(v, group), _ptr(bias), _strides(bias, False),
                            _ptr(dout), _strides(dout, group), _ptr(stats),
                            _ptr(dq), _strides(dq, group), _stream()))
    return dq
