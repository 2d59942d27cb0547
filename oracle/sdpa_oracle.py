"""ctypes front end of the fp64 CPU oracle (sdpa_oracle.c).

TEST INFRASTRUCTURE ONLY.  The test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers; the GPU library and its
Python binding never import this module.

Layouts (all float64 numpy arrays, C-contiguous):
  batch mode:   q [B,H,S_q,d_qk]  k [B,H,S_kv,d_qk]  v [B,H,S_kv,d_v]
                bias [B,H,S_q,S_kv]  dout/o [B,H,S_q,d_v]  lse/D [B,H,S_q]
  varlen mode:  q [T_q,H,d_qk]  k [T_kv,H,d_qk]  v [T_kv,H,d_v]
                dout/o [T_q,H,d_v]  lse/D [H,T_q]
                with cu_seqlens_q / cu_seqlens_kv int arrays of length n+1.
In varlen mode the dropout counter's batch index is the sequence index.

`heads` optionally restricts the work to a list of (b, h) pairs; outputs of
the other heads are left as NaN so a test cannot mistake them for results.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


class _Head(ctypes.Structure):
    _fields_ = [
        ("sq", ctypes.c_int64), ("skv", ctypes.c_int64),
        ("dqk", ctypes.c_int64), ("dv", ctypes.c_int64),
        ("scale", ctypes.c_double), ("causal", ctypes.c_int32),
        ("p_drop", ctypes.c_float),
        ("seed", ctypes.c_uint64), ("offset", ctypes.c_uint64),
        ("bh", ctypes.c_uint32),
        ("q", _dp), ("k", _dp), ("v", _dp), ("bias", _dp), ("dout", _dp),
        ("ld_q", ctypes.c_int64), ("ld_k", ctypes.c_int64),
        ("ld_v", ctypes.c_int64), ("ld_bias", ctypes.c_int64),
        ("ld_do", ctypes.c_int64),
        ("o", _dp), ("lse", _dp), ("dq", _dp), ("dk", _dp), ("dv_out", _dp),
        ("dbias", _dp), ("dvec", _dp),
        ("ld_o", ctypes.c_int64), ("ld_dq", ctypes.c_int64),
        ("ld_dk", ctypes.c_int64), ("ld_dv", ctypes.c_int64),
        ("ld_dbias", ctypes.c_int64),
        ("keep", ctypes.POINTER(ctypes.c_uint8)), ("ld_keep", ctypes.c_int64),
        ("band", ctypes.c_int32), ("band_off", ctypes.c_int64),
        ("band_lo", ctypes.c_int64), ("band_hi", ctypes.c_int64),
        ("alibi", ctypes.c_int32), ("alibi_slope", ctypes.c_double),
        ("alibi_off", ctypes.c_int64),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        _lib = ctypes.CDLL(_LIB_PATH)
        _lib.oracle_fwd.argtypes = [ctypes.POINTER(_Head), ctypes.c_int64, ctypes.c_int]
        _lib.oracle_bwd.argtypes = [ctypes.POINTER(_Head), ctypes.c_int64, ctypes.c_int]
        _lib.oracle_philox4x32_10.argtypes = [ctypes.POINTER(ctypes.c_uint32)] * 3
        _lib.oracle_keep_bit.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32,
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
        _lib.oracle_keep_bit.restype = ctypes.c_int
        _lib.oracle_drop_threshold.argtypes = [ctypes.c_float]
        _lib.oracle_drop_threshold.restype = ctypes.c_int
        _lib.oracle_max_threads.restype = ctypes.c_int
    return _lib


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def philox4x32_10(counter, key):
    """Philox4x32-10 block function: 4 counter words, 2 key words -> 4 words."""
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in counter])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    o = (ctypes.c_uint32 * 4)()
    lib().oracle_philox4x32_10(c, k, o)
    return [int(x) for x in o]


def drop_threshold(p: float) -> int:
    return int(lib().oracle_drop_threshold(ctypes.c_float(p)))


def keep_bit(seed, offset, bh, i, j, p):
    return int(lib().oracle_keep_bit(seed, offset, bh, i, j, drop_threshold(p)))


def _ptr(a, off=0):
    if a is None:
        return ctypes.cast(None, _dp)
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return ctypes.cast(a.ctypes.data + 8 * off, _dp)


def _as64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


_UNBOUNDED = 1 << 62


def _band(causal, bottom_right, window_left, window_right):
    """(lo, hi) of the visible band j - i - off, or None for the plain
    (unmasked or top-left causal) cases."""
    if not bottom_right and window_left is None and window_right is None:
        return None
    lo = -int(window_left) if window_left is not None else -_UNBOUNDED
    hi = int(window_right) if window_right is not None else _UNBOUNDED
    if causal:
        hi = min(hi, 0)
    return lo, hi


def _heads(q, k, v, bias, dout, outs, *, scale, causal, p_drop, seed, offset,
           cu_q, cu_kv, select, band=None, bottom_right=False, alibi=None):
    """Build the list of head descriptors for batch or varlen layout."""
    heads = []
    keep = outs.get("keep")
    if cu_q is None:
        B, H, Sq, Dqk = q.shape
        Skv, Dv = k.shape[2], v.shape[3]
        pairs = select if select is not None else [(b, h) for b in range(B) for h in range(H)]
        for (b, h) in pairs:
            hd = _Head()
            hd.sq, hd.skv, hd.dqk, hd.dv = Sq, Skv, Dqk, Dv
            base_q = ((b * H + h) * Sq)
            base_k = ((b * H + h) * Skv)
            hd.q, hd.ld_q = _ptr(q, base_q * Dqk), Dqk
            hd.k, hd.ld_k = _ptr(k, base_k * Dqk), Dqk
            hd.v, hd.ld_v = _ptr(v, base_k * Dv), Dv
            hd.bias, hd.ld_bias = (_ptr(bias, base_q * Skv), Skv) if bias is not None else (_ptr(None), 0)
            hd.dout, hd.ld_do = (_ptr(dout, base_q * Dv), Dv) if dout is not None else (_ptr(None), 0)
            hd.o, hd.ld_o = (_ptr(outs["o"], base_q * Dv), Dv) if "o" in outs else (_ptr(None), 0)
            hd.lse = _ptr(outs["lse"], base_q) if "lse" in outs else _ptr(None)
            hd.dvec = _ptr(outs["D"], base_q) if "D" in outs else _ptr(None)
            if "dq" in outs:
                hd.dq, hd.ld_dq = _ptr(outs["dq"], base_q * Dqk), Dqk
                hd.dk, hd.ld_dk = _ptr(outs["dk"], base_k * Dqk), Dqk
                hd.dv_out, hd.ld_dv = _ptr(outs["dv"], base_k * Dv), Dv
            if "dbias" in outs:
                hd.dbias, hd.ld_dbias = _ptr(outs["dbias"], base_q * Skv), Skv
            if keep is not None:
                hd.keep = ctypes.cast(keep.ctypes.data + base_q * Skv, ctypes.POINTER(ctypes.c_uint8))
                hd.ld_keep = Skv
            hd.bh = b * H + h
            heads.append(hd)
    else:
        Tq, H, Dqk = q.shape
        Tkv = k.shape[0]
        Dv = v.shape[2]
        n = len(cu_q) - 1
        pairs = select if select is not None else [(b, h) for b in range(n) for h in range(H)]
        for (b, h) in pairs:
            sq0, sq1 = int(cu_q[b]), int(cu_q[b + 1])
            sk0, sk1 = int(cu_kv[b]), int(cu_kv[b + 1])
            hd = _Head()
            hd.sq, hd.skv, hd.dqk, hd.dv = sq1 - sq0, sk1 - sk0, Dqk, Dv
            hd.q, hd.ld_q = _ptr(q, (sq0 * H + h) * Dqk), H * Dqk
            hd.k, hd.ld_k = _ptr(k, (sk0 * H + h) * Dqk), H * Dqk
            hd.v, hd.ld_v = _ptr(v, (sk0 * H + h) * Dv), H * Dv
            assert bias is None, "bias with varlen is not part of the method's varlen mode here"
            hd.bias = _ptr(None)
            hd.dout, hd.ld_do = (_ptr(dout, (sq0 * H + h) * Dv), H * Dv) if dout is not None else (_ptr(None), 0)
            hd.o, hd.ld_o = (_ptr(outs["o"], (sq0 * H + h) * Dv), H * Dv) if "o" in outs else (_ptr(None), 0)
            hd.lse = _ptr(outs["lse"], h * Tq + sq0) if "lse" in outs else _ptr(None)
            hd.dvec = _ptr(outs["D"], h * Tq + sq0) if "D" in outs else _ptr(None)
            if "dq" in outs:
                hd.dq, hd.ld_dq = _ptr(outs["dq"], (sq0 * H + h) * Dqk), H * Dqk
                hd.dk, hd.ld_dk = _ptr(outs["dk"], (sk0 * H + h) * Dqk), H * Dqk
                hd.dv_out, hd.ld_dv = _ptr(outs["dv"], (sk0 * H + h) * Dv), H * Dv
            hd.bh = b * H + h
            heads.append(hd)
    if alibi is not None:
        # (slopes [B, H], alignment bottom-right?) for each head descriptor
        slopes, align_br = alibi
        for hd, (b, h) in zip(heads, pairs):
            hd.alibi = 1
            hd.alibi_slope = float(slopes[b, h])
            hd.alibi_off = hd.skv - hd.sq if align_br else 0
    for hd in heads:
        hd.scale = float(scale)
        hd.causal = 1 if causal else 0
        if band is not None:
            hd.band = 1
            hd.band_off = hd.skv - hd.sq if bottom_right else 0
            hd.band_lo, hd.band_hi = band
        hd.p_drop = float(p_drop)
        hd.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
        hd.offset = int(offset) & 0xFFFFFFFFFFFFFFFF
    return heads


def _alibi(alibi_slopes, n_batch, n_heads, causal, bottom_right, window_left, window_right):
    """(slopes [B, H], bottom-right alignment) for the ALiBi term, or None.
    A slope vector [H] is shared by every batch entry.  The alignment is the
    mask's (bottom-right or top-left) and bottom-right when there is no mask,
    as CK builds its position encoding from the mask or, without one, from
    the bottom-right corner."""
    if alibi_slopes is None:
        return None
    sl = np.asarray(alibi_slopes, dtype=np.float64)
    if sl.ndim == 1:
        sl = np.broadcast_to(sl, (n_batch, n_heads))
    assert sl.shape == (n_batch, n_heads)
    masked = causal or window_left is not None or window_right is not None
    return sl, (bottom_right or not masked)


def unpack_int4(packed, signed):
    """4-bit codes from bytes holding two codes each: code 2i of a row is the
    low nibble of byte i, code 2i + 1 its high nibble (the low-nibble-first
    packing of sub-byte data types in oneDNN's memory descriptors, which the
    micro SDPA host driver accepts for key / value quantization).  Signed
    codes are 4-bit two's complement (-8 .. 7), unsigned codes 0 .. 15.
    packed uint8 [..., D / 2] -> int64 [..., D]."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    lo, hi = b & 0xF, (b >> 4) & 0xF
    codes = np.stack([lo, hi], axis=-1).reshape(b.shape[:-1] + (2 * b.shape[-1],))
    if signed:
        codes = np.where(codes >= 8, codes - 16, codes)
    return codes


def dequantize_kv(codes, scales, group_size, zero_points=None):
    """K or V from 8-bit integer codes with one scale (and optionally one
    integer zero point) per token and per group of `group_size` consecutive
    head-dim elements: x_c = (code_c - zp_{c // g}) * scale_{c // g}.  This is
    the grouped key / value quantization of the oneDNN micro SDPA host driver
    (key scales grouped along the head dimension per key, value scales
    grouped along the head dimension per value row, zero points subtracted
    before scaling).  codes [..., D]; scales, zero_points [..., D / g]."""
    x = np.asarray(codes, dtype=np.float64)
    d = x.shape[-1]
    assert d % group_size == 0 and scales.shape[-1] == d // group_size
    if zero_points is not None:
        x = x - np.repeat(np.asarray(zero_points, dtype=np.float64), group_size, axis=-1)
    return x * np.repeat(np.asarray(scales, dtype=np.float64), group_size, axis=-1)


def _run(fn, heads, threads):
    arr = (_Head * len(heads))(*heads)
    getattr(lib(), fn)(arr, len(heads), int(threads))


def _kv_ratio(q, k, group):
    """Query heads per key/value head (grouped-query attention).  Query head h
    reads key/value head h // ratio: Composable Kernel's i_nhead /
    nhead_ratio_qk in FmhaBwdDQDKDVKernel's pointer set-up; oneDNN's
    kv_group_size = query heads / key-value heads in init_conf_common."""
    ax = 1
    hq, hk = q.shape[ax], k.shape[ax]
    assert hq % hk == 0, "query heads must be a multiple of key/value heads"
    return hq // hk


def _repeat_kv(t, r):
    """Key/value tensor with each head repeated r times along the head axis,
    so that query head h sees head h // r (plain grouped-query definition)."""
    return t if r == 1 else np.repeat(t, r, axis=1)


def _sum_groups(t, r, complete):
    """Per-query-head gradient [.., H, ..] summed over each group of r
    consecutive heads (ascending order, fp64) into [.., H/r, ..].  Groups
    with a head outside `complete` are NaN."""
    if r == 1:
        return t
    shp = list(t.shape)
    shp[1:2] = [shp[1] // r, r]
    out = np.zeros(shp[:2] + shp[3:])
    tt = t.reshape(shp)
    for j in range(r):
        out += tt[:, :, j]
    for hk in range(out.shape[1]):
        if not complete(hk):
            out[:, hk] = np.nan
    return out


def fwd(q, k, v, *, scale, causal=False, bias=None, p_drop=0.0, seed=0, offset=0,
        cu_seqlens_q=None, cu_seqlens_kv=None, heads=None, threads=0, want_keep=False,
        bottom_right=False, window_left=None, window_right=None, alibi_slopes=None):
    """Forward definition.  Returns dict(o=..., lse=..., [keep=...]).
    k and v may have fewer heads than q (grouped-query attention).  The mask
    is top-left causal, or with bottom_right / window_left / window_right the
    band lo <= j - i - off <= hi described in the C source.  alibi_slopes
    ([B, H] or [H]) adds -slope |j - i - off| to the scores in place of a
    bias (see _alibi for the alignment)."""
    q, k, v, bias = _as64(q), _as64(k), _as64(v), _as64(bias)
    r = _kv_ratio(q, k, cu_seqlens_q is not None)
    k, v = np.ascontiguousarray(_repeat_kv(k, r)), np.ascontiguousarray(_repeat_kv(v, r))
    if cu_seqlens_q is None:
        B, H, Sq, _ = q.shape
        outs = {"o": np.full((B, H, Sq, v.shape[3]), np.nan),
                "lse": np.full((B, H, Sq), np.nan)}
        if want_keep:
            outs["keep"] = np.zeros((B, H, Sq, k.shape[2]), dtype=np.uint8)
    else:
        assert not want_keep
        Tq, H, _ = q.shape
        outs = {"o": np.full((Tq, H, v.shape[2]), np.nan),
                "lse": np.full((H, Tq), np.nan)}
    hs = _heads(q, k, v, bias, None, outs, scale=scale, causal=causal, p_drop=p_drop,
                seed=seed, offset=offset, cu_q=cu_seqlens_q, cu_kv=cu_seqlens_kv, select=heads,
                band=_band(causal, bottom_right, window_left, window_right),
                bottom_right=bottom_right,
                alibi=_alibi(alibi_slopes, q.shape[0] if cu_seqlens_q is None else len(cu_seqlens_q) - 1,
                             q.shape[1], causal, bottom_right, window_left, window_right))
    _run("oracle_fwd", hs, threads)
    return outs


def bwd(q, k, v, dout, *, scale, causal=False, bias=None, p_drop=0.0, seed=0, offset=0,
        cu_seqlens_q=None, cu_seqlens_kv=None, heads=None, threads=0, want_dbias=None,
        bottom_right=False, window_left=None, window_right=None, alibi_slopes=None):
    """Backward definition (recomputes O and LSE itself).

    Returns dict(o, lse, D, dq, dk, dv[, dbias]).  With fewer key/value heads
    than query heads, dk and dv of key/value head hk are the sums of the
    per-query-head gradients over its group (NaN for groups only partly in
    `heads`)."""
    q, k, v, bias, dout = _as64(q), _as64(k), _as64(v), _as64(bias), _as64(dout)
    r = _kv_ratio(q, k, cu_seqlens_q is not None)
    k, v = np.ascontiguousarray(_repeat_kv(k, r)), np.ascontiguousarray(_repeat_kv(v, r))
    if want_dbias is None:
        want_dbias = bias is not None
    if cu_seqlens_q is None:
        B, H, Sq, _ = q.shape
        Skv = k.shape[2]
        outs = {"o": np.full((B, H, Sq, v.shape[3]), np.nan),
                "lse": np.full((B, H, Sq), np.nan), "D": np.full((B, H, Sq), np.nan),
                "dq": np.full(q.shape, np.nan), "dk": np.full(k.shape, np.nan),
                "dv": np.full(v.shape, np.nan)}
        if want_dbias:
            outs["dbias"] = np.full((B, H, Sq, Skv), np.nan)
    else:
        Tq, H, _ = q.shape
        outs = {"o": np.full((Tq, H, v.shape[2]), np.nan),
                "lse": np.full((H, Tq), np.nan), "D": np.full((H, Tq), np.nan),
                "dq": np.full(q.shape, np.nan), "dk": np.full(k.shape, np.nan),
                "dv": np.full(v.shape, np.nan)}
    hs = _heads(q, k, v, bias, dout, outs, scale=scale, causal=causal, p_drop=p_drop,
                seed=seed, offset=offset, cu_q=cu_seqlens_q, cu_kv=cu_seqlens_kv, select=heads,
                band=_band(causal, bottom_right, window_left, window_right),
                bottom_right=bottom_right,
                alibi=_alibi(alibi_slopes, q.shape[0] if cu_seqlens_q is None else len(cu_seqlens_q) - 1,
                             q.shape[1], causal, bottom_right, window_left, window_right))
    _run("oracle_bwd", hs, threads)
    if r > 1:
        nb = q.shape[0] if cu_seqlens_q is None else len(cu_seqlens_q) - 1
        sel = None if heads is None else set(heads)
        def complete(hk):
            return sel is None or all((b, hk * r + j) in sel for b in range(nb) for j in range(r))
        if cu_seqlens_q is None:
            outs["dk"] = _sum_groups(outs["dk"], r, complete)
            outs["dv"] = _sum_groups(outs["dv"], r, complete)
        else:  # [T, H, D]: heads on axis 1 as well
            outs["dk"] = _sum_groups(outs["dk"], r, complete)
            outs["dv"] = _sum_groups(outs["dv"], r, complete)
    return outs
