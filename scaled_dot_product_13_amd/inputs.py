"""Seeded synthetic inputs for the attention workloads.

This module only draws random tensors and describes workload shapes; it
holds none of the attention arithmetic.  Both the GPU tests/benchmark and
the CPU oracle are fed from it.

Recipe: a torch CPU generator seeded with `seed` draws, in order,
(group mode only) the sequence lengths with randint(lo, hi+1), then
Q, K, V, [bias], dO as float32 standard normals, each then rounded to the io
dtype (round to nearest even).  Tensors are dense BHSD (batch mode) or packed
THD with cu_seqlens = [0, cumsum(lengths)] (group mode); K and V use the
same lengths unless explicit key/value lengths are given.

Quantized K/V (kv_quant = (group_size, with_zero_points[, format])): with
format "s8" (the default) K and V are int8 codes clip(round(40 z), -127,
127), z standard normal, with fp32 scales U(0.02, 0.03) per token and group
of head-dim elements (about what a per-group max-abs quantizer gives for
N(0, 1) data) and, optionally, int8 zero points randint(-8, 9); drawn in the
order codes K, scales K, [zero points K], codes V, scales V, [zero points V],
in place of the K and V normals.  With format "s4" the codes are
clip(round(3.5 z), -8, 7), with "u4" that plus 8, clipped to 0 .. 15, the
scales U(0.25, 0.32), and the codes are stored two per byte, code 2i in the
low nibble of byte i (uint8 tensors with a last dimension of d / 2).
"""
from dataclasses import dataclass, field
from typing import Optional

import torch

DROPOUT_SEED = 0x9E3779B97F4A7C15

_IO = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class Workload:
    name: str
    dtype: str
    b: int
    h: int
    s_q: int
    s_kv: int
    d_qk: int
    d_v: int
    causal: bool = False
    bias: bool = False
    dropout_p: float = 0.0
    seed: int = 0
    # group (varlen) mode: number of sequences and the length range
    varlen: Optional[tuple] = None  # (n_seq, lo, hi)
    scale: Optional[float] = None
    h_kv: Optional[int] = None  # key/value heads (grouped-query); None = h
    # mask band beyond top-left causal: key j is visible from row i iff
    # -window_left <= j - i - off <= window_right (None = unbounded side,
    # causal caps the right side at 0), off = s_kv - s_q with bottom_right
    bottom_right: bool = False
    window_left: Optional[int] = None
    window_right: Optional[int] = None
    kv_quant: Optional[tuple] = None  # (group_size, with_zero_points[, "s8" | "s4" | "u4"])
    extra: dict = field(default_factory=dict)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else self.d_qk ** -0.5


# The five workloads of the benchmark suite (seed 1000 + index).
WORKLOADS = {
    1: Workload("fp32 B1 H2 S128 d64", "f32", 1, 2, 128, 128, 64, 64, seed=1001),
    2: Workload("bf16 causal B4 H16 S2048 d128", "bf16", 4, 16, 2048, 2048, 128, 128,
                causal=True, seed=1002),
    3: Workload("fp16 bias B2 H32 Sq1024 Skv4096 dqk192 dv128", "f16", 2, 32, 1024, 4096,
                192, 128, bias=True, seed=1003),
    4: Workload("bf16 varlen 16 seqs L~U[64,4096] H16 d128 causal", "bf16", 16, 16, 4096, 4096,
                128, 128, causal=True, varlen=(16, 64, 4096), seed=1004),
    5: Workload("bf16 causal dropout0.1 B2 H16 S4096 d128", "bf16", 2, 16, 4096, 4096, 128, 128,
                causal=True, dropout_p=0.1, seed=1005),
}


# Thin-query (decode) workload: one new token per sequence attending to a
# long key/value cache, grouped-query heads (4 query heads per key/value
# head), bottom-right causal as a decoder step is.
DECODE = Workload("bf16 decode B16 H32 Hkv8 Sq1 Skv8192 d128", "bf16", 16, 32, 1, 8192, 128, 128,
                  causal=True, bottom_right=True, h_kv=8, seed=1006)
# The same step over an int8 K/V cache: scales per token and group of 32
# head-dim elements, no zero points.
DECODE_Q8 = Workload("bf16 decode int8-KV g32 B16 H32 Hkv8 Sq1 Skv8192 d128", "bf16", 16, 32, 1,
                     8192, 128, 128, causal=True, bottom_right=True, h_kv=8, seed=1007,
                     kv_quant=(32, False))
# And over a signed 4-bit K/V cache (two codes per byte), scales per token
# and group of 32 head-dim elements, no zero points.
DECODE_Q4 = Workload("bf16 decode int4-KV g32 B16 H32 Hkv8 Sq1 Skv8192 d128", "bf16", 16, 32, 1,
                     8192, 128, 128, causal=True, bottom_right=True, h_kv=8, seed=1008,
                     kv_quant=(32, False, "s4"))


def make_inputs(wl: Workload, lengths=None, kv_lengths=None):
    """Draw the workload's tensors on the CPU.  Returns a dict with
    q, k, v, dout, [bias], [lengths, cu_seqlens, max_seqlen and their _kv
    twins] and the io dtype."""
    g = torch.Generator().manual_seed(wl.seed)
    io = _IO[wl.dtype]
    out = {"dtype": io}
    if wl.varlen is not None:
        n, lo, hi = wl.varlen
        if lengths is None:
            lengths = torch.randint(lo, hi + 1, (n,), generator=g)
        else:
            lengths = torch.as_tensor(lengths, dtype=torch.int64)
        kv_lengths = lengths if kv_lengths is None else torch.as_tensor(kv_lengths, dtype=torch.int64)
        assert len(kv_lengths) == len(lengths)

        def cumulative(ls):
            cu = torch.zeros(len(ls) + 1, dtype=torch.int32)
            cu[1:] = torch.cumsum(ls, 0).to(torch.int32)
            return cu
        cu, cu_kv = cumulative(lengths), cumulative(kv_lengths)
        T, Tk = int(cu[-1]), int(cu_kv[-1])
        hk = wl.h_kv or wl.h
        shp_q, shp_k, shp_v, shp_o = (T, wl.h, wl.d_qk), (Tk, hk, wl.d_qk), (Tk, hk, wl.d_v), (T, wl.h, wl.d_v)
        out["lengths"] = lengths
        out["cu_seqlens"] = cu
        out["max_seqlen"] = int(lengths.max()) if len(lengths) else 0
        out["kv_lengths"] = kv_lengths
        out["cu_seqlens_kv"] = cu_kv
        out["max_seqlen_kv"] = int(kv_lengths.max()) if len(kv_lengths) else 0
    else:
        hk = wl.h_kv or wl.h
        shp_q = (wl.b, wl.h, wl.s_q, wl.d_qk)
        shp_k = (wl.b, hk, wl.s_kv, wl.d_qk)
        shp_v = (wl.b, hk, wl.s_kv, wl.d_v)
        shp_o = (wl.b, wl.h, wl.s_q, wl.d_v)
    out["q"] = torch.randn(shp_q, generator=g, dtype=torch.float32).to(io)
    if wl.kv_quant is None:
        out["k"] = torch.randn(shp_k, generator=g, dtype=torch.float32).to(io)
        out["v"] = torch.randn(shp_v, generator=g, dtype=torch.float32).to(io)
    else:
        gs, with_zp = wl.kv_quant[:2]
        fmt = wl.kv_quant[2] if len(wl.kv_quant) > 2 else "s8"
        for name, shp in (("k", shp_k), ("v", shp_v)):
            z = torch.randn(shp, generator=g, dtype=torch.float32)
            sshp = shp[:-1] + (shp[-1] // gs,)
            if fmt == "s8":
                out[name] = torch.clamp(torch.round(40.0 * z), -127, 127).to(torch.int8)
                out[name + "_scales"] = 0.02 + 0.01 * torch.rand(sshp, generator=g, dtype=torch.float32)
            else:
                c = torch.round(3.5 * z)
                c = torch.clamp(c, -8, 7) if fmt == "s4" else torch.clamp(c + 8, 0, 15)
                nib = (c.to(torch.int64) & 15).to(torch.uint8)  # storage: low nibble first
                out[name] = nib[..., 0::2] | (nib[..., 1::2] << 4)
                out[name + "_scales"] = 0.25 + 0.07 * torch.rand(sshp, generator=g, dtype=torch.float32)
            out[name + "_zp"] = (torch.randint(-8, 9, sshp, generator=g).to(torch.int8)
                                 if with_zp else None)
    if wl.bias:
        out["bias"] = torch.randn((wl.b, wl.h, wl.s_q, wl.s_kv), generator=g,
                                  dtype=torch.float32).to(io)
    out["dout"] = torch.randn(shp_o, generator=g, dtype=torch.float32).to(io)
    return out


def small(dtype="bf16", b=1, h=2, s_q=200, s_kv=200, d_qk=128, d_v=128, causal=False,
          bias=False, dropout_p=0.0, seed=7, varlen=None, scale=None, h_kv=None,
          bottom_right=False, window_left=None, window_right=None, kv_quant=None) -> Workload:
    """A small workload (parity-test size) with the same recipe."""
    return Workload(f"small-{dtype}", dtype, b, h, s_q, s_kv, d_qk, d_v, causal=causal, bias=bias,
                    dropout_p=dropout_p, seed=seed, varlen=varlen, scale=scale, h_kv=h_kv,
                    bottom_right=bottom_right, window_left=window_left,
                    window_right=window_right, kv_quant=kv_quant)
