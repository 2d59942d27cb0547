"""Pins of the fp64 CPU oracle against facts that do not come from the oracle.

Every test here runs on the CPU.  What pins what:
  - Philox4x32-10: published known-answer vectors, and rocRAND's engine run
    on the host.
  - keep mask: drop-rate statistics, seed/offset sensitivity, p = 0 identity.
  - forward: closed forms (S_kv = 1, Q = 0, causal prefix means), key
    permutation invariance, and torch's float64 scaled_dot_product_attention
    library routine; LSE against torch.logsumexp.
  - backward: central finite differences of L = sum(dO o O) through the
    oracle's own forward, torch float64 autograd of the forward, and
    invariants (row sums of dS vanish, sum_j dK_j = 0, sum_j dV_j = sum_i dO_i).
  - group mode: equals batch mode run sequence by sequence.
  - quantized K/V: per-group symmetric int8 quantization of real data
    dequantizes to within half a step (the rounding bound); shifting codes
    and zero points together changes nothing; unit scales are the identity.
  - ALiBi: slope 0 is the plain forward; a very steep slope leaves only the
    key on the aligned diagonal (O_i = V_{i+off}); under a top-left causal
    mask it equals a per-key bias slope * j (the -slope * i part is constant
    along a row and cancels in the softmax); central differences.
  - mutation check: deliberately broken builds of the oracle fail the pins.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle.sdpa_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- Philox ----
def _kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            v = [int(x, 16) for x in line.split()]
            rows.append((v[0:4], v[4:6], v[6:10]))
    return rows


def test_philox_known_answers():
    rows = _kat()
    assert len(rows) == 3
    for ctr, key, want in rows:
        assert O.philox4x32_10(ctr, key) == want


def test_philox_matches_rocrand_engine(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "rpc"
    r = subprocess.run([hipcc, "-O1", os.path.join(ROOT, "tests", "rocrand_philox_check.cpp"),
                        "-o", str(exe)], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("rocRAND header not usable: " + r.stderr[-300:])
    rng = np.random.default_rng(5)
    cases = []
    for _ in range(64):
        c = [int(rng.integers(0, 2**32)), int(rng.integers(0, 2**30)),
             int(rng.integers(0, 2**32)), int(rng.integers(0, 2**32))]
        k = [int(rng.integers(0, 2**32)), int(rng.integers(0, 2**32))]
        cases.append((c, k))
    inp = "".join("%x %x %x %x %x %x\n" % (*c, *k) for c, k in cases)
    out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout
    got = [[int(x, 16) for x in line.split()] for line in out.strip().splitlines()]
    for (c, k), g in zip(cases, got):
        assert O.philox4x32_10(c, k) == g


def test_drop_threshold_values():
    assert O.drop_threshold(0.0) == 0
    assert O.drop_threshold(0.1) == 26       # round(25.6)
    assert O.drop_threshold(0.5) == 128
    assert O.drop_threshold(0.999) == 255


def test_keep_bit_layout_reproduces_known_answer_bytes():
    """The keep decision's position-to-byte mapping, pinned bit for bit to
    the Random123 known-answer vectors.  Each KAT counter (c0, c1, c2, c3)
    and key (k0, k1) is read as key position j = 4 c0 + (j & 3), query
    position i = 4 c1 + (i & 3), head index b*H + h = c2, offset = c3 and
    seed = k0 + 2^32 k1.  For every (i & 3, j & 3) the random byte is
    recovered by sweeping the drop threshold t = round(256 p) over 0..255
    (p = t / 256): the element is kept iff byte >= t, so the byte is the
    largest t that still keeps it.  It must equal byte (j & 3) of output
    word (i & 3).  Swapping i and j, or the word and byte indices, fails."""
    for ctr, key, want in _kat():
        seed = key[0] | (key[1] << 32)
        for ii in range(4):
            for jj in range(4):
                i, j = 4 * ctr[1] + ii, 4 * ctr[0] + jj
                kept = [O.keep_bit(seed, ctr[3], ctr[2], i, j, t / 256.0) for t in range(256)]
                assert kept[0] == 1
                byte = max(t for t in range(256) if kept[t])
                # monotone: kept exactly for t <= byte
                assert kept == [1] * (byte + 1) + [0] * (255 - byte)
                assert byte == (want[ii] >> (8 * jj)) & 0xFF, (ctr, ii, jj)


def test_keep_mask_statistics_and_sensitivity():
    B, H, S = 1, 2, 256
    q = _rand((B, H, S, 16), 1)
    k = _rand((B, H, S, 16), 2)
    v = _rand((B, H, S, 16), 3)
    seed = 0x9E3779B97F4A7C15
    r0 = O.fwd(q, k, v, scale=0.25, p_drop=0.1, seed=seed, offset=0, want_keep=True)["keep"]
    n = r0.size
    rate = 1.0 - r0.mean()
    p = 26 / 256
    assert abs(rate - p) < 6 * math.sqrt(p * (1 - p) / n)
    r1 = O.fwd(q, k, v, scale=0.25, p_drop=0.1, seed=seed, offset=1, want_keep=True)["keep"]
    r2 = O.fwd(q, k, v, scale=0.25, p_drop=0.1, seed=seed + 1, offset=0, want_keep=True)["keep"]
    # independent masks disagree on about 2 p (1 - p) of the elements
    for other in (r1, r2):
        frac = (other != r0).mean()
        assert abs(frac - 2 * p * (1 - p)) < 0.02
    # the two heads use different counters
    assert (r0[0, 0] != r0[0, 1]).mean() > 0.1


def test_dropout_zero_is_identity():
    q, k, v = _rand((1, 2, 37, 8), 4), _rand((1, 2, 41, 8), 5), _rand((1, 2, 41, 6), 6)
    a = O.fwd(q, k, v, scale=0.3, p_drop=0.0)
    b = O.fwd(q, k, v, scale=0.3)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])


# ------------------------------------------------------- forward pins -------
def test_single_key_gives_v():
    q, k, v = _rand((2, 3, 9, 5), 7), _rand((2, 3, 1, 5), 8), _rand((2, 3, 1, 4), 9)
    bias = _rand((2, 3, 9, 1), 10)
    r = O.fwd(q, k, v, scale=0.7, bias=bias)
    assert np.allclose(r["o"], np.broadcast_to(v, r["o"].shape), atol=1e-12, rtol=0)
    s00 = 0.7 * np.einsum("bhid,bhjd->bhij", q, k)[..., 0] + bias[..., 0]
    assert np.allclose(r["lse"], s00, atol=1e-12, rtol=0)


def test_zero_query_gives_mean_of_values():
    q = np.zeros((1, 2, 7, 5))
    k, v = _rand((1, 2, 11, 5), 11), _rand((1, 2, 11, 3), 12)
    r = O.fwd(q, k, v, scale=0.5)
    assert np.allclose(r["o"], v.mean(axis=2, keepdims=True).repeat(7, axis=2), atol=1e-12, rtol=0)
    assert np.allclose(r["lse"], math.log(11), atol=1e-12, rtol=0)


def test_causal_zero_query_gives_prefix_means():
    q = np.zeros((1, 1, 9, 4))
    k, v = _rand((1, 1, 9, 4), 13), _rand((1, 1, 9, 3), 14)
    r = O.fwd(q, k, v, scale=0.5, causal=True)
    want = np.cumsum(v, axis=2) / np.arange(1, 10)[None, None, :, None]
    assert np.allclose(r["o"], want, atol=1e-12, rtol=0)
    assert np.allclose(r["lse"][0, 0], np.log(np.arange(1, 10)), atol=1e-12, rtol=0)
    # row 0 sees only key 0
    assert np.allclose(r["o"][0, 0, 0], v[0, 0, 0], atol=1e-15)


def test_causal_with_more_keys_than_queries_is_top_left():
    q, k, v = _rand((1, 1, 4, 3), 15), _rand((1, 1, 9, 3), 16), _rand((1, 1, 9, 2), 17)
    r = O.fwd(q, k, v, scale=1.0, causal=True)
    # row i of a top-left causal mask sees keys 0..i only
    for i in range(4):
        sub = O.fwd(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], scale=1.0)
        assert np.allclose(r["o"][0, 0, i], sub["o"][0, 0, 0], atol=1e-14)


def test_key_permutation_invariance():
    q, k, v = _rand((1, 2, 13, 6), 18), _rand((1, 2, 17, 6), 19), _rand((1, 2, 17, 5), 20)
    perm = np.random.default_rng(21).permutation(17)
    a = O.fwd(q, k, v, scale=0.4)
    b = O.fwd(q, k[:, :, perm], v[:, :, perm], scale=0.4)
    assert np.allclose(a["o"], b["o"], atol=1e-12, rtol=0)
    assert np.allclose(a["lse"], b["lse"], atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("with_bias", [False, True])
def test_forward_matches_torch_sdpa_float64(causal, with_bias):
    B, H, Sq, Skv, Dq, Dv = 2, 3, 19, 23 if not causal else 19, 7, 5
    q, k, v = _rand((B, H, Sq, Dq), 22), _rand((B, H, Skv, Dq), 23), _rand((B, H, Skv, Dv), 24)
    bias = _rand((B, H, Sq, Skv), 25) if with_bias else None
    scale = 0.37
    r = O.fwd(q, k, v, scale=scale, causal=causal, bias=bias)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    mask = None
    if with_bias:
        mask = torch.from_numpy(bias)
    if causal and with_bias:
        tri = torch.ones(Sq, Skv, dtype=torch.bool).tril()
        mask = mask.masked_fill(~tri, float("-inf"))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    else:
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                               is_causal=causal, scale=scale)
    assert np.allclose(r["o"], ref.numpy(), atol=1e-12, rtol=0)
    s = scale * torch.einsum("bhid,bhjd->bhij", tq, tk)
    if with_bias:
        s = s + torch.from_numpy(bias)
    if causal:
        s = s.masked_fill(~torch.ones(Sq, Skv, dtype=torch.bool).tril(), float("-inf"))
    assert np.allclose(r["lse"], torch.logsumexp(s, -1).numpy(), atol=1e-12, rtol=0)


def test_dropout_applies_scaled_keep_mask_after_normalisation():
    B, H, S, D = 1, 2, 21, 6
    q, k, v = _rand((B, H, S, D), 26), _rand((B, H, S, D), 27), _rand((B, H, S, D), 28)
    p = 0.3
    r = O.fwd(q, k, v, scale=0.5, causal=True, p_drop=p, seed=99, offset=3, want_keep=True)
    plain = O.fwd(q, k, v, scale=0.5, causal=True)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    s = 0.5 * torch.einsum("bhid,bhjd->bhij", tq, tk)
    s = s.masked_fill(~torch.ones(S, S, dtype=torch.bool).tril(), float("-inf"))
    P = torch.softmax(s, -1)
    keep = torch.from_numpy(r["keep"].astype(np.float64))
    z = keep / (1.0 - np.float64(np.float32(p)))
    assert np.allclose(r["o"], (P * z @ tv).numpy(), atol=1e-12, rtol=0)
    assert np.array_equal(r["lse"], plain["lse"])  # LSE from the undropped P


# ------------------------------------------------------ backward pins -------
def _loss(q, k, v, dout, bias, **kw):
    return float(np.sum(O.fwd(q, k, v, bias=bias, **kw)["o"] * dout))


@pytest.mark.parametrize("causal,with_bias,p", [(False, False, 0.0), (True, False, 0.0),
                                                 (False, True, 0.0), (True, True, 0.25)])
def test_backward_central_differences(causal, with_bias, p):
    B, H, Sq, Skv, Dq, Dv = 1, 2, 5, 7 if not causal else 5, 3, 4
    q, k, v = _rand((B, H, Sq, Dq), 30), _rand((B, H, Skv, Dq), 31), _rand((B, H, Skv, Dv), 32)
    dout = _rand((B, H, Sq, Dv), 33)
    bias = _rand((B, H, Sq, Skv), 34) if with_bias else None
    kw = dict(scale=0.6, causal=causal, p_drop=p, seed=5, offset=0)
    g = O.bwd(q, k, v, dout, bias=bias, **kw)
    eps = 1e-6
    targets = [("dq", q), ("dk", k), ("dv", v)] + ([("dbias", bias)] if with_bias else [])
    for name, x in targets:
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(q, k, v, dout, bias, **kw)
            x[idx] = old - eps
            lm = _loss(q, k, v, dout, bias, **kw)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(num - g[name])) / max(1e-3, np.max(np.abs(num)))
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("causal,with_bias,p", [(False, True, 0.0), (True, False, 0.0),
                                                 (True, True, 0.2)])
def test_backward_matches_torch_autograd_float64(causal, with_bias, p):
    B, H, Sq, Skv, Dq, Dv = 2, 2, 11, 13 if not causal else 11, 5, 4
    q, k, v = _rand((B, H, Sq, Dq), 40), _rand((B, H, Skv, Dq), 41), _rand((B, H, Skv, Dv), 42)
    dout = _rand((B, H, Sq, Dv), 43)
    bias = _rand((B, H, Sq, Skv), 44) if with_bias else None
    scale = 0.45
    kw = dict(scale=scale, causal=causal, p_drop=p, seed=77, offset=9)
    g = O.bwd(q, k, v, dout, bias=bias, **kw)
    keep = O.fwd(q, k, v, bias=bias, want_keep=True, **kw)["keep"] if p > 0 else None
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    tb = torch.tensor(bias, requires_grad=True) if with_bias else None
    s = scale * tq @ tk.transpose(-1, -2)
    if with_bias:
        s = s + tb
    if causal:
        s = s.masked_fill(~torch.ones(Sq, Skv, dtype=torch.bool).tril(), float("-inf"))
    P = torch.softmax(s, -1)
    if p > 0:
        P = P * (torch.from_numpy(keep.astype(np.float64)) / (1.0 - np.float64(np.float32(p))))
    out = P @ tv
    out.backward(torch.from_numpy(dout))
    assert np.allclose(g["o"], out.detach().numpy(), atol=1e-12, rtol=0)
    assert np.allclose(g["dq"], tq.grad.numpy(), atol=1e-10, rtol=0)
    assert np.allclose(g["dk"], tk.grad.numpy(), atol=1e-10, rtol=0)
    assert np.allclose(g["dv"], tv.grad.numpy(), atol=1e-10, rtol=0)
    if with_bias:
        assert np.allclose(g["dbias"], tb.grad.numpy(), atol=1e-10, rtol=0)


@pytest.mark.parametrize("hkv,causal,with_bias,p", [(1, True, False, 0.0), (2, False, True, 0.0),
                                                     (2, True, False, 0.25)])
def test_grouped_query_heads_match_torch_autograd_float64(hkv, causal, with_bias, p):
    # grouped-query attention: query head h reads key/value head h // (H/hkv);
    # torch composes it with index_select along heads, whose autograd sums
    # the gradient over each group
    B, H, Sq, Skv, Dq, Dv = 2, 4, 9, 12 if not causal else 9, 5, 3
    q, dout = _rand((B, H, Sq, Dq), 60), _rand((B, H, Sq, Dv), 63)
    k, v = _rand((B, hkv, Skv, Dq), 61), _rand((B, hkv, Skv, Dv), 62)
    bias = _rand((B, H, Sq, Skv), 64) if with_bias else None
    scale = 0.5
    kw = dict(scale=scale, causal=causal, p_drop=p, seed=17, offset=4)
    g = O.bwd(q, k, v, dout, bias=bias, **kw)
    assert g["dk"].shape == k.shape and g["dv"].shape == v.shape
    keep = O.fwd(q, k, v, bias=bias, want_keep=True, **kw)["keep"] if p > 0 else None
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    idx = torch.arange(H) // (H // hkv)
    kk, vv = tk.index_select(1, idx), tv.index_select(1, idx)
    s = scale * tq @ kk.transpose(-1, -2)
    if with_bias:
        s = s + torch.from_numpy(bias)
    if causal:
        s = s.masked_fill(~torch.ones(Sq, Skv, dtype=torch.bool).tril(), float("-inf"))
    P = torch.softmax(s, -1)
    if p > 0:
        P = P * (torch.from_numpy(keep.astype(np.float64)) / (1.0 - np.float64(np.float32(p))))
    out = P @ vv
    out.backward(torch.from_numpy(dout))
    assert np.allclose(g["o"], out.detach().numpy(), atol=1e-12, rtol=0)
    assert np.allclose(g["dq"], tq.grad.numpy(), atol=1e-10, rtol=0)
    assert np.allclose(g["dk"], tk.grad.numpy(), atol=1e-10, rtol=0)
    assert np.allclose(g["dv"], tv.grad.numpy(), atol=1e-10, rtol=0)


def test_grouped_query_heads_central_differences():
    # MQA (one key/value head for three query heads), causal, on a tiny shape
    B, H, S, Dq, Dv = 1, 3, 4, 3, 2
    q, dout = _rand((B, H, S, Dq), 70), _rand((B, H, S, Dv), 73)
    k, v = _rand((B, 1, S, Dq), 71), _rand((B, 1, S, Dv), 72)
    kw = dict(scale=0.7, causal=True)
    g = O.bwd(q, k, v, dout, **kw)
    eps = 1e-6
    for name, x in (("dk", k), ("dv", v), ("dq", q)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + eps
            lp = _loss(q, k, v, dout, None, **kw)
            x[i] = old - eps
            lm = _loss(q, k, v, dout, None, **kw)
            x[i] = old
            num[i] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(num - g[name])) / max(1e-3, np.max(np.abs(num)))
        assert err < 1e-6, (name, err)


# ------------------------------------------------------------ band masks ----
def test_bottom_right_causal_is_top_left_when_square():
    q, k, v = _rand((1, 2, 9, 4), 80), _rand((1, 2, 9, 4), 81), _rand((1, 2, 9, 3), 82)
    a = O.fwd(q, k, v, scale=0.5, causal=True)
    b = O.fwd(q, k, v, scale=0.5, causal=True, bottom_right=True)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])


def test_bottom_right_causal_equals_last_rows_of_a_longer_query():
    # Rows are independent: bottom-right alignment of s_q queries against
    # s_kv keys is top-left causal attention of a query sequence extended to
    # s_kv rows (any values in the extra leading rows), keeping the last s_q.
    Sq, Skv = 5, 11
    q, k, v = _rand((1, 2, Sq, 4), 83), _rand((1, 2, Skv, 4), 84), _rand((1, 2, Skv, 3), 85)
    qq = np.concatenate([_rand((1, 2, Skv - Sq, 4), 86), q], axis=2)
    a = O.fwd(q, k, v, scale=0.6, causal=True, bottom_right=True)
    b = O.fwd(qq, k, v, scale=0.6, causal=True)
    assert np.allclose(a["o"], b["o"][:, :, Skv - Sq:], atol=1e-12, rtol=0)
    assert np.allclose(a["lse"], b["lse"][:, :, Skv - Sq:], atol=1e-12, rtol=0)


def test_bottom_right_rows_without_keys():
    # s_q > s_kv: the first s_q - s_kv rows see no key (O = 0, LSE = -inf, no gradient)
    Sq, Skv = 7, 4
    q, do = _rand((1, 1, Sq, 3), 87), _rand((1, 1, Sq, 2), 88)
    k, v = _rand((1, 1, Skv, 3), 89), _rand((1, 1, Skv, 2), 90)
    g = O.bwd(q, k, v, do, scale=0.5, causal=True, bottom_right=True)
    n = Sq - Skv
    assert np.all(g["o"][0, 0, :n] == 0) and np.all(np.isneginf(g["lse"][0, 0, :n]))
    assert np.all(g["dq"][0, 0, :n] == 0)
    assert np.isfinite(g["lse"][0, 0, n:]).all()


@pytest.mark.parametrize("wl,wr,causal", [(2, None, True), (1, 2, False), (0, 0, False),
                                          (None, 1, False)])
def test_sliding_window_rows_are_softmax_over_their_key_slice(wl, wr, causal):
    # each row's output is plain softmax attention over exactly the keys in
    # its window, computed row by row with torch on the sliced K, V
    Sq, Skv, scale = 8, 8, 0.7
    q, k, v = _rand((1, 1, Sq, 4), 91), _rand((1, 1, Skv, 4), 92), _rand((1, 1, Skv, 3), 93)
    r = O.fwd(q, k, v, scale=scale, causal=causal, window_left=wl, window_right=wr)
    for i in range(Sq):
        lo = 0 if wl is None else max(0, i - wl)
        hi = Skv - 1 if wr is None else min(Skv - 1, i + wr)
        if causal:
            hi = min(hi, i)
        tq = torch.from_numpy(q[0, 0, i:i + 1])
        tk, tv = torch.from_numpy(k[0, 0, lo:hi + 1]), torch.from_numpy(v[0, 0, lo:hi + 1])
        s = scale * tq @ tk.T
        assert np.allclose(r["o"][0, 0, i], (torch.softmax(s, -1) @ tv).numpy()[0], atol=1e-12, rtol=0)
        assert np.isclose(r["lse"][0, 0, i], torch.logsumexp(s, -1).item(), atol=1e-12, rtol=0)


def test_unbounded_window_is_the_plain_mask():
    q, k, v = _rand((1, 2, 9, 4), 94), _rand((1, 2, 12, 4), 95), _rand((1, 2, 12, 3), 96)
    a = O.fwd(q, k, v, scale=0.5, causal=True)
    b = O.fwd(q, k, v, scale=0.5, causal=True, window_left=100)
    c = O.fwd(q, k, v, scale=0.5)
    d = O.fwd(q, k, v, scale=0.5, window_left=50, window_right=50)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(c["o"], d["o"])


def test_band_backward_central_differences():
    B, H, Sq, Skv, Dq, Dv = 1, 1, 5, 7, 3, 2
    q, k, v = _rand((B, H, Sq, Dq), 97), _rand((B, H, Skv, Dq), 98), _rand((B, H, Skv, Dv), 99)
    dout = _rand((B, H, Sq, Dv), 100)
    kw = dict(scale=0.6, causal=True, bottom_right=True, window_left=2)
    g = O.bwd(q, k, v, dout, **kw)
    eps = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + eps
            lp = _loss(q, k, v, dout, None, **kw)
            x[i] = old - eps
            lm = _loss(q, k, v, dout, None, **kw)
            x[i] = old
            num[i] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(num - g[name])) / max(1e-3, np.max(np.abs(num)))
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("p", [0.0, 0.3])
def test_backward_invariants(p):
    B, H, S, D = 1, 3, 29, 8
    q, k, v, dout = (_rand((B, H, S, D), 50 + i) for i in range(4))
    bias = _rand((B, H, S, S), 55)
    g = O.bwd(q, k, v, dout, bias=bias, scale=0.3, causal=True, p_drop=p, seed=3)
    # softmax shift invariance: every row of dS sums to zero
    assert np.allclose(g["dbias"].sum(-1), 0.0, atol=1e-12)
    # hence sum over keys of dK vanishes
    assert np.allclose(g["dk"].sum(2), 0.0, atol=1e-11)
    if p == 0.0:
        # rows of P sum to one: sum_j dV_j = sum_i dO_i
        assert np.allclose(g["dv"].sum(2), dout.sum(2), atol=1e-11)
    # D from the backward equals rowsum(dO o O) with O from the forward
    f = O.fwd(q, k, v, bias=bias, scale=0.3, causal=True, p_drop=p, seed=3)
    assert np.allclose(g["D"], np.sum(dout * f["o"], -1), atol=1e-12, rtol=0)
    assert np.allclose(g["lse"], f["lse"], atol=0, rtol=0)


# ----------------------------------------------------------------- ALiBi ----
def test_alibi_zero_slope_is_the_plain_forward():
    B, H, Sq, Skv, D = 2, 3, 9, 13, 8
    q, k, v = _rand((B, H, Sq, D), 201), _rand((B, H, Skv, D), 202), _rand((B, H, Skv, D), 203)
    for kw in (dict(), dict(causal=True), dict(causal=True, bottom_right=True, window_left=3)):
        a = O.fwd(q, k, v, scale=0.4, alibi_slopes=np.zeros((B, H)), **kw)
        b = O.fwd(q, k, v, scale=0.4, **kw)
        assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"]), kw


@pytest.mark.parametrize("causal,bottom_right,sq,skv", [(False, False, 7, 12), (True, False, 9, 9),
                                                       (True, True, 6, 11), (False, False, 10, 10)])
def test_alibi_steep_slope_keeps_only_the_diagonal_key(causal, bottom_right, sq, skv):
    # with slope >> |scores| every row's weight sits on the key j = i + off:
    # bottom-right without a mask (off = s_kv - s_q), the mask's alignment
    # otherwise
    B, H, D = 1, 2, 5
    q, k, v = _rand((B, H, sq, D), 211, 0.1), _rand((B, H, skv, D), 212, 0.1), _rand((B, H, skv, D), 213)
    slope = 80.0
    f = O.fwd(q, k, v, scale=0.5, causal=causal, bottom_right=bottom_right,
              alibi_slopes=np.full(H, slope))
    off = skv - sq if (bottom_right or not causal) else 0
    for i in range(sq):
        j = i + off
        assert 0 <= j < skv
        assert np.allclose(f["o"][0, :, i], v[0, :, j], atol=1e-12, rtol=0), i
        s_diag = 0.5 * np.einsum("hd,hd->h", q[0, :, i], k[0, :, j])
        assert np.allclose(f["lse"][0, :, i], s_diag, atol=1e-12, rtol=0), i


def test_alibi_top_left_causal_is_a_per_key_bias():
    # -slope (i - j) = slope j - slope i on the visible keys j <= i; the
    # second term is constant along a row
    B, H, S, D = 2, 2, 11, 6
    q, k, v, dout = (_rand((B, H, S, D), 221 + i) for i in range(4))
    slopes = np.array([[0.3, 1.1], [0.05, 0.7]])
    a = O.bwd(q, k, v, dout, scale=0.45, causal=True, alibi_slopes=slopes)
    key_bias = np.broadcast_to(slopes[:, :, None, None] * np.arange(S)[None, None, None, :],
                               (B, H, S, S)).copy()
    b = O.bwd(q, k, v, dout, scale=0.45, causal=True, bias=key_bias, want_dbias=False)
    for name in ("o", "dq", "dk", "dv"):
        assert np.allclose(a[name], b[name], atol=1e-12, rtol=1e-12), name
    row_const = slopes[:, :, None] * np.arange(S)[None, None, :]
    assert np.allclose(a["lse"], b["lse"] - row_const, atol=1e-12, rtol=0)


def test_alibi_backward_central_differences():
    B, H, Sq, Skv, Dq, Dv = 1, 2, 4, 6, 3, 4
    q, k, v = _rand((B, H, Sq, Dq), 231), _rand((B, H, Skv, Dq), 232), _rand((B, H, Skv, Dv), 233)
    dout = _rand((B, H, Sq, Dv), 234)
    kw = dict(scale=0.6, alibi_slopes=np.array([[0.25, 0.9]]))
    g = O.bwd(q, k, v, dout, **kw)
    eps = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + eps
            lp = _loss(q, k, v, dout, None, **kw)
            x[i] = old - eps
            lm = _loss(q, k, v, dout, None, **kw)
            x[i] = old
            num[i] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(num - g[name])) / max(1e-3, np.max(np.abs(num)))
        assert err < 1e-6, (name, err)


# --------------------------------------------------------- quantized K/V ----
@pytest.mark.parametrize("group", [16, 32, 128])
def test_dequantize_is_within_half_a_step_of_the_quantized_data(group):
    # a test-side symmetric quantizer: scale = max|x| / 127 per token and
    # group, code = round(x / scale); dequantizing must land within scale / 2
    x = _rand((2, 3, 40, 128), 241)
    xg = x.reshape(2, 3, 40, 128 // group, group)
    scale = np.abs(xg).max(-1) / 127.0
    codes = np.clip(np.rint(xg / scale[..., None]), -127, 127).astype(np.int8).reshape(x.shape)
    xr = O.dequantize_kv(codes, scale, group)
    bound = np.repeat(scale, group, axis=-1) / 2
    assert np.all(np.abs(xr - x) <= bound * (1 + 1e-12))
    # and the quantization is not trivially coarse: errors use the whole step
    assert np.max(np.abs(xr - x) / bound) > 0.9


def test_dequantize_zero_point_shift_and_identity():
    rng = np.random.default_rng(251)
    codes = rng.integers(-100, 100, size=(4, 7, 64)).astype(np.int8)
    zp = rng.integers(-20, 20, size=(4, 7, 4)).astype(np.int8)
    sc = rng.uniform(0.01, 0.2, size=(4, 7, 4))
    a = O.dequantize_kv(codes, sc, 16, zp)
    c = 7
    b = O.dequantize_kv((codes.astype(np.int16) + c), sc, 16, zp.astype(np.int16) + c)
    assert np.array_equal(a, b)
    assert np.array_equal(O.dequantize_kv(codes, np.ones((4, 7, 1)), 64), codes.astype(np.float64))
    # one group per 16 columns: column c uses group c // 16
    one = np.zeros((1, 1, 64), dtype=np.int8)
    one[0, 0, 17] = 1
    g = np.array([[[1.0, 3.0, 5.0, 7.0]]])
    assert O.dequantize_kv(one, g, 16)[0, 0, 17] == 3.0


def _pack_nibbles_by_arithmetic(codes):
    """Test-side packer, written with integer arithmetic rather than bit
    operations: byte i = (code 2i mod 16) + 16 (code 2i+1 mod 16)."""
    c = np.asarray(codes, dtype=np.int64) % 16
    return (c[..., 0::2] + 16 * c[..., 1::2]).astype(np.uint8)


@pytest.mark.parametrize("signed", [True, False])
def test_unpack_int4_inverts_the_packing(signed):
    # every code value in every position, packed by a different method
    rng = np.random.default_rng(271 + signed)
    lo, hi = (-8, 8) if signed else (0, 16)
    codes = rng.integers(lo, hi, size=(3, 5, 128))
    codes[0, 0, :16] = np.arange(lo, hi)
    codes[0, 1, 1:17:2] = np.arange(lo, hi)[:8]
    assert np.array_equal(O.unpack_int4(_pack_nibbles_by_arithmetic(codes), signed), codes)


def test_unpack_int4_byte_table():
    # all 256 bytes: the low nibble is the even code, the high nibble the odd
    # one; signed codes are 4-bit two's complement
    b = np.arange(256, dtype=np.uint8)[None, :]
    u = O.unpack_int4(b, False)[0]
    s = O.unpack_int4(b, True)[0]
    for v in range(256):
        assert (u[2 * v], u[2 * v + 1]) == (v % 16, v // 16)
        assert (s[2 * v] - u[2 * v]) % 16 == 0 and -8 <= s[2 * v] <= 7
        assert (s[2 * v + 1] - u[2 * v + 1]) % 16 == 0 and -8 <= s[2 * v + 1] <= 7
    assert s[2 * 0x8F] == -1 and s[2 * 0x8F + 1] == -8 and s[2 * 0x07] == 7


@pytest.mark.parametrize("group", [32, 128])
def test_int4_dequantize_is_within_half_a_step(group):
    # a test-side symmetric 4-bit quantizer (scale = max|x| / 7, codes in
    # -7 .. 7), packed, unpacked by the oracle and dequantized: within half a
    # step of the data
    x = _rand((2, 3, 40, 128), 281)
    xg = x.reshape(2, 3, 40, 128 // group, group)
    scale = np.abs(xg).max(-1) / 7.0
    codes = np.clip(np.rint(xg / scale[..., None]), -7, 7).astype(np.int64).reshape(x.shape)
    xr = O.dequantize_kv(O.unpack_int4(_pack_nibbles_by_arithmetic(codes), True), scale, group)
    bound = np.repeat(scale, group, axis=-1) / 2
    assert np.all(np.abs(xr - x) <= bound * (1 + 1e-12))
    assert np.max(np.abs(xr - x) / bound) > 0.9


# ------------------------------------------------------------ group mode ----
def test_group_mode_equals_batch_mode_per_sequence():
    H, D = 2, 6
    lens = [5, 1, 12, 7]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    q, k, v, dout = (_rand((T, H, D), 60 + i) for i in range(4))
    kw = dict(scale=0.5, causal=True, p_drop=0.2, seed=11, offset=2)
    gf = O.fwd(q, k, v, cu_seqlens_q=cu, cu_seqlens_kv=cu, **kw)
    gb = O.bwd(q, k, v, dout, cu_seqlens_q=cu, cu_seqlens_kv=cu, **kw)
    for n, L in enumerate(lens):
        sl = slice(cu[n], cu[n + 1])
        def bhsd(x):
            return np.ascontiguousarray(x[sl].transpose(1, 0, 2))[None]
        # the batch-mode run of one sequence must use batch index n for the RNG:
        # build a batch of n+1 copies and read entry n
        rep = lambda x: np.repeat(bhsd(x), n + 1, axis=0)
        bf = O.fwd(rep(q), rep(k), rep(v), heads=[(n, h) for h in range(H)], **kw)
        bb = O.bwd(rep(q), rep(k), rep(v), rep(dout), heads=[(n, h) for h in range(H)], **kw)
        assert np.array_equal(gf["o"][sl].transpose(1, 0, 2), bf["o"][n])
        assert np.array_equal(gf["lse"][:, sl], bf["lse"][n])
        for name in ("dq", "dk", "dv"):
            assert np.array_equal(gb[name][sl].transpose(1, 0, 2), bb[name][n])


# --------------------------------------------------------- mutation check ----
MUTANTS = {
    # a dropped bias term
    "bias": ("+ (h->bias ? h->bias[i * h->ld_bias + j] : 0.0)", ""),
    # an off-by-one causal boundary
    "causal": ("        l = i;\n", "        l = i - 1;\n"),
    # an off-by-one left window edge
    "window": ("int64_t lo = i + h->band_off + h->band_lo,", "int64_t lo = i + h->band_off + h->band_lo + 1,"),
    # the bottom-right diagonal shifted
    "bottom_right": ("hi = i + h->band_off + h->band_hi;", "hi = i + h->band_off + h->band_hi + 1;"),
    # a wrong sign in dS
    "dS": ("double dS = s[j] * (z[j] * dot - D);", "double dS = s[j] * (z[j] * dot + D);"),
    # a transposed operand in dK
    "dK": ("dkj[c] += h->scale * dS * qi[c];", "dkj[c] += h->scale * dS * kj[c];"),
    # dropout rescale forgotten
    "rescale": ("double rescale = 1.0 / (1.0 - (double)h->p_drop);", "double rescale = 1.0;"),
    # a wrong Philox word order
    "philox": ("uint32_t n1 = lo1;", "uint32_t n1 = lo0;"),
    # the keep counter with query and key positions swapped
    "keep_counter": ("uint32_t ctr[4] = {(uint32_t)(j >> 2), (uint32_t)(i >> 2), bh,",
                     "uint32_t ctr[4] = {(uint32_t)(i >> 2), (uint32_t)(j >> 2), bh,"),
    # the keep byte taken with word and byte indices swapped
    "keep_byte": ("uint32_t byte = (r[i & 3] >> (8 * (j & 3))) & 0xffu;",
                  "uint32_t byte = (r[j & 3] >> (8 * (i & 3))) & 0xffu;"),
    # ALiBi with the wrong sign, without the absolute value, or misaligned
    "alibi_sign": ("s[j] -= h->alibi_slope", "s[j] += h->alibi_slope"),
    "alibi_abs": ("fabs((double)(j - i - h->alibi_off))", "((double)(j - i - h->alibi_off))"),
    "alibi_off": ("(j - i - h->alibi_off)", "(j - i + h->alibi_off)"),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_oracle_mistakes(mutant, tmp_path):
    """Build a deliberately broken copy of the oracle and check that at least
    one of the pins above fails against it."""
    src = open(os.path.join(ROOT, "oracle", "sdpa_oracle.c")).read()
    old, new = MUTANTS[mutant]
    assert old in src
    mdir = tmp_path / "oracle"
    mdir.mkdir()
    (mdir / "sdpa_oracle.c").write_text(src.replace(old, new))
    for f in ("sdpa_oracle.py", "__init__.py", "build.py"):
        shutil.copy(os.path.join(ROOT, "oracle", f), mdir / f)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                    str(mdir / "sdpa_oracle.c"), "-o", str(mdir / "liboracle.so"), "-lm"],
                   check=True)
    code = (
        "import sys; sys.path.insert(0, %r); sys.path.insert(1, %r)\n"
        "import oracle.sdpa_oracle as O; assert O.__file__.startswith(%r)\n"
        "import tests.test_oracle_pins as T\n"
        "T.O = O\n"
        "import inspect\n"
        "fails = 0\n"
        "for name, fn in sorted(vars(T).items()):\n"
        "    if not name.startswith('test_') or name == 'test_pins_catch_planted_oracle_mistakes':\n"
        "        continue\n"
        "    if name == 'test_philox_matches_rocrand_engine':\n"
        "        continue\n"
        "    params = getattr(fn, 'pytestmark', [])\n"
        "    combos = [()]\n"
        "    for m in params:\n"
        "        if m.name == 'parametrize':\n"
        "            names = [n.strip() for n in m.args[0].split(',')]\n"
        "            combos = [c + (dict(zip(names, v if isinstance(v, tuple) else (v,))),) for c in combos for v in m.args[1]]\n"
        "    for c in combos:\n"
        "        kw = {}\n"
        "        for d in c: kw.update(d)\n"
        "        try:\n"
        "            fn(**kw)\n"
        "        except Exception:\n"
        "            fails += 1\n"
        "print('FAILS', fails)\n"
    ) % (str(tmp_path), ROOT, str(mdir))
    r = subprocess.run(["python", "-c", code], capture_output=True, text=True, cwd=str(tmp_path))
    assert "FAILS" in r.stdout, r.stderr[-2000:]
    n = int(r.stdout.split("FAILS")[1].split()[0])
    assert n > 0, f"no pin caught the planted mistake {mutant!r}"
