"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``check_*`` function raises AssertionError when the oracle disagrees with a closed form,
an invariant, a library routine, a page-printed figure, a hand-derived case, or the independent
numpy decoder.  ``tests/test_oracle_pins.py`` runs them against the oracle, and
``tests/test_oracle_mutants.py`` runs them against deliberately broken copies of the oracle to
show that each plausible mistake is caught by at least one of them.
"""
from __future__ import annotations

import math
import os
from dataclasses import replace
from fractions import Fraction

import numpy as np
import scipy.special
import torch

import oracle as O
import synth as S

from np_decoder import NumpyDecoder, bf16_bits_to_f32, logical_kv

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                out[k] = int(v)
    return out


def _rng(seed):
    return np.random.default_rng(seed)


def _f16_bits(vals):
    return np.asarray(vals, np.float16).view(np.uint16)


# ----------------------------------------------------------------------------- number formats
def check_f16_decode_exhaustive():
    """All 65536 binary16 patterns against numpy's binary16 -> binary32 conversion, bit for bit."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = O.f16_to_f32(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def check_bf16_round_nearest_even():
    """Tie cases by hand, then random values against torch's bf16 rounding."""
    ties = {0x3F808000: 0x3F80, 0x3F818000: 0x3F82, 0x3F80C000: 0x3F81, 0x3F807FFF: 0x3F80,
            0x7F800000: 0x7F80, 0xFF800000: 0xFF80, 0x7F7FFFFF: 0x7F80, 0x00000000: 0x0000,
            0x80000000: 0x8000}
    for fbits, want in ties.items():
        f = np.array([fbits], np.uint32).view(np.float32)
        assert int(O.f32_to_bf16(f)[0]) == want, hex(fbits)
    r = _rng(1)
    x = (r.standard_normal(4000) * np.exp(r.uniform(-30, 30, 4000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16(x), ref)


# ----------------------------------------------------------------------------- dequant + GEMV
def check_int4_codes_by_hand():
    """Per-weight INT4 contract: mask 4 bits, subtract the zero point 8, times the group's fp16
    scale.  Byte j of a row holds k = 2j (bits 0-3) and k = 2j+1 (bits 4-7)."""
    K = 128
    W = np.full((1, K // 2), 0x88, np.uint8)          # every code 8 -> level 0
    W[0, 0] = 0x1F                                      # k=0: 15 -> +7 ; k=1: 1 -> -7
    W[0, 32] = 0x0F                                     # k=64: 15 -> +7 ; k=65: 0 -> -8
    S_ = _f16_bits([1.0, 2.0]).reshape(1, 2)
    w = O.dequant_row("q4", W, S_, 0, K, 64)
    want = np.zeros(K, np.float32)
    want[0], want[1], want[64], want[65] = 7.0, -7.0, 14.0, -16.0
    assert np.array_equal(w, want)
    # a scale that is not a power of two: the product stays exact in fp32
    s3 = np.float16(0.0133)
    S3 = np.array([[s3.view(np.uint16), s3.view(np.uint16)]], np.uint16)
    w3 = O.dequant_row("q4", W, S3, 0, K, 64)
    assert w3[0] == np.float32(7) * np.float32(s3) and w3[65] == np.float32(-8) * np.float32(s3)


def check_int8_onehot():
    """x = e_k gives column k of the dequantised matrix: fl32(q * s), bit for bit."""
    r = _rng(2)
    N, K = 37, 48
    q = r.integers(-127, 128, (N, K)).astype(np.int8)
    s = ((0.02 / 127) * r.uniform(0.5, 1.5, N)).astype(np.float32)
    for k in (0, 1, 17, K - 1):
        x = np.zeros(K, np.float32); x[k] = 1.0
        y = O.gemv("q8", q, s, x)
        assert np.array_equal(y, q[:, k].astype(np.float32) * s)


def check_gemv_ones_closed_form():
    """x = 1: y_n = sum_g s_g * sum_{k in g} (nib - 8), exact rational arithmetic."""
    r = _rng(3)
    N, K, grp = 9, 192, 64
    W = r.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sv = r.uniform(0.005, 0.02, (N, K // grp)).astype(np.float16)
    y = O.gemv("q4", W, sv.view(np.uint16), np.ones(K, np.float32), group=grp)
    for n in range(N):
        tot = Fraction(0)
        for g in range(K // grp):
            lev = 0
            for k in range(g * grp, (g + 1) * grp):
                byte = int(W[n, k // 2])
                lev += ((byte >> 4) if k % 2 else (byte & 15)) - 8
            tot += Fraction(float(sv[n, g])) * lev
        assert y[n] == np.float32(float(tot)), n
    # int8: sum of fp32 products; the closed form s * sum(q) holds to fp32 rounding of each term
    q = r.integers(-127, 128, (N, K)).astype(np.int8)
    s = np.full(N, np.float32(0.02 / 127))
    y8 = O.gemv("q8", q, s, np.ones(K, np.float32))
    exact = s.astype(np.float64) * q.astype(np.int64).sum(1)
    bound = np.abs(q).astype(np.float64).sum(1) * float(s[0]) * 2.0 ** -24 + np.abs(exact) * 2.0 ** -24
    assert np.all(np.abs(y8 - exact) <= bound + 1e-30)


def check_gemv_bruteforce():
    """Both formats, with bias and residual, against an independent numpy dequant + fp64 matmul."""
    from np_decoder import dequant
    r = _rng(4)
    for wfmt, grp in (("q8", 64), ("q4", 64), ("q4", 32)):
        N, K = 45, 192
        if wfmt == "q8":
            W = r.integers(-127, 128, (N, K)).astype(np.int8)
            Sc = ((0.02 / 127) * r.uniform(0.5, 1.5, N)).astype(np.float32)
        else:
            W = r.integers(0, 256, (N, K // 2)).astype(np.uint8)
            Sc = r.uniform(0.005, 0.02, (N, K // grp)).astype(np.float16).view(np.uint16)
        x = r.standard_normal(K).astype(np.float32)
        b = (0.02 * r.standard_normal(N)).astype(np.float32)
        res = r.standard_normal(N).astype(np.float32)
        y = O.gemv(wfmt, W, Sc, x, bias=b, residual=res, group=grp)
        ref = dequant(wfmt, W, Sc, grp) @ x.astype(np.float64) + b + res
        assert np.allclose(y, ref, rtol=1e-6, atol=1e-6), wfmt
        y0 = O.gemv(wfmt, W, Sc, x, group=grp)
        assert np.allclose(y0, dequant(wfmt, W, Sc, grp) @ x.astype(np.float64), rtol=1e-6, atol=1e-6)


# ----------------------------------------------------------------------------- INT8 activations
def check_act_i8_by_hand():
    """Per-group symmetric INT8 activations, worked by hand: with max|x| = 127 the inverse scale
    is exactly 1, so q is x rounded to nearest with ties to even (62.5 -> 62, 1.5 -> 2,
    -2.5 -> -2, -0.5 -> 0); with max|x| = 1 the inverse scale is 127 and 0.5 -> 63.5 -> 64."""
    x = np.array([127, 62.5, -0.5, 1.5, -2.5, 0, 3.25, -126.75,
                  0.5, -1.0, 0.25, 0.125, 0, 0, 0, 0], np.float32)
    qv, sx = O.quantize_act_i8(x, group=8)
    assert list(qv[:8]) == [127, 62, 0, 2, -2, 0, 3, -127], list(qv[:8])
    assert list(qv[8:12]) == [64, -127, 32, 16] and list(qv[12:]) == [0] * 4
    assert sx[0] == np.float32(1.0) and sx[1] == np.float32(1.0) / np.float32(127.0)
    # a group of zeros has scale 0 and codes 0
    q0, s0 = O.quantize_act_i8(np.zeros(64, np.float32))
    assert not q0.any() and s0[0] == 0.0


def check_act_i8_invariants():
    """For every nonzero group: the largest |q| is 127, q is the binary32 product x * (127/amax)
    rounded to nearest-even, and |x - q*s| <= s/2 up to the rounding of the scale."""
    r = _rng(11)
    x = (r.standard_normal(64 * 7) * r.uniform(0.01, 30.0, 64 * 7)).astype(np.float32)
    x[64:128] = 0.0
    qv, sx = O.quantize_act_i8(x)
    for g in range(7):
        xg, qg = x[g * 64:(g + 1) * 64].astype(np.float64), qv[g * 64:(g + 1) * 64].astype(np.int64)
        if g == 1:
            assert sx[g] == 0 and not qg.any()
            continue
        amax = np.abs(xg).max()
        assert np.abs(qg).max() == 127
        assert sx[g] == np.float32(amax) / np.float32(127)
        t = (x[g * 64:(g + 1) * 64] * (np.float32(127) / np.float32(amax))).astype(np.float32)
        assert np.array_equal(qg, np.clip(np.rint(t), -127, 127).astype(np.int64))
        assert np.all(np.abs(xg - qg * float(sx[g])) <= 0.5 * float(sx[g]) * (1 + 1e-5))


def check_gemv_a8_against_dequantized_activations():
    """The INT8-activation GEMV is the real GEMV on the dequantised activations q[k] * s[k // group]:
    checked against numpy dequant + fp64 matmul, both formats, with bias and residual; and when
    x holds integers with max |x| = 127 per group, quantisation is the identity (q = x, s = 1), so the
    result equals the exact rational value of the fp-activation GEMV."""
    from np_decoder import dequant
    r = _rng(12)
    for wfmt, grp in (("q8", 64), ("q4", 64), ("q4", 32)):
        N, K = 37, 256
        if wfmt == "q8":
            W = r.integers(-127, 128, (N, K)).astype(np.int8)
            Sc = ((0.02 / 127) * r.uniform(0.5, 1.5, N)).astype(np.float32)
        else:
            W = r.integers(0, 256, (N, K // 2)).astype(np.uint8)
            Sc = r.uniform(0.005, 0.02, (N, K // grp)).astype(np.float16).view(np.uint16)
        x = r.standard_normal(K).astype(np.float32)
        qv, sx = O.quantize_act_i8(x, group=grp)
        b = (0.02 * r.standard_normal(N)).astype(np.float32)
        res = r.standard_normal(N).astype(np.float32)
        xh = qv.astype(np.float64) * np.repeat(sx.astype(np.float64), grp)
        Wd = dequant(wfmt, W, Sc, grp)
        y = O.gemv_a8(wfmt, W, Sc, qv, sx, bias=b, residual=res, group=grp)
        assert np.allclose(y, Wd @ xh + b + res, rtol=1e-6, atol=1e-6), wfmt
        y0 = O.gemv_a8(wfmt, W, Sc, qv, sx, group=grp)
        assert np.allclose(y0, Wd @ xh, rtol=1e-6, atol=1e-7), wfmt
        # the quantisation error of the activations bounds the distance to the fp-activation GEMV
        yf = O.gemv(wfmt, W, Sc, x, group=grp)
        bound = np.abs(Wd) @ np.repeat(sx.astype(np.float64), grp) * 0.5
        assert np.all(np.abs(y0.astype(np.float64) - yf) <= bound * (1 + 1e-4) + 1e-6), wfmt
        # integer activations, 127 in every group: exact
        xi = r.integers(-126, 127, K).astype(np.float32)
        xi[::grp] = 127.0
        qi, si = O.quantize_act_i8(xi, group=grp)
        assert np.array_equal(qi.astype(np.float32), xi) and np.all(si == 1.0)
        yi = O.gemv_a8(wfmt, W, Sc, qi, si, group=grp)
        for n in range(0, N, 5):
            if wfmt == "q8":  # row scale times an integer sum (the numpy dequant rounds w to fp32)
                exact = Fraction(float(Sc[n])) * int((W[n].astype(np.int64) * xi.astype(np.int64)).sum())
            else:  # fp16 scale times a small integer level is exact in fp64
                exact = sum((Fraction(float(v)) for v in Wd[n] * xi.astype(np.float64)), Fraction(0))
            assert yi[n] == np.float32(float(exact)), (wfmt, n)


# ----------------------------------------------------------------------------- sampling
def _np_philox_words(ctr, key):
    """Philox4x64-10 words of one counter from numpy's generator (it advances the counter before
    each block, so it is started one below)."""
    c = (ctr[0] | (ctr[1] << 64) | (ctr[2] << 128) | (ctr[3] << 192)) - 1
    bg = np.random.Philox(key=key[0] | (key[1] << 64), counter=c % (1 << 256))
    return bg.random_raw(4)


def check_philox_against_numpy():
    """Philox4x64-10 equals numpy's implementation; the all-zero case is the published known-answer
    vector of the Random123 distribution."""
    assert [int(v) for v in O.philox4x64_10([0, 0, 0, 0], [0, 0])] == [
        0x16554D9ECA36314C, 0xDB20FE9D672D0FDC, 0xD7E772CEE186176B, 0x7E68B68AEC7BA23B]
    r = _rng(21)
    for _ in range(12):
        ctr = [int(v) for v in r.integers(0, 2 ** 63, 4, dtype=np.int64)]
        ctr[0] |= 1
        key = [int(v) for v in r.integers(0, 2 ** 63, 2, dtype=np.int64)]
        assert np.array_equal(O.philox4x64_10(ctr, key), _np_philox_words(ctr, key))


def check_sample_uniform_against_numpy():
    """u of token i at a step: word i mod 4 of the block (i // 4, step, 0, 0) keyed (seed, 0), as
    ((word >> 11) + 0.5) 2^-53."""
    for seed, step in ((0, 0), (7, 1), (2 ** 40 + 3, 12345)):
        for i in (0, 1, 2, 3, 4, 7, 150001):
            w = int(_np_philox_words([i // 4, step, 0, 0], [seed, 0])[i % 4])
            assert O.sample_uniform(seed, step, i) == ((w >> 11) + 0.5) * 2.0 ** -53
            assert 0.0 < O.sample_uniform(seed, step, i) < 1.0


def _np_sample(lg, T, k, p, seed, step):
    """Independent reading of the sampler: stable sort, cumulative mass, Gumbel keys from numpy's
    Philox and Python's libm log."""
    lg = np.asarray(lg, np.float32)
    if T <= 0:
        return int(np.argmax(lg))
    V = lg.size
    order = np.argsort(-lg.astype(np.float64), kind="stable")
    keep = order
    if 0 < k < V:
        keep = keep[:k]
    if p < 1.0:
        z = lg[keep].astype(np.float64) / T
        e = np.exp(z - z[0])
        cum = np.cumsum(e)  # (summed in the same order as the oracle's loop)
        tot = e.sum()
        n = int(np.argmax(cum >= p * tot)) + 1
        keep = keep[:n]
    best, bi = None, None
    for i in sorted(int(v) for v in keep):
        w = int(_np_philox_words([i // 4, step, 0, 0], [seed, 0])[i % 4])
        u = ((w >> 11) + 0.5) * 2.0 ** -53
        key = np.float32(float(lg[i]) / T - math.log(-math.log(u)))
        if best is None or key > best:
            best, bi = key, i
    return bi


def check_sample_against_numpy_reading():
    r = _rng(22)
    lg = (2.0 * r.standard_normal(300)).astype(np.float32)
    lg[[5, 77]] = lg.max()  # a tie at the top
    for T, k, p in ((1.0, 0, 1.0), (0.6, 20, 0.95), (0.7, 0, 0.5), (1.3, 50, 1.0), (0.0, 20, 0.9), (2.0, 300, 0.99)):
        for step in (0, 1, 9):
            assert O.sample(lg, T, k, p, seed=11, step=step) == _np_sample(lg, T, k, p, 11, step), (T, k, p, step)


def check_sample_special_cases():
    """Greedy limits: temperature 0, top-k 1 and a vanishing top-p all give the argmax; top-k >= V
    keeps everything; with equal logits top-k keeps the smallest indices, and a top-p mass that
    lands exactly on a prefix boundary stops there."""
    r = _rng(23)
    lg = r.standard_normal(1000).astype(np.float32)
    am = int(np.argmax(lg))
    for step in range(5):
        assert O.sample(lg, 0.0, seed=1, step=step) == am
        assert O.sample(lg, 0.8, top_k=1, seed=1, step=step) == am
        assert O.sample(lg, 0.8, top_p=1e-12, seed=1, step=step) == am
        assert O.sample(lg, 0.8, top_k=1000, seed=1, step=step) == O.sample(lg, 0.8, seed=1, step=step)
    eq = np.zeros(8, np.float32)
    got_k = {O.sample(eq, 1.0, top_k=3, seed=5, step=s) for s in range(200)}
    assert got_k == {0, 1, 2}
    got_p = {O.sample(eq, 1.0, top_p=0.5, seed=5, step=s) for s in range(200)}  # mass 4/8 reached at 4
    assert got_p == {0, 1, 2, 3}


def _chi2(counts, probs, n):
    exp = np.asarray(probs) * n
    return float(((np.asarray(counts) - exp) ** 2 / exp).sum())


def check_sample_frequencies():
    """Gumbel-max draws follow the softmax of l / T over the kept set (chi-square, 20000 steps,
    a bound a correct sampler exceeds with probability below 1e-6)."""
    lg = np.array([1.0, 2.0, 0.5, 2.0, -1.0, 0.0], np.float32)
    n = 20000
    for T, k, keep in ((1.0, 0, [0, 1, 2, 3, 4, 5]), (0.5, 3, [0, 1, 3])):
        z = lg[keep].astype(np.float64) / T
        pr = np.exp(z - z.max())
        pr /= pr.sum()
        cnt = np.zeros(len(keep))
        for step in range(n):
            t = O.sample(lg, T, top_k=k, seed=99, step=step)
            assert t in keep, (T, k, t)
            cnt[keep.index(t)] += 1
        assert _chi2(cnt, pr, n) < 40.0, (T, k, cnt, pr * n)


# ----------------------------------------------------------------------------- RMSNorm
def check_rmsnorm_closed_forms():
    r = _rng(5)
    dim, eps = 64, 1e-6
    g = (1 + 0.1 * r.standard_normal(dim)).astype(np.float32)
    for c in (0.7, 1e-3, 25.0):
        y = O.rmsnorm(np.full(dim, c, np.float32), g, eps)
        want = g.astype(np.float64) * np.float32(c) / math.sqrt(float(np.float32(c)) ** 2 + eps)
        assert np.allclose(y, want, rtol=2e-7, atol=0), c
    x = r.standard_normal((3, dim)).astype(np.float32)
    y = O.rmsnorm(x, g, eps).astype(np.float64)
    ms = np.mean(x.astype(np.float64) ** 2, axis=1)
    assert np.allclose(np.mean((y / g) ** 2, axis=1), ms / (ms + eps), rtol=1e-6)
    y2 = O.rmsnorm(1000.0 * x, g, eps)
    assert np.allclose(y2, y, rtol=2e-6, atol=1e-7)


# ----------------------------------------------------------------------------- RoPE
def check_rope_invariants():
    r = _rng(6)
    D, base = 128, 1e6
    x = r.standard_normal((5, D)).astype(np.float32)
    assert np.array_equal(O.rope(x, 0, base), x)                      # R(0) = I
    y = O.rope(x, 32768, base)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-6)
    q, k = x[0], x[1]
    for m, n in ((1000, 400), (4096, 4095), (17, 0), (32768, 3)):
        lhs = float(O.rope(q, m, base).astype(np.float64) @ O.rope(k, n, base).astype(np.float64))
        rhs = float(O.rope(q, m - n, base).astype(np.float64) @ k.astype(np.float64))
        assert abs(lhs - rhs) <= 1e-5 * np.linalg.norm(q) * np.linalg.norm(k), (m, n)


def check_rope_textbook_cases():
    # D = 2: the textbook 2x2 rotation by angle pos (theta_0 = base^0 = 1)
    for pos in (1, 3, 1000):
        v = np.array([0.6, -1.3], np.float32)
        R = np.array([[math.cos(pos), -math.sin(pos)], [math.sin(pos), math.cos(pos)]])
        assert np.allclose(O.rope(v, pos, 1e6), R @ v.astype(np.float64), rtol=1e-6, atol=1e-7)
    # D = 8, pairs (i, i + 4), theta_i = base^(-2i/8)
    base = 100.0
    for i in range(4):
        e = np.zeros(8, np.float32); e[i] = 1.0
        pos = 20
        phi = pos * base ** (-2.0 * i / 8)
        want = np.zeros(8); want[i] = math.cos(phi); want[i + 4] = math.sin(phi)
        assert np.allclose(O.rope(e, pos, base), want, atol=1e-7), i
        e2 = np.zeros(8, np.float32); e2[i + 4] = 1.0
        want2 = np.zeros(8); want2[i] = -math.sin(phi); want2[i + 4] = math.cos(phi)
        assert np.allclose(O.rope(e2, pos, base), want2, atol=1e-7), i


# ----------------------------------------------------------------------------- SwiGLU
def check_swiglu_identities():
    r = _rng(7)
    g = (3 * r.standard_normal(1000)).astype(np.float32)
    u = r.standard_normal(1000).astype(np.float32)
    m = O.swiglu(g, u)
    ref = g.astype(np.float64) * scipy.special.expit(g.astype(np.float64)) * u
    assert np.allclose(m, ref, rtol=1e-6, atol=1e-12)
    assert np.all(O.swiglu(np.zeros(4, np.float32), np.full(4, 5.0, np.float32)) == 0)
    one = np.ones_like(g)
    assert np.allclose(O.swiglu(-g, one).astype(np.float64), O.swiglu(g, one).astype(np.float64) - g,
                       rtol=0, atol=2e-6 * (1 + np.abs(g)))
    big = np.full(3, 40.0, np.float32)
    assert np.allclose(O.swiglu(big, np.full(3, 2.0, np.float32)), 80.0, rtol=1e-7)


# ----------------------------------------------------------------------------- paged KV + attention
def _pool(r, P, Hkv, D, fmt, ps=16):
    a = r.standard_normal((P, Hkv, ps, D)).astype(np.float32)
    if fmt == "bf16":
        return torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return a


def _logical(pool, pt, T, fmt, ps=16):
    t = np.arange(T)
    a = pool[pt[t // ps], :, t % ps, :]
    if fmt == "bf16":
        a = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    return a.astype(np.float64)            # [T][Hkv][D]


def check_attention_bruteforce():
    r = _rng(8)
    Hq, Hkv, D = 4, 2, 8
    for fmt in ("f32", "bf16"):
        for T in (1, 2, 5, 17, 49):
            P = -(-T // 16) + 1
            pt = r.permutation(P).astype(np.int32)
            kp, vp = _pool(r, P, Hkv, D, fmt), _pool(r, P, Hkv, D, fmt)
            q = (2 * r.standard_normal((Hq, D))).astype(np.float32)
            out, probs = O.attention(q, kp, vp, fmt, pt, T, probs=True)
            Kl, Vl = _logical(kp, pt, T, fmt), _logical(vp, pt, T, fmt)
            for h in range(Hq):
                j = h // (Hq // Hkv)
                p = scipy.special.softmax(Kl[:, j, :] @ q[h].astype(np.float64) / math.sqrt(D))
                assert np.allclose(out[h], p @ Vl[:, j, :], rtol=1e-6, atol=1e-7), (fmt, T, h)
                assert np.allclose(probs[h], p, rtol=1e-6, atol=1e-9)
            assert np.allclose(probs.astype(np.float64).sum(1), 1.0, atol=1e-6)


def check_attention_special_cases():
    r = _rng(9)
    Hq, Hkv, D, fmt = 6, 2, 8, "f32"
    P = 4
    pt = np.array([2, 0, 3, 1], np.int32)
    kp, vp = _pool(r, P, Hkv, D, fmt), _pool(r, P, Hkv, D, fmt)
    q = r.standard_normal((Hq, D)).astype(np.float32)
    # T = 1: the only probability is exactly 1, so out is v of token 0 bit for bit
    out = O.attention(q, kp, vp, fmt, pt, 1)
    for h in range(Hq):
        assert np.array_equal(out[h], vp[pt[0], h // 3, 0, :])
    # equal scores (q = 0): the mean of V
    T = 37
    out = O.attention(np.zeros((Hq, D), np.float32), kp, vp, fmt, pt, T)
    Vl = _logical(vp, pt, T, fmt)
    for h in range(Hq):
        assert np.allclose(out[h], Vl[:, h // 3, :].mean(0), rtol=1e-6, atol=1e-7)
    # GQA map: V of KV head j constant c_j -> every query head of group j returns c_j
    vc = np.zeros_like(vp)
    vc[:, 0], vc[:, 1] = 1.5, -4.0
    out = O.attention(q, kp, vc, fmt, pt, T)
    assert np.allclose(out[:3], 1.5, rtol=1e-6) and np.allclose(out[3:], -4.0, rtol=1e-6)
    # the same logical context behind two different page tables gives the same output
    pt2 = np.array([1, 3, 0, 2], np.int32)
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[pt2], vp2[pt2] = kp[pt], vp[pt]
    assert np.array_equal(O.attention(q, kp, vp, fmt, pt, T), O.attention(q, kp2, vp2, fmt, pt2, T))


def check_kv_layout_against_page_figures():
    """16 KiB pages, 4 KiB per KV-head slice, 1 KB of K per token per layer (Qwen2.5-7B shape)."""
    dims = read_golden("qwen25_7b_dims.txt")
    Hkv, D, ps = dims["n_kv_heads"], dims["head_dim"], dims["page_tokens"]
    P = 3
    pool = np.zeros((P, Hkv, ps, D), np.uint16)
    pt = np.array([2, 0, 1], np.int32)
    t = 16 + 5                                       # logical page 1 -> physical page 0, slot 5
    kv = np.ones((Hkv, D), np.float32)
    O.kv_store(pool, "bf16", pt, ps, t, kv)
    nz = np.flatnonzero(pool.view(np.uint8).reshape(-1))
    assert nz.size == dims["kv_bytes_per_token_per_layer"]          # 4 * 128 * 2 bytes
    page_bytes = pool[0].nbytes
    assert page_bytes == dims["kv_page_bytes"] and page_bytes % dims["page_alignment_bytes"] == 0
    assert pool[0, 0].nbytes == dims["kv_head_slice_bytes"]
    assert nz.min() == 0 * page_bytes + 5 * D * 2                    # physical page 0, head 0, slot 5
    for j in range(Hkv):
        off = j * dims["kv_head_slice_bytes"] + 5 * D * 2
        assert np.all(pool.view(np.uint8).reshape(-1)[off:off + 2 * D] != 0)
    assert O.kv_store is not None and float(O.lib().orc_kv_load(
        O._p(pool), 2, O._p(pt), ps, Hkv, D, t, 3, 127)) == 1.0


def check_workload_shapes_against_pages():
    d7 = read_golden("qwen25_7b_dims.txt")
    for name in ("qwen2.5-7b-q4", "qwen2.5-7b-q4-32k"):
        wl = S.WORKLOADS[name]
        assert (wl.n_layers, wl.hidden, wl.inter, wl.vocab) == (
            d7["n_layers"], d7["hidden"], d7["inter"], d7["vocab"])
        assert (wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.page_size) == (
            d7["n_heads"], d7["n_kv_heads"], d7["head_dim"], d7["page_tokens"])
    d15 = read_golden("qwen25_15b_meta.txt")
    wl = S.WORKLOADS["qwen2.5-1.5b-q8"]
    assert (wl.n_layers, wl.n_heads, wl.n_kv_heads) == (d15["n_layers"], d15["n_heads"], d15["n_kv_heads"])
    assert S.WORKLOADS["qwen2.5-7b-q4-32k"].ctx <= d15["context_length"]


# ----------------------------------------------------------------------------- argmax
def check_argmax_ties():
    assert O.argmax(np.array([1, 3, 3, 2], np.float32)) == 1
    assert O.argmax(np.array([5, 5], np.float32)) == 0
    assert O.argmax(np.array([np.nan, 1, 2], np.float32)) == 2
    assert O.argmax(np.array([-1, -1, -1], np.float32)) == 0
    v = np.zeros(152064, np.float32); v[[9, 70000, 152063]] = 4.0
    assert O.argmax(v) == 9


# ----------------------------------------------------------------------------- decode step
def _zero_scales(model):
    for P in model["layers"]:
        for s in ("sq", "sk", "sv", "so", "sg", "su", "sd"):
            P[s] = np.zeros_like(P[s])
    if "s_lm" in model:
        model["s_lm"] = np.zeros_like(model["s_lm"])
    return model


def check_decode_zero_weights_identity():
    """With every weight scale 0 each layer is the identity on h, bit for bit; logits are 0 and
    the greedy token is 0 (smallest index among equal maxima)."""
    for wfmt in ("q8", "q4"):
        wl = S.tiny(wfmt)
        m = _zero_scales(S.make_model(wl))
        kv = S.make_kv(wl, 16)
        r = O.OracleDecoder(m, kv).step(wl.ctx, m["token"], trace=True)
        e = m["embed"][m["token"]].astype(np.uint32) << 16
        for row in r["trace"]:
            assert np.array_equal(row.view(np.uint32), e)
        assert np.all(r["logits"] == 0) and r["token"] == 0


def check_decode_against_numpy(steps: int = 3):
    """The C oracle against the independent numpy decoder on tiny models, several steps."""
    variants = [S.tiny("q8"), S.tiny("q4"), S.tiny("q8", qk_norm=True, qkv_bias=False),
                S.tiny("q4", kv_fmt="f32", shuffled_pages=True)]
    for wl in variants:
        m = S.make_model(wl)
        kv = S.make_kv(wl, 32)
        od = O.OracleDecoder(m, kv)
        kl, vl = logical_kv(kv, wl, wl.n_layers)
        nd = NumpyDecoder(m, kl, vl)
        tok = m["token"]
        for s in range(steps):
            pos = wl.ctx + s
            a = od.step(pos, tok, trace=True)
            b = nd.step(pos, tok)
            scale = np.abs(b["trace"]).max(axis=1, keepdims=True)
            assert np.all(np.abs(a["trace"] - b["trace"]) <= 1e-5 * scale), (wl.name, s)
            assert np.allclose(a["logits"], b["logits"], rtol=0, atol=1e-5 * np.abs(b["logits"]).max())
            srt = np.sort(b["logits"].astype(np.float64))
            if srt[-1] - srt[-2] > 1e-5 * abs(srt[-1]):
                assert a["token"] == b["token"], (wl.name, s)
            tok = b["token"]


def check_decode_kv_pre_and_forced_codes():
    """The step's exposure of the new token's cache entries, against the independent numpy
    decoder: kv_pre equals numpy's fp32 k, v before the bf16 rounding; forcing every layer's own
    codes reproduces the plain step bit for bit; forcing a code one bf16 step away stores exactly
    that code, and the step then equals numpy's step with the same cache entry replaced."""
    wl = S.tiny("q4", shuffled_pages=True)
    m = S.make_model(wl)
    kv = S.make_kv(wl, 32)
    pos, tok, L = wl.ctx, m["token"], wl.n_layers
    pg, sl = int(kv["page_table"][pos // wl.page_size]), pos % wl.page_size
    od = O.OracleDecoder(m, kv)
    a = od.step(pos, tok, trace=True, kv_pre=True)
    kl, vl = logical_kv(kv, wl, L)
    nd = NumpyDecoder(m, kl, vl)
    nd.step(pos, tok)
    for l in range(L):
        for i in range(2):
            want = np.asarray(nd.pre[l][i], np.float64)
            assert np.all(np.abs(a["kv_pre"][l, i] - want) <= 1e-5 * np.abs(want).max()), (l, i)
    own = {l: (od.k[l][pg, :, sl, :].copy(), od.v[l][pg, :, sl, :].copy()) for l in range(L)}
    b = O.OracleDecoder(m, kv).step(pos, tok, trace=True, kv_force=own)
    assert np.array_equal(a["trace"].view(np.uint32), b["trace"].view(np.uint32))
    assert np.array_equal(a["logits"].view(np.uint32), b["logits"].view(np.uint32))
    moved_k = own[0][0].copy()
    moved_k[1, 2] += 1   # the next bf16 code of the same sign
    od3 = O.OracleDecoder(m, kv)
    c = od3.step(pos, tok, trace=True, kv_force={0: (moved_k, own[0][1])})
    assert np.array_equal(od3.k[0][pg, :, sl, :], moved_k)
    assert np.array_equal(od3.v[0][pg, :, sl, :], own[0][1])

    def hook(l, k, v):
        if l == 0:
            k = bf16_bits_to_f32(moved_k)
        return k, v

    nd3 = NumpyDecoder(m, *logical_kv(kv, wl, L))
    r = nd3.step(pos, tok, kv_hook=hook)
    scale = np.abs(r["trace"]).max(axis=1, keepdims=True)
    assert np.all(np.abs(c["trace"] - r["trace"]) <= 1e-5 * scale)
    assert not np.array_equal(c["trace"][1:], a["trace"][1:])   # the moved code changed the step


def check_decode_batch_against_numpy():
    """Batched step: every running slot equals the independent numpy decoder of that sequence alone
    (its own block table into the shared pool, its own position and token); an idle slot is left
    untouched; a block allocated on demand when a sequence crosses a page boundary is used."""
    wl = S.tiny("q4", shuffled_pages=True)
    m = S.make_model(wl)
    ctxs = [15, 20, 9]
    kv = S.make_kv_batch(wl, ctxs, max_blocks=4, spare_pages=3)
    tables = kv["block_tables"].copy()
    free = list(kv["free_pages"])
    od = O.OracleDecoder(m, {"page_table": tables[0], "k": kv["k"], "v": kv["v"]})
    nds = []
    for b, c in enumerate(ctxs):
        one = {"page_table": tables[b], "ctx": c, "k": kv["k"], "v": kv["v"]}
        kl, vl = logical_kv(one, wl, wl.n_layers)
        nds.append(NumpyDecoder(m, kl, vl))
    toks = np.array([m["token"], 3, 11], np.int32)
    pos = np.array(ctxs, np.int32)
    h = np.zeros((3, wl.hidden), np.float32)
    for step in range(3):
        active = [True, step != 1, True]  # slot 1 sits out the second step
        ps = np.where(active, pos, -1).astype(np.int32)
        for b in range(3):  # on-demand block for the token about to be written
            if active[b] and tables[b, pos[b] // wl.page_size] < 0:
                tables[b, pos[b] // wl.page_size] = free.pop()
        h_idle = h[1].copy()
        nxt, lg = od.step_batch(tables, ps, toks, h)
        for b in range(3):
            if not active[b]:
                assert nxt[b] == -1 and np.array_equal(h[b], h_idle)
                continue
            ref = nds[b].step(int(pos[b]), int(toks[b]))
            assert np.allclose(lg[b], ref["logits"], rtol=0, atol=1e-5 * np.abs(ref["logits"]).max()), (step, b)
            hl = ref["trace"][-1]
            assert np.all(np.abs(h[b] - hl) <= 1e-5 * np.abs(hl).max()), (step, b)
            srt = np.sort(ref["logits"].astype(np.float64))
            if srt[-1] - srt[-2] > 1e-5 * abs(srt[-1]):
                assert nxt[b] == ref["token"], (step, b)
            toks[b] = ref["token"]
            pos[b] += 1
    assert (tables >= 0).sum() == sum(-(-(c + 1) // wl.page_size) for c in ctxs) + 1  # slot 0 crossed a page


def check_prefill_against_numpy():
    """Prefill of a 21-token prompt after 9 cached tokens (crossing a page boundary): the last
    position's logits and the KV of every prompt position against the independent numpy decoder
    stepping through the prompt."""
    wl = S.tiny("q4", shuffled_pages=True)
    m = S.make_model(wl)
    ctx, T = 9, 21
    kv = S.make_kv(wl, ctx + T + 4, ctx=ctx)
    wl9 = replace(wl, ctx=ctx)
    od = O.OracleDecoder(m, kv)
    kl, vl = logical_kv(kv, wl9, wl.n_layers)
    nd = NumpyDecoder(m, kl, vl)
    toks = (np.arange(T) * 7 + 3) % wl.vocab
    r = od.prefill(ctx, toks)
    ref = None
    for t in range(T):
        ref = nd.step(ctx + t, int(toks[t]))
    assert np.allclose(r["logits"], ref["logits"], rtol=0, atol=1e-5 * np.abs(ref["logits"]).max())
    srt = np.sort(ref["logits"].astype(np.float64))
    if srt[-1] - srt[-2] > 1e-5 * abs(srt[-1]):
        assert r["token"] == ref["token"]
    pt = kv["page_table"]
    for l in range(wl.n_layers):
        for t in range(ctx, ctx + T):
            for pool, lst in ((od.k[l], nd.K[l]), (od.v[l], nd.V[l])):
                got = pool[pt[t // wl.page_size], :, t % wl.page_size, :]
                got = got.astype(np.float32) if wl.kv_fmt == "f32" else bf16_bits_to_f32(got)
                want = np.asarray(lst[t], np.float32)
                assert np.allclose(got, want, rtol=0, atol=1e-5 * max(1e-30, np.abs(want).max())), (l, t)


ALL_CHECKS = [
    check_f16_decode_exhaustive, check_bf16_round_nearest_even, check_int4_codes_by_hand,
    check_int8_onehot, check_gemv_ones_closed_form, check_gemv_bruteforce,
    check_act_i8_by_hand, check_act_i8_invariants, check_gemv_a8_against_dequantized_activations,
    check_philox_against_numpy, check_sample_uniform_against_numpy, check_sample_against_numpy_reading,
    check_sample_special_cases, check_sample_frequencies,
    check_rmsnorm_closed_forms, check_rope_invariants, check_rope_textbook_cases,
    check_swiglu_identities, check_attention_bruteforce, check_attention_special_cases,
    check_kv_layout_against_page_figures, check_workload_shapes_against_pages, check_argmax_ties,
    check_decode_zero_weights_identity, check_decode_against_numpy, check_decode_kv_pre_and_forced_codes,
    check_decode_batch_against_numpy,
    check_prefill_against_numpy,
]
