"""INT8-activation GEMV ("Path A") through the C ABI against the CPU oracle.

Bars: the activation quantisation is bit-exact (every decision is taken in binary32 on both sides,
the division correctly rounded); the GEMV on the same INT8 activations is within 2e-5 of the
oracle's max-abs output (fp32 accumulation of exact integer run sums vs fp64), and bit-exact where
every product and partial sum is exact in fp32.
"""
import numpy as np
import pytest

import oracle
from gpu_util import dev, host, rel_max_err, sync

q = pytest.importorskip("quantized_gemv_gqa_amd")

pytestmark = pytest.mark.gpu


def _acts(rng, K, group):
    """Activations of mixed magnitude per group, one all-zero group, one group of exact ties."""
    ng = K // group
    x = (rng.standard_normal(K) * np.repeat(rng.uniform(0.01, 40.0, ng), group)).astype(np.float32)
    if ng >= 3:
        x[group:2 * group] = 0.0
        # amax 127: the inverse scale is 1 and every x + 0.5 is a tie (nearest even decides)
        t = rng.integers(-126, 126, group).astype(np.float32) + 0.5
        t[0] = 127.0
        x[2 * group:3 * group] = t
    return x


@pytest.mark.parametrize("K,group", [(3584, 64), (18944, 64), (4096, 128), (896, 32), (4864, 64), (128, 128),
                                     (4096, 4096)])
def test_quantize_act_i8_bit_exact(K, group):
    rng = np.random.default_rng(K + group)
    x = _acts(rng, K, group)
    qd, sd = q.quantize_act_i8(dev(x), group)
    sync()
    qr, sr = oracle.quantize_act_i8(x, group)
    assert np.array_equal(host(qd), qr)
    assert np.array_equal(host(sd).view(np.uint32), sr.view(np.uint32))


def _weights(rng, wfmt, N, K, group):
    if wfmt == "q8":
        W = rng.integers(-127, 128, (N, K)).astype(np.int8)
        return W, ((0.02 / 127) * rng.uniform(0.5, 1.5, N)).astype(np.float32)
    W = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    return W, rng.uniform(0.005, 0.02, (N, K // group)).astype(np.float16).view(np.uint16)


def _pack(wfmt, W, S, group):
    return q.pack_q8(dev(W), dev(S)) if wfmt == "q8" else q.pack_q4(dev(W), dev(S), group)


A8_SHAPES = [
    # Qwen2.5-7B shape, INT4 groups of 64: fused qkv, o, gate/up, down, lm head
    ("q4", 4608, 3584, 64), ("q4", 3584, 3584, 64), ("q4", 37888, 3584, 64), ("q4", 3584, 18944, 64),
    ("q4", 152064, 3584, 64),
    # int8 rows (Qwen2.5-1.5B and Qwen3-8B shapes), activation groups of 64
    ("q8", 2048, 1536, 64), ("q8", 1536, 8960, 64), ("q8", 6144, 4096, 64), ("q8", 4096, 12288, 64),
    # other groups, ragged rows, short K
    ("q4", 1000, 320, 32), ("q4", 65, 256, 128), ("q8", 200, 64, 32), ("q8", 1, 4096, 4096), ("q4", 4097, 128, 64),
]


@pytest.mark.parametrize("wfmt,N,K,group", A8_SHAPES)
@pytest.mark.parametrize("split", [True, False])
def test_gemv_a8_parity(wfmt, N, K, group, split):
    rng = np.random.default_rng(N * 3 + K + group)
    W, S = _weights(rng, wfmt, N, K, group)
    x = _acts(rng, K, group)
    b = (0.02 * rng.standard_normal(N)).astype(np.float32)
    r = rng.standard_normal(N).astype(np.float32)
    Wp, Sp = _pack(wfmt, W, S, group)
    qd, sd = q.quantize_act_i8(dev(x), group)
    ws = q.gemv_workspace(wfmt, N, K) if split else None
    y0 = q.gemv_a8(wfmt, Wp, Sp, qd, sd, N, workspace=ws, group=group)
    y1 = q.gemv_a8(wfmt, Wp, Sp, qd, sd, N, bias=dev(b), residual=dev(r), workspace=ws, group=group)
    sync()
    qr, sr = oracle.quantize_act_i8(x, group)
    assert np.array_equal(host(qd), qr)
    ref0 = oracle.gemv_a8(wfmt, W, S, qr, sr, group=group)
    ref1 = oracle.gemv_a8(wfmt, W, S, qr, sr, bias=b, residual=r, group=group)
    assert rel_max_err(host(y0), ref0) <= 2e-5
    assert rel_max_err(host(y1), ref1) <= 2e-5
    if split:
        assert not host(ws)[:262144].any()  # arrival counters back at zero


@pytest.mark.parametrize("wfmt,N,K", [("q4", 300, 18944), ("q8", 300, 4096), ("q4", 64, 256)])
def test_gemv_a8_exact_case_bit_exact(wfmt, N, K):
    """Integer activations with 127 in every group (q = x, s = 1) and power-of-two weight scales:
    every product and partial sum is an exact fp32 value, so any summation order gives the oracle's
    result bit for bit."""
    rng = np.random.default_rng(7)
    group = 64
    W, S = _weights(rng, wfmt, N, K, group)
    if wfmt == "q8":
        S = np.full(N, 2.0 ** -10, np.float32)
    else:
        S = np.full(S.shape, 2.0 ** -6, np.float16).view(np.uint16)
    x = rng.integers(-127, 128, K).astype(np.float32)
    x[::group] = 127.0
    Wp, Sp = _pack(wfmt, W, S, group)
    qd, sd = q.quantize_act_i8(dev(x), group)
    y = q.gemv_a8(wfmt, Wp, Sp, qd, sd, N, workspace=q.gemv_workspace(wfmt, N, K), group=group)
    sync()
    assert np.array_equal(host(qd).astype(np.float32), x) and np.all(host(sd) == 1.0)
    ref = oracle.gemv_a8(wfmt, W, S, host(qd), host(sd), group=group)
    assert np.array_equal(host(y).view(np.uint32), ref.view(np.uint32))


def test_gemv_a8_against_fp_activation_gemv():
    """Path A differs from the fp32-activation GEMV by at most the activation rounding:
    |y_a8 - y_fp| <= sum_k |w[n][k]| s[k / group] / 2 (plus fp32 accumulation)."""
    rng = np.random.default_rng(9)
    wfmt, N, K, group = "q4", 4608, 3584, 64
    W, S = _weights(rng, wfmt, N, K, group)
    x = rng.standard_normal(K).astype(np.float32)
    Wp, Sp = _pack(wfmt, W, S, group)
    ws = q.gemv_workspace(wfmt, N, K)
    qd, sd = q.quantize_act_i8(dev(x), group)
    ya = host(q.gemv_a8(wfmt, Wp, Sp, qd, sd, N, workspace=ws, group=group))
    yf = host(q.gemv(wfmt, Wp, Sp, dev(x), N, workspace=ws, group=group))
    sync()
    sx = host(sd).astype(np.float64)
    absw = np.abs(np.stack([oracle.dequant_row(wfmt, W, S, n, K) for n in range(N)]).astype(np.float64))
    bound = absw @ np.repeat(sx, group) * 0.5
    assert np.all(np.abs(ya.astype(np.float64) - yf) <= bound * (1 + 1e-3) + 1e-4 * np.abs(yf).max())


def test_gemv_a8_rejects_bad_group():
    x = dev(np.ones(96, np.float32))
    with pytest.raises(q.QdecError):
        q.quantize_act_i8(x, 64)  # 96 is not a multiple of 64
