"""The allocation-free INT4 GEMV (qdec_gemv_q4_noalloc) against qdec_gemv_q4 with a workspace.

Both run the same kernels on the same split plan, so y must be equal bit for bit.  Two calls in
a row on the allocation-free entry point, the second on a smaller, ragged matrix with another
group size, check that the shared static scratch carries nothing from one call into the next;
both are also held to the GEMV parity bar against the oracle (max-abs error over max-abs
reference <= 2e-5).  A shape beyond the static scratch is refused before any HIP call, which is
checked without a GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev, host, rel_max_err

q = pytest.importorskip("quantized_gemv_gqa_amd")

SCRATCH_BYTES = 768 * 1024


def _case(rng, N, K, group):
    W = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    S = rng.uniform(0.005, 0.02, (N, K // group)).astype(np.float16).view(np.uint16)
    x = rng.standard_normal(K).astype(np.float32)
    b = (0.02 * rng.standard_normal(N)).astype(np.float32)
    r = rng.standard_normal(N).astype(np.float32)
    return W, S, x, b, r


def test_noalloc_refuses_shapes_beyond_its_static_scratch():
    L = q.lib()
    N, K = 8256, 4096  # 129 tiles of 64 rows split 16 ways: 2064 units of partial sums
    assert L.qdec_gemv_workspace_bytes(q.W_Q4, N, K) > SCRATCH_BYTES
    # the refusal precedes every HIP call, so aligned stand-in addresses suffice
    Wp, Sp, x, y = 1 << 24, 1 << 25, 1 << 26, 1 << 27
    st = L.qdec_gemv_q4_noalloc(Wp, Sp, 64, x, None, None, y, N, K, None)
    assert st == q.QDEC_EINVAL
    assert b"static" in L.qdec_last_error()
    # the largest decode shapes fit: gate/up of Qwen2.5-7B and of Qwen2.5-1.5B
    assert L.qdec_gemv_workspace_bytes(q.W_Q4, 37888, 3584) <= SCRATCH_BYTES
    assert L.qdec_gemv_workspace_bytes(q.W_Q4, 17920, 1536) <= SCRATCH_BYTES


@pytest.mark.gpu
def test_noalloc_gemv_equals_workspace_gemv_on_consecutive_calls():
    rng = np.random.default_rng(20240607)
    # qkv of Qwen2.5-7B (72 tiles, split 14 ways), then a smaller matrix with a ragged last tile
    cases = [(4608, 3584, 64), (1000, 1024, 128)]
    data, packed, got = [], [], []
    for N, K, group in cases:
        W, S, x, b, r = _case(rng, N, K, group)
        data.append((W, S, x, b, r))
        Wp, Sp = q.pack_q4(dev(W), dev(S), group)
        packed.append((Wp, Sp, dev(x), dev(b), dev(r)))
    torch.cuda.synchronize()
    for (N, K, group), (Wp, Sp, x, b, r) in zip(cases, packed):
        print("qdec_gemv_q4_noalloc N=%d K=%d group=%d" % (N, K, group), flush=True)
        got.append(q.gemv_q4_noalloc(Wp, Sp, x, N, bias=b, residual=r, group=group))
    torch.cuda.synchronize()
    for (N, K, group), (Wp, Sp, x, b, r), y, (W, S, xh, bh, rh) in zip(cases, packed, got, data):
        ws = q.gemv_workspace("q4", N, K)
        ref = q.gemv("q4", Wp, Sp, x, N, bias=b, residual=r, workspace=ws, group=group)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), "N=%d K=%d: differs from qdec_gemv_q4 with a workspace" % (N, K)
        want = oracle.gemv("q4", W, S, xh, bias=bh, residual=rh, group=group)
        assert rel_max_err(host(y), want) <= 2e-5
