"""On-GPU sampling (qdec_sample) against the CPU oracle.

Bar: the token is identical.  Every decision on both sides is a comparison of fp32 logits, of
fp32-rounded keys computed from the same fp64 expression, or of fp64 sums taken in the same order,
so the two sides agree exactly (the only freedom is a last-ulp difference of fp64 exp/log between
the device and host math libraries, which cannot flip a decision except at an exact boundary).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev, host, sync

q = pytest.importorskip("quantized_gemv_gqa_amd")

pytestmark = pytest.mark.gpu


def _logits(rng, V):
    """Heavy-tailed logits (a few dominant tokens, a long flat tail), ties at the top and at the
    typical top-k boundaries."""
    lg = (1.5 * rng.standard_normal(V)).astype(np.float32)
    hot = rng.choice(V, size=min(V, 40), replace=False)
    lg[hot] += rng.uniform(4.0, 9.0, hot.size).astype(np.float32)
    order = np.argsort(-lg, kind="stable")
    if V > 300:
        lg[order[1]] = lg[order[0]]          # tie at the top
        lg[order[20]] = lg[order[19]]        # tie across the top-20 boundary
        lg[order[50:53]] = lg[order[49]]     # ties across the top-50 boundary
    return lg


PARAMS = [(0.0, 0, 1.0), (1.0, 0, 1.0), (0.6, 20, 0.95), (0.7, 50, 1.0), (1.0, 256, 0.9), (1.3, 1, 1.0),
          (0.8, 200, 0.5), (0.9, 255, 1.0), (2.0, 20, 0.99), (0.5, 64, 0.7)]


@pytest.mark.parametrize("V", [152064, 151936, 4864, 300, 5])
def test_sample_matches_oracle(V):
    rng = np.random.default_rng(V)
    lg = _logits(rng, V)
    d = dev(lg)
    ws = q.sample_workspace()
    step = torch.zeros(1, dtype=torch.int32, device="cuda")
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    for T, k, p in PARAMS:
        T32, p32 = float(np.float32(T)), float(np.float32(p))
        for s in (0, 1, 7, 123456):
            step.fill_(s)
            q.sample(d, T32, k, p32, seed=2024, step=step, token=tok, workspace=ws)
            sync()
            want = oracle.sample(lg, T32, k, p32, seed=2024, step=s)
            assert int(host(tok)[0]) == want, (V, T, k, p, s)


def test_sample_equal_logits_and_null_step():
    """All logits equal: top-k keeps the smallest indices; a NULL step pointer draws at step 0."""
    lg = np.zeros(1000, np.float32)
    d = dev(lg)
    ws = q.sample_workspace()
    got = set()
    for seed in range(40):
        t = int(host(q.sample(d, 1.0, 3, 1.0, seed=seed, workspace=ws))[0])
        assert t == oracle.sample(lg, 1.0, 3, 1.0, seed=seed, step=0)
        got.add(t)
    assert got == {0, 1, 2}


def test_sample_frequencies_follow_softmax():
    """5000 draws at steps 0..4999: chi-square against softmax(l / T) over the top-k set."""
    lg = np.array([1.0, 2.0, 0.5, 2.0, -1.0, 0.0, 1.5, -0.5], np.float32)
    d = dev(lg)
    ws = q.sample_workspace()
    step = torch.zeros(1, dtype=torch.int32, device="cuda")
    toks = torch.empty(5000, dtype=torch.int32, device="cuda")
    for s in range(5000):
        step.fill_(s)
        q.sample(d, 0.8, 5, 1.0, seed=7, step=step, token=toks[s:s + 1], workspace=ws)
    sync()
    t = host(toks)
    keep = [1, 3, 6, 0, 2]  # the five largest logits
    assert set(t.tolist()) <= set(keep)
    z = lg[keep].astype(np.float64) / float(np.float32(0.8))
    pr = np.exp(z - z.max())
    pr /= pr.sum()
    cnt = np.array([(t == i).sum() for i in keep], np.float64)
    chi2 = float(((cnt - 5000 * pr) ** 2 / (5000 * pr)).sum())
    assert chi2 < 35.0, (cnt, 5000 * pr)
    for s in (0, 17, 4999):
        assert t[s] == oracle.sample(lg, float(np.float32(0.8)), 5, 1.0, seed=7, step=s)


def test_sample_in_graph_replays():
    """Captured with a step counter that the graph itself advances: each replay draws the next
    step's token, equal to the eager result at that step."""
    V = 152064
    rng = np.random.default_rng(5)
    lg = _logits(rng, V)
    d = dev(lg)
    ws = q.sample_workspace()
    step = torch.zeros(1, dtype=torch.int32, device="cuda")
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    log = torch.zeros(8, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        q.sample(d, 0.7, 40, 0.9, seed=99, step=step, token=tok, workspace=ws)
        sync()
        with torch.cuda.graph(g, stream=s):
            q.sample(d, 0.7, 40, 0.9, seed=99, step=step, token=tok, workspace=ws)
            log.index_copy_(0, step.long(), tok)
            step.add_(1)
        step.zero_()
        for _ in range(8):
            g.replay()
        sync()
    T32, p32 = float(np.float32(0.7)), float(np.float32(0.9))
    want = [oracle.sample(lg, T32, 40, p32, seed=99, step=i) for i in range(8)]
    assert host(log).tolist() == want
    assert int(host(step)[0]) == 8


def test_sample_rejects_unsupported():
    d = dev(np.zeros(1000, np.float32))
    with pytest.raises(q.QdecError):
        q.sample(d, 1.0, 0, 0.9)  # top-p over the whole vocabulary
    with pytest.raises(q.QdecError):
        q.sample(d, 1.0, 300, 1.0)
