"""Batched decode (several sequences, one token each, shared paged KV pool) against the oracle.

Bars: the skinny GEMM per column like the GEMV (max-abs error over max-abs reference <= 2e-5);
the batched step per running slot like the single step (hidden 1e-3 relative, logits 2e-2
max-abs, greedy tokens equal unless the oracle's top-2 margin is inside the logits bar); idle slots
untouched; slot placement in the pool does not change results (bitwise).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev, host, rel_max_err, sync

q = pytest.importorskip("quantized_gemv_gqa_amd")

pytestmark = pytest.mark.gpu

HIDDEN_TOL = 1e-3
LOGIT_TOL = 2e-2


def _weights(rng, wfmt, N, K, group=64):
    if wfmt == "q8":
        W = rng.integers(-127, 128, (N, K)).astype(np.int8)
        return W, ((0.02 / 127) * rng.uniform(0.5, 1.5, N)).astype(np.float32)
    W = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    return W, rng.uniform(0.005, 0.02, (N, K // group)).astype(np.float16).view(np.uint16)


GEMM_SHAPES = [("q4", 4608, 3584), ("q4", 3584, 3584), ("q4", 37888, 3584), ("q4", 3584, 18944),
               ("q8", 6144, 4096), ("q8", 1536, 8960), ("q4", 1000, 320), ("q8", 200, 64), ("q4", 65, 128)]


@pytest.mark.parametrize("wfmt,N,K", GEMM_SHAPES)
@pytest.mark.parametrize("nb", [1, 3, 8])
@pytest.mark.parametrize("split", [True, False])
def test_gemm_parity(wfmt, N, K, nb, split):
    rng = np.random.default_rng(N + K + nb)
    W, S = _weights(rng, wfmt, N, K)
    X = rng.standard_normal((nb, K)).astype(np.float32)
    b = (0.02 * rng.standard_normal(N)).astype(np.float32)
    R = rng.standard_normal((nb, N)).astype(np.float32)
    Wp, Sp = (q.pack_q8(dev(W), dev(S)) if wfmt == "q8" else q.pack_q4(dev(W), dev(S), 64))
    ws = q.gemm_workspace(wfmt, N, K, nb) if split else None
    Y0 = q.gemm(wfmt, Wp, Sp, dev(X), N, workspace=ws)
    Y1 = q.gemm(wfmt, Wp, Sp, dev(X), N, bias=dev(b), residual=dev(R), workspace=ws)
    sync()
    for c in range(nb):
        assert rel_max_err(host(Y0)[c], oracle.gemv(wfmt, W, S, X[c])) <= 2e-5, c
        assert rel_max_err(host(Y1)[c], oracle.gemv(wfmt, W, S, X[c], bias=b, residual=R[c])) <= 2e-5, c
    if split:
        assert not host(ws)[:262144].any()


class Batch:
    """One batched workload on both sides: device pools/tables and the oracle's copy."""

    def __init__(self, name, ctxs, n_layers=2, max_blocks=None, spare=8, num_splits=8):
        wl = synth.WORKLOADS[name] if isinstance(name, str) else name
        self.wl = wl
        self.model = synth.make_model(wl, n_layers=n_layers)
        mb = max_blocks or max(-(-(c + 8) // 16) for c in ctxs) + 1
        self.kv = synth.make_kv_batch(wl, ctxs, mb, n_layers=n_layers, spare_pages=spare)
        self.tables = self.kv["block_tables"].copy()
        self.free = list(self.kv["free_pages"])
        self.orc = oracle.OracleDecoder(self.model, {"page_table": self.tables[0], "k": self.kv["k"], "v": self.kv["v"]})
        self.dm = q.upload_model(self.model)
        dt = torch.int16 if wl.kv_fmt == "bf16" else None
        self.kp = [dev(a, dt) for a in self.kv["k"]]
        self.vp = [dev(a, dt) for a in self.kv["v"]]
        B = len(ctxs)
        self.B = B
        self.d_tables = dev(self.tables)
        self.d_pos = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.d_tok = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.gpu = q.BatchDecode(self.dm, self.kp, self.vp, self.d_tables, self.d_pos, self.d_tok, num_splits=num_splits)
        self.h_orc = np.zeros((B, wl.hidden), np.float32)

    def map_blocks(self, pos):
        for b, p in enumerate(pos):
            if p >= 0 and self.tables[b, p // 16] < 0:
                self.tables[b, p // 16] = self.free.pop()
        self.d_tables.copy_(torch.from_numpy(self.tables))


def _check_slots(bt, pos, toks, ref_next, ref_lg, where):
    lg = host(bt.gpu.logits)
    hg = host(bt.gpu.hidden)
    tg = host(bt.d_tok)
    for b in range(bt.B):
        if pos[b] < 0:
            continue
        assert float(np.abs(lg[b] - ref_lg[b]).max()) <= LOGIT_TOL, (where, b)
        assert rel_max_err(hg[b], bt.h_orc[b]) <= HIDDEN_TOL, (where, b)
        if tg[b] != ref_next[b]:
            srt = np.sort(ref_lg[b].astype(np.float64))
            assert srt[-1] - srt[-2] <= LOGIT_TOL, (where, b, tg[b], ref_next[b])
    return tg


def test_batch_step_matches_oracle():
    """Four slots of different lengths: slot 1 sits out step 1 and crosses a page boundary into a
    block mapped on demand, slot 3 joins at step 2; eager first, then graph replays with the slots
    changed in device memory between them."""
    ctxs = [40, 15, 100, 63]
    bt = Batch("qwen2.5-7b-q4", ctxs)
    toks = np.array([bt.model["token"], 5, 77, 1234], np.int32)
    pos = np.array(ctxs, np.int32)
    plan = [[1, 1, 1, 0], [1, 0, 1, 0], [1, 1, 1, 1], [1, 1, 0, 1]]
    with torch.cuda.stream(torch.cuda.Stream()):
        for s, act in enumerate(plan):
            ps = np.where(np.array(act) > 0, pos, -1).astype(np.int32)
            bt.map_blocks(ps)
            bt.d_pos.copy_(torch.from_numpy(ps))
            bt.d_tok.copy_(torch.from_numpy(toks))
            idle_before = {b: (host(bt.gpu.hidden)[b].copy(), host(bt.gpu.logits)[b].copy()) for b in range(4) if ps[b] < 0}
            bt.gpu.step(q.STEP_EAGER if s == 0 else q.STEP_GRAPH)
            sync()
            nxt, lg = bt.orc.step_batch(bt.tables, ps, toks, bt.h_orc)
            tg = _check_slots(bt, ps, toks, nxt, lg, "step %d" % s)
            pg = host(bt.d_pos)
            for b in range(4):
                if ps[b] < 0:
                    hb, lb = idle_before[b]
                    assert pg[b] == -1 and np.array_equal(host(bt.gpu.hidden)[b], hb)
                    assert np.array_equal(host(bt.gpu.logits)[b], lb)
                else:
                    assert pg[b] == ps[b] + 1
                    toks[b] = tg[b]
                    pos[b] += 1
    assert bt.gpu.kernel_count == 1 + 5 * 2 + 3


def test_batch_long_contexts_at_the_split_cap():
    """Eight sequences near 4096 tokens with the split count batch_splits picks there: 8 sequences
    x 4 KV heads x 8 splits = 256 attention workgroups, the cap.  Two layers of the Qwen2.5-7B
    shape, an eager step then a graph replay, against the oracle."""
    ctxs = [4096 - 37 * b for b in range(8)]
    S = q.batch_splits(8, 4, max(ctxs))
    assert S * 8 * 4 == 256, S
    bt = Batch("qwen2.5-7b-q4", ctxs, num_splits=S)
    rng = np.random.default_rng(4096)
    toks = rng.integers(0, bt.wl.vocab, 8).astype(np.int32)
    pos = np.array(ctxs, np.int32)
    with torch.cuda.stream(torch.cuda.Stream()):
        for s in range(2):
            bt.map_blocks(pos)
            bt.d_pos.copy_(torch.from_numpy(pos))
            bt.d_tok.copy_(torch.from_numpy(toks))
            bt.gpu.step(q.STEP_EAGER if s == 0 else q.STEP_GRAPH)
            sync()
            nxt, lg = bt.orc.step_batch(bt.tables, pos, toks, bt.h_orc)
            tg = _check_slots(bt, pos, toks, nxt, lg, "step %d" % s)
            assert np.array_equal(host(bt.d_pos), pos + 1)
            toks = tg.copy()
            pos = pos + 1


@pytest.mark.parametrize("wfmt", ["q4", "q8"])
@pytest.mark.parametrize("ctxs", [[33], [20, 33], [20, 33, 7], [5, 9, 17, 30, 41, 47, 64, 70]])
def test_batch_wide_hidden_matches_oracle(wfmt, ctxs):
    """Hidden 4160 (65 tiles of 64 rows): each folded RMSNorm adds more than 64 per-tile sums of
    squares per column, and the last tile is ragged for the norm's producers; 1, 2, 3 and 8 slots
    take the one-, two-, four- and eight-column GEMMs."""
    from dataclasses import replace
    wl = replace(synth.WORKLOADS["qwen2.5-7b-q4"], name="wide-h4160-" + wfmt, hidden=4160, inter=512, vocab=1000,
                 wfmt=wfmt, ctx=64, shuffled_pages=True, seed=1010)
    bt = Batch(wl, ctxs, n_layers=1)
    B = len(ctxs)
    toks = (np.arange(B, dtype=np.int32) * 97 + 3) % wl.vocab
    pos = np.array(ctxs, np.int32)
    with torch.cuda.stream(torch.cuda.Stream()):
        for s in range(2):
            bt.map_blocks(pos)
            bt.d_pos.copy_(torch.from_numpy(pos))
            bt.d_tok.copy_(torch.from_numpy(toks))
            bt.gpu.step(q.STEP_GRAPH)
            sync()
            nxt, lg = bt.orc.step_batch(bt.tables, pos, toks, bt.h_orc)
            tg = _check_slots(bt, pos, toks, nxt, lg, "step %d" % s)
            toks = tg.astype(np.int32)
            pos = pos + 1


def test_batch_placement_does_not_matter():
    """Three slots with the same context values and token but different physical pages give the
    same results bit for bit."""
    ctx = 37
    bt = Batch("qwen2.5-7b-q4", [ctx, ctx, ctx], spare=4)
    # give every slot slot 0's context values (copy its pages into the others' pages)
    for l in range(2):
        for pool in (bt.kp[l], bt.vp[l]):
            for b in (1, 2):
                for blk in range(-(-(ctx + 1) // 16)):
                    pool[int(bt.tables[b, blk])] = pool[int(bt.tables[0, blk])]
    sync()
    ps = np.full(3, ctx, np.int32)
    bt.d_pos.copy_(torch.from_numpy(ps))
    bt.d_tok.fill_(int(bt.model["token"]))
    with torch.cuda.stream(torch.cuda.Stream()):
        bt.gpu.step(q.STEP_GRAPH)
        sync()
    lg, hg = host(bt.gpu.logits), host(bt.gpu.hidden)
    for b in (1, 2):
        assert np.array_equal(lg[b].view(np.uint32), lg[0].view(np.uint32))
        assert np.array_equal(hg[b].view(np.uint32), hg[0].view(np.uint32))
