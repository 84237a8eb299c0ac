"""Whole-step parity of qdec_decode_step against the CPU oracle.

Bars (from the decode-step contract): per-layer hidden states max-abs error over max-abs reference
<= 1e-3; logits max-abs error <= 2e-2; greedy tokens identical, except where the oracle's own
top-1/top-2 margin is inside the logits tolerance (then the step is a tie and both tokens are
correct); graph replay bitwise equal to eager launches.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import host, rel_max_err, sync

q = pytest.importorskip("quantized_gemv_gqa_amd")

pytestmark = pytest.mark.gpu

HIDDEN_TOL = 1e-3
LOGIT_TOL = 2e-2


class Pair:
    """One workload on both sides: GPU decode state and the oracle, from the same host bytes."""

    def __init__(self, wl, n_layers=None, extra_tokens=72, trace=True, log_len=0, pos0=None,
                 num_splits=None):
        self.wl = wl
        self.model = synth.make_model(wl, n_layers=n_layers)
        ctx = wl.ctx if pos0 is None else pos0
        self.kv = synth.make_kv(wl, ctx + extra_tokens, n_layers=n_layers, ctx=ctx)
        self.pos0 = ctx
        self.orc = oracle.OracleDecoder(self.model, self.kv)
        self.dm = q.upload_model(self.model)
        self.dk = q.upload_kv(self.kv, wl.kv_fmt)
        self.gpu = q.DecodeStep(self.dm, self.dk, pos0=ctx, token0=self.model.get("token", 0), trace=trace,
                                log_len=log_len, h0=self.model.get("h0"), num_splits=num_splits)

    def oracle_step(self, pos, token):
        return self.orc.step(pos, token, trace=True)


def check_step(gpu: "q.DecodeStep", ref: dict, wl, where: str):
    tr = host(gpu.trace)
    for l in range(tr.shape[0]):
        e = rel_max_err(tr[l], ref["trace"][l])
        assert e <= HIDDEN_TOL, "%s: hidden after layer %d rel err %.3g" % (where, l, e)
    if wl.has_lm_head:
        lg = host(gpu.logits)
        e = float(np.abs(lg - ref["logits"]).max())
        assert e <= LOGIT_TOL, "%s: logits max abs err %.3g" % (where, e)
        tok = int(host(gpu.token)[0])
        if tok != ref["token"]:
            srt = np.sort(ref["logits"].astype(np.float64))
            margin = srt[-1] - srt[-2]
            assert margin <= LOGIT_TOL, "%s: token %d vs oracle %d (margin %.3g)" % (where, tok, ref["token"], margin)
        return tok
    return None


def test_single_layer_step():
    """One Qwen2-style layer (hidden 896, int8 rows, fp32 contiguous KV of 256 tokens)."""
    wl = synth.WORKLOADS["layer-h896-q8"]
    p = Pair(wl)
    p.gpu.step(q.STEP_EAGER)
    sync()
    ref = p.oracle_step(p.pos0, 0)
    check_step(p.gpu, ref, wl, "layer")
    assert int(host(p.gpu.pos)[0]) == p.pos0 + 1
    # the appended K and V at the new position match the oracle's to the hidden-state bar
    t = p.pos0
    pg = p.kv["page_table"][t // 16]
    for name, mine, theirs in (("k", p.dk["k"][0], p.orc.k[0]), ("v", p.dk["v"][0], p.orc.v[0])):
        got = host(mine)[pg, :, t % 16, :]
        want = theirs[pg, :, t % 16, :]
        assert rel_max_err(got, want) <= HIDDEN_TOL, name
        # every other slot is untouched
        other = host(mine).copy()
        other[pg, :, t % 16, :] = 0
        base = p.kv[name][0].copy()
        base[pg, :, t % 16, :] = 0
        assert np.array_equal(other, base), name


@pytest.mark.parametrize("name,n_layers", [("qwen2.5-1.5b-q8", 2), ("qwen2.5-7b-q4", 2), ("qwen3-8b-q8", 2),
                                           ("qwen2.5-7b-q4-32k", 1)])
def test_truncated_model_steps(name, n_layers):
    """Full widths and vocab, few layers: three steps (eager, graph, graph) against the oracle."""
    wl = synth.WORKLOADS[name]
    p = Pair(wl, n_layers=n_layers)
    tok = p.model["token"]
    with torch.cuda.stream(torch.cuda.Stream()):
        for s, mode in enumerate((q.STEP_EAGER, q.STEP_GRAPH, q.STEP_GRAPH)):
            p.gpu.step(mode)
            sync()
            ref = p.oracle_step(p.pos0 + s, tok)
            gtok = check_step(p.gpu, ref, wl, "%s step %d" % (name, s))
            tok = gtok  # teacher-force with the GPU token (identical unless a tie)
            p.gpu.token.fill_(tok)
        sync()


MODES = (q.STEP_EAGER, q.STEP_GRAPH, q.STEP_EAGER | q.STEP_PER_OP, q.STEP_GRAPH | q.STEP_PER_OP)


def test_graph_replay_equals_eager_bitwise():
    """Same device code either way: graph replays and the two-launch layer kernels must reproduce
    per-op eager launches bit for bit, across a page boundary (positions 15 -> 16 -> 17), with pos
    and token read from device memory."""
    wl = synth.WORKLOADS["qwen2.5-7b-q4"]
    model = synth.make_model(wl, n_layers=2)
    kv = synth.make_kv(wl, 64, n_layers=2, ctx=15)
    dm = q.upload_model(model)
    outs = {}
    for mode in MODES:
        dk = q.upload_kv(kv, wl.kv_fmt)
        st = q.DecodeStep(dm, dk, pos0=15, token0=model["token"], trace=True, log_len=8, num_splits=3)
        res = []
        with torch.cuda.stream(torch.cuda.Stream()):
            for _ in range(4):
                st.step(mode)
                sync()
                res.append((host(st.logits).copy(), host(st.trace).copy(), int(host(st.token)[0])))
        assert st.read_error() == 0, mode
        outs[mode] = (res, host(st.token_log).copy(), int(host(st.pos)[0]), [host(t).copy() for t in dk["k"]])
        st.close()
    re, le, pe, ke = outs[q.STEP_EAGER | q.STEP_PER_OP]
    assert pe == 19 and list(le[:4]) == [r[2] for r in re]
    for mode in MODES:
        rg, lg, pg, kg = outs[mode]
        assert pg == pe and np.array_equal(le, lg), mode
        for a, b in zip(re, rg):
            assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32)), mode
            assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32)), mode
            assert a[2] == b[2], mode
        for a, b in zip(ke, kg):
            assert np.array_equal(a, b), mode


@pytest.mark.parametrize("name", ["qwen2.5-1.5b-q8", "qwen3-8b-q8"])
def test_layer_kernels_equal_per_op_bitwise(name):
    """The other fused-layer shapes (6 and 4 q heads per KV head, int8 weights, q/k norm) against
    per-op launches, bit for bit, and the step's error word stays clear."""
    wl = synth.WORKLOADS[name]
    model = synth.make_model(wl, n_layers=2)
    kv = synth.make_kv(wl, 40, n_layers=2, ctx=30)
    dm = q.upload_model(model)
    outs = {}
    for mode in (q.STEP_GRAPH, q.STEP_GRAPH | q.STEP_PER_OP):
        dk = q.upload_kv(kv, wl.kv_fmt)
        st = q.DecodeStep(dm, dk, pos0=30, token0=model["token"], trace=True, num_splits=2)
        assert st.layer_blocks > 0, "this shape must get the fused attention launch"
        res = []
        with torch.cuda.stream(torch.cuda.Stream()):
            for _ in range(3):
                st.step(mode)
                sync()
                res.append((host(st.logits).copy().view(np.uint32), host(st.trace).copy().view(np.uint32)))
        assert st.read_error() == 0
        outs[mode] = res
        st.close()
    for a, b in zip(outs[q.STEP_GRAPH], outs[q.STEP_GRAPH | q.STEP_PER_OP]):
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_fused_attention_launch_is_used_at_full_size(name):
    """Every workload whose shape the fused attention launch supports (head dim 128, 4/6/7/8 q
    heads per KV head) gets it at its full size and default splits: a plan that stops fitting
    would otherwise fall back to per-op launches silently."""
    wl = synth.WORKLOADS[name]
    G = wl.n_heads // wl.n_kv_heads
    model = synth.make_model(wl, n_layers=1)
    kv = synth.make_kv(wl, 40, n_layers=1, ctx=30)
    start = {"token0": model["token"]} if "token" in model else {"h0": model["h0"]}
    st = q.DecodeStep(q.upload_model(model), q.upload_kv(kv, wl.kv_fmt), pos0=30, **start)
    want = wl.head_dim == 128 and G in (4, 6, 7, 8)
    assert (st.layer_blocks > 0) == want, (name, st.layer_blocks)
    st.close()


def test_step_errors_are_reported():
    wl = synth.WORKLOADS["layer-h896-q8"]
    p = Pair(wl)
    with pytest.raises(q.QdecError):
        p.gpu.step(mode=7)
    with pytest.raises(q.QdecError):
        p.gpu.step(q.STEP_GRAPH, stream=torch.cuda.default_stream())  # capture needs its own stream


def test_step_sampling_matches_sampler_on_its_logits():
    """Sampling inside the step: the logits meet the logits bar against the oracle, and the token
    is exactly the sampler's draw (oracle) from those logits at draw counter = step count; graph
    replays draw fresh numbers; greedy comes back when the temperature is set to 0."""
    wl = synth.WORKLOADS["qwen2.5-7b-q4"]
    p = Pair(wl, n_layers=2, trace=False, log_len=8)
    T32, p32 = float(np.float32(0.7)), float(np.float32(0.9))
    p.gpu.set_sampling(0.7, 40, 0.9, seed=5)
    tok = p.model["token"]
    toks = []
    with torch.cuda.stream(torch.cuda.Stream()):
        for s, mode in enumerate((q.STEP_EAGER, q.STEP_GRAPH, q.STEP_GRAPH, q.STEP_GRAPH)):
            p.gpu.step(mode)
            sync()
            ref = p.oracle_step(p.pos0 + s, tok)
            lg = host(p.gpu.logits)
            assert float(np.abs(lg - ref["logits"]).max()) <= LOGIT_TOL
            gtok = int(host(p.gpu.token)[0])
            assert gtok == oracle.sample(lg, T32, 40, p32, seed=5, step=s), s
            toks.append(gtok)
            tok = gtok
        p.gpu.set_sampling(0.0)
        p.gpu.step(q.STEP_GRAPH)
        sync()
        assert int(host(p.gpu.token)[0]) == int(np.argmax(host(p.gpu.logits)))
    assert host(p.gpu.token_log)[:4].tolist() == toks
    assert int(host(p.gpu.step_count)[0]) == 5 and int(host(p.gpu.pos)[0]) == p.pos0 + 5


@pytest.mark.parametrize("name", ["qwen2.5-7b-q4", "qwen2.5-1.5b-q8", "qwen3-8b-q8", "qwen2.5-7b-q4-32k"])
def test_full_model_graph_steps_match_oracle(name):
    """Whole models in the benchmarked launch configuration (the Qwen2.5-7B-shape INT4 model with
    its 4096-token shuffled paged bf16 context is the benchmark itself): every layer, default
    attention splits, no per-layer trace, hipGraph replay.  Three steps, each against the oracle
    continuing from the GPU's token: final hidden state, every logit and the greedy token to the
    step bars."""
    wl = synth.WORKLOADS[name]
    p = Pair(wl, extra_tokens=8, trace=False)
    assert p.gpu.cfg.num_splits == q.default_splits(wl.n_kv_heads, wl.ctx)
    tok = p.model["token"]
    with torch.cuda.stream(torch.cuda.Stream()):
        for s in range(3):
            p.gpu.step(q.STEP_GRAPH)
            sync()
            ref = p.orc.step(p.pos0 + s, tok)
            e = rel_max_err(host(p.gpu.hidden), ref["h"])
            assert e <= HIDDEN_TOL, "step %d: final hidden rel err %.3g" % (s, e)
            lg = host(p.gpu.logits)
            e = float(np.abs(lg - ref["logits"]).max())
            assert e <= LOGIT_TOL, "step %d: logits max abs err %.3g" % (s, e)
            gtok = int(host(p.gpu.token)[0])
            if gtok != ref["token"]:
                srt = np.sort(ref["logits"].astype(np.float64))
                assert srt[-1] - srt[-2] <= LOGIT_TOL, (s, gtok, ref["token"])
            tok = gtok
            p.gpu.token.fill_(tok)
    assert int(host(p.gpu.pos)[0]) == p.pos0 + 3
