"""Whole-model greedy decode over 64 steps against the CPU oracle, in the benchmarked launch
configuration (every layer, default attention splits, hipGraph replay), with the per-layer trace.

Bars (the decode-step contract): per-layer hidden states max-abs error over max-abs reference
<= 1e-3 at every step; logits max-abs error <= 2e-2 at every step; greedy tokens identical at
every step, except where the oracle's own top-1/top-2 margin is inside the logits tolerance.  At
such a tie both tokens are correct and both sides continue with the oracle's token (teacher
forcing), so the run measures drift, not divergence after a tie.

The new token's k and v are rounded to bf16 when they enter the cache.  Where the GPU's fp32 value
and the oracle's lie on either side of a bf16 rounding midpoint, both codes are correct; a few
such ties happen at most steps.  Left alone, the two caches drift apart by them, and a later query
that attends strongly to such a token (in these synthetic models the appended tokens' k and v are
several times larger than the N(0,1) context, so queries attend mostly to them) sees the
difference.  They are resolved like token ties: the stored vectors are held to the hidden-state
bar (each differing code a correct bf16 rounding of a value within 1e-3 of the vector's max of the
oracle's unrounded value), and the GPU's codes then replace the oracle's, so each step is compared
from identical caches (if the step itself misses a bar, the oracle's step is first run again with
the GPU's codes forced, layer by layer).

The synthetic Qwen2.5-7B-shape model's greedy sequence is a fixed point (one token repeated), so
a free run re-checks one token id; a second run feeds 64 distinct seeded token ids to both sides
(teacher forcing throughout), so every step embeds and attends a different token.

The greedy argmax fused into the lm head's epilogue is checked for its tie rule (smallest index
among the maxima, across tiles of different reduction groups) with constructed lm-head rows.
"""
import time

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
KV_TOL = HIDDEN_TOL   # stored k, v: the hidden-state bar (x the vector's max |value|) beyond bf16 rounding
STEPS = 64


def _margin(logits):
    srt = np.sort(np.asarray(logits, np.float64))
    return float(srt[-1] - srt[-2])


def _bf16(code):
    return (np.asarray(code, np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16_half_step(v):
    """Half the spacing of bf16 values around v (8 significant bits; subnormal spacing 2^-133)."""
    _, e = np.frexp(np.abs(v))
    return np.where(v == 0, 2.0 ** -134, 0.5 * np.ldexp(1.0, np.maximum(e - 8, -133)))


def is_valid_rounding(gpu_codes, orc_codes, pre):
    """Where the GPU's stored bf16 codes for the new token differ from the oracle's, each GPU
    code must be a correct bf16 rounding of a value within KV_TOL x the vector's max |value| of
    the oracle's value before rounding: the stored k and v are held to the hidden-state bar,
    beyond the rounding to bf16 that the cache format imposes.  (At a rounding tie the two codes
    are neighbours around the oracle's value; downstream of one, a layer's inputs differ within
    the hidden-state bar, and so do its k and v.)  Returns (all valid, details of the differences
    that are not)."""
    diff = np.flatnonzero(gpu_codes.ravel() != orc_codes.ravel())
    g, o, x = gpu_codes.ravel()[diff], orc_codes.ravel()[diff], np.asarray(pre, np.float64).ravel()
    gv = _bf16(g)
    tol = KV_TOL * np.abs(x).max()
    bad = np.abs(gv - x[diff]) > tol + _bf16_half_step(gv)
    info = [(int(i), hex(int(a)), hex(int(c)), float(v), float(tol))
            for i, a, c, v in zip(diff[bad], g[bad], o[bad], x[diff][bad])][:4]
    return bool(not bad.any()), info


class Run:
    """One workload on both sides from the same host bytes: GPU step handle with the per-layer
    trace, and the oracle with its own copy of the KV cache."""

    def __init__(self, name):
        wl = synth.WORKLOADS[name]
        self.wl = wl
        model = synth.make_model(wl)
        kv = synth.make_kv(wl, wl.ctx + STEPS + 8)
        self.model = model
        self.pt = kv["page_table"]
        self.orc = oracle.OracleDecoder(model, kv)
        self.dk = q.upload_kv(kv, wl.kv_fmt)
        self.gpu = q.DecodeStep(q.upload_model(model), self.dk, pos0=wl.ctx, token0=model["token"], trace=True,
                                log_len=STEPS)
        assert self.gpu.cfg.num_splits == q.default_splits(wl.n_kv_heads, wl.ctx)
        self.forced_steps = []   # steps whose oracle step was run again with forced codes
        self.synced = []         # steps whose valid differing codes were copied into the oracle's cache

    def failure(self, s, ref):
        """The first bar the GPU's step misses against `ref`, or None."""
        tr = host(self.gpu.trace)
        for l in range(tr.shape[0]):
            e = rel_max_err(tr[l], ref["trace"][l])
            if e > HIDDEN_TOL:
                return "step %d: hidden after layer %d rel err %.3g" % (s, l, e)
        e = float(np.abs(host(self.gpu.logits) - ref["logits"]).max())
        if e > LOGIT_TOL:
            return "step %d: logits max abs err %.3g" % (s, e)
        return None

    def _code_diffs(self, pos, ref, skip=()):
        """Layers whose new-token cache codes differ between GPU and oracle:
        [(l, all valid, gpu k codes, gpu v codes, invalid k details, invalid v details)]."""
        pg, sl = int(self.pt[pos // 16]), pos % 16
        out = []
        for l in range(self.wl.n_layers):
            if l in skip:
                continue
            gk = self.dk["k"][l][pg, :, sl, :].cpu().numpy().view(np.uint16)
            gv = self.dk["v"][l][pg, :, sl, :].cpu().numpy().view(np.uint16)
            ok, ov = self.orc.k[l][pg, :, sl, :], self.orc.v[l][pg, :, sl, :]
            if np.array_equal(gk, ok) and np.array_equal(gv, ov):
                continue
            tk, ik = is_valid_rounding(gk, ok, ref["kv_pre"][l, 0])
            tv, iv = is_valid_rounding(gv, ov, ref["kv_pre"][l, 1])
            out.append((l, tk and tv, gk, gv, ik, iv))
        return out

    def oracle_step(self, s, pos, tok):
        """The oracle's step at pos, checked against the GPU's, after which both caches hold the
        same codes for the new token.

        Each layer's new k and v are rounded to bf16 on both sides; where the codes differ, each
        differing GPU code must be a correct rounding of a value within the hidden-state bar of
        the oracle's unrounded value (is_valid_rounding).  If every difference is valid and the GPU meets the
        bars, the GPU's codes are copied into the oracle's cache, so later
        steps attend over identical caches.  Otherwise (a bar missed, or a difference that is not
        valid) the layers are resolved in order: the first layer whose codes differ must
        differ by valid roundings only, the GPU's codes are forced into the oracle's step for it and the
        oracle's step is run again, until the codes agree in every layer; then the bars must
        hold."""
        ref = self.orc.step(pos, tok, trace=True, kv_pre=True)
        why = self.failure(s, ref)
        diffs = self._code_diffs(pos, ref)
        pg, sl = int(self.pt[pos // 16]), pos % 16
        if why is None and all(t for (_, t, *_r) in diffs):
            for (l, _, gk, gv, _ik, _iv) in diffs:
                self.orc.k[l][pg, :, sl, :] = gk
                self.orc.v[l][pg, :, sl, :] = gv
            if diffs:
                self.synced.append((s, [d[0] for d in diffs]))
            return ref
        tr = host(self.gpu.trace)
        errs = ["%.2g" % rel_max_err(tr[l], ref["trace"][l]) for l in range(min(6, tr.shape[0]))]
        summary = [(d[0], bool(d[1]), len(d[4]), len(d[5])) for d in diffs][:8]
        forced = {}
        for _ in range(self.wl.n_layers):
            diffs = self._code_diffs(pos, ref, skip=forced)
            if not diffs:
                break
            l, tie, gk, gv, ik, iv = diffs[0]
            assert tie, "step %d (%s): layer %d cache codes are not valid roundings: k %s v %s; hidden errs %s; " \
                        "diffs (layer, valid, bad k, bad v) %s; forced %s" % (s, why, l, ik, iv, errs, summary, sorted(forced))
            forced[l] = (gk, gv)
            ref = self.orc.step(pos, tok, trace=True, kv_pre=True, kv_force=forced)
        self.forced_steps.append((s, sorted(forced)))
        why2 = self.failure(s, ref)
        assert why2 is None, "%s; after forcing the GPU's cache codes of layers %s: %s" % (why, sorted(forced), why2)
        return ref


def _progress(name, s, t0):
    """One line per step (seen under pytest -s): a step of a large model with its oracle takes
    seconds of CPU time."""
    print("%s step %d done, %.1f s" % (name, s, time.time() - t0), flush=True)


@pytest.mark.parametrize("name", ["qwen2.5-7b-q4", "qwen2.5-1.5b-q8", "qwen3-8b-q8", "qwen2.5-7b-q4-32k"])
def test_greedy_64_steps_match_oracle(name):
    """64 free-running greedy steps on both sides, graph replay, every layer checked every step."""
    t0 = time.time()
    r = Run(name)
    pos0 = r.wl.ctx
    tok = r.model["token"]
    gpu_toks, ties = [], []
    with torch.cuda.stream(torch.cuda.Stream()):
        for s in range(STEPS):
            r.gpu.step(q.STEP_GRAPH)
            sync()
            ref = r.oracle_step(s, pos0 + s, tok)
            gtok = int(host(r.gpu.token)[0])
            gpu_toks.append(gtok)
            if gtok != ref["token"]:
                m = _margin(ref["logits"])
                assert m <= LOGIT_TOL, "%s step %d: token %d vs oracle %d (margin %.3g)" % (
                    name, s, gtok, ref["token"], m)
                ties.append((s, gtok, ref["token"], m))
                r.gpu.token.fill_(ref["token"])  # continue both sides from the oracle's token
            tok = ref["token"]
            _progress(name, s, t0)
        sync()
    assert r.gpu.read_error() == 0
    assert int(host(r.gpu.pos)[0]) == pos0 + STEPS
    assert host(r.gpu.token_log).tolist() == gpu_toks
    print("%s: %d/%d greedy tokens identical, token ties %s, cache codes synced at %d steps, forced at %s, "
          "first tokens %s" % (name, STEPS - len(ties), STEPS, ties, len(r.synced), r.forced_steps, gpu_toks[:8]))


def test_teacher_forced_64_distinct_tokens():
    """The Qwen2.5-7B-shape INT4 model fed 64 distinct seeded token ids on both sides (the
    token, position, KV append and attention differ at every step): per-layer hidden states and
    logits at every step, and each step's greedy token against the oracle's."""
    t0 = time.time()
    r = Run("qwen2.5-7b-q4")
    pos0 = r.wl.ctx
    toks = np.random.default_rng(20261202).choice(r.wl.vocab, STEPS, replace=False).astype(np.int32)
    argmax_equal = 0
    with torch.cuda.stream(torch.cuda.Stream()):
        for s in range(STEPS):
            r.gpu.token.fill_(int(toks[s]))
            r.gpu.step(q.STEP_GRAPH)
            sync()
            ref = r.oracle_step(s, pos0 + s, int(toks[s]))
            gtok = int(host(r.gpu.token)[0])
            if gtok == ref["token"]:
                argmax_equal += 1
            else:
                assert _margin(ref["logits"]) <= LOGIT_TOL, (s, gtok, ref["token"])
            _progress("teacher-forced", s, t0)
        sync()
    assert r.gpu.read_error() == 0
    print("teacher-forced: %d/%d greedy tokens identical, %d distinct outputs, cache codes synced at %d steps, "
          "forced at %s" % (argmax_equal, STEPS, len(set(host(r.gpu.token_log).tolist())), len(r.synced), r.forced_steps))


def _lm_tie_model(kind):
    """A one-layer Qwen2.5-7B-shape INT4 model whose lm head has all scales zero except for a few
    rows: `kind` "zero" leaves every logit exactly 0; "tie" gives three rows of one code row
    with equal scales (equal logits, tiles in reduction groups 36, 16 and 36) and two rows with
    the scales negated (the negated logit), so the maximum is attained by exactly one of the two
    sets, at indices in different tiles and groups."""
    wl = synth.WORKLOADS["qwen2.5-7b-q4"]
    model = synth.make_model(wl, n_layers=1)
    W, S = model["w_lm"], model["s_lm"]
    S[:] = 0
    pos_rows, neg_rows = [], []
    if kind == "tie":
        src = 64 * 100 + 5
        pos_rows = [64 * 100 + 5, 64 * 2000 + 7, 64 * 164 + 40]   # tiles 100, 2000, 164
        neg_rows = [64 * 37 + 1, 64 * 1500 + 63]                   # tiles 37, 1500
        code, scale = W[src].copy(), synth.f16_uniform(S.shape[1], 99, 1, 0.005, 0.02)
        for rw in pos_rows:
            W[rw], S[rw] = code, scale
        for rw in neg_rows:
            W[rw], S[rw] = code, scale ^ np.uint16(0x8000)
    return wl, model, pos_rows, neg_rows


@pytest.mark.parametrize("kind", ["zero", "tie"])
def test_lm_head_argmax_tie_rule(kind):
    """The greedy token written by the lm head's epilogue is the smallest index among equal maxima,
    also when the equal logits sit in tiles that the two-level reduction handles in different
    groups; all-zero logits give token 0."""
    wl, model, pos_rows, neg_rows = _lm_tie_model(kind)
    kv = synth.make_kv(wl, wl.ctx + 8, n_layers=1)
    st = q.DecodeStep(q.upload_model(model), q.upload_kv(kv, wl.kv_fmt), pos0=wl.ctx, token0=model["token"])
    with torch.cuda.stream(torch.cuda.Stream()):
        for mode in (q.STEP_EAGER, q.STEP_GRAPH):
            st.pos.fill_(wl.ctx)
            st.token.fill_(model["token"])
            st.step(mode)
            sync()
            lg = host(st.logits)
            tok = int(host(st.token)[0])
            ref = oracle.OracleDecoder(model, kv).step(wl.ctx, model["token"])
            assert float(np.abs(lg - ref["logits"]).max()) <= LOGIT_TOL
            if kind == "zero":
                assert not lg.any() and tok == 0 and ref["token"] == 0
                continue
            v = lg[pos_rows[0]]
            assert v != 0.0
            assert all(lg[rw] == v for rw in pos_rows) and all(lg[rw] == -v for rw in neg_rows)
            winners = pos_rows if v > 0 else neg_rows
            assert np.flatnonzero(lg == lg.max()).tolist() == sorted(winners)
            assert tok == min(winners) == ref["token"], (tok, winners, ref["token"])
    assert st.read_error() == 0
    st.close()


def test_kv_slot_overrun_sets_error_word():
    """A step at a position with no cache slot (an unmapped page-table entry, or past the page
    table) stores nothing, reports error 2 through the step's error word, and every kernel ends
    normally: the next step at a valid position runs clean."""
    wl = synth.WORKLOADS["qwen2.5-7b-q4"]
    model = synth.make_model(wl, n_layers=2)
    kv = synth.make_kv(wl, 48, n_layers=2, ctx=30)   # 3 pages: positions 0 .. 47
    kv["page_table"] = kv["page_table"].copy()
    kv["page_table"][2] = -1                          # positions 32 .. 47 unmapped
    dk = q.upload_kv(kv, wl.kv_fmt)
    st = q.DecodeStep(q.upload_model(model), dk, pos0=30, token0=model["token"])
    k_before = [host(t).copy() for t in dk["k"]]
    with torch.cuda.stream(torch.cuda.Stream()):
        for mode in (q.STEP_EAGER, q.STEP_GRAPH, q.STEP_EAGER | q.STEP_PER_OP):
            for pos, want in ((31, 0), (32, 2), (47, 2), (48, 2), (31, 0)):
                st.pos.fill_(pos)
                st.step(mode)
                sync()
                assert st.read_error() == want, (mode, pos)
    # only position 31 (page 1, slot 15) was ever written
    for before, t in zip(k_before, dk["k"]):
        after = host(t)
        pg = int(kv["page_table"][1])
        diff = np.argwhere(after.view(np.int16) != before.view(np.int16))
        assert all(int(d[0]) == pg and int(d[2]) == 15 for d in diff)
    st.close()
