"""Decode-step benchmark, one MI355X.  Default workload: the Qwen2.5-7B-shaped INT4 (groups of
64) model, paged bf16 KV of 4096 tokens, batch 1, greedy, one hipGraph replay per token;
`--workload` selects any other decode workload (the Qwen2.5-1.5B and Qwen3-8B shapes with INT8
weights, the 32K-context attention-stress case, or the single Qwen2-style layer, timed
cache-resident and cold).

Prints one JSON line.  `value` is decode throughput (tokens/s) over K timed graph replays with
the inputs resident in HBM; `kernels` gives every kernel role's duration (HIP events after each
launch of a few eager steps, on the launch stream), algorithmic bytes, GB/s and share of the
step; `roofline` is the role with the largest share; `cpu_baseline` times the CPU oracle on a
bounded sample (whole decode steps) of the same workload, and `oracle_token_check` compares its
greedy tokens with the GPU's from the same state.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
METRIC = "decode ms/token + achieved HBM GB/s (% of peak), Qwen2.5-7B-shape INT4, 1 GPU"
# HBM traffic of the dominant kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE counter runs, scaled by
# the same counters on a plain copy of known size; valid only for the kernel sources it was taken on
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kernel_traffic_qwen25_7b_q4.json")
KERNEL_SOURCES = ("quantized_gemv_gqa_amd/csrc/gemv.hip", "quantized_gemv_gqa_amd/csrc/layer.hip",
                  "quantized_gemv_gqa_amd/csrc/qdec_device.h", "quantized_gemv_gqa_amd/csrc/qdec_attention.h",
                  "quantized_gemv_gqa_amd/csrc/qdec_internal.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(role: str):
    """HBM bytes per launch of a kernel role from the committed counter record, or None if absent
    or taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch", {}).get(role)


def step_bytes(wl, T: int) -> int:
    """Algorithmic HBM bytes of one decode step at T = pos + 1 attended keys: every quantized
    weight and scale once, biases and norm gains, one embedding row, the lm head, the KV read
    (each KV byte once per KV head) and the new token's K/V write."""
    H, I, D = wl.hidden, wl.inter, wl.head_dim
    qd, kvd = wl.n_heads * D, wl.n_kv_heads * D
    mats = [(qd + 2 * kvd, H), (H, qd), (2 * I, H), (H, I)]

    def wbytes(N, K):
        if wl.wfmt == "q4":
            return N * K // 2 + N * (K // wl.group) * 2
        return N * K + N * 4

    per_layer = sum(wbytes(N, K) for N, K in mats) + 2 * H * 4
    if wl.qkv_bias:
        per_layer += (qd + 2 * kvd) * 4
    if wl.qk_norm:
        per_layer += 2 * D * 4
    kvb = 4 if wl.kv_fmt == "f32" else 2
    per_layer += 2 * kvd * kvb * T + 2 * kvd * kvb
    total = wl.n_layers * per_layer
    if wl.has_lm_head:
        total += wbytes(wl.vocab, H) + H * 4 + H * 2
    return total


def gemv_ab(wl, reps: int = 40, replays: int = 5):
    """A/B of the two GEMV activation paths at the workload's GEMV shapes: fp32 activations
    (qdec_gemv_*) against INT8 activations (qdec_quantize_act_i8 + qdec_gemv_*_a8).  Each shape
    streams copies of its weights totalling >= 1 GiB in rotation, so every launch reads HBM.
    `reps` launches are captured in one HIP graph (as in the decode step: no host launch cost
    between kernels); the per-launch time is the replays' HIP-event time over all launches."""
    import quantized_gemv_gqa_amd as q
    dev = "cuda:0"
    H, I, D = wl.hidden, wl.inter, wl.head_dim
    shapes = [("qkv", (wl.n_heads + 2 * wl.n_kv_heads) * D, H), ("o", H, wl.n_heads * D), ("gate_up", 2 * I, H),
              ("down", H, I)]
    if wl.has_lm_head:
        shapes.append(("lm_head", wl.vocab, H))
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    stream = torch.cuda.Stream()
    rows = []
    for name, N, K in shapes:
        wf = q.W_Q4 if wl.wfmt == "q4" else q.W_Q8
        wbytes = q.lib().qdec_packed_weight_bytes(wf, N, K)
        sbytes = q.lib().qdec_packed_scale_bytes(wf, N, K, wl.group)
        copies = max(2, -(-(1 << 30) // (wbytes + sbytes)))
        Ws, Ss = [], []
        for _ in range(copies):  # any bytes are valid codes; scales of the synthetic model's range
            Ws.append(torch.randint(0, 256, (wbytes,), dtype=torch.uint8, device=dev, generator=gen))
            if wl.wfmt == "q4":
                Ss.append((torch.rand(sbytes // 2, device=dev, generator=gen) * 0.015 + 0.005).half().view(torch.int16))
            else:
                Ss.append(torch.rand(sbytes // 4, device=dev, generator=gen) * (0.02 / 127))
        x = torch.randn(K, device=dev, generator=gen)
        y = torch.empty(N, device=dev)
        qa = torch.empty(K, dtype=torch.int8, device=dev)
        sx = torch.empty(K // wl.group, device=dev)
        ws = q.gemv_workspace(wl.wfmt, N, K, dev)
        torch.cuda.synchronize()

        def fp(i):
            q.gemv(wl.wfmt, Ws[i % copies], Ss[i % copies], x, N, y=y, workspace=ws, group=wl.group)

        def a8(i):
            q.gemv_a8(wl.wfmt, Ws[i % copies], Ss[i % copies], qa, sx, N, y=y, workspace=ws, group=wl.group)

        def quant(i):
            q.quantize_act_i8(x, wl.group, q=qa, sx=sx)

        def both(i):
            quant(i)
            a8(i)

        us = {}
        for key, fn in (("fp32_act", fp), ("quantize", quant), ("int8_act_gemv", a8), ("int8_act_total", both)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                fn(0)  # eager once (the first launch of a kernel loads its code object)
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=stream):
                    for i in range(reps):
                        fn(i)
                g.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(replays):
                    g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
            us[key] = e0.elapsed_time(e1) * 1e3 / (replays * reps)
            del g
        wsb = (wbytes + sbytes) * N // (((N + 63) // 64) * 64)  # unpadded weights + scales
        fp_bytes = wsb + 4 * K + 4 * N
        a8_bytes = wsb + K + 4 * (K // wl.group) + 4 * N
        rows.append({"gemv": name, "N": N, "K": K, "weight_copies": copies,
                     "us_fp32_act": us["fp32_act"], "us_int8_act_gemv": us["int8_act_gemv"],
                     "us_quantize": us["quantize"], "us_int8_act_total": us["int8_act_total"],
                     "gbps_fp32_act": fp_bytes / (us["fp32_act"] * 1e-6) / 1e9,
                     "gbps_int8_act_gemv": a8_bytes / (us["int8_act_gemv"] * 1e-6) / 1e9,
                     "speedup_gemv_only": us["fp32_act"] / us["int8_act_gemv"],
                     "speedup_with_quantize": us["fp32_act"] / us["int8_act_total"]})
        del Ws, Ss
        torch.cuda.empty_cache()
    return rows


def batch_bench(wl, B: int, K: int, W: int):
    """Batched decode: B sequences of the workload's context, one token each per step, one hipGraph
    replay per step over a shared paged KV pool with per-sequence block tables (blocks for the
    timed positions mapped before the timed region).  Throughput counts all B tokens of a step."""
    import quantized_gemv_gqa_amd as q
    import synth
    dev = "cuda:0"
    torch.cuda.set_device(0)
    t0 = time.time()
    model = synth.make_model(wl)
    ctxs = [wl.ctx] * B
    max_blocks = -(-(wl.ctx + W + K + 1) // 16)
    kv = synth.make_kv_batch(wl, ctxs, max_blocks, spare_pages=B * (max_blocks - (wl.ctx + 1 + 15) // 16))
    gen_s = time.time() - t0
    tables, free = kv["block_tables"].copy(), list(kv["free_pages"])
    for b in range(B):  # map every block the run will write (the host's on-demand allocation, done ahead)
        for blk in range(max_blocks):
            if tables[b, blk] < 0:
                tables[b, blk] = free.pop()
    dm = q.upload_model(model, dev)
    dt = torch.int16 if wl.kv_fmt == "bf16" else None
    kp = [torch.from_numpy(a.view(np.int16) if dt is not None else a).to(dev) for a in kv["k"]]
    vp = [torch.from_numpy(a.view(np.int16) if dt is not None else a).to(dev) for a in kv["v"]]
    del kv
    d_tables = torch.from_numpy(tables).to(dev)
    d_pos = torch.full((B,), wl.ctx, dtype=torch.int32, device=dev)
    d_tok = torch.full((B,), int(model.get("token", 0)), dtype=torch.int32, device=dev)
    splits = q.batch_splits(B, wl.n_kv_heads, wl.ctx)
    bd = q.BatchDecode(dm, kp, vp, d_tables, d_pos, d_tok, num_splits=splits, device=dev)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(W):
            bd.step(q.STEP_GRAPH)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            bd.step(q.STEP_GRAPH)
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    assert int(d_pos.min().item()) == wl.ctx + W + K
    # algorithmic bytes of a step: every weight once, each sequence's KV once
    T0 = wl.ctx + W + 1
    one = sum(step_bytes(wl, T0 + i) for i in range(K)) / K
    kv_one = 2 * wl.n_layers * wl.n_kv_heads * wl.head_dim * (2 if wl.kv_fmt == "bf16" else 4) * (T0 + K / 2)
    step_b = one + (B - 1) * kv_one
    return {"metric": "batched decode tokens/s, Qwen2.5-7B-shape INT4, 1 GPU", "value": B * K / (ms * K * 1e-3),
            "unit": "tokens/s", "batch": B, "steps": K, "warmup": W, "ms_per_step": ms, "higher_is_better": True,
            "data": "synthetic", "dtype": "f32",
            "config": {"workload": wl.name, "sequences": B, "context_each": wl.ctx, "kv": "one shared paged bf16 pool, "
                       "per-sequence block tables", "submission": "hipGraph replay per step",
                       "kernels_per_step": bd.kernel_count, "num_splits": splits},
            "step_bytes": step_b, "step_gbps": step_b / (ms * 1e-3) / 1e9, "gen_s": gen_s}


def prefill_bench(wl, T: int, reps: int, warmup: int):
    """Time to first token for a T-token prompt on an empty sequence: qdec_prefill on the step
    handle (every layer's projections on the matrix cores, attention, KV stored, lm head and the
    greedy first token), HIP events around each call on its stream; the position is reset to 0
    between calls, outside the timed region."""
    import quantized_gemv_gqa_amd as q
    import synth
    dev = "cuda:0"
    torch.cuda.set_device(0)
    t0 = time.time()
    model = synth.make_model(wl)
    kv = synth.make_kv(wl, T + 16, ctx=0)
    gen_s = time.time() - t0
    dm = q.upload_model(model, dev)
    dk = q.upload_kv(kv, wl.kv_fmt, dev)
    st = q.DecodeStep(dm, dk, pos0=0, token0=0, log_len=4, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    tokens = torch.randint(0, wl.vocab, (T,), dtype=torch.int32, device=dev, generator=gen)
    stream = torch.cuda.Stream()
    times = []
    with torch.cuda.stream(stream):
        for i in range(warmup + reps):
            st.pos.zero_()
            st.step_count.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st.prefill(tokens)
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= warmup:
                times.append(e0.elapsed_time(e1))
    assert int(st.pos.item()) == T
    ms = sum(times) / len(times)
    H, I, D = wl.hidden, wl.inter, wl.head_dim
    params = (wl.n_heads + 2 * wl.n_kv_heads) * D * H + H * wl.n_heads * D + 2 * I * H + H * I
    gemm_flop = 2.0 * T * params * wl.n_layers
    attn_flop = 2.0 * 2 * wl.n_layers * wl.n_heads * D * (T * (T + 1) / 2)
    return {"metric": "prefill time to first token, Qwen2.5-7B-shape INT4, 1 GPU", "value": ms, "unit": "ms",
            "higher_is_better": False, "prompt_tokens": T, "reps": reps, "warmup": warmup,
            "prefill_tokens_per_s": T / (ms * 1e-3), "dtype": "f16 matrix inputs as fp16 pairs, f32 accumulation",
            "data": "synthetic",
            "config": {"workload": wl.name, "layers": wl.n_layers, "context_before": 0},
            "roofline": {"bound": "mfma", "achieved": gemm_flop / (ms * 1e-3) / 1e12, "peak": 2500.0,
                         "unit": "TFLOP/s", "frac": gemm_flop / (ms * 1e-3) / 1e12 / 2500.0,
                         "note": "algorithmic GEMM flops (2 T x weights per layer) over the whole prefill time; "
                                 "the pair split issues 3 (INT4) matrix products per fragment"},
            "gemm_flop": gemm_flop, "attn_flop": attn_flop, "ms_each": times, "gen_s": gen_s}


def kernel_roles(wl, n_kernels: int, sampling: bool = False):
    """Role of each kernel of one step, in launch order: the embedding, then per layer either
    the fused attention launch + gate/up + down, or the five per-op launches, then the lm head
    (+ the two sampling launches), or the position update of a model without one."""
    L = wl.n_layers
    tail = ["lm_head"] + (["sample", "sample"] if sampling else []) if wl.has_lm_head else ["finish"]
    fused = 1 + 3 * L + len(tail)
    per_op = 1 + 5 * L + len(tail)
    if n_kernels == fused:
        body = ["attn_layer", "gate_up", "down"] * L
    elif n_kernels == per_op:
        body = ["qkv", "attention", "o", "gate_up", "down"] * L
    else:
        raise RuntimeError("unexpected kernel count %d for %d layers" % (n_kernels, L))
    return ["embed"] + body + tail


def role_bytes(wl, T: int) -> dict:
    """Algorithmic HBM bytes each kernel role moves at T attended keys (step_bytes split by kernel)."""
    H, I, D = wl.hidden, wl.inter, wl.head_dim
    qd, kvd = wl.n_heads * D, wl.n_kv_heads * D

    def wbytes(N, K):
        if wl.wfmt == "q4":
            return N * K // 2 + N * (K // wl.group) * 2
        return N * K + N * 4

    kvb = 4 if wl.kv_fmt == "f32" else 2
    qkv = wbytes(qd + 2 * kvd, H) + H * 4 + ((qd + 2 * kvd) * 4 if wl.qkv_bias else 0) + (2 * D * 4 if wl.qk_norm else 0)
    att = 2 * kvd * kvb * T + 2 * kvd * kvb
    o = wbytes(H, qd)
    r = {"embed": H * 2 if wl.has_lm_head else 0, "qkv": qkv, "attention": att, "o": o, "attn_layer": qkv + att + o,
         "gate_up": wbytes(2 * I, H) + H * 4, "down": wbytes(H, I), "finish": 0, "sample": 0}
    if wl.has_lm_head:
        r["lm_head"] = wbytes(wl.vocab, H) + H * 4
    return r


ROLE_NAMES = {"attn_layer": "fused attention launch (qkv GEMV + RoPE/KV append + split attention + merge + o GEMV)",
              "gate_up": "gate/up GEMV + SwiGLU", "down": "down GEMV + residual", "lm_head": "lm head GEMV + greedy argmax",
              "embed": "embedding row", "qkv": "qkv GEMV", "attention": "split attention + merge", "o": "o GEMV",
              "finish": "position update", "sample": "sampling"}


def per_kernel_roofline(wl, st, stream, reps: int):
    """Per-kernel durations of `reps` eager steps (a HIP event after every launch, on the launch
    stream), grouped by role: average microseconds, algorithmic bytes and GB/s of each role, and
    its share of the summed kernel time."""
    times = []
    T0 = int(st.pos.item()) + 1
    for _ in range(reps):
        times.append(st.kernel_times(stream=stream))
    n = len(times[0])
    roles = kernel_roles(wl, n, sampling=False)
    rb = role_bytes(wl, T0 + reps // 2)
    acc = {}
    for t in times:
        for role, us in zip(roles, t):
            a = acc.setdefault(role, [0.0, 0])
            a[0] += us
            a[1] += 1
    total = sum(sum(t) for t in times) / reps
    out = []
    for role, (us_sum, cnt) in acc.items():
        per_step = us_sum / reps
        avg = us_sum / cnt
        b = rb.get(role, 0)
        out.append({"role": role, "kernel": ROLE_NAMES.get(role, role), "launches_per_step": cnt // reps,
                    "us_per_launch": avg, "bytes_per_launch": b,
                    "gbps": (b / (avg * 1e-6) / 1e9) if b else None,
                    "frac_of_peak": (b / (avg * 1e-6) / 1e9 / HBM_PEAK_GBPS) if b else None,
                    "share_of_step": per_step / total})
    out.sort(key=lambda r: -r["share_of_step"])
    return out, total


def stream_read_gbps(dev, stream, gib: float = 2.0, reps: int = 8, warm: int = 3):
    """Plain streaming read of `gib` GiB (qdec_stream_read), HIP events around `reps` reads after
    `warm` untimed ones (the first reads of a fresh buffer run up to 30 % slower)."""
    import quantized_gemv_gqa_amd as q
    buf = torch.empty(int(gib * (1 << 30)) // 16 * 4, dtype=torch.int32, device=dev)
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    with torch.cuda.stream(stream):
        for _ in range(warm):
            q.stream_read(buf, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            q.stream_read(buf, sink)
        e1.record(stream)
        torch.cuda.synchronize()
    nbytes = buf.numel() * 4
    del buf
    return nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def describe(wl) -> dict:
    return {"workload": wl.name, "layers": wl.n_layers, "hidden": wl.hidden, "heads": [wl.n_heads, wl.n_kv_heads],
            "head_dim": wl.head_dim, "inter": wl.inter, "vocab": wl.vocab,
            "weights": ("int4 g%d zp8 fp16 scales" % wl.group) if wl.wfmt == "q4" else "int8 per-row fp32 scales",
            "kv": "%s, 16-token pages%s" % ("paged bf16" if wl.kv_fmt == "bf16" else "fp32",
                                            ", shuffled" if wl.shuffled_pages else ", identity page table"),
            "context": wl.ctx, "batch": 1}


def layer_bench(wl, K: int, W: int, copies: int):
    """The single-layer workload (no embedding or lm head): its 15 MB of weights fit in the 256 MB
    last-level cache, so it is timed both as is (cache-resident) and cold, over `copies` rotating
    copies of the layer (one step handle and graph each, replayed round-robin)."""
    import quantized_gemv_gqa_amd as q
    import synth
    dev = "cuda:0"
    torch.cuda.set_device(0)
    model = synth.make_model(wl)
    kv = synth.make_kv(wl, wl.ctx + W + K + 16)
    stream = torch.cuda.Stream()
    res = {}
    for label, n in (("cache_resident", 1), ("cold", copies)):
        steps = []
        for _ in range(n):
            dm = q.upload_model(model, dev)
            dk = q.upload_kv(kv, wl.kv_fmt, dev)
            steps.append(q.DecodeStep(dm, dk, pos0=wl.ctx, h0=model["h0"], device=dev))
        with torch.cuda.stream(stream):
            for i in range(max(W, n)):
                steps[i % n].step(q.STEP_GRAPH)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(K):
                steps[i % n].step(q.STEP_GRAPH)
            e1.record(stream)
            torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / K
        err = max(st.read_error() for st in steps)
        assert err == 0, "step error word %d" % err
        b = step_bytes(wl, wl.ctx + 1)
        res[label] = {"copies": n, "us_per_step": us, "gbps": b / (us * 1e-6) / 1e9,
                      "frac_of_peak": b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        del steps
        torch.cuda.empty_cache()
    return {"metric": METRIC.replace("Qwen2.5-7B-shape INT4", "single Qwen2-style layer"),
            "value": res["cold"]["gbps"], "unit": "GB/s", "steps": K, "warmup": W, "higher_is_better": True,
            "dtype": "f32", "data": "synthetic", "config": describe(wl), "step_bytes": step_bytes(wl, wl.ctx + 1),
            "layer_step": res}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="qwen2.5-7b-q4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--eager-steps", type=int, default=8, help="eager (kernel-by-kernel) steps timed after the graph")
    ap.add_argument("--kernel-steps", type=int, default=6, help="eager steps with an event after every kernel")
    ap.add_argument("--cold-copies", type=int, default=48, help="single-layer workload: rotating weight copies")
    ap.add_argument("--calib-copy-mib", type=int, default=512,
                    help="size of one plain device copy run after the timed region (counter calibration)")
    ap.add_argument("--sampling", default="",
                    help="T,top_k,top_p: sample each token on the GPU (seed 1234) instead of greedy argmax")
    ap.add_argument("--prefill", type=int, default=0,
                    help="instead of the decode step: time to first token for a prompt of this many tokens")
    ap.add_argument("--batch", type=int, default=0,
                    help="instead of the batch-1 step: batched decode of this many sequences (1..8)")
    ap.add_argument("--gemv-ab", action="store_true",
                    help="instead of the decode step: A/B of fp32- vs INT8-activation GEMVs at the workload's shapes")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build runs the decode step on a single MI355X; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import quantized_gemv_gqa_amd as q
    import synth

    wl = synth.WORKLOADS[args.workload]
    if args.prefill:
        print(json.dumps(prefill_bench(wl, args.prefill, max(1, min(args.steps, 10)), min(args.warmup, 2))))
        return
    if args.batch:
        print(json.dumps(batch_bench(wl, args.batch, args.steps, args.warmup)))
        return
    if args.gemv_ab:
        torch.cuda.set_device(0)
        print(json.dumps({"workload": wl.name, "weights": wl.wfmt, "group": wl.group, "gemv_ab": gemv_ab(wl)}))
        return
    if not wl.has_lm_head:
        print(json.dumps(layer_bench(wl, args.steps, args.warmup, args.cold_copies)))
        return
    K, W, E, KT = args.steps, args.warmup, args.eager_steps, args.kernel_steps
    n_all = W + K + E + KT
    max_ctx = wl.ctx + n_all + 16
    t0 = time.time()
    model = synth.make_model(wl)
    kv = synth.make_kv(wl, max_ctx)
    gen_s = time.time() - t0
    dev = "cuda:0"
    torch.cuda.set_device(0)
    dm = q.upload_model(model, dev)
    dk = q.upload_kv(kv, wl.kv_fmt, dev)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    st = q.DecodeStep(dm, dk, pos0=wl.ctx, token0=model.get("token", 0), log_len=n_all, device=dev)
    sampling = None
    if args.sampling:
        T_s, k_s, p_s = args.sampling.split(",")
        sampling = {"temperature": float(T_s), "top_k": int(k_s), "top_p": float(p_s), "seed": 1234}
        st.set_sampling(sampling["temperature"], sampling["top_k"], sampling["top_p"], sampling["seed"])
    with torch.cuda.stream(stream):
        for _ in range(W):
            st.step(q.STEP_GRAPH)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record(stream)
        for _ in range(K):
            st.step(q.STEP_GRAPH)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / K
    err_word = st.read_error()
    assert err_word == 0, "the timed steps set the step error word (%d)" % err_word
    pos_end = int(st.pos.item())
    assert pos_end == wl.ctx + W + K, pos_end
    T0 = wl.ctx + W + 1
    bytes_timed = sum(step_bytes(wl, T0 + i) for i in range(K))
    gbps_step = bytes_timed / (e0.elapsed_time(e1) * 1e-3) / 1e9

    # eager submission (every kernel launched from the host) for comparison with graph replay
    with torch.cuda.stream(stream):
        st.step(q.STEP_EAGER)
        torch.cuda.synchronize()
        e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e2.record(stream)
        for _ in range(E - 1):
            st.step(q.STEP_EAGER)
        e3.record(stream)
        torch.cuda.synchronize()
    ms_eager = e2.elapsed_time(e3) / max(1, E - 1)

    # per-kernel durations (HIP events on the launch stream), grouped by role
    kernels = []
    kernel_sum_us = None
    if sampling is None and KT > 0:
        kernels, kernel_sum_us = per_kernel_roofline(wl, st, stream, KT)
    err_word = st.read_error()
    assert err_word == 0, "the eager steps set the step error word (%d)" % err_word

    stream_gbps = stream_read_gbps(dev, stream)
    # one plain copy of known size (read + write of calib-copy-mib MiB), the reference the HBM
    # byte counters are scaled by when this command runs under rocprofv3 --pmc
    if args.calib_copy_mib > 0:
        src = torch.empty(args.calib_copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    tokens = st.token_log.cpu().numpy()

    cfg = describe(wl)
    cfg.update({"submission": "hipGraph replay per token", "kernels_per_step": st.kernel_count,
                "num_splits": st.cfg.num_splits, "next_token": sampling or "greedy"})
    out = {
        "metric": METRIC if wl.name == "qwen2.5-7b-q4" else METRIC.replace("Qwen2.5-7B-shape INT4", wl.name),
        "value": K / (e0.elapsed_time(e1) * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": cfg,
        "step_bytes": bytes_timed / K,
        "step_gbps": gbps_step,
        "step_frac_of_peak": gbps_step / HBM_PEAK_GBPS,
        "stream_read_gbps": stream_gbps,
        "step_frac_of_stream_read": gbps_step / stream_gbps,
        "eager_ms_per_step": ms_eager,
        "error_word": 0,
        "wall_s_timed": wall,
    }
    if kernels:
        top = kernels[0]
        out["roofline"] = {"bound": "hbm", "kernel": top["kernel"], "achieved": top["gbps"], "peak": HBM_PEAK_GBPS,
                           "unit": "GB/s", "frac": top["frac_of_peak"], "traffic": measured_traffic(top["role"]),
                           "bytes_per_launch": top["bytes_per_launch"], "us_per_launch": top["us_per_launch"],
                           "share_of_step": top["share_of_step"], "kernel_source_hash": kernel_source_hash(),
                           "timing": "HIP events after every launch of %d eager steps, on the launch stream" % KT}
        out["kernels"] = kernels
        out["kernel_sum_ms_per_step"] = kernel_sum_us / 1e3
    out["tokens_head"] = [int(t) for t in tokens[:8]]

    if not args.no_cpu_baseline:
        import oracle
        nthreads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count() or 1
        od = oracle.OracleDecoder(model, kv, nthreads=nthreads)
        tok = model.get("token", 0)
        n, t_cpu = 0, 0.0
        orc_tokens, margins = [], []
        while t_cpu < args.cpu_seconds and n < min(64, W + K):
            c0 = time.perf_counter()
            r = od.step(wl.ctx + n, tok, logits=True)
            t_cpu += time.perf_counter() - c0
            tok = r["token"]
            orc_tokens.append(int(tok))
            srt = np.sort(r["logits"].astype(np.float64))
            margins.append(float(srt[-1] - srt[-2]))
            n += 1
        out["cpu_baseline"] = {"value": n / t_cpu, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
                               "sample": "%d whole decode steps of the same model from position %d (greedy)" % (n, wl.ctx)}
        if sampling is None:
            gpu_t = [int(t) for t in tokens[:n]]
            same = sum(int(a == b) for a, b in zip(gpu_t, orc_tokens))
            first_diff = next((i for i, (a, b) in enumerate(zip(gpu_t, orc_tokens)) if a != b), None)
            out["oracle_token_check"] = {"steps": n, "identical": same, "first_difference": first_diff,
                                         "min_oracle_margin": min(margins),
                                         "note": "GPU greedy tokens of the warm-up and timed steps against the oracle's "
                                                 "decode of the same model from the same state"}
    out["gen_s"] = gen_s
    print(json.dumps(out))


if __name__ == "__main__":
    main()
