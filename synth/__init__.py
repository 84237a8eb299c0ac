"""Seeded synthetic inputs for the batch-1 quantized GQA decode step.

This module draws the random inputs (weights, scales, biases, norm gains, prior
KV context, page tables, start token) and nothing else: it holds no step of the
decode method.  The CPU oracle and the GPU path both consume the arrays built
here, and neither imports the other.

Workload shapes follow the five decode workloads this project measures (a
single Qwen2-style layer at hidden 896; Qwen2.5-1.5B, Qwen2.5-7B and Qwen3-8B
shapes; a 32K-context Qwen2.5-7B attention-stress case).  The per-block tensor
list (attn_norm, q/k/v with bias, attn_output, ffn_norm, ffn_gate/up/down,
output_norm, output) is the Qwen2 block of the naive-CUDA Qwen engine post
(part 1, the GGUF "Tensor Data" figure).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_SRC = os.path.join(_HERE, "synth.c")


def build(force: bool = False) -> str:
    """Compile the generator with gcc (host only)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def _L():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P, I64, U64, D, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_int
        lib.synth_draw.argtypes = [U64, U64, U64]
        lib.synth_draw.restype = U64
        lib.synth_fill_u8.argtypes = [P, I64, U64, U64]
        lib.synth_fill_i8.argtypes = [P, I64, U64, U64, I, I]
        lib.synth_fill_f32_normal.argtypes = [P, I64, U64, U64, D, D]
        lib.synth_fill_f32_uniform.argtypes = [P, I64, U64, U64, D, D]
        lib.synth_fill_f16_uniform.argtypes = [P, I64, U64, U64, D, D]
        lib.synth_fill_bf16_normal.argtypes = [P, I64, U64, U64, D, D]
        lib.synth_permutation.argtypes = [P, I64, U64, U64]
        lib.synth_fill_kv.argtypes = [P, I, P, I, I64, I, I, U64, U64, D]
        lib.synth_tied_embedding.argtypes = [P, P, P, I64, I64]
        for f in ("synth_fill_u8", "synth_fill_i8", "synth_fill_f32_normal", "synth_fill_f32_uniform",
                  "synth_fill_f16_uniform", "synth_fill_bf16_normal", "synth_permutation",
                  "synth_fill_kv", "synth_tied_embedding"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------------------- streams
# Tensor ids: per-layer tensors use layer * 64 + slot, globals use GLOBAL * 64 + slot.
_LAYER_SLOTS = {n: i for i, n in enumerate(
    ["wq", "sq", "bq", "wk", "sk", "bk", "wv", "sv", "bv", "wo", "so", "wg", "sg", "wu", "su",
     "wd", "sd", "g_attn", "g_ffn", "g_q", "g_k", "k_cache", "v_cache"])}
_GLOBAL = 1 << 20
_GLOBAL_SLOTS = {n: i for i, n in enumerate(
    ["embed", "g_out", "w_lm", "s_lm", "h0", "token", "pages"])}


def stream_id(name: str, layer: int | None = None) -> int:
    if layer is None:
        return _GLOBAL * 64 + _GLOBAL_SLOTS[name]
    return layer * 64 + _LAYER_SLOTS[name]


# ----------------------------------------------------------------------------- fills
def u8(n, seed, sid):
    a = np.empty(n, np.uint8); _L().synth_fill_u8(_p(a), n, seed, sid); return a


def i8(n, seed, sid, lo=-127, hi=127):
    a = np.empty(n, np.int8); _L().synth_fill_i8(_p(a), n, seed, sid, lo, hi); return a


def f32_normal(n, seed, sid, mean=0.0, std=1.0):
    a = np.empty(n, np.float32); _L().synth_fill_f32_normal(_p(a), n, seed, sid, mean, std); return a


def f32_uniform(n, seed, sid, lo, hi):
    a = np.empty(n, np.float32); _L().synth_fill_f32_uniform(_p(a), n, seed, sid, lo, hi); return a


def f16_uniform(n, seed, sid, lo, hi):
    a = np.empty(n, np.uint16); _L().synth_fill_f16_uniform(_p(a), n, seed, sid, lo, hi); return a


def bf16_normal(n, seed, sid, mean=0.0, std=1.0):
    a = np.empty(n, np.uint16); _L().synth_fill_bf16_normal(_p(a), n, seed, sid, mean, std); return a


def permutation(n, seed, sid):
    a = np.empty(n, np.int32); _L().synth_permutation(_p(a), n, seed, sid); return a


def draw(seed: int, sid: int, i: int) -> int:
    return int(_L().synth_draw(seed, sid, i))


# ----------------------------------------------------------------------------- workloads
@dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    inter: int
    vocab: int                # 0: no embedding / lm_head (single-layer case)
    wfmt: str                 # "q8": int8 per output row, fp32 scale; "q4": nibbles, fp16 scale per group
    kv_fmt: str               # "f32" or "bf16"
    ctx: int                  # prior context tokens already in the cache at step 0
    steps: int = 64           # greedy steps
    group: int = 64           # q4 group size along K
    eps: float = 1e-6
    rope_base: float = 1e6
    page_size: int = 16
    shuffled_pages: bool = False
    qkv_bias: bool = True
    qk_norm: bool = False
    tied: bool = False
    seed: int = 1000
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def has_lm_head(self) -> bool:
        return self.vocab > 0

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def n_qkv(self) -> int:
        return self.q_dim + 2 * self.kv_dim


WORKLOADS = {
    # one Qwen2-style layer, hidden 896, 14/2 heads of 64, MLP 4864, int8 rows, fp32 contiguous KV of 256 tokens
    "layer-h896-q8": Workload("layer-h896-q8", 1, 896, 14, 2, 64, 4864, 0, "q8", "f32", 256,
                              steps=1, seed=1000),
    # Qwen2.5-1.5B shape, int8 rows, tied bf16 embedding, bf16 contiguous KV of 1024 tokens
    "qwen2.5-1.5b-q8": Workload("qwen2.5-1.5b-q8", 28, 1536, 12, 2, 128, 8960, 151936, "q8", "bf16",
                                1024, tied=True, seed=1001),
    # Qwen2.5-7B shape, int4 groups of 64 with fp16 scales, paged bf16 KV of 4096 tokens, shuffled pages
    "qwen2.5-7b-q4": Workload("qwen2.5-7b-q4", 28, 3584, 28, 4, 128, 18944, 152064, "q4", "bf16",
                              4096, shuffled_pages=True, seed=1002),
    # Qwen3-8B shape, int8 rows, per-head q/k RMSNorm, no q/k/v bias, bf16 KV of 4096 tokens
    "qwen3-8b-q8": Workload("qwen3-8b-q8", 36, 4096, 32, 8, 128, 12288, 151936, "q8", "bf16", 4096,
                            qkv_bias=False, qk_norm=True, seed=1003),
    # Qwen2.5-7B shape at 32768 tokens of paged context: the KV stream rivals the weight stream
    "qwen2.5-7b-q4-32k": Workload("qwen2.5-7b-q4-32k", 28, 3584, 28, 4, 128, 18944, 152064, "q4",
                                  "bf16", 32768, shuffled_pages=True, seed=1004),
}


def tiny(wfmt: str = "q8", **kw) -> Workload:
    """A tiny model for brute-force checks (hidden 16, 4/2 heads of 4, MLP 24, vocab 50, 2 layers)."""
    base = Workload("tiny-" + wfmt, 2, 16, 4, 2, 4, 24, 50, wfmt, "bf16", 5, steps=3,
                    group=8 if wfmt == "q4" else 64, seed=7)
    return replace(base, **kw)


# ----------------------------------------------------------------------------- model
def _weight(wl: Workload, rows: int, cols: int, seed: int, wname: str, sname: str, layer,
            row_scale_jitter: bool):
    if wl.wfmt == "q8":
        w = i8(rows * cols, seed, stream_id(wname, layer)).reshape(rows, cols)
        if row_scale_jitter:
            s = (0.02 / 127) * f32_uniform(rows, seed, stream_id(sname, layer), 0.5, 1.5)
            s = s.astype(np.float32)
        else:
            s = np.full(rows, np.float32(0.02 / 127), np.float32)
        return w, s
    assert wl.wfmt == "q4" and cols % wl.group == 0 and cols % 2 == 0
    w = u8(rows * cols // 2, seed, stream_id(wname, layer)).reshape(rows, cols // 2)
    s = f16_uniform(rows * (cols // wl.group), seed, stream_id(sname, layer), 0.005, 0.02)
    return w, s.reshape(rows, cols // wl.group)


def _gain(n, seed, sid):
    # RMSNorm gains: 1 + 0.1 * N(0,1), so that a dropped gain is visible
    return f32_normal(n, seed, sid, 1.0, 0.1)


def make_model(wl: Workload, seed: int | None = None, n_layers: int | None = None,
               row_scale_jitter: bool = False) -> dict:
    """Host arrays of one synthetic model, as the per-block tensor list.

    q8 weights: int8 [N][K] uniform on [-127, 127], fp32 row scale 0.02/127 (or that times
    U(0.5, 1.5) per row with row_scale_jitter).  q4 weights: uint8 [N][K/2], byte j of a row
    holds k = 2j in bits 0-3 and k = 2j+1 in bits 4-7, nibbles uniform on 0..15 (zero point 8),
    fp16 scales [N][K/group] uniform on [0.005, 0.02).
    """
    seed = wl.seed if seed is None else seed
    L = wl.n_layers if n_layers is None else n_layers
    H, I, qd, kvd = wl.hidden, wl.inter, wl.q_dim, wl.kv_dim
    layers = []
    for l in range(L):
        d = {}
        d["wq"], d["sq"] = _weight(wl, qd, H, seed, "wq", "sq", l, row_scale_jitter)
        d["wk"], d["sk"] = _weight(wl, kvd, H, seed, "wk", "sk", l, row_scale_jitter)
        d["wv"], d["sv"] = _weight(wl, kvd, H, seed, "wv", "sv", l, row_scale_jitter)
        if wl.qkv_bias:
            d["bq"] = f32_normal(qd, seed, stream_id("bq", l), 0.0, 0.02)
            d["bk"] = f32_normal(kvd, seed, stream_id("bk", l), 0.0, 0.02)
            d["bv"] = f32_normal(kvd, seed, stream_id("bv", l), 0.0, 0.02)
        d["wo"], d["so"] = _weight(wl, H, qd, seed, "wo", "so", l, row_scale_jitter)
        d["wg"], d["sg"] = _weight(wl, I, H, seed, "wg", "sg", l, row_scale_jitter)
        d["wu"], d["su"] = _weight(wl, I, H, seed, "wu", "su", l, row_scale_jitter)
        d["wd"], d["sd"] = _weight(wl, H, I, seed, "wd", "sd", l, row_scale_jitter)
        d["g_attn"] = _gain(H, seed, stream_id("g_attn", l))
        d["g_ffn"] = _gain(H, seed, stream_id("g_ffn", l))
        if wl.qk_norm:
            d["g_q"] = _gain(wl.head_dim, seed, stream_id("g_q", l))
            d["g_k"] = _gain(wl.head_dim, seed, stream_id("g_k", l))
        layers.append(d)
    m = {"layers": layers, "workload": wl, "seed": seed}
    if wl.has_lm_head:
        V = wl.vocab
        m["g_out"] = _gain(H, seed, stream_id("g_out"))
        m["w_lm"], m["s_lm"] = _weight(wl, V, H, seed, "w_lm", "s_lm", None, row_scale_jitter)
        if wl.tied:
            assert wl.wfmt == "q8"
            E = np.empty((V, H), np.uint16)
            _L().synth_tied_embedding(_p(E), _p(m["w_lm"]), _p(m["s_lm"]), V, H)
        else:
            E = bf16_normal(V * H, seed, stream_id("embed"), 0.0, 0.02).reshape(V, H)
        m["embed"] = E
        m["token"] = draw(seed, stream_id("token"), 0) % V
    else:
        m["h0"] = f32_normal(H, seed, stream_id("h0"), 0.0, 1.0)
    return m


def n_pages(wl: Workload, max_ctx: int) -> int:
    return -(-max_ctx // wl.page_size)


def make_kv(wl: Workload, max_ctx: int, seed: int | None = None, n_layers: int | None = None,
            ctx: int | None = None) -> dict:
    """Page table and per-layer K/V pools, the prior context filled with N(0,1) values.

    Pool layout per layer: [n_pages][n_kv_heads][page_size][head_dim] (fp32 or bf16 bits); the
    page table maps logical page p (tokens 16p..16p+15) to a physical page.  Shuffled workloads
    use a seeded permutation, the others the identity.
    """
    seed = wl.seed if seed is None else seed
    L = wl.n_layers if n_layers is None else n_layers
    ctx = wl.ctx if ctx is None else ctx
    assert max_ctx >= ctx + 1
    P = n_pages(wl, max_ctx)
    pt = permutation(P, seed, stream_id("pages")) if wl.shuffled_pages else np.arange(P, dtype=np.int32)
    dt = np.float32 if wl.kv_fmt == "f32" else np.uint16
    fmt = 1 if wl.kv_fmt == "f32" else 2
    shape = (P, wl.n_kv_heads, wl.page_size, wl.head_dim)
    kp, vp = [], []
    for l in range(L):
        for name, lst in (("k_cache", kp), ("v_cache", vp)):
            a = np.zeros(shape, dt)
            _L().synth_fill_kv(_p(a), fmt, _p(pt), wl.page_size, ctx, wl.n_kv_heads, wl.head_dim,
                               seed, stream_id(name, l), 1.0)
            lst.append(a)
    return {"page_table": pt, "k": kp, "v": vp, "max_ctx": max_ctx, "ctx": ctx}


def make_kv_batch(wl: Workload, ctxs, max_blocks: int, seed: int | None = None, n_layers: int | None = None,
                  spare_pages: int = 0) -> dict:
    """Shared per-layer K/V pools for a batch of sequences with their own block tables.

    Sequence b holds ctxs[b] prior tokens (N(0,1) values, a different draw per sequence) in the
    blocks its table row maps; the pool's physical pages are dealt to the sequences through a seeded
    permutation, each sequence getting max_blocks of them (row b, unused rows entries -1 past
    `spare_pages` pages left free for on-demand allocation).  Returns the block tables
    [B][max_blocks], the pools, and the free page list.
    """
    seed = wl.seed if seed is None else seed
    L = wl.n_layers if n_layers is None else n_layers
    B = len(ctxs)
    need = [-(-(c + 1) // wl.page_size) for c in ctxs]  # blocks holding the context and the next token
    assert all(n <= max_blocks for n in need)
    P = sum(need) + spare_pages
    perm = permutation(P, seed, stream_id("pages"))
    tables = np.full((B, max_blocks), -1, np.int32)
    o = 0
    for b in range(B):
        tables[b, :need[b]] = perm[o:o + need[b]]
        o += need[b]
    free = [int(v) for v in perm[o:]]
    dt = np.float32 if wl.kv_fmt == "f32" else np.uint16
    fmt = 1 if wl.kv_fmt == "f32" else 2
    shape = (P, wl.n_kv_heads, wl.page_size, wl.head_dim)
    kp, vp = [], []
    for l in range(L):
        for name, lst in (("k_cache", kp), ("v_cache", vp)):
            a = np.zeros(shape, dt)
            for b in range(B):
                row = np.ascontiguousarray(tables[b])
                _L().synth_fill_kv(_p(a), fmt, _p(row), wl.page_size, int(ctxs[b]), wl.n_kv_heads, wl.head_dim,
                                   seed + 7919 * (b + 1), stream_id(name, l), 1.0)
            lst.append(a)
    return {"block_tables": tables, "k": kp, "v": vp, "free_pages": free, "ctxs": list(ctxs)}
