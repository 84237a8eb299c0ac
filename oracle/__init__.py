"""CPU oracle for the batch-1 quantized GQA decode step (numpy marshalling over plain C).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The GPU library never links or calls it.

The arithmetic lives in ``qdec_oracle.c`` (fp64 plain definitions, one function per step of
the method, each citing the page it follows).  This file only converts numpy arrays to C
pointers and back.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRCS = [os.path.join(_HERE, "qdec_oracle.c"), os.path.join(_HERE, "qdec_oracle.h")]

W_Q8, W_Q4 = 1, 2
KV_F32, KV_BF16 = 1, 2


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O3, no fast-math, no FMA contraction: IEEE semantics kept)."""
    stale = not os.path.exists(_SO) or any(os.path.getmtime(_SO) < os.path.getmtime(s) for s in _SRCS)
    if force or stale:
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", _SRCS[0], "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class _Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "inter", "vocab",
        "wfmt", "group", "kv_fmt", "page_size",
        "has_bias", "has_qk_norm", "has_embedding", "has_lm_head")] + [
        ("eps", ctypes.c_double), ("rope_base", ctypes.c_double)]


_P = ctypes.c_void_p


class _Layer(ctypes.Structure):
    _fields_ = [(n, _P) for n in (
        "wq", "sq", "wk", "sk", "wv", "sv", "wo", "so", "wg", "sg", "wu", "su", "wd", "sd",
        "bq", "bk", "bv", "g_attn", "g_ffn", "g_q", "g_k", "k_pool", "v_pool")]


class _Head(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("embed", "g_out", "w_lm", "s_lm")]


_lib = None


def use_library(path: str | None) -> None:
    """Load the oracle from another build of its source (None: the default build)."""
    global _lib
    _lib = None
    lib(path)


def lib(path: str | None = None):
    global _lib
    if _lib is None:
        L = ctypes.CDLL(path or build())
        I, I64, D, F, U16 = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_float, ctypes.c_uint16
        L.orc_f16_to_f32.argtypes = [U16]; L.orc_f16_to_f32.restype = F
        L.orc_f32_to_bf16.argtypes = [F]; L.orc_f32_to_bf16.restype = U16
        L.orc_bf16_to_f32.argtypes = [U16]; L.orc_bf16_to_f32.restype = F
        L.orc_dequant_row.argtypes = [I, _P, _P, I, I64, I, _P]; L.orc_dequant_row.restype = None
        L.orc_gemv.argtypes = [I, _P, _P, I, _P, _P, _P, _P, I, I, I]; L.orc_gemv.restype = None
        L.orc_quantize_act_i8.argtypes = [_P, I, I, _P, _P]; L.orc_quantize_act_i8.restype = None
        L.orc_gemv_a8.argtypes = [I, _P, _P, I, _P, _P, _P, _P, _P, I, I, I]; L.orc_gemv_a8.restype = None
        L.orc_rmsnorm.argtypes = [_P, _P, _P, I, I, D]; L.orc_rmsnorm.restype = None
        L.orc_rope.argtypes = [_P, I, I, I, D]; L.orc_rope.restype = None
        L.orc_swiglu.argtypes = [_P, _P, _P, I]; L.orc_swiglu.restype = None
        L.orc_kv_store.argtypes = [_P, I, _P, I, I, I, I, _P]; L.orc_kv_store.restype = None
        L.orc_kv_load.argtypes = [_P, I, _P, I, I, I, I, I, I]; L.orc_kv_load.restype = F
        L.orc_attention.argtypes = [_P, _P, _P, I, _P, I, I, I, I, I, D, _P, _P]
        L.orc_attention.restype = None
        L.orc_argmax.argtypes = [_P, I]; L.orc_argmax.restype = I
        L.orc_decode_batch.argtypes = [_P, _P, _P, I, _P, I, _P, _P, _P, _P, _P, I]
        L.orc_decode_batch.restype = None
        L.orc_prefill.argtypes = [_P, _P, _P, _P, I, _P, I, _P, _P, I]; L.orc_prefill.restype = I
        U64 = ctypes.c_uint64
        L.orc_philox4x64_10.argtypes = [_P, _P, _P]; L.orc_philox4x64_10.restype = None
        L.orc_sample_uniform.argtypes = [U64, I64, I64]; L.orc_sample_uniform.restype = D
        L.orc_sample.argtypes = [_P, I, D, I, D, U64, I64]; L.orc_sample.restype = I
        L.orc_decode_step.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Layer),
                                      ctypes.POINTER(_Head), _P, I, I, _P, _P, _P, I]
        L.orc_decode_step.restype = I
        L.orc_decode_step_kv.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Layer),
                                         ctypes.POINTER(_Head), _P, I, I, _P, _P, _P, I, _P, _P, _P]
        L.orc_decode_step_kv.restype = I
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle needs C-contiguous numpy"
    return a.ctypes.data_as(_P)


def _fmt(wfmt) -> int:
    return {"q8": W_Q8, "q4": W_Q4, W_Q8: W_Q8, W_Q4: W_Q4}[wfmt]


def _kvfmt(kv) -> int:
    return {"f32": KV_F32, "bf16": KV_BF16, KV_F32: KV_F32, KV_BF16: KV_BF16}[kv]


# ----------------------------------------------------------------------------- number formats
def f16_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, np.uint16).ravel()
    return np.array([lib().orc_f16_to_f32(int(v)) for v in b], np.float32)


def f32_to_bf16(x) -> np.ndarray:
    a = np.ascontiguousarray(x, np.float32).ravel()
    return np.array([lib().orc_f32_to_bf16(float(v)) for v in a], np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- ops
def dequant_row(wfmt, W, S, row, K, group=64) -> np.ndarray:
    w = np.empty(K, np.float32)
    lib().orc_dequant_row(_fmt(wfmt), _p(W), _p(S), group, row, K, _p(w))
    return w


def gemv(wfmt, W, S, x, bias=None, residual=None, group=64, nthreads=0) -> np.ndarray:
    W = np.ascontiguousarray(W); S = np.ascontiguousarray(S)
    x = np.ascontiguousarray(x, np.float32)
    N = W.shape[0]
    K = x.shape[0]
    y = np.empty(N, np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    r = None if residual is None else np.ascontiguousarray(residual, np.float32)
    lib().orc_gemv(_fmt(wfmt), _p(W), _p(S), group, _p(x), _p(b), _p(r), _p(y), N, K,
                   nthreads or int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count() or 1)
    return y


def quantize_act_i8(x, group=64):
    """INT8 activations with one scale per group (Path A); returns (q int8 [K], s float32 [K/group])."""
    x = np.ascontiguousarray(x, np.float32)
    K = x.shape[0]
    assert K % group == 0
    q = np.empty(K, np.int8)
    s = np.empty(K // group, np.float32)
    lib().orc_quantize_act_i8(_p(x), K, group, _p(q), _p(s))
    return q, s


def gemv_a8(wfmt, W, S, q, sx, bias=None, residual=None, group=64, nthreads=0) -> np.ndarray:
    """GEMV with INT8 activations (q, per-group sx from quantize_act_i8)."""
    W = np.ascontiguousarray(W); S = np.ascontiguousarray(S)
    q = np.ascontiguousarray(q, np.int8); sx = np.ascontiguousarray(sx, np.float32)
    N = W.shape[0]
    K = q.shape[0]
    y = np.empty(N, np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    r = None if residual is None else np.ascontiguousarray(residual, np.float32)
    lib().orc_gemv_a8(_fmt(wfmt), _p(W), _p(S), group, _p(q), _p(sx), _p(b), _p(r), _p(y), N, K,
                      nthreads or int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count() or 1)
    return y


def rmsnorm(x, gamma=None, eps=1e-6) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    x2 = x.reshape(-1, x.shape[-1])
    y = np.empty_like(x2)
    g = None if gamma is None else np.ascontiguousarray(gamma, np.float32)
    lib().orc_rmsnorm(_p(x2), _p(g), _p(y), x2.shape[0], x2.shape[1], eps)
    return y.reshape(x.shape)


def rope(x, pos, base=1e6) -> np.ndarray:
    y = np.array(x, np.float32, copy=True, order="C")
    y2 = y.reshape(-1, y.shape[-1])
    lib().orc_rope(_p(y2), y2.shape[0], y2.shape[1], int(pos), float(base))
    return y


def swiglu(g, u) -> np.ndarray:
    g = np.ascontiguousarray(g, np.float32); u = np.ascontiguousarray(u, np.float32)
    m = np.empty_like(g)
    lib().orc_swiglu(_p(g), _p(u), _p(m), g.size)
    return m


def kv_store(pool, kv_fmt, page_table, page_size, t, kv) -> None:
    Hkv, D = pool.shape[1], pool.shape[3]
    kv = np.ascontiguousarray(kv, np.float32)
    lib().orc_kv_store(_p(pool), _kvfmt(kv_fmt), _p(page_table), page_size, Hkv, D, int(t), _p(kv))


def attention(q, k_pool, v_pool, kv_fmt, page_table, T, page_size=16, scale=None, probs=False):
    """q [Hq][D]; pools [pages][Hkv][page_size][D]; returns out [Hq][D] (and probs [Hq][T])."""
    q = np.ascontiguousarray(q, np.float32)
    Hq, D = q.shape
    Hkv = k_pool.shape[1]
    out = np.empty((Hq, D), np.float32)
    pr = np.empty((Hq, T), np.float32) if probs else None
    sc = 1.0 / np.sqrt(D) if scale is None else scale
    pt = np.ascontiguousarray(page_table, np.int32)
    lib().orc_attention(_p(q), _p(k_pool), _p(v_pool), _kvfmt(kv_fmt), _p(pt), page_size, int(T),
                        Hq, Hkv, D, float(sc), _p(out), _p(pr))
    return (out, pr) if probs else out


def philox4x64_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, np.uint64)
    k = np.ascontiguousarray(key, np.uint64)
    out = np.empty(4, np.uint64)
    lib().orc_philox4x64_10(_p(c), _p(k), _p(out))
    return out


def sample_uniform(seed: int, step: int, i: int) -> float:
    return float(lib().orc_sample_uniform(seed, step, i))


def sample(logits, temperature: float, top_k: int = 0, top_p: float = 1.0, seed: int = 0, step: int = 0) -> int:
    """Temperature / top-k / top-p sampling with a Gumbel-max draw keyed by (seed, step)."""
    v = np.ascontiguousarray(logits, np.float32)
    return int(lib().orc_sample(_p(v), v.size, temperature, top_k, top_p, seed, step))


def argmax(v) -> int:
    v = np.ascontiguousarray(v, np.float32)
    return int(lib().orc_argmax(_p(v), v.size))


# ----------------------------------------------------------------------------- decode step
class OracleDecoder:
    """Holds one synthetic model and its own copy of the KV cache; steps it on the CPU."""

    def __init__(self, model: dict, kv: dict, copy_kv: bool = True, nthreads: int = 0):
        wl = model["workload"]
        self.wl = wl
        self.nthreads = nthreads or int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count() or 1
        layers = model["layers"]
        self._keep = [model]
        self.k = [a.copy() if copy_kv else a for a in kv["k"][: len(layers)]]
        self.v = [a.copy() if copy_kv else a for a in kv["v"][: len(layers)]]
        self.page_table = np.ascontiguousarray(kv["page_table"], np.int32)
        c = _Config()
        c.n_layers, c.hidden, c.n_heads, c.n_kv_heads = len(layers), wl.hidden, wl.n_heads, wl.n_kv_heads
        c.head_dim, c.inter, c.vocab = wl.head_dim, wl.inter, wl.vocab
        c.wfmt, c.group, c.kv_fmt, c.page_size = _fmt(wl.wfmt), wl.group, _kvfmt(wl.kv_fmt), wl.page_size
        c.has_bias, c.has_qk_norm = int(wl.qkv_bias), int(wl.qk_norm)
        c.has_embedding = c.has_lm_head = int(wl.has_lm_head)
        c.eps, c.rope_base = wl.eps, wl.rope_base
        self.cfg = c
        arr = (_Layer * len(layers))()
        for i, d in enumerate(layers):
            L = arr[i]
            for n in ("wq", "sq", "wk", "sk", "wv", "sv", "wo", "so", "wg", "sg", "wu", "su", "wd",
                      "sd", "g_attn", "g_ffn"):
                setattr(L, n, _p(d[n]))
            for n in ("bq", "bk", "bv", "g_q", "g_k"):
                setattr(L, n, _p(d[n]) if n in d else None)
            L.k_pool, L.v_pool = _p(self.k[i]), _p(self.v[i])
        self.layers = arr
        hd = _Head()
        if wl.has_lm_head:
            hd.embed, hd.g_out = _p(model["embed"]), _p(model["g_out"])
            hd.w_lm, hd.s_lm = _p(model["w_lm"]), _p(model["s_lm"])
        self.head = hd
        self.h = np.zeros(wl.hidden, np.float32) if wl.has_lm_head else model["h0"].copy()

    def prefill(self, pos0: int, tokens):
        """Prompt tokens at positions pos0 .. pos0 + T - 1 (stores their KV); returns the last
        position's greedy token, logits and residual stream."""
        tk = np.ascontiguousarray(tokens, np.int32)
        lg = np.empty(self.wl.vocab, np.float32)
        nxt = lib().orc_prefill(ctypes.byref(self.cfg), self.layers, ctypes.byref(self.head), _p(self.page_table),
                                int(pos0), _p(tk), tk.size, _p(self.h), _p(lg), self.nthreads)
        return {"token": nxt, "logits": lg, "h": self.h.copy()}

    def step_batch(self, block_tables, pos, tokens, h):
        """Batched step: row b of block_tables [B][max_blocks], pos[b] (< 0: idle), tokens[b], residual
        streams h [B][H] (updated in place).  Returns (next tokens [B], logits [B][V])."""
        bt = np.ascontiguousarray(block_tables, np.int32)
        B, mb = bt.shape
        ps = np.ascontiguousarray(pos, np.int32)
        tk = np.ascontiguousarray(tokens, np.int32)
        assert h.dtype == np.float32 and h.flags.c_contiguous and h.shape == (B, self.wl.hidden)
        lg = np.zeros((B, self.wl.vocab), np.float32)
        nxt = np.full(B, -1, np.int32)
        lib().orc_decode_batch(ctypes.byref(self.cfg), self.layers, ctypes.byref(self.head), B, _p(bt), mb, _p(ps),
                               _p(tk), _p(h), _p(lg), _p(nxt), self.nthreads)
        return nxt, lg

    def step(self, pos: int, token: int = 0, trace: bool = False, logits: bool = True, kv_pre: bool = False,
             kv_force: dict | None = None):
        """One decode step.  kv_pre: also return the new token's fp32 k, v per layer before they are
        rounded into the cache ("kv_pre", [L][2][Hkv][D]).  kv_force: {layer: (k_codes, v_codes)}
        of bf16 codes ([Hkv][D] uint16) stored as the new token's entries of those layers instead
        of the rounding (teacher forcing of a rounding tie)."""
        wl = self.wl
        L = self.cfg.n_layers
        tr = np.empty((L + 1, wl.hidden), np.float32) if trace else None
        lg = np.empty(wl.vocab, np.float32) if (logits and wl.has_lm_head) else None
        pre = np.empty((L, 2, wl.n_kv_heads, wl.head_dim), np.float32) if kv_pre else None
        force = mask = None
        if kv_force:
            assert wl.kv_fmt == "bf16", "forced cache codes are bf16"
            force = np.zeros((L, 2, wl.n_kv_heads, wl.head_dim), np.uint16)
            mask = np.zeros(L, np.uint8)
            for l, (kc, vc) in kv_force.items():
                force[l, 0], force[l, 1], mask[l] = kc, vc, 1
        nxt = lib().orc_decode_step_kv(ctypes.byref(self.cfg), self.layers, ctypes.byref(self.head),
                                       _p(self.page_table), int(pos), int(token), _p(self.h), _p(tr),
                                       _p(lg), self.nthreads, _p(pre), _p(force), _p(mask))
        return {"token": nxt, "trace": tr, "logits": lg, "h": self.h.copy(), "kv_pre": pre}
