"""An independent fp64 numpy decoder for tiny models (test code only).

It is written separately from the C oracle, from the same plain definitions, so that the two
can check each other on tiny shapes: vectorised numpy instead of loops, a logical (unpaged)
KV list instead of page-table indexing, and library routines (numpy's fp16 decode, torch's
bf16 rounding, scipy's softmax and expit) instead of hand-written ones.
"""
from __future__ import annotations

import numpy as np
import scipy.special
import torch


def bf16_round(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(b, np.uint16).view(np.int16)).view(torch.bfloat16).to(
        torch.float32).numpy()


def dequant(wfmt: str, W: np.ndarray, S: np.ndarray, group: int = 64) -> np.ndarray:
    if wfmt == "q8":
        return (W.astype(np.float32) * S.astype(np.float32)[:, None]).astype(np.float64)
    N = W.shape[0]
    nib = np.stack([W & 0x0F, W >> 4], axis=-1).reshape(N, -1).astype(np.int64)
    sc = np.repeat(S.view(np.float16).astype(np.float64), group, axis=1)
    return (nib - 8) * sc


def rmsnorm(x, g, eps):
    x = np.asarray(x, np.float64)
    return (np.asarray(g, np.float64) * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps))


def rope(x, pos, base):
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    half = D // 2
    theta = base ** (-np.arange(half) * 2.0 / D)
    c, s = np.cos(pos * theta), np.sin(pos * theta)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def f32(x):
    return np.asarray(x, np.float64).astype(np.float32)


class NumpyDecoder:
    def __init__(self, model: dict, kv_logical_k: np.ndarray, kv_logical_v: np.ndarray):
        """kv_logical_*: [L][ctx][Hkv][D] fp32 values of the prior context (already bf16-exact)."""
        self.m = model
        self.wl = model["workload"]
        self.K = [list(k) for k in kv_logical_k]
        self.V = [list(v) for v in kv_logical_v]

    def step(self, pos: int, token: int, kv_hook=None):
        """kv_hook(l, k, v) -> (k, v): replaces the new token's stored (rounded) entries of layer l;
        self.pre[l] keeps that layer's k, v before the rounding."""
        wl, m = self.wl, self.m
        self.pre = []
        H, Hq, Hkv, D = wl.hidden, wl.n_heads, wl.n_kv_heads, wl.head_dim
        G = Hq // Hkv
        grp = wl.group
        h = bf16_bits_to_f32(m["embed"][token]) if wl.has_lm_head else m["h0"].copy()
        trace = [f32(h)]
        for l, P in enumerate(m["layers"]):
            a = f32(rmsnorm(h, P["g_attn"], wl.eps))
            q = dequant(wl.wfmt, P["wq"], P["sq"], grp) @ a
            k = dequant(wl.wfmt, P["wk"], P["sk"], grp) @ a
            v = dequant(wl.wfmt, P["wv"], P["sv"], grp) @ a
            if wl.qkv_bias:
                q, k, v = q + P["bq"], k + P["bk"], v + P["bv"]
            q, k, v = f32(q).reshape(Hq, D), f32(k).reshape(Hkv, D), f32(v).reshape(Hkv, D)
            if wl.qk_norm:
                q, k = f32(rmsnorm(q, P["g_q"], wl.eps)), f32(rmsnorm(k, P["g_k"], wl.eps))
            q, k = f32(rope(q, pos, wl.rope_base)), f32(rope(k, pos, wl.rope_base))
            self.pre.append((k.copy(), v.copy()))
            if wl.kv_fmt == "bf16":
                k, v = bf16_round(k), bf16_round(v)
            if kv_hook is not None:
                k, v = kv_hook(l, k, v)
            assert len(self.K[l]) == pos
            self.K[l].append(k); self.V[l].append(v)
            Kt = np.stack(self.K[l]).astype(np.float64)   # [T][Hkv][D]
            Vt = np.stack(self.V[l]).astype(np.float64)
            att = np.empty((Hq, D))
            for hh in range(Hq):
                j = hh // G
                sc = Kt[:, j, :] @ q[hh].astype(np.float64) / np.sqrt(D)
                p = scipy.special.softmax(sc)
                att[hh] = p @ Vt[:, j, :]
            att = f32(att).reshape(-1)
            h = f32(dequant(wl.wfmt, P["wo"], P["so"], grp) @ att + h)
            b = f32(rmsnorm(h, P["g_ffn"], wl.eps))
            g = f32(dequant(wl.wfmt, P["wg"], P["sg"], grp) @ b)
            u = f32(dequant(wl.wfmt, P["wu"], P["su"], grp) @ b)
            mm = f32(g.astype(np.float64) * scipy.special.expit(g.astype(np.float64)) * u)
            h = f32(dequant(wl.wfmt, P["wd"], P["sd"], grp) @ mm + h)
            trace.append(h)
        out = {"trace": np.stack(trace), "h": h}
        if wl.has_lm_head:
            hn = f32(rmsnorm(h, m["g_out"], wl.eps))
            logits = f32(dequant(wl.wfmt, m["w_lm"], m["s_lm"], grp) @ hn)
            out["logits"] = logits
            out["token"] = int(np.argmax(logits))
        return out


def logical_kv(kv: dict, wl, n_layers: int):
    """Gather the prior context of a paged pool into logical [L][ctx][Hkv][D] fp32 arrays."""
    pt = kv["page_table"]
    ctx = kv["ctx"]
    t = np.arange(ctx)
    outk, outv = [], []
    for l in range(n_layers):
        for src, dst in ((kv["k"][l], outk), (kv["v"][l], outv)):
            a = src[pt[t // wl.page_size], :, t % wl.page_size, :]   # [ctx][Hkv][D]
            a = a.astype(np.float32) if wl.kv_fmt == "f32" else bf16_bits_to_f32(a)
            dst.append(a)
    return outk, outv
