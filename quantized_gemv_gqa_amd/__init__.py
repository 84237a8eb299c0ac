"""Python binding of libqdec: batch-1 quantized GQA decode step on AMD MI355X (gfx950).

Argument marshalling only.  Every step of the decode path runs in the HIP kernels of
``libqdec.so`` (sources under ``csrc/``); PyTorch only provides device memory and streams.
The library must be built (``__graft_entry__.build()``); importing this package without it
raises, and no operation has a CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
LIB_PATH = os.path.join(_HERE, "libqdec.so")
CSRC = os.path.join(_HERE, "csrc")
INCLUDE = os.path.join(_ROOT, "include")

QDEC_OK, QDEC_EINVAL, QDEC_EUNSUPPORTED, QDEC_EHIP, QDEC_ESTATE = 0, -1, -2, -3, -4
W_Q8, W_Q4 = 1, 2
KV_F32, KV_BF16 = 1, 2
STEP_EAGER, STEP_GRAPH = 0, 1
STEP_PER_OP = 4  # flag for EAGER / GRAPH: one launch per operation instead of two per layer
PAGE = 16
TILE = 64

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build_library(jobs: int = 8, verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libqdec.so in-tree."""
    objdir = os.path.join(_ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = ["hipcc", *HIP_FLAGS, "-I", INCLUDE, "-c", src, "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0), verbose)
    while procs:
        _wait(procs.pop(0), verbose)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _wait(item, verbose):
    cmd, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError("hipcc failed: %s\n%s" % (" ".join(cmd), text))
    if verbose and text.strip():
        print(text)


# ----------------------------------------------------------------------------- ctypes structs
_P = ctypes.c_void_p
_I = ctypes.c_int


class QdecConfig(ctypes.Structure):
    _fields_ = [(n, _I) for n in (
        "n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "inter", "vocab",
        "wfmt", "group", "kv_fmt", "page_size", "n_pages", "has_qkv_bias", "has_qk_norm",
        "num_splits")] + [("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float)]


class QdecLayerWeights(ctypes.Structure):
    _fields_ = [(n, _P) for n in (
        "w_qkv", "s_qkv", "b_qkv", "w_o", "s_o", "w_gu", "s_gu", "w_down", "s_down",
        "g_attn", "g_ffn", "g_q", "g_k")]


class QdecModel(ctypes.Structure):
    _fields_ = [("layers", ctypes.POINTER(QdecLayerWeights)), ("embed", _P), ("g_out", _P),
                ("w_lm", _P), ("s_lm", _P)]


class QdecBatchState(ctypes.Structure):
    _fields_ = [("k_pools", ctypes.POINTER(_P)), ("v_pools", ctypes.POINTER(_P)), ("block_tables", _P),
                ("max_batch", _I), ("max_blocks", _I), ("pos", _P), ("tokens", _P), ("hidden", _P), ("logits", _P),
                ("workspace", _P), ("workspace_bytes", ctypes.c_size_t)]


class QdecState(ctypes.Structure):
    _fields_ = [("k_pools", ctypes.POINTER(_P)), ("v_pools", ctypes.POINTER(_P)),
                ("page_table", _P), ("pos", _P), ("token", _P), ("hidden", _P), ("logits", _P),
                ("trace", _P), ("token_log", _P), ("step_count", _P), ("log_len", _I),
                ("workspace", _P), ("workspace_bytes", ctypes.c_size_t)]


_lib = None


def lib():
    """The loaded libqdec.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libqdec.so is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        S, Z = ctypes.c_int, ctypes.c_size_t
        F = ctypes.c_float
        L.qdec_last_error.restype = ctypes.c_char_p
        L.qdec_version.restype = ctypes.c_char_p
        L.qdec_packed_weight_bytes.argtypes = [_I, _I, _I]; L.qdec_packed_weight_bytes.restype = Z
        L.qdec_packed_scale_bytes.argtypes = [_I, _I, _I, _I]; L.qdec_packed_scale_bytes.restype = Z
        L.qdec_pack_q8.argtypes = [_P, _P, _I, _I, _P, _P, _P]; L.qdec_pack_q8.restype = S
        L.qdec_pack_q4.argtypes = [_P, _P, _I, _I, _I, _P, _P, _P]; L.qdec_pack_q4.restype = S
        L.qdec_gemv_workspace_bytes.argtypes = [_I, _I, _I]; L.qdec_gemv_workspace_bytes.restype = Z
        L.qdec_gemv_q8.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _P, Z, _P]; L.qdec_gemv_q8.restype = S
        L.qdec_gemv_q4.argtypes = [_P, _P, _I, _P, _P, _P, _P, _I, _I, _P, Z, _P]; L.qdec_gemv_q4.restype = S
        L.qdec_gemv_q4_noalloc.argtypes = [_P, _P, _I, _P, _P, _P, _P, _I, _I, _P]
        L.qdec_gemv_q4_noalloc.restype = S
        L.qdec_quantize_act_i8.argtypes = [_P, _I, _I, _P, _P, _P]; L.qdec_quantize_act_i8.restype = S
        L.qdec_gemv_q8_a8.argtypes = [_P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _P, Z, _P]
        L.qdec_gemv_q8_a8.restype = S
        L.qdec_gemv_q4_a8.argtypes = [_P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _P, Z, _P]
        L.qdec_gemv_q4_a8.restype = S
        L.qdec_gemm_workspace_bytes.argtypes = [_I, _I, _I, _I]; L.qdec_gemm_workspace_bytes.restype = Z
        L.qdec_gemm_q8.argtypes = [_P, _P, _P, _I, _I, _P, _P, _P, _I, _I, _I, _P, Z, _P]; L.qdec_gemm_q8.restype = S
        L.qdec_gemm_q4.argtypes = [_P, _P, _I, _P, _I, _I, _P, _P, _P, _I, _I, _I, _P, Z, _P]; L.qdec_gemm_q4.restype = S
        L.qdec_batch_workspace_bytes.argtypes = [ctypes.POINTER(QdecConfig), _I]
        L.qdec_batch_workspace_bytes.restype = Z
        L.qdec_batch_create.argtypes = [ctypes.POINTER(QdecConfig), ctypes.POINTER(QdecModel),
                                        ctypes.POINTER(QdecBatchState), ctypes.POINTER(_P)]
        L.qdec_batch_create.restype = S
        L.qdec_batch_decode_step.argtypes = [_P, _I, _P]; L.qdec_batch_decode_step.restype = S
        L.qdec_batch_kernel_count.argtypes = [_P]; L.qdec_batch_kernel_count.restype = _I
        L.qdec_batch_destroy.argtypes = [_P]; L.qdec_batch_destroy.restype = None
        L.qdec_gemm_mfma.argtypes = [_I, _P, _P, _I, _P, _P, _I, _I, _P, _P, _P, _I, _I, _I, _P]
        L.qdec_gemm_mfma.restype = S
        L.qdec_prefill_workspace_bytes.argtypes = [ctypes.POINTER(QdecConfig), _I]
        L.qdec_prefill_workspace_bytes.restype = Z
        L.qdec_prefill.argtypes = [_P, _P, _I, _P, Z, _P]; L.qdec_prefill.restype = S
        L.qdec_sample_workspace_bytes.argtypes = []; L.qdec_sample_workspace_bytes.restype = Z
        L.qdec_sample.argtypes = [_P, _I, F, _I, F, ctypes.c_uint64, _P, _P, _P, Z, _P]; L.qdec_sample.restype = S
        L.qdec_rmsnorm_rope.argtypes = [_P, _P, _P, _I, _I, F, F, _P, _P]; L.qdec_rmsnorm_rope.restype = S
        L.qdec_swiglu.argtypes = [_P, _P, _P, _I, _P]; L.qdec_swiglu.restype = S
        L.qdec_argmax.argtypes = [_P, _I, _P, _P]; L.qdec_argmax.restype = S
        L.qdec_stream_read.argtypes = [_P, Z, _P, _P]; L.qdec_stream_read.restype = S
        L.qdec_attn_workspace_bytes.argtypes = [_I, _I, _I]; L.qdec_attn_workspace_bytes.restype = Z
        L.qdec_attn_decode_paged.argtypes = [_P, _P, _P, _P, _P, _I, _P, _I, _I, _P, _I, _I, _I, F,
                                             _I, _P, Z, _P, _P]
        L.qdec_attn_decode_paged.restype = S
        L.qdec_step_workspace_bytes.argtypes = [ctypes.POINTER(QdecConfig)]
        L.qdec_step_workspace_bytes.restype = Z
        L.qdec_step_create.argtypes = [ctypes.POINTER(QdecConfig), ctypes.POINTER(QdecModel),
                                       ctypes.POINTER(QdecState), ctypes.POINTER(_P)]
        L.qdec_step_create.restype = S
        L.qdec_decode_step.argtypes = [_P, _I, _P]; L.qdec_decode_step.restype = S
        L.qdec_step_set_sampling.argtypes = [_P, F, _I, F, ctypes.c_uint64]; L.qdec_step_set_sampling.restype = S
        L.qdec_step_kernel_count.argtypes = [_P]; L.qdec_step_kernel_count.restype = _I
        L.qdec_step_kernel_times.argtypes = [_P, _I, _P, _I, _P]; L.qdec_step_kernel_times.restype = _I
        L.qdec_step_layer_blocks.argtypes = [_P]; L.qdec_step_layer_blocks.restype = _I
        L.qdec_step_layer_timeline.argtypes = [_P, _P]; L.qdec_step_layer_timeline.restype = S
        L.qdec_step_mlp_timeline.argtypes = [_P, _P, ctypes.POINTER(_I)]; L.qdec_step_mlp_timeline.restype = S
        L.qdec_step_destroy.argtypes = [_P]; L.qdec_step_destroy.restype = None
        L.qdec_step_read_error.argtypes = [_P, ctypes.POINTER(_I)]; L.qdec_step_read_error.restype = S
        _lib = L
    return _lib


EXPORTED = [
    "qdec_last_error", "qdec_version", "qdec_packed_weight_bytes", "qdec_packed_scale_bytes",
    "qdec_pack_q8", "qdec_pack_q4", "qdec_gemv_workspace_bytes", "qdec_gemv_q8", "qdec_gemv_q4",
    "qdec_gemv_q4_noalloc",
    "qdec_quantize_act_i8", "qdec_gemv_q8_a8", "qdec_gemv_q4_a8", "qdec_sample_workspace_bytes", "qdec_sample",
    "qdec_gemm_workspace_bytes", "qdec_gemm_q8", "qdec_gemm_q4", "qdec_batch_workspace_bytes", "qdec_batch_create",
    "qdec_batch_decode_step", "qdec_batch_kernel_count", "qdec_batch_destroy", "qdec_prefill_workspace_bytes",
    "qdec_prefill", "qdec_gemm_mfma",
    "qdec_rmsnorm_rope", "qdec_swiglu", "qdec_argmax", "qdec_stream_read", "qdec_attn_workspace_bytes",
    "qdec_attn_decode_paged", "qdec_step_workspace_bytes", "qdec_step_create", "qdec_decode_step",
    "qdec_step_kernel_count", "qdec_step_kernel_times", "qdec_step_layer_blocks", "qdec_step_layer_timeline", "qdec_step_mlp_timeline", "qdec_step_set_sampling", "qdec_step_destroy", "qdec_step_read_error",
]


class QdecError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().qdec_last_error().decode(errors="replace")
        super().__init__("%s failed with status %d: %s" % (where, status, msg))
        self.status = status


def _check(status: int, where: str):
    if status != QDEC_OK:
        raise QdecError(status, where)


def _ptr(t):
    if t is None:
        return None
    assert t.is_cuda and t.is_contiguous(), "qdec needs contiguous device tensors"
    return t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


# ----------------------------------------------------------------------------- packing
def pack_q8(W: torch.Tensor, scale: torch.Tensor, stream=None):
    """int8 [N][K] + fp32 [N] (device, row-major) -> packed tile64 weights and padded scales."""
    N, K = W.shape
    Wp = torch.empty(lib().qdec_packed_weight_bytes(W_Q8, N, K), dtype=torch.uint8, device=W.device)
    Sp = torch.empty(lib().qdec_packed_scale_bytes(W_Q8, N, K, 0) // 4, dtype=torch.float32, device=W.device)
    _check(lib().qdec_pack_q8(_ptr(W), _ptr(scale), N, K, _ptr(Wp), _ptr(Sp), _stream(stream)), "qdec_pack_q8")
    return Wp, Sp


def pack_q4(W: torch.Tensor, scale: torch.Tensor, group: int = 64, stream=None):
    """uint8 [N][K/2] + fp16 bits [N][K/group] (device, row-major) -> packed weights and scales."""
    N, K = W.shape[0], W.shape[1] * 2
    Wp = torch.empty(lib().qdec_packed_weight_bytes(W_Q4, N, K), dtype=torch.uint8, device=W.device)
    nb = lib().qdec_packed_scale_bytes(W_Q4, N, K, group)
    Sp = torch.empty(max(nb, 2) // 2, dtype=torch.int16, device=W.device)
    _check(lib().qdec_pack_q4(_ptr(W), _ptr(scale), N, K, group, _ptr(Wp), _ptr(Sp), _stream(stream)),
           "qdec_pack_q4")
    return Wp, Sp


def pack(wfmt: str, W: torch.Tensor, scale: torch.Tensor, group: int = 64, stream=None):
    return pack_q8(W, scale, stream) if wfmt == "q8" else pack_q4(W, scale, group, stream)


def gemv_workspace(wfmt: str, N: int, K: int, device="cuda"):
    nb = lib().qdec_gemv_workspace_bytes(W_Q8 if wfmt == "q8" else W_Q4, N, K)
    return torch.zeros(nb, dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------- per-op calls
def gemv(wfmt: str, Wp, Sp, x, N: int, bias=None, residual=None, y=None, workspace=None,
         group: int = 64, stream=None):
    K = x.numel()
    if y is None:
        y = torch.empty(N, dtype=torch.float32, device=x.device)
    ws, wsb = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel())
    if wfmt == "q8":
        st = lib().qdec_gemv_q8(_ptr(Wp), _ptr(Sp), _ptr(x), _ptr(bias), _ptr(residual), _ptr(y), N, K,
                                ws, wsb, _stream(stream))
    else:
        st = lib().qdec_gemv_q4(_ptr(Wp), _ptr(Sp), group, _ptr(x), _ptr(bias), _ptr(residual), _ptr(y),
                                N, K, ws, wsb, _stream(stream))
    _check(st, "qdec_gemv_" + wfmt)
    return y


def gemv_q4_noalloc(Wp, Sp, x, N: int, bias=None, residual=None, y=None, group: int = 64, stream=None):
    """qdec_gemv_q4 without a workspace: the library's static per-GPU scratch holds the split-K state."""
    K = x.numel()
    if y is None:
        y = torch.empty(N, dtype=torch.float32, device=x.device)
    _check(lib().qdec_gemv_q4_noalloc(_ptr(Wp), _ptr(Sp), group, _ptr(x), _ptr(bias), _ptr(residual), _ptr(y), N, K,
                                      _stream(stream)), "qdec_gemv_q4_noalloc")
    return y


def quantize_act_i8(x, group: int = 64, q=None, sx=None, stream=None):
    """INT8 activations with one fp32 scale per group of `group` k (Path A)."""
    K = x.numel()
    if q is None:
        q = torch.empty(K, dtype=torch.int8, device=x.device)
    if sx is None:
        sx = torch.empty(K // group, dtype=torch.float32, device=x.device)
    _check(lib().qdec_quantize_act_i8(_ptr(x), K, group, _ptr(q), _ptr(sx), _stream(stream)), "qdec_quantize_act_i8")
    return q, sx


def gemv_a8(wfmt: str, Wp, Sp, q, sx, N: int, bias=None, residual=None, y=None, workspace=None,
            group: int = 64, stream=None):
    """GEMV on INT8 activations (q, sx from quantize_act_i8 with the same group)."""
    K = q.numel()
    if y is None:
        y = torch.empty(N, dtype=torch.float32, device=q.device)
    ws, wsb = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel())
    if wfmt == "q8":
        st = lib().qdec_gemv_q8_a8(_ptr(Wp), _ptr(Sp), _ptr(q), _ptr(sx), group, _ptr(bias), _ptr(residual),
                                   _ptr(y), N, K, ws, wsb, _stream(stream))
    else:
        st = lib().qdec_gemv_q4_a8(_ptr(Wp), _ptr(Sp), group, _ptr(q), _ptr(sx), _ptr(bias), _ptr(residual),
                                   _ptr(y), N, K, ws, wsb, _stream(stream))
    _check(st, "qdec_gemv_%s_a8" % wfmt)
    return y


def gemm(wfmt: str, Wp, Sp, X, N: int, bias=None, residual=None, Y=None, workspace=None, group: int = 64,
         stream=None):
    """Skinny GEMM: Y [nb][N] = W X[b] for the rows of X [nb][K] (nb <= 8)."""
    nb, K = X.shape
    if Y is None:
        Y = torch.empty((nb, N), dtype=torch.float32, device=X.device)
    ws, wsb = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel())
    if wfmt == "q8":
        st = lib().qdec_gemm_q8(_ptr(Wp), _ptr(Sp), _ptr(X), K, nb, _ptr(bias), _ptr(residual), _ptr(Y), Y.shape[1], N,
                                K, ws, wsb, _stream(stream))
    else:
        st = lib().qdec_gemm_q4(_ptr(Wp), _ptr(Sp), group, _ptr(X), K, nb, _ptr(bias), _ptr(residual), _ptr(Y),
                                Y.shape[1], N, K, ws, wsb, _stream(stream))
    _check(st, "qdec_gemm_" + wfmt)
    return Y


def gemm_mfma(wfmt: str, Wp, Sp, X16, N: int, X16lo=None, bias=None, residual=None, Y=None, group: int = 64,
              stream=None):
    """Prefill GEMM: Y [M][N] = W X[m] for activations X = X16 + X16lo ([M][K] torch.float16 each)."""
    M, K = X16.shape
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X16.device)
    _check(lib().qdec_gemm_mfma(W_Q8 if wfmt == "q8" else W_Q4, _ptr(Wp), _ptr(Sp), group, _ptr(X16), _ptr(X16lo), K, M,
                                _ptr(bias), _ptr(residual), _ptr(Y), Y.shape[1], N, K, _stream(stream)), "qdec_gemm_mfma")
    return Y


def gemm_workspace(wfmt: str, N: int, K: int, nb: int, device="cuda"):
    nbytes = lib().qdec_gemm_workspace_bytes(W_Q8 if wfmt == "q8" else W_Q4, N, K, nb)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def sample_workspace(device="cuda"):
    return torch.empty(lib().qdec_sample_workspace_bytes(), dtype=torch.uint8, device=device)


def sample(logits, temperature: float, top_k: int = 0, top_p: float = 1.0, seed: int = 0, step=None,
           token=None, workspace=None, stream=None):
    """Next token from device logits (temperature / top-k / top-p, Gumbel-max draw keyed by
    (seed, *step)); returns the device int32 token tensor."""
    if token is None:
        token = torch.empty(1, dtype=torch.int32, device=logits.device)
    if workspace is None:
        workspace = sample_workspace(logits.device)
    _check(lib().qdec_sample(_ptr(logits), logits.numel(), temperature, top_k, top_p, seed, _ptr(step), _ptr(token),
                             _ptr(workspace), workspace.numel(), _stream(stream)), "qdec_sample")
    return token


def rmsnorm_rope(x, gamma=None, eps: float = 1e-6, rope_base: float = 0.0, pos=None, out=None, stream=None):
    rows, dim = x.shape
    y = torch.empty_like(x) if out is None else out
    _check(lib().qdec_rmsnorm_rope(_ptr(x), _ptr(gamma), _ptr(y), rows, dim, eps, rope_base, _ptr(pos),
                                   _stream(stream)), "qdec_rmsnorm_rope")
    return y


def swiglu(g, u, out=None, stream=None):
    m = torch.empty_like(g) if out is None else out
    _check(lib().qdec_swiglu(_ptr(g), _ptr(u), _ptr(m), g.numel(), _stream(stream)), "qdec_swiglu")
    return m


def argmax(logits, stream=None):
    tok = torch.empty(1, dtype=torch.int32, device=logits.device)
    _check(lib().qdec_argmax(_ptr(logits), logits.numel(), _ptr(tok), _stream(stream)), "qdec_argmax")
    return tok


def stream_read(src, sink=None, stream=None):
    """Bandwidth reference: read every byte of the device tensor `src` once (qdec_stream_read)."""
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=src.device)
    _check(lib().qdec_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)),
           "qdec_stream_read")
    return sink


def attn_workspace(n_heads: int, head_dim: int, num_splits: int, device="cuda"):
    nb = lib().qdec_attn_workspace_bytes(n_heads, head_dim, num_splits)
    return torch.zeros(nb, dtype=torch.uint8, device=device)


def attn_decode_paged(q, k_pool, v_pool, kv_fmt: str, page_table, pos, n_kv_heads: int,
                      k_new=None, v_new=None, num_splits: int = 16, sm_scale=None, workspace=None,
                      out=None, stream=None):
    """q [Hq][D]; pools [pages][Hkv][16][D] (fp32 or bf16-bits int16); pos: int32 [1] device."""
    Hq, D = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / (D ** 0.5)
    if workspace is None:
        workspace = attn_workspace(Hq, D, num_splits, q.device)
    o = torch.empty_like(q) if out is None else out
    fmt = KV_F32 if kv_fmt == "f32" else KV_BF16
    _check(lib().qdec_attn_decode_paged(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), fmt,
                                        _ptr(page_table), k_pool.shape[0], PAGE, _ptr(pos), Hq, n_kv_heads, D,
                                        float(sm_scale), num_splits, _ptr(workspace), workspace.numel(),
                                        _ptr(o), _stream(stream)), "qdec_attn_decode_paged")
    return o


# ----------------------------------------------------------------------------- model upload
def _to_dev(a, device, dtype=None):
    import numpy as np
    if a.dtype == np.uint16:  # fp16 / bf16 bit patterns travel as int16
        a = a.view(np.int16)
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None and t.dtype != dtype:
        t = t.view(dtype)
    return t.to(device)


def interleave_gate_up(g: torch.Tensor, u: torch.Tensor) -> torch.Tensor:
    """Row order of the fused gate/up matrix: per 64-row tile, 32 gate rows then the same 32 up rows."""
    I = g.shape[0]
    assert I % 32 == 0 and u.shape == g.shape
    rest = g.shape[1:]
    return torch.stack([g.reshape(I // 32, 32, *rest), u.reshape(I // 32, 32, *rest)], dim=1).reshape(2 * I, *rest)


def upload_model(model: dict, device="cuda", stream=None) -> dict:
    """Host model arrays (row-major interchange layout) -> packed device tensors for the step."""
    wl = model["workload"]
    grp = wl.group
    sdt = torch.int16 if wl.wfmt == "q4" else None
    layers = []
    for P in model["layers"]:
        d = {}
        wq = torch.cat([_to_dev(P[n], device) for n in ("wq", "wk", "wv")])
        sq = torch.cat([_to_dev(P[n], device, sdt) for n in ("sq", "sk", "sv")])
        d["w_qkv"], d["s_qkv"] = pack(wl.wfmt, wq, sq, grp, stream)
        if wl.qkv_bias:
            d["b_qkv"] = torch.cat([_to_dev(P[n], device) for n in ("bq", "bk", "bv")])
        d["w_o"], d["s_o"] = pack(wl.wfmt, _to_dev(P["wo"], device), _to_dev(P["so"], device, sdt), grp, stream)
        wgu = interleave_gate_up(_to_dev(P["wg"], device), _to_dev(P["wu"], device))
        sgu = interleave_gate_up(_to_dev(P["sg"], device, sdt), _to_dev(P["su"], device, sdt))
        d["w_gu"], d["s_gu"] = pack(wl.wfmt, wgu.contiguous(), sgu.contiguous(), grp, stream)
        d["w_down"], d["s_down"] = pack(wl.wfmt, _to_dev(P["wd"], device), _to_dev(P["sd"], device, sdt), grp,
                                        stream)
        d["g_attn"], d["g_ffn"] = _to_dev(P["g_attn"], device), _to_dev(P["g_ffn"], device)
        if wl.qk_norm:
            d["g_q"], d["g_k"] = _to_dev(P["g_q"], device), _to_dev(P["g_k"], device)
        layers.append(d)
        del wq, sq, wgu, sgu
    out = {"layers": layers, "workload": wl}
    if wl.has_lm_head:
        out["embed"] = _to_dev(model["embed"], device, torch.int16)
        out["g_out"] = _to_dev(model["g_out"], device)
        out["w_lm"], out["s_lm"] = pack(wl.wfmt, _to_dev(model["w_lm"], device),
                                        _to_dev(model["s_lm"], device, sdt), grp, stream)
    return out


def upload_kv(kv: dict, kv_fmt: str, device="cuda") -> dict:
    dt = torch.int16 if kv_fmt == "bf16" else None
    return {"page_table": _to_dev(kv["page_table"], device),
            "k": [_to_dev(a, device, dt) for a in kv["k"]],
            "v": [_to_dev(a, device, dt) for a in kv["v"]]}


def default_splits(n_kv_heads: int, ctx: int, pages_per_split: int = 4) -> int:
    """Attention split count: at most `pages_per_split` KV pages per split (the context is dealt
    to the splits first, so a split's keys sit on its first waves, one per SIMD of the compute
    unit), rounded up to a multiple of 4 so a context that grows by a few pages keeps the same
    count, at most 64 (past that a longer context gives each wave more keys).  Measured on
    MI355X, ms per step: Qwen2.5-7B shape at 4096 tokens, 64 splits 1.546-1.550, 60 1.551, 56
    1.549-1.553, 48 1.561-1.564; Qwen2.5-1.5B shape at 1024 tokens, 16 splits 1.065-1.067, 20
    1.054-1.058, 24 1.064, 32 1.070-1.072, 64 1.089-1.093."""
    pages = max(1, -(-(ctx + 1) // PAGE))
    s = -(-pages // pages_per_split)
    s = -(-s // 4) * 4
    return int(max(1, min(s, 64)))


# ----------------------------------------------------------------------------- decode steps
def batch_splits(batch: int, n_kv_heads: int, ctx: int) -> int:
    """Attention splits for a batch: the batch-1 choice, capped so that batch * KV heads * splits
    stays near 256 workgroups (one per compute unit; each is latency-bound, so more of them only
    queue).  Measured at 4096 tokens, Qwen2.5-7B shape: 8 sequences 8 splits 4.11 ms per step, 16
    splits 4.54 ms, 4 splits 4.42 ms; 4 sequences 16 splits 3.23 ms, 8 splits 3.36 ms, 24 splits
    3.54 ms; 2 sequences 32 splits 2.86 ms, 16 splits 2.93 ms."""
    return int(max(1, min(default_splits(n_kv_heads, ctx), 256 // max(1, batch * n_kv_heads))))


class BatchDecode:
    """Batched decode of up to 8 sequences over one shared paged KV pool (libqdec batch handle).

    The caller keeps `block_tables` ([max_batch][max_blocks] int32, device), `pos` and `tokens`
    ([max_batch] int32, device) up to date between steps: a slot with pos < 0 is idle, and the block
    of the position about to be written must be mapped before the step."""

    def __init__(self, dev_model: dict, k_pools, v_pools, block_tables, pos, tokens, num_splits: int = 8,
                 device="cuda"):
        """num_splits: attention splits per (sequence, KV head); batch_splits() gives a choice that
        keeps about two attention workgroups per compute unit."""
        wl = dev_model["workload"]
        self.wl = wl
        L = len(dev_model["layers"])
        B, mb = block_tables.shape
        c = QdecConfig()
        c.n_layers, c.hidden, c.n_heads, c.n_kv_heads = L, wl.hidden, wl.n_heads, wl.n_kv_heads
        c.head_dim, c.inter, c.vocab = wl.head_dim, wl.inter, wl.vocab
        c.wfmt, c.group = (W_Q8 if wl.wfmt == "q8" else W_Q4), wl.group
        c.kv_fmt, c.page_size = (KV_F32 if wl.kv_fmt == "f32" else KV_BF16), PAGE
        c.n_pages = k_pools[0].shape[0]
        c.has_qkv_bias, c.has_qk_norm = int(wl.qkv_bias), int(wl.qk_norm)
        c.num_splits = num_splits
        c.rms_eps, c.rope_base = wl.eps, wl.rope_base
        self.cfg = c
        self.block_tables, self.pos, self.tokens = block_tables, pos, tokens
        self._keep = [dev_model, k_pools, v_pools]
        self.layer_arr = (QdecLayerWeights * L)()
        for i, d in enumerate(dev_model["layers"]):
            lw = self.layer_arr[i]
            for n in ("w_qkv", "s_qkv", "w_o", "s_o", "w_gu", "s_gu", "w_down", "s_down", "g_attn", "g_ffn"):
                setattr(lw, n, _ptr(d[n]))
            for n in ("b_qkv", "g_q", "g_k"):
                setattr(lw, n, _ptr(d.get(n)))
        m = QdecModel()
        m.layers = self.layer_arr
        m.embed, m.g_out = _ptr(dev_model["embed"]), _ptr(dev_model["g_out"])
        m.w_lm, m.s_lm = _ptr(dev_model["w_lm"]), _ptr(dev_model["s_lm"])
        self.model = m
        self.hidden = torch.zeros((B, wl.hidden), dtype=torch.float32, device=device)
        self.logits = torch.zeros((B, wl.vocab), dtype=torch.float32, device=device)
        nbytes = lib().qdec_batch_workspace_bytes(ctypes.byref(c), B)
        if nbytes == 0:
            raise QdecError(QDEC_EINVAL, "qdec_batch_workspace_bytes")
        self.workspace = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        self.kp = (_P * L)(*[_ptr(t) for t in k_pools[:L]])
        self.vp = (_P * L)(*[_ptr(t) for t in v_pools[:L]])
        s = QdecBatchState()
        s.k_pools, s.v_pools = self.kp, self.vp
        s.block_tables, s.max_batch, s.max_blocks = _ptr(block_tables), B, mb
        s.pos, s.tokens, s.hidden, s.logits = _ptr(pos), _ptr(tokens), _ptr(self.hidden), _ptr(self.logits)
        s.workspace, s.workspace_bytes = _ptr(self.workspace), nbytes
        self.state = s
        h = _P()
        _check(lib().qdec_batch_create(ctypes.byref(c), ctypes.byref(m), ctypes.byref(s), ctypes.byref(h)),
               "qdec_batch_create")
        self.handle = h

    def step(self, mode: int = STEP_EAGER, stream=None):
        _check(lib().qdec_batch_decode_step(self.handle, mode, _stream(stream)), "qdec_batch_decode_step")

    @property
    def kernel_count(self) -> int:
        return lib().qdec_batch_kernel_count(self.handle)

    def close(self):
        if getattr(self, "handle", None):
            lib().qdec_batch_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class DecodeStep:
    """Owns the device state of one decode stream and a libqdec step handle."""

    def __init__(self, dev_model: dict, dev_kv: dict, pos0: int, token0: int = 0, num_splits: int | None = None,
                 trace: bool = False, log_len: int = 0, h0=None, device="cuda"):
        wl = dev_model["workload"]
        self.wl = wl
        self.device = device
        L = len(dev_model["layers"])
        self.n_layers = L
        c = QdecConfig()
        c.n_layers, c.hidden, c.n_heads, c.n_kv_heads = L, wl.hidden, wl.n_heads, wl.n_kv_heads
        c.head_dim, c.inter, c.vocab = wl.head_dim, wl.inter, wl.vocab
        c.wfmt, c.group = (W_Q8 if wl.wfmt == "q8" else W_Q4), wl.group
        c.kv_fmt, c.page_size = (KV_F32 if wl.kv_fmt == "f32" else KV_BF16), PAGE
        c.n_pages = dev_kv["k"][0].shape[0]
        c.has_qkv_bias, c.has_qk_norm = int(wl.qkv_bias), int(wl.qk_norm)
        c.num_splits = num_splits or default_splits(wl.n_kv_heads, pos0)
        c.rms_eps, c.rope_base = wl.eps, wl.rope_base
        self.cfg = c
        self._keep = [dev_model, dev_kv]
        self.layer_arr = (QdecLayerWeights * L)()
        for i, d in enumerate(dev_model["layers"]):
            lw = self.layer_arr[i]
            for n in ("w_qkv", "s_qkv", "w_o", "s_o", "w_gu", "s_gu", "w_down", "s_down", "g_attn", "g_ffn"):
                setattr(lw, n, _ptr(d[n]))
            for n in ("b_qkv", "g_q", "g_k"):
                setattr(lw, n, _ptr(d.get(n)))
        m = QdecModel()
        m.layers = self.layer_arr
        if wl.has_lm_head:
            m.embed, m.g_out = _ptr(dev_model["embed"]), _ptr(dev_model["g_out"])
            m.w_lm, m.s_lm = _ptr(dev_model["w_lm"]), _ptr(dev_model["s_lm"])
        self.model = m
        i32 = dict(dtype=torch.int32, device=device)
        self.pos = torch.tensor([pos0], **i32)
        self.token = torch.tensor([token0], **i32)
        self.hidden = torch.zeros(wl.hidden, dtype=torch.float32, device=device)
        if h0 is not None:
            self.hidden.copy_(torch.from_numpy(h0))
        self.logits = torch.zeros(max(wl.vocab, 1), dtype=torch.float32, device=device)
        self.trace = torch.zeros((L + 1, wl.hidden), dtype=torch.float32, device=device) if trace else None
        self.token_log = torch.full((max(log_len, 1),), -1, **i32) if log_len else None
        self.step_count = torch.zeros(1, **i32)
        ws_bytes = lib().qdec_step_workspace_bytes(ctypes.byref(c))
        if ws_bytes == 0:
            raise QdecError(QDEC_EINVAL, "qdec_step_workspace_bytes")
        self.workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=device)
        self.kp = (_P * L)(*[_ptr(t) for t in dev_kv["k"][:L]])
        self.vp = (_P * L)(*[_ptr(t) for t in dev_kv["v"][:L]])
        s = QdecState()
        s.k_pools, s.v_pools = self.kp, self.vp
        s.page_table, s.pos, s.token = _ptr(dev_kv["page_table"]), _ptr(self.pos), _ptr(self.token)
        s.hidden, s.logits = _ptr(self.hidden), (_ptr(self.logits) if wl.has_lm_head else None)
        s.trace = _ptr(self.trace)
        s.token_log, s.step_count = _ptr(self.token_log), _ptr(self.step_count)
        s.log_len = log_len
        s.workspace, s.workspace_bytes = _ptr(self.workspace), ws_bytes
        self.state = s
        h = _P()
        _check(lib().qdec_step_create(ctypes.byref(c), ctypes.byref(m), ctypes.byref(s), ctypes.byref(h)),
               "qdec_step_create")
        self.handle = h

    def step(self, mode: int = STEP_EAGER, stream=None):
        _check(lib().qdec_decode_step(self.handle, mode, _stream(stream)), "qdec_decode_step")

    def prefill(self, tokens, stream=None, workspace=None):
        """Run the prompt `tokens` (int32 device tensor) at positions pos .. pos + n - 1: stores its
        KV, sets token to the greedy next token and advances pos by n (libqdec qdec_prefill)."""
        n = tokens.numel()
        if workspace is None:
            nbytes = lib().qdec_prefill_workspace_bytes(ctypes.byref(self.cfg), n)
            if nbytes == 0:
                raise QdecError(QDEC_EUNSUPPORTED, "qdec_prefill_workspace_bytes")
            if getattr(self, "_pws", None) is None or self._pws.numel() < nbytes:
                self._pws = torch.zeros(nbytes, dtype=torch.uint8, device=tokens.device)
            workspace = self._pws
        _check(lib().qdec_prefill(self.handle, _ptr(tokens), n, _ptr(workspace), workspace.numel(), _stream(stream)),
               "qdec_prefill")

    def set_sampling(self, temperature: float, top_k: int = 0, top_p: float = 1.0, seed: int = 0):
        """Sample later tokens (temperature / top-k / top-p, draw counter = step_count) instead of
        taking the greedy argmax; temperature <= 0 goes back to greedy.  Drops captured graphs."""
        _check(lib().qdec_step_set_sampling(self.handle, temperature, top_k, top_p, seed), "qdec_step_set_sampling")

    @property
    def kernel_count(self) -> int:
        return lib().qdec_step_kernel_count(self.handle)

    def kernel_times(self, per_op: bool = False, stream=None):
        """One eager step with a HIP event after every kernel: the list of kernel durations in
        microseconds, in launch order (the step advances like any other)."""
        import numpy as np
        buf = np.zeros(8 + 8 * self.n_layers, np.float32)
        n = lib().qdec_step_kernel_times(self.handle, STEP_EAGER | (STEP_PER_OP if per_op else 0),
                                         buf.ctypes.data_as(_P), buf.size, _stream(stream))
        if n < 0:
            raise QdecError(n, "qdec_step_kernel_times")
        return buf[:n].tolist()

    @property
    def layer_blocks(self) -> int:
        """Workgroups of the fused attention launch (0: the step has none)."""
        return lib().qdec_step_layer_blocks(self.handle)

    def layer_timeline(self, ts=None):
        """Record per-wave clock marks of the fused attention launches of later steps into `ts`
        (int64 device tensor [n_layers][blocks][8][16], zeroed by the caller); None stops."""
        _check(lib().qdec_step_layer_timeline(self.handle, _ptr(ts)), "qdec_step_layer_timeline")
        self._tl = ts

    def mlp_units(self):
        """(gate/up units, down units): wave jobs of the two MLP GEMV launches of a layer."""
        u = (_I * 2)()
        _check(lib().qdec_step_mlp_timeline(self.handle, None, u), "qdec_step_mlp_timeline")
        return int(u[0]), int(u[1])

    def mlp_timeline(self, ts=None):
        """Record per-unit clock marks of the gate/up and down launches of later steps into `ts`
        (int64 device tensor [n_layers][gate/up units + down units][8], zeroed by the caller);
        None stops."""
        _check(lib().qdec_step_mlp_timeline(self.handle, _ptr(ts), None), "qdec_step_mlp_timeline")
        self._mtl = ts

    def read_error(self) -> int:
        """The step's device error flag (a bounded wait gave up), cleared after reading."""
        f = _I()
        _check(lib().qdec_step_read_error(self.handle, ctypes.byref(f)), "qdec_step_read_error")
        return int(f.value)

    def close(self):
        if getattr(self, "handle", None):
            lib().qdec_step_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
