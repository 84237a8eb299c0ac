"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function the
public header declares, sizes its buffers as documented, and rejects bad arguments before any
HIP call."""
import ctypes
import os
import re

import pytest

q = pytest.importorskip("quantized_gemv_gqa_amd")

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qdec.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qdec_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(q.LIB_PATH):
        pytest.skip("libqdec.so not built")
    return q.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 19
    for n in names:
        assert hasattr(L, n), n
    assert set(q.EXPORTED) == set(names)


def test_version_and_error_string(L):
    assert b"gfx950" in L.qdec_version()
    assert isinstance(L.qdec_last_error(), bytes)


def test_packed_sizes(L):
    # tiles of 64 rows, zero padded: N = 100 -> 128 rows
    assert L.qdec_packed_weight_bytes(q.W_Q8, 100, 64) == 128 * 64
    assert L.qdec_packed_weight_bytes(q.W_Q4, 100, 64) == 128 * 32
    assert L.qdec_packed_scale_bytes(q.W_Q8, 100, 64, 0) == 128 * 4
    assert L.qdec_packed_scale_bytes(q.W_Q4, 100, 128, 64) == 128 * 2 * 2
    assert L.qdec_packed_weight_bytes(7, 100, 64) == 0       # unknown layout id
    assert L.qdec_packed_scale_bytes(q.W_Q4, 100, 100, 64) == 0  # K not a multiple of group
    # Qwen2.5-7B shape, INT4 groups of 64: the packed lm_head is exactly V * H / 2 bytes
    assert L.qdec_packed_weight_bytes(q.W_Q4, 152064, 3584) == 152064 * 3584 // 2
    assert L.qdec_packed_scale_bytes(q.W_Q4, 152064, 3584, 64) == 152064 * 56 * 2


def test_workspace_sizes(L):
    assert L.qdec_attn_workspace_bytes(28, 128, 64) == 8192 + 64 * 28 * 130 * 4
    assert L.qdec_attn_workspace_bytes(0, 128, 64) == 0
    assert L.qdec_gemv_workspace_bytes(q.W_Q4, 4608, 3584) > 0
    assert L.qdec_gemv_workspace_bytes(9, 4608, 3584) == 0


FAKE = 1 << 32  # a 256-byte aligned address that is never dereferenced by a rejected call


def _err(L):
    return L.qdec_last_error().decode()


def test_gemv_rejects_bad_arguments(L):
    st = L.qdec_gemv_q8(None, FAKE, FAKE, None, None, FAKE, 10, 64, None, 0, None)
    assert st == q.QDEC_EINVAL and "null" in _err(L)
    st = L.qdec_gemv_q8(FAKE, FAKE, FAKE, None, None, FAKE + 4096, 10, 60, None, 0, None)
    assert st == q.QDEC_EINVAL and "multiple of 16" in _err(L)
    st = L.qdec_gemv_q4(FAKE, FAKE, 48, FAKE, None, None, FAKE + 4096, 10, 96, None, 0, None)
    assert st == q.QDEC_EUNSUPPORTED and "group" in _err(L)
    st = L.qdec_gemv_q4(FAKE, FAKE, 64, FAKE, None, None, FAKE + 4096, 10, 96, None, 0, None)
    assert st == q.QDEC_EINVAL and "multiple of group" in _err(L)
    st = L.qdec_gemv_q4(FAKE + 8, FAKE, 64, FAKE, None, None, FAKE + 4096, 10, 128, None, 0, None)
    assert st == q.QDEC_EINVAL and "aligned" in _err(L)
    st = L.qdec_gemv_q4(FAKE, FAKE, 64, FAKE, None, None, FAKE + 64, 10, 128, None, 0, None)
    assert st == q.QDEC_EINVAL and "overlap" in _err(L)
    st = L.qdec_gemv_q4(FAKE, FAKE, 64, FAKE, None, None, FAKE + 4096, 10, 128, FAKE, 16, None)
    assert st == q.QDEC_EINVAL and "workspace too small" in _err(L)


def test_int8_activation_calls_reject_bad_arguments(L):
    assert L.qdec_quantize_act_i8(None, 128, 64, FAKE, FAKE, None) == q.QDEC_EINVAL
    st = L.qdec_quantize_act_i8(FAKE, 128, 48, FAKE + 4096, FAKE + 8192, None)
    assert st == q.QDEC_EUNSUPPORTED and "group" in _err(L)
    st = L.qdec_quantize_act_i8(FAKE, 96, 64, FAKE + 4096, FAKE + 8192, None)
    assert st == q.QDEC_EINVAL and "multiple of group" in _err(L)
    st = L.qdec_quantize_act_i8(FAKE, 128, 64, FAKE + 256, FAKE + 8192, None)
    assert st == q.QDEC_EINVAL and "overlap" in _err(L)
    st = L.qdec_gemv_q8_a8(FAKE, FAKE, None, FAKE, 64, None, None, FAKE, 10, 128, None, 0, None)
    assert st == q.QDEC_EINVAL and "null" in _err(L)
    st = L.qdec_gemv_q8_a8(FAKE, FAKE, FAKE, FAKE, 16, None, None, FAKE, 10, 128, None, 0, None)
    assert st == q.QDEC_EUNSUPPORTED and "group" in _err(L)
    st = L.qdec_gemv_q4_a8(FAKE, FAKE, 64, FAKE, FAKE, None, None, FAKE, 10, 96, None, 0, None)
    assert st == q.QDEC_EINVAL and "multiple of group" in _err(L)
    st = L.qdec_gemv_q4_a8(FAKE, FAKE, 64, FAKE + 4, FAKE, None, None, FAKE, 10, 128, None, 0, None)
    assert st == q.QDEC_EINVAL and "aligned" in _err(L)
    st = L.qdec_gemv_q4_a8(FAKE, FAKE, 64, FAKE, FAKE, None, None, FAKE, 10, 128, FAKE, 16, None)
    assert st == q.QDEC_EINVAL and "workspace too small" in _err(L)


def test_sample_rejects_bad_arguments(L):
    WS = L.qdec_sample_workspace_bytes()
    assert WS > 0
    ok = dict(logits=FAKE, V=1000, temperature=0.7, top_k=20, top_p=0.9, seed=1, step=None, token=FAKE + 8192,
              workspace=FAKE, workspace_bytes=WS, stream=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.qdec_sample(*a.values())
    assert call(logits=None) == q.QDEC_EINVAL
    assert call(V=0) == q.QDEC_EINVAL
    assert call(temperature=float("nan")) == q.QDEC_EINVAL
    assert call(top_p=0.0) == q.QDEC_EINVAL and "top_p" in _err(L)
    assert call(top_p=1.5) == q.QDEC_EINVAL
    assert call(top_k=-1) == q.QDEC_EINVAL
    assert call(top_k=0) == q.QDEC_EUNSUPPORTED and "top_p < 1" in _err(L)
    assert call(top_k=300) == q.QDEC_EUNSUPPORTED
    assert call(top_k=300, top_p=1.0) == q.QDEC_EUNSUPPORTED
    assert call(workspace=FAKE + 16) == q.QDEC_EINVAL
    assert call(workspace_bytes=WS - 1) == q.QDEC_EINVAL and "too small" in _err(L)


def test_batch_and_gemm_validation(L):
    c = _cfg(n_pages=600)
    assert L.qdec_batch_workspace_bytes(ctypes.byref(c), 8) > 0
    assert L.qdec_batch_workspace_bytes(ctypes.byref(c), 9) == 0
    assert L.qdec_batch_workspace_bytes(ctypes.byref(c), 0) == 0
    assert L.qdec_batch_create(None, None, None, None) == q.QDEC_EINVAL
    assert L.qdec_gemm_workspace_bytes(q.W_Q4, 4608, 3584, 8) > L.qdec_gemm_workspace_bytes(q.W_Q4, 4608, 3584, 2)
    assert L.qdec_gemm_workspace_bytes(q.W_Q4, 4608, 3584, 9) == 0
    st = L.qdec_gemm_q4(FAKE, FAKE, 64, FAKE, 128, 9, None, None, FAKE + (1 << 20), 10, 10, 128, None, 0, None)
    assert st == q.QDEC_EINVAL and "nb" in _err(L)
    st = L.qdec_gemm_q4(FAKE, FAKE, 64, FAKE, 126, 2, None, None, FAKE + (1 << 20), 10, 10, 126, None, 0, None)
    assert st == q.QDEC_EINVAL
    st = L.qdec_gemm_q8(FAKE, FAKE, FAKE, 128, 2, None, None, FAKE + 256, 10, 10, 128, None, 0, None)
    assert st == q.QDEC_EINVAL and "overlap" in _err(L)


def test_pack_rejects_bad_arguments(L):
    assert L.qdec_pack_q8(None, FAKE, 4, 16, FAKE, FAKE, None) == q.QDEC_EINVAL
    assert L.qdec_pack_q8(FAKE, FAKE, 4, 24, FAKE, FAKE, None) == q.QDEC_EINVAL
    assert L.qdec_pack_q4(FAKE, FAKE, 4, 96, 96, FAKE, FAKE, None) == q.QDEC_EUNSUPPORTED
    assert L.qdec_pack_q4(FAKE, FAKE, 4, 96, 64, FAKE, FAKE, None) == q.QDEC_EINVAL


def test_small_ops_reject_bad_arguments(L):
    assert L.qdec_rmsnorm_rope(FAKE, None, FAKE, 4, 130 * 2, 1e-6, 0.0, None, None) == q.QDEC_EINVAL
    assert L.qdec_rmsnorm_rope(FAKE, None, FAKE, 4, 7, 1e-6, 0.0, None, None) == q.QDEC_EINVAL
    st = L.qdec_rmsnorm_rope(FAKE, None, FAKE, 4, 64, 1e-6, 10000.0, None, None)
    assert st == q.QDEC_EINVAL and "pos" in _err(L)
    assert L.qdec_swiglu(FAKE, None, FAKE, 8, None) == q.QDEC_EINVAL
    assert L.qdec_swiglu(FAKE, FAKE, FAKE, 0, None) == q.QDEC_EINVAL
    assert L.qdec_argmax(FAKE, 0, FAKE, None) == q.QDEC_EINVAL


def _attn(L, **kw):
    a = dict(q=FAKE, k_new=None, v_new=None, k_pool=FAKE, v_pool=FAKE, kv_fmt=q.KV_BF16, page_table=FAKE,
             n_pages=4, page_size=16, pos=FAKE, n_heads=28, n_kv_heads=4, head_dim=128, sm_scale=0.088,
             num_splits=8, workspace=FAKE, workspace_bytes=1 << 20, out=FAKE, stream=None)
    a.update(kw)
    return L.qdec_attn_decode_paged(*a.values())


def test_attention_rejects_bad_arguments(L):
    assert _attn(L, kv_fmt=3) == q.QDEC_EUNSUPPORTED
    assert _attn(L, page_size=8) == q.QDEC_EUNSUPPORTED
    assert _attn(L, n_heads=30) == q.QDEC_EINVAL            # 30 % 4 != 0
    assert _attn(L, n_heads=36) == q.QDEC_EUNSUPPORTED      # 9 q heads per kv head
    assert _attn(L, head_dim=96) == q.QDEC_EUNSUPPORTED
    assert _attn(L, num_splits=0) == q.QDEC_EINVAL
    assert _attn(L, num_splits=257) == q.QDEC_EINVAL
    assert _attn(L, k_new=FAKE) == q.QDEC_EINVAL            # k_new without v_new
    assert _attn(L, workspace_bytes=100) == q.QDEC_EINVAL
    assert _attn(L, sm_scale=float("nan")) == q.QDEC_EINVAL
    assert _attn(L, out=None) == q.QDEC_EINVAL


def test_kv_pools_over_4gib_are_refused(L):
    """A layer's K or V pool is addressed with 32-bit byte offsets: pools of 4 GiB or more are
    refused by every entry point that takes one, instead of reading zeros or wrong rows."""
    # 8 KV heads x 16 x 128 x 2 B = 32 KiB per bf16 page: 131072 pages is exactly 4 GiB
    # (the accepted size still stops at the too-small workspace, so nothing is launched)
    st = _attn(L, n_heads=32, n_kv_heads=8, n_pages=131071, workspace_bytes=100)
    assert st == q.QDEC_EINVAL and "workspace" in _err(L)
    st = _attn(L, n_heads=32, n_kv_heads=8, n_pages=131072, workspace_bytes=100)
    assert st == q.QDEC_EUNSUPPORTED and "4 GiB" in _err(L)
    # fp32 pages are twice as large
    assert _attn(L, n_heads=32, n_kv_heads=8, kv_fmt=q.KV_F32, n_pages=65536, workspace_bytes=100) == q.QDEC_EUNSUPPORTED
    big = dict(n_heads=32, n_kv_heads=8, num_splits=8)
    assert L.qdec_step_workspace_bytes(ctypes.byref(_cfg(n_pages=131071, **big))) > 0
    assert L.qdec_step_workspace_bytes(ctypes.byref(_cfg(n_pages=131072, **big))) == 0
    assert L.qdec_batch_workspace_bytes(ctypes.byref(_cfg(n_pages=131071, **big)), 8) > 0
    assert L.qdec_batch_workspace_bytes(ctypes.byref(_cfg(n_pages=131072, **big)), 8) == 0


def _cfg(**kw):
    c = q.QdecConfig()
    base = dict(n_layers=28, hidden=3584, n_heads=28, n_kv_heads=4, head_dim=128, inter=18944,
                vocab=152064, wfmt=q.W_Q4, group=64, kv_fmt=q.KV_BF16, page_size=16, n_pages=260,
                has_qkv_bias=1, has_qk_norm=0, num_splits=64, rms_eps=1e-6, rope_base=1e6)
    base.update(kw)
    for k, v in base.items():
        setattr(c, k, v)
    return c


def test_step_config_validation(L):
    ok = L.qdec_step_workspace_bytes(ctypes.byref(_cfg()))
    assert ok > 0
    for bad in (dict(wfmt=5), dict(kv_fmt=0), dict(page_size=32), dict(head_dim=80), dict(group=48),
                dict(n_heads=27), dict(inter=18940), dict(num_splits=0), dict(num_splits=300),
                dict(rope_base=0.0)):
        assert L.qdec_step_workspace_bytes(ctypes.byref(_cfg(**bad))) == 0, bad
    h = ctypes.c_void_p()
    m = q.QdecModel()
    s = q.QdecState()
    assert L.qdec_step_create(ctypes.byref(_cfg()), ctypes.byref(m), ctypes.byref(s),
                              ctypes.byref(h)) == q.QDEC_EINVAL
    assert L.qdec_decode_step(None, 0, None) == q.QDEC_EINVAL
    assert L.qdec_step_kernel_count(None) == 0
    L.qdec_step_destroy(None)
