"""The C-ABI library loads on the CPU, exports every entry point of include/csa.h,
sizes workspaces, and rejects bad arguments on the host before any launch.

No compute call is made here (there is no GPU): every call below fails its host
checks, which run before anything touches device memory.
"""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

csa = pytest.importorskip("context_sparse_attention_amd")
from context_sparse_attention_amd import _binding as B  # noqa: E402


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"moba_gate_topk", "dsa_indexer_topk", "sparse_attn_fwd_shard", "summary_merge",
            "mla_v_up_proj", "csa_last_error"} <= set(names)
    for name in names:
        assert hasattr(B.lib, name), f"{name} missing from libcsa.so"


class FakeLayout:
    """A layout whose device pointers are never dereferenced by the host checks."""

    def __init__(self, cu, n_q):
        self.cu_host = np.asarray(cu, np.int32)
        fake = 1 << 20
        self._c = B.LayoutC(n_q, int(self.cu_host[-1]), fake, fake, len(cu) - 1, fake,
                            self.cu_host.ctypes.data_as(ctypes.c_void_p).value)

    @property
    def c(self):
        return ctypes.byref(self._c)


def t3(n, h, d, dtype=B.CSA_BF16, sn=None, sh=None, data=1 << 20):
    return B.Tensor3(data, dtype, n, h, d, sn if sn is not None else h * d,
                     sh if sh is not None else d)


def call_gate(q, k, L, block=64, topk=3, ws_bytes=1 << 30, ws=1 << 24):
    st = B.lib.moba_gate_topk(ctypes.byref(q), ctypes.byref(k), L.c, block, topk, 1 << 20,
                              None, ws, ws_bytes, None)
    return st, B.lib.csa_last_error().decode()


def test_workspace_sizes_are_positive_and_monotone():
    L1 = FakeLayout([0, 4096], 1024)
    L2 = FakeLayout([0, 8192], 1024)
    a = B.lib.moba_gate_topk_workspace_size(L1.c, 8, 128, 512)
    b = B.lib.moba_gate_topk_workspace_size(L2.c, 8, 128, 512)
    assert 0 < a < b and a % 256 == 0
    assert B.lib.dsa_indexer_topk_workspace_size(L2.c, 2048) >= 1024 * 8192 * 4
    assert B.lib.sparse_attn_fwd_shard_workspace_size(L2.c, 0, 32, 8, 128, 5, 512) > 0
    assert B.lib.moba_gate_topk_workspace_size(None, 8, 128, 512) == 0


def test_gate_rejects_bad_arguments():
    L = FakeLayout([0, 100, 256], 64)
    q, k = t3(64, 4, 64), t3(256, 2, 64)
    st, msg = call_gate(q, t3(256, 3, 64), L)
    assert st == 1 and "multiple" in msg
    st, msg = call_gate(q, t3(200, 2, 64), L)
    assert st == 1 and "n_kv" in msg
    st, msg = call_gate(t3(64, 4, 64, dtype=B.CSA_F32), k, L)
    assert st == 1 and "dtype" in msg
    st, msg = call_gate(q, k, L, topk=40)
    assert st == 2
    st, msg = call_gate(q, k, L, block=0)
    assert st == 1
    st, msg = call_gate(q, k, L, ws_bytes=16)
    assert st == 3 and "workspace" in msg
    st, msg = call_gate(q, k, L, ws=(1 << 24) + 8)
    assert st == 3
    st, msg = call_gate(t3(64, 4, 60), t3(256, 2, 60), L)
    assert st == 2
    st, msg = call_gate(t3(64, 4, 64, data=(1 << 20) + 2), k, L)
    assert st == 1 and "aligned" in msg
    bad_cu = FakeLayout([0, 300, 256], 64)
    st, msg = call_gate(q, k, bad_cu)
    assert st == 1 and "cu_seqlens" in msg


def test_attention_rejects_bad_arguments():
    L = FakeLayout([0, 512], 128)
    q, k, v = t3(128, 4, 64), t3(512, 2, 64), t3(512, 2, 64)

    def call(mode=0, idx_heads=1, width=4, block=64, scale=0.125, out_dtype=1, vv=None):
        st = B.lib.sparse_attn_fwd_shard(ctypes.byref(q), ctypes.byref(k), ctypes.byref(vv or v),
                                         L.c, mode, 1 << 20, idx_heads, width, block, scale,
                                         1 << 20, out_dtype, None, 1 << 24, 1 << 30, None)
        return st, B.lib.csa_last_error().decode()

    assert call(mode=5)[0] == 1
    assert call(idx_heads=3)[0] == 1
    assert call(width=0)[0] == 1
    assert call(block=0)[0] == 1
    assert call(scale=float("nan"))[0] == 1
    assert call(out_dtype=7)[0] == 1
    assert call(vv=t3(512, 1, 64))[0] == 1
    assert call(vv=t3(512, 2, 1024))[0] == 2


def test_merge_rejects_bad_arguments():
    st = B.lib.summary_merge(2, 4, 8, 1 << 20, 1 << 20, 1 << 20, None, None, None, None, 0,
                             None, None)
    assert st == 1 and "no output" in B.lib.csa_last_error().decode()
    st = B.lib.summary_merge(2, 4, 8, 1 << 20, 1 << 20, 1 << 20, 1 << 20, None, None, None,
                             0, None, None)
    assert st == 1 and "together" in B.lib.csa_last_error().decode()


def test_indexer_rejects_bad_arguments():
    L = FakeLayout([0, 1024], 16)
    iq, ik = t3(16, 64, 128), t3(1024, 1, 128)

    def call(iq_=iq, ik_=ik, topk=8, w_stride=64):
        st = B.lib.dsa_indexer_topk(ctypes.byref(iq_), ctypes.byref(ik_), 1 << 20, w_stride,
                                    L.c, topk, 1 << 20, None, 1 << 24, 1 << 30, None)
        return st, B.lib.csa_last_error().decode()

    assert call(topk=0)[0] == 1
    assert call(ik_=t3(1024, 2, 128))[0] == 1
    assert call(iq_=t3(16, 64, 256), ik_=t3(1024, 1, 256))[0] == 2
    assert call(w_stride=10)[0] == 1


def test_up_projection_rejects_bad_arguments():
    def call(o=None, w=None, out=1 << 20, out_dtype=1):
        o = o or t3(64, 8, 512)
        w = w or t3(8, 128, 512)
        st = B.lib.mla_v_up_proj(ctypes.byref(o), ctypes.byref(w), out, out_dtype, None)
        return st, B.lib.csa_last_error().decode()

    assert call(w=t3(4, 128, 512))[0] == 1           # head counts differ
    assert call(w=t3(8, 128, 256))[0] == 1           # latent widths differ
    assert call(w=t3(8, 48, 512))[0] == 2            # output width not a multiple of 32
    assert call(o=t3(64, 8, 544), w=t3(8, 128, 544))[0] == 2  # latent width not a multiple of 64
    assert call(out_dtype=7)[0] == 1
    assert call(out=None)[0] == 1
    assert call(out=(1 << 20) + 8)[0] == 1           # misaligned output


def test_noalloc_gate_rejects_shapes_beyond_its_scratch_on_the_host():
    # 8192 one-token blocks x 8 heads x 128 dims of block means: beyond the fixed
    # scratch, so the call returns before touching the device
    L = FakeLayout([0, 8192], 64)
    q, k = t3(64, 8, 128), t3(8192, 8, 128)
    assert B.lib.moba_gate_topk_workspace_size(L.c, 8, 128, 1) > B.GATE_SCRATCH_BYTES
    st = B.lib.moba_gate_topk_noalloc(ctypes.byref(q), ctypes.byref(k), L.c, 1, 2, 1 << 20,
                                      None, None)
    assert st == 2 and "scratch" in B.lib.csa_last_error().decode()
    # ordinary argument errors are the workspace call's
    st = B.lib.moba_gate_topk_noalloc(ctypes.byref(q), ctypes.byref(t3(8192, 3, 128)), L.c,
                                      64, 2, 1 << 20, None, None)
    assert st == 1


def kernel_of(q, k, v, L, mode, idx_heads, width, block=0, scale=0.1, out=B.CSA_BF16):
    name = B.lib.sparse_attn_fwd_shard_kernel(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                              L.c, mode, idx_heads, width, block, scale, out)
    return None if name is None else name.decode()


def test_kernel_family_query_names_the_path_each_shape_takes():
    # the DSA shard: 128 heads over one 576-wide latent key, value = its first 512 columns
    L = FakeLayout([0, 16384], 4096)
    k = t3(16384, 1, 576)
    v = t3(16384, 1, 512, sn=576, sh=576)
    assert kernel_of(t3(4096, 128, 576), k, v, L, B.CSA_SEL_TOKEN, 1, 2048) == "token_mfma"
    # per-head index rows in token mode: the general kernel
    assert kernel_of(t3(4096, 128, 576), k, v, L, B.CSA_SEL_TOKEN, 128, 16) == "generic"
    # the 32K GQA MoBA shard
    L = FakeLayout([0, 32768], 8192)
    kv = t3(32768, 8, 128)
    assert kernel_of(t3(8192, 32, 128), kv, kv, L, B.CSA_SEL_BLOCK, 32, 5, 1024) == "block_mfma"
    # blocks not a multiple of 64, fp32 inputs, or a non-positive scale: the general kernel
    assert kernel_of(t3(8192, 32, 128), kv, kv, L, B.CSA_SEL_BLOCK, 32, 5, 48) == "generic"
    f32 = t3(32768, 8, 128, dtype=B.CSA_F32)
    assert kernel_of(t3(8192, 32, 128, dtype=B.CSA_F32), f32, f32, L, B.CSA_SEL_BLOCK, 32, 5,
                     1024) == "generic"
    assert kernel_of(t3(8192, 32, 128), kv, kv, L, B.CSA_SEL_BLOCK, 32, 5, 1024,
                     scale=-0.1) == "generic"
    # rejected arguments: NULL and an error text
    assert kernel_of(t3(8192, 32, 128), kv, kv, L, 7, 32, 5, 1024) is None
    assert "mode" in B.lib.csa_last_error().decode()
