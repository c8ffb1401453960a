"""ctypes marshalling for libcsa.so (see include/csa.h for the contract)."""

import ctypes
import math
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libcsa.so")

if not os.path.exists(library_path):
    raise ImportError(
        f"{library_path} is not built; run `python context_sparse_attention_amd/build.py` "
        "(or __graft_entry__.build()) first. There is no fallback path.")

lib = ctypes.CDLL(library_path)

CSA_OK = 0
CSA_F32, CSA_BF16 = 0, 1
CSA_SEL_BLOCK, CSA_SEL_TOKEN = 0, 1


class CsaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"csa status {status}: {message}")
        self.status = status


class Tensor3(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("n", ctypes.c_int64),
                ("h", ctypes.c_int32), ("d", ctypes.c_int32), ("stride_n", ctypes.c_int64),
                ("stride_h", ctypes.c_int64)]


class LayoutC(ctypes.Structure):
    _fields_ = [("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32),
                ("q_pos", ctypes.c_void_p), ("q_seq", ctypes.c_void_p),
                ("n_seq", ctypes.c_int32), ("cu_seqlens", ctypes.c_void_p),
                ("cu_seqlens_host", ctypes.c_void_p)]


_P = ctypes.c_void_p
_T3 = ctypes.POINTER(Tensor3)
_LP = ctypes.POINTER(LayoutC)
_sz = ctypes.c_size_t
_i32, _i64, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float

lib.csa_last_error.restype = ctypes.c_char_p
lib.csa_last_error.argtypes = []
lib.moba_gate_topk_workspace_size.restype = _sz
lib.moba_gate_topk_workspace_size.argtypes = [_LP, _i32, _i32, _i32]
lib.moba_gate_topk.restype = ctypes.c_int
lib.moba_gate_topk.argtypes = [_T3, _T3, _LP, _i32, _i32, _P, _P, _P, _sz, _P]
lib.moba_gate_topk_noalloc.restype = ctypes.c_int
lib.moba_gate_topk_noalloc.argtypes = [_T3, _T3, _LP, _i32, _i32, _P, _P, _P]
lib.dsa_indexer_topk_workspace_size.restype = _sz
lib.dsa_indexer_topk_workspace_size.argtypes = [_LP, _i32]
lib.dsa_indexer_topk.restype = ctypes.c_int
lib.dsa_indexer_topk.argtypes = [_T3, _T3, _P, _i64, _LP, _i32, _P, _P, _P, _sz, _P]
lib.sparse_attn_fwd_shard_workspace_size.restype = _sz
lib.sparse_attn_fwd_shard_workspace_size.argtypes = [_LP, _i32, _i32, _i32, _i32, _i32, _i32]
lib.sparse_attn_fwd_shard.restype = ctypes.c_int
lib.sparse_attn_fwd_shard.argtypes = [_T3, _T3, _T3, _LP, _i32, _P, _i32, _i32, _i32, _f32,
                                      _P, _i32, _P, _P, _sz, _P]
lib.sparse_attn_bwd_shard_workspace_size.restype = _sz
lib.sparse_attn_bwd_shard_workspace_size.argtypes = [_LP, _i32, _i32, _i32, _i32, _i32, _i32,
                                                     _i32, _i32, _i32]
lib.sparse_attn_bwd_shard_kernel.restype = ctypes.c_char_p
lib.sparse_attn_bwd_shard_kernel.argtypes = [_LP, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                             _i32, _i32]
lib.sparse_attn_bwd_shard.restype = ctypes.c_int
lib.sparse_attn_bwd_shard.argtypes = [_T3, _T3, _T3, _LP, _i32, _P, _i32, _i32, _i32, _f32,
                                      _T3, _T3, _P, _P, _P, _P, _P, _sz, _P]
lib.sparse_attn_fwd_shard_kernel.restype = ctypes.c_char_p
lib.sparse_attn_fwd_shard_kernel.argtypes = [_T3, _T3, _T3, _LP, _i32, _i32, _i32, _i32, _f32,
                                             _i32]
lib.csa_trace_begin.restype = ctypes.c_int
lib.csa_trace_begin.argtypes = [ctypes.c_int]
lib.csa_trace_collect.restype = ctypes.c_int
lib.csa_trace_collect.argtypes = [ctypes.POINTER(ctypes.c_float),
                                  ctypes.POINTER(ctypes.c_char_p), ctypes.c_int]
lib.summary_merge.restype = ctypes.c_int
lib.summary_merge.argtypes = [_i32, _i64, _i32, _P, _P, _P, _P, _P, _P, _P, _i32, _P, _P]
lib.mla_v_up_proj.restype = ctypes.c_int
lib.mla_v_up_proj.argtypes = [_T3, _T3, _P, _i32, _P]


def _check(status):
    if status != CSA_OK:
        raise CsaError(status, lib.csa_last_error().decode())


def _dtype_code(t):
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _tensor3(t):
    """[n, h, d] (or [n, d] as [n, 1, d]) torch tensor -> Tensor3 (strides in elements)."""
    if t.dim() == 2:
        n, d = t.shape
        return Tensor3(t.data_ptr(), _dtype_code(t), n, 1, d, t.stride(0), d)
    if t.dim() != 3:
        raise ValueError("expected a 2-D or 3-D tensor")
    if t.stride(2) != 1:
        raise ValueError("last dimension must be contiguous")
    n, h, d = t.shape
    return Tensor3(t.data_ptr(), _dtype_code(t), n, h, d, t.stride(0), t.stride(1))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


class Layout:
    """Shard layout: global position and sequence id of each local row, packed-sequence starts."""

    def __init__(self, q_pos, q_seq, cu_seqlens, device="cuda"):
        self.cu_host = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        self.q_pos = torch.as_tensor(np.asarray(q_pos, np.int32), device=device)
        self.q_seq = torch.as_tensor(np.asarray(q_seq, np.int32), device=device)
        self.cu = torch.as_tensor(self.cu_host, device=device)
        self.n_q = int(self.q_pos.numel())
        self.n_kv = int(self.cu_host[-1])
        self.n_seq = len(self.cu_host) - 1
        self._c = LayoutC(self.n_q, self.n_kv, self.q_pos.data_ptr(), self.q_seq.data_ptr(),
                          self.n_seq, self.cu.data_ptr(),
                          self.cu_host.ctypes.data_as(ctypes.c_void_p).value)

    @property
    def c(self):
        return ctypes.byref(self._c)


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _given(t, shape, dtype, dev, name):
    """A caller-supplied output tensor, checked for shape, dtype, device and contiguity."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != dev or \
            not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {dtype} tensor of shape "
                         f"{tuple(shape)} on {dev}")
    return t


def _out(t, shape, dtype, dev, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    return _given(t, shape, dtype, dev, name)


def moba_gate_topk(q, k, layout, block_size, topk, return_score=False, idx=None,
                   score=None):
    """idx [n_q, Hq, topk+1] int32 (block start positions), optionally the gate scores.

    ``idx`` / ``score`` may be given as preallocated outputs (every element is written).
    """
    dev = q.device
    shape = (layout.n_q, q.shape[1], topk + 1)
    idx = _out(idx, shape, torch.int32, dev, "idx")
    if return_score or score is not None:
        score = _out(score, shape, torch.float32, dev, "score")
    ws_bytes = lib.moba_gate_topk_workspace_size(layout.c, k.shape[1], k.shape[2], block_size)
    ws = _workspace(ws_bytes, dev)
    _check(lib.moba_gate_topk(ctypes.byref(_tensor3(q)), ctypes.byref(_tensor3(k)), layout.c,
                              block_size, topk, idx.data_ptr(), _ptr(score), ws.data_ptr(),
                              ws.numel(), _stream()))
    return (idx, score) if (return_score or score is not None) else idx


def moba_gate_topk_noalloc(q, k, layout, block_size, topk, idx, score=None):
    """moba_gate_topk into caller-given outputs, with the library's fixed scratch
    instead of a workspace (nothing is allocated); returns idx (and score)."""
    dev = q.device
    shape = (layout.n_q, q.shape[1], topk + 1)
    _given(idx, shape, torch.int32, dev, "idx")
    if score is not None:
        _given(score, shape, torch.float32, dev, "score")
    _check(lib.moba_gate_topk_noalloc(ctypes.byref(_tensor3(q)), ctypes.byref(_tensor3(k)),
                                      layout.c, block_size, topk, idx.data_ptr(), _ptr(score),
                                      _stream()))
    return idx if score is None else (idx, score)


GATE_SCRATCH_BYTES = 16 * 1024 * 1024  # CSA_GATE_SCRATCH_BYTES of include/csa.h


def dsa_indexer_topk(iq, ik, w, layout, topk, return_score=False, idx=None, score=None):
    """idx [n_q, topk] int32 (key positions), optionally the selected logits.

    ``idx`` / ``score`` may be given as preallocated outputs (every element is written).
    """
    dev = iq.device
    if w.dtype != torch.float32 or w.stride(1) != 1:
        raise ValueError("w must be float32 with a contiguous head dimension")
    shape = (layout.n_q, topk)
    idx = _out(idx, shape, torch.int32, dev, "idx")
    if return_score or score is not None:
        score = _out(score, shape, torch.float32, dev, "score")
    ws_bytes = lib.dsa_indexer_topk_workspace_size(layout.c, topk)
    ws = _workspace(ws_bytes, dev)
    _check(lib.dsa_indexer_topk(ctypes.byref(_tensor3(iq)), ctypes.byref(_tensor3(ik)),
                                w.data_ptr(), w.stride(0), layout.c, topk, idx.data_ptr(),
                                _ptr(score), ws.data_ptr(), ws.numel(), _stream()))
    return (idx, score) if (return_score or score is not None) else idx


def sparse_attn_fwd_shard(q, k, v, layout, mode, idx, block_size=0, softmax_scale=None,
                          out_dtype=None, return_lse=True, out=None, lse=None):
    """out [n_q, Hq, Dv] (and lse [n_q, Hq]) of the shard's rows over their selected chunks.

    ``idx`` is [n_q, idx_heads, W] (or [n_q, W] for idx_heads = 1), int32, contiguous.
    ``out`` / ``lse`` may be given as preallocated outputs (every element is written).
    """
    dev = q.device
    if idx.dim() == 2:
        idx = idx.unsqueeze(1)
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 tensor")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(q.shape[2])
    hq, dv = q.shape[1], v.shape[2]
    if out is not None:
        out_dtype = out.dtype
    out_dtype = out_dtype or q.dtype
    out = _out(out, (layout.n_q, hq, dv), out_dtype, dev, "out")
    if return_lse or lse is not None:
        lse = _out(lse, (layout.n_q, hq), torch.float32, dev, "lse")
    ws_bytes = lib.sparse_attn_fwd_shard_workspace_size(layout.c, mode, hq, k.shape[1], dv,
                                                        idx.shape[2], block_size)
    ws = _workspace(ws_bytes, dev)
    _check(lib.sparse_attn_fwd_shard(ctypes.byref(_tensor3(q)), ctypes.byref(_tensor3(k)),
                                     ctypes.byref(_tensor3(v)), layout.c, mode, idx.data_ptr(),
                                     idx.shape[1], idx.shape[2], block_size,
                                     float(softmax_scale), out.data_ptr(), _dtype_code(out),
                                     _ptr(lse), ws.data_ptr(), ws.numel(), _stream()))
    return (out, lse) if (return_lse or lse is not None) else out


def sparse_attn_fwd_shard_kernel(q, k, v, layout, mode, idx_heads, idx_width, block_size=0,
                                 softmax_scale=None, out_dtype=None):
    """The kernel family sparse_attn_fwd_shard runs for these arguments:
    "block_mfma", "token_mfma" or "generic"."""
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(q.shape[2])
    out_dtype = out_dtype or q.dtype
    name = lib.sparse_attn_fwd_shard_kernel(
        ctypes.byref(_tensor3(q)), ctypes.byref(_tensor3(k)), ctypes.byref(_tensor3(v)),
        layout.c, mode, idx_heads, idx_width, block_size, float(softmax_scale),
        CSA_BF16 if out_dtype == torch.bfloat16 else CSA_F32)
    if name is None:
        raise CsaError(1, lib.csa_last_error().decode())
    return name.decode()


def sparse_attn_bwd_shard_workspace_size(q, k, v, layout, mode, idx_heads, idx_width,
                                         block_size=0):
    """Workspace bytes of sparse_attn_bwd_shard for these tensors' shapes and dtype."""
    return lib.sparse_attn_bwd_shard_workspace_size(
        layout.c, mode, _dtype_code(q), q.shape[1], k.shape[1], q.shape[2], v.shape[2],
        idx_heads, idx_width, block_size)


def sparse_attn_bwd_shard_kernel(q, k, v, layout, mode, idx_heads, idx_width, block_size=0):
    """The kernel family sparse_attn_bwd_shard runs: "block_mfma", "token_mfma" or
    "generic"."""
    name = lib.sparse_attn_bwd_shard_kernel(
        layout.c, mode, _dtype_code(q), q.shape[1], k.shape[1], q.shape[2], v.shape[2],
        idx_heads, idx_width, block_size)
    if name is None:
        raise CsaError(1, lib.csa_last_error().decode())
    return name.decode()


def sparse_attn_bwd_shard(q, k, v, layout, mode, idx, out, dout, lse, block_size=0,
                          softmax_scale=None, dq=None, dk=None, dv=None):
    """(dq, dk, dv) float32 of the forward's arguments, output, lse and dL/dout.

    ``idx`` as in sparse_attn_fwd_shard.  ``dq`` / ``dk`` / ``dv`` may be given as
    preallocated float32 outputs (every element is written).
    """
    dev = q.device
    if idx.dim() == 2:
        idx = idx.unsqueeze(1)
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 tensor")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(q.shape[2])
    hq, hkv = q.shape[1], k.shape[1]
    dq = _out(dq, (layout.n_q, hq, q.shape[2]), torch.float32, dev, "dq")
    dk = _out(dk, (layout.n_kv, hkv, k.shape[2]), torch.float32, dev, "dk")
    dv = _out(dv, (layout.n_kv, hkv, v.shape[2]), torch.float32, dev, "dv")
    ws_bytes = sparse_attn_bwd_shard_workspace_size(q, k, v, layout, mode, idx.shape[1],
                                                    idx.shape[2], block_size)
    ws = _workspace(ws_bytes, dev)
    _check(lib.sparse_attn_bwd_shard(ctypes.byref(_tensor3(q)), ctypes.byref(_tensor3(k)),
                                     ctypes.byref(_tensor3(v)), layout.c, mode, idx.data_ptr(),
                                     idx.shape[1], idx.shape[2], block_size,
                                     float(softmax_scale), ctypes.byref(_tensor3(out)),
                                     ctypes.byref(_tensor3(dout)), lse.data_ptr(),
                                     dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                                     ws.numel(), _stream()))
    return dq, dk, dv


def summary_merge(m, l, z, finalize=True, merged=False, o_dtype=torch.float32):
    """Merge [P, R] / [P, R, dv] fp32 summaries; returns the requested outputs as a dict."""
    for t in (m, l, z):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("summaries must be contiguous float32")
    n_parts, n_rows, dv = z.shape
    dev = z.device
    res = {}
    mo = lo = zo = o = lse = None
    if merged:
        mo = torch.empty(n_rows, dtype=torch.float32, device=dev)
        lo = torch.empty(n_rows, dtype=torch.float32, device=dev)
        zo = torch.empty((n_rows, dv), dtype=torch.float32, device=dev)
        res.update(m=mo, l=lo, z=zo)
    if finalize:
        o = torch.empty((n_rows, dv), dtype=o_dtype, device=dev)
        lse = torch.empty(n_rows, dtype=torch.float32, device=dev)
        res.update(o=o, lse=lse)
    _check(lib.summary_merge(n_parts, n_rows, dv, m.data_ptr(), l.data_ptr(), z.data_ptr(),
                             _ptr(mo), _ptr(lo), _ptr(zo), _ptr(o),
                             CSA_BF16 if o_dtype == torch.bfloat16 else CSA_F32, _ptr(lse),
                             _stream()))
    return res


def mla_v_up_proj(o, w, out_dtype=None):
    """out [n_q, Hq, Dv] = per head o [n_q, Hq, Dl] @ w[h]^T, w [Hq, Dv, Dl] (bf16)."""
    out_dtype = out_dtype or o.dtype
    out = torch.empty((o.shape[0], o.shape[1], w.shape[1]), dtype=out_dtype, device=o.device)
    _check(lib.mla_v_up_proj(ctypes.byref(_tensor3(o)), ctypes.byref(_tensor3(w)),
                             out.data_ptr(), _dtype_code(out), _stream()))
    return out


def trace_begin(max_records):
    """Record HIP event pairs around each call's dominant kernel (see csa.h)."""
    _check(lib.csa_trace_begin(int(max_records)))


def trace_collect(max_records=4096):
    """[(kernel name, elapsed ms)] of the recorded launches, in order; rewinds the ring."""
    ms = (ctypes.c_float * max_records)()
    names = (ctypes.c_char_p * max_records)()
    n = lib.csa_trace_collect(ms, names, max_records)
    return [(names[i].decode(), float(ms[i])) for i in range(n)]
