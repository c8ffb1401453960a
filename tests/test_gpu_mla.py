"""GPU parity of mla_v_up_proj (absorbed-MLA value up-projection) against the
fp64 oracle (MI355X only).

Tolerance, from the arithmetic: the products of bf16 values are exact in fp32,
and an fp32 sum of Dl of them is within (Dl - 1) 2^-24 sum |o w| of the exact
sum; a bf16 output adds half an ulp, 2^-8 |x|.
"""

import numpy as np
import pytest
import torch

import oracle
from csa_inputs import up_projection_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import context_sparse_attention_amd as csa


def _say(*a):
    print("[case]", *a, flush=True)


def _bound(o, w, ref, out_dtype):
    dl = o.shape[2]
    mag = np.einsum("ihc,hdc->ihd", np.abs(o.astype(np.float64)), np.abs(w.astype(np.float64)))
    b = (dl - 1) * 2.0 ** -24 * mag + 1e-30
    if out_dtype == torch.bfloat16:
        b = b + 2.0 ** -8 * np.abs(ref)
    return b


def _check(o_np, w_np, out, out_dtype, rows=None):
    rows = np.arange(o_np.shape[0]) if rows is None else rows
    ref = oracle.v_up_proj(o_np[rows], w_np)
    got = out.float().cpu().numpy()[rows]
    err = np.abs(got - ref)
    bound = _bound(o_np[rows], w_np, ref, out_dtype)
    assert np.all(err <= bound), f"max excess {(err - bound).max():.3e}, max err {err.max():.3e}"
    assert err.max() <= 2e-2  # the bf16 output tolerance of the shard's outputs
    return err.max()


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n_q,hq,dl,dv", [(1, 2, 512, 128), (130, 8, 512, 128),
                                          (300, 3, 64, 64), (77, 5, 192, 96), (40, 16, 512, 32)])
def test_up_projection_small(n_q, hq, dl, dv, out_dtype):
    _say("up-proj", n_q, hq, dl, dv, out_dtype)
    o_np, w_np = up_projection_inputs(n_q, hq, dl, dv)
    o = torch.from_numpy(o_np).cuda().to(torch.bfloat16)
    w = torch.from_numpy(w_np).cuda().to(torch.bfloat16)
    out = csa.mla_v_up_proj(o, w, out_dtype=out_dtype)
    torch.cuda.synchronize()
    _check(o_np, w_np, out, out_dtype)


def test_up_projection_strided_latent_view():
    # the latent output read through a view whose rows are wider than Dl
    _say("up-proj strided view")
    n_q, hq, dl, dv = 96, 4, 512, 128
    o_np, w_np = up_projection_inputs(n_q, hq, dl, dv, seed=12)
    big = torch.zeros((n_q, hq, dl + 64), dtype=torch.bfloat16, device="cuda")
    big[:, :, :dl] = torch.from_numpy(o_np).cuda().to(torch.bfloat16)
    big[:, :, dl:] = float("nan")  # never read
    w = torch.from_numpy(w_np).cuda().to(torch.bfloat16)
    out = csa.mla_v_up_proj(big[:, :, :dl], w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(o_np, w_np, out, torch.float32)


def test_up_projection_empty():
    o = torch.zeros((0, 8, 512), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((8, 128, 512), dtype=torch.bfloat16, device="cuda")
    out = csa.mla_v_up_proj(o, w)
    torch.cuda.synchronize()
    assert out.shape == (0, 8, 128)


def test_up_projection_dsa_shape_sampled_rows():
    # the DSA workload's shard: 4096 rows x 128 heads, latent 512 -> 128 channels
    _say("up-proj DSA shape")
    n_q, hq, dl, dv = 4096, 128, 512, 128
    o_np, w_np = up_projection_inputs(n_q, hq, dl, dv, seed=13)
    o = torch.from_numpy(o_np).cuda().to(torch.bfloat16)
    w = torch.from_numpy(w_np).cuda().to(torch.bfloat16)
    out = csa.mla_v_up_proj(o, w)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(n_q, 96, replace=False))
    rows = np.concatenate([[0, 127, 128, n_q - 1], rows])
    _check(o_np, w_np, out, torch.bfloat16, rows)


def test_absorbed_path_end_to_end():
    # indexer -> latent attention (value = the first dv key columns) -> up-projection,
    # against the oracle attending, on the GPU's own selection, over each head's
    # up-projected values (the softmax weights do not depend on the values)
    from csa_inputs import tiny_token_workload
    _say("absorbed path end to end")
    t = tiny_token_workload(seed=31, lengths=(320,), hq=16, dqk=128, dv=64, hi=4, di=32,
                            topk=40, dtype="bf16")
    lay = csa.Layout(t.q_pos, t.q_seq, t.cu_seqlens)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)

    q, k = dev(t.q), dev(t.k)
    iq, ik = dev(t.iq), dev(t.ik)
    idx = csa.dsa_indexer_topk(iq, ik, torch.from_numpy(t.w).cuda(), lay, t.topk)
    o_lat, _ = csa.sparse_attn_fwd_shard(q, k, k[..., : t.dv], lay, csa.CSA_SEL_TOKEN, idx,
                                         softmax_scale=t.scale, out_dtype=torch.float32)
    _, w_np = up_projection_inputs(1, t.hq, t.dv, 32, seed=32)
    up = csa.mla_v_up_proj(o_lat.to(torch.bfloat16), dev(w_np), out_dtype=torch.float32)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    k_rep = np.repeat(t.k, t.hq, axis=1)
    v_proj = np.einsum("jc,hdc->jhd", t.value[:, 0, :].astype(np.float64), w_np)
    ref, _ = oracle.shard_forward(t.q, k_rep, v_proj, t.q_pos, t.q_seq, t.cu_seqlens, "token",
                                  idx_np[:, None, :], t.scale)
    err = np.abs(up.cpu().numpy() - ref).max()
    assert err <= 2e-2, f"max abs error {err:.3e}"
