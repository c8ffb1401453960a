"""Benchmark: one step = selection + sparse attention of one context-parallel shard.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step runs the whole hot path once over one synthetic batch already resident
in HBM: ``moba_gate_topk`` then ``sparse_attn_fwd_shard`` (block mode) for the
MoBA workloads, ``dsa_indexer_topk`` then ``sparse_attn_fwd_shard`` (token
mode) for the DSA workload.  The default workload is the 8K-token MoBA shard
(16 heads, D=128, last 2048 queries, blocks of 512, top-3 + own block).

Printed: one JSON line.  ``value`` is effective TFLOP/s of the whole step
(selected permitted query-key pairs x 2 x (Dqk + Dv) per second), timed over
replays of the step captured as a HIP graph (the same library calls; every
checked replay reproduces the eager output bit for bit); ``--no-graph`` times
the eager calls instead, whose step time is also reported.  Extra fields:
per-stage times (warm and with caches flushed), the roofline of the attention
kernel, and the fp64 CPU oracle timed on a bounded sample of rows.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective sparse-attn TFLOP/s per shard (+ gate/top-k HBM GB/s), % of roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    # the GPU's clocks rise over tens of milliseconds of load: 500 warm-up steps
    # (~50 ms of the 8K step) measured 2.6% faster than 3 at the same timed steps
    p.add_argument("--warmup", type=int, default=500)
    p.add_argument("--workload", default="moba_mha_8k")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-cold", action="store_true")
    p.add_argument("--no-graph", action="store_true",
                   help="time the eager calls instead of a captured HIP graph of the step")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain device-to-device copy of known size (the reference "
                        "for scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return p.parse_args()


# Source files of each attention kernel; the HBM traffic of a kernel, taken
# from counter runs, is reported only while these files are unchanged.
KERNEL_SOURCES = {
    "k_bm_attn": ["attn_block_mfma.hip"],
    "k_tok_attn": ["attn_token_mfma.hip", "mfma.hpp"],
    "k_attn_generic": ["attn_generic.hip"],
}
COMMON_SOURCES = ["common.hpp", "attention.hpp"]
COPY_BYTES = 1 << 30


def source_sha(kernel):
    """sha256 (16 hex digits) of the kernel's source files and the shared headers."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "context_sparse_attention_amd", "csrc")
    for f in KERNEL_SOURCES.get(kernel, []) + COMMON_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from profiles/traffic.json, or None.

    The file holds FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of each kernel
    and workload, and what the same counters read for a plain copy of
    COPY_BYTES; a kernel's bytes are its counters divided by the copy's
    counter-per-byte.  An entry counts only if its source hash matches.
    """
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    cal = t["calibration"]
    for e in t["kernels"]:
        if e["kernel"] == kernel and e["workload"] == workload and \
                e["source_sha"] == source_sha(kernel):
            return e["fetch_kib"] * 1024 / cal["fetch_per_byte"] + \
                e["write_kib"] * 1024 / cal["write_per_byte"]
    return None


def copy_calibration():
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 3}), flush=True)


def permitted_bounds(w):
    cu = w.cu_seqlens.astype(np.int64)
    seq = w.q_seq.astype(np.int64)
    pos = w.q_pos.astype(np.int64)
    ok = (seq >= 0) & (seq < len(cu) - 1)
    s = np.clip(seq, 0, len(cu) - 2)
    lo, end = cu[s], cu[s + 1]
    ok &= (pos >= lo) & (pos < end)
    return lo, pos, end, ok


def effective_pairs(w, idx, split=False):
    """Selected permitted (query head, key) pairs of the step.

    With split=True (block mode) also returns the pairs of full blocks lying
    strictly before the row's position, the work of the query-tile kernel.
    """
    lo, pos, end, ok = permitted_bounds(w)
    idx = idx.astype(np.int64)
    if idx.ndim == 2:
        idx = idx[:, None, :]
    lo_, pos_, end_ = lo[:, None, None], pos[:, None, None], end[:, None, None]
    valid = ok[:, None, None] & (idx >= lo_) & (idx <= pos_)
    full = 0
    if w.mode == "block":
        valid &= ((idx - lo_) % w.block_size) == 0
        n = np.minimum(np.minimum(idx + w.block_size, end_), pos_ + 1) - idx
        pairs = np.where(valid, n, 0).sum()
        full = np.where(valid & (idx + w.block_size - 1 < pos_), n, 0).sum()
    else:
        pairs = valid.sum()
    if idx.shape[1] == 1:
        pairs *= w.hq
        full *= w.hq
    return (int(pairs), int(full)) if split else int(pairs)


def selection_bytes(w):
    """Algorithmic HBM bytes of the selection stage (read once, written once)."""
    lo, pos, end, ok = permitted_bounds(w)
    if w.mode == "block":
        B = w.block_size
        # blocks ending at or before the latest own-block start of each sequence
        need = {}
        for i in np.nonzero(ok)[0]:
            s = int(w.q_seq[i])
            own_start = lo[i] + ((pos[i] - lo[i]) // B) * B
            need[s] = max(need.get(s, 0), int(own_start - lo[i]))
        key_tokens = sum(need.values())
        esz = 2 if w.dtype == "bf16" else 4
        kbytes = key_tokens * w.hkv * w.dqk * esz
        qbytes = w.n_q * w.hq * w.dqk * esz
        ibytes = w.n_q * w.hq * (w.topk + 1) * 4
        return {"total": kbytes + qbytes + ibytes, "keys": kbytes, "queries": qbytes,
                "indices": ibytes}
    n = np.where(ok, pos - lo + 1, 0)
    logits = int(n.sum()) * 4
    ibytes = w.n_q * w.topk * 4
    return {"total": logits + ibytes, "logits": logits, "indices": ibytes,
            "indexer_flops": int(n.sum()) * w.iq.shape[1] * w.iq.shape[2] * 2}


def cpu_baseline(w, seconds):
    """fp64 oracle on a bounded random sample of rows, one BLAS thread."""
    from threadpoolctl import threadpool_limits
    import oracle

    rng = np.random.default_rng(0)
    order = rng.permutation(w.n_q)
    done_pairs, rows_done, t_sel, t_att = 0, 0, 0.0, 0.0
    with threadpool_limits(limits=1):
        t_start = time.perf_counter()
        for start in range(0, w.n_q, 8):
            rows = np.sort(order[start:start + 8])
            t0 = time.perf_counter()
            if w.mode == "block":
                gate = oracle.gate_scores(w.q[rows], w.k, w.q_pos[rows], w.q_seq[rows],
                                          w.cu_seqlens, w.block_size)
                idx = oracle.select_blocks(gate, w.topk)
            else:
                idx, _, _ = oracle.indexer_topk(w.iq[rows], w.ik, w.w[rows], w.q_pos[rows],
                                                w.q_seq[rows], w.cu_seqlens, w.topk)
                idx = idx[:, None, :]
            t1 = time.perf_counter()
            oracle.shard_forward(w.q[rows], w.k, w.value, w.q_pos[rows], w.q_seq[rows],
                                 w.cu_seqlens, w.mode, idx, w.scale, w.block_size)
            t2 = time.perf_counter()
            t_sel += t1 - t0
            t_att += t2 - t1
            sub = _SubRows(w, rows)
            done_pairs += effective_pairs(sub, idx)
            rows_done += len(rows)
            if time.perf_counter() - t_start > seconds:
                break
    flops = done_pairs * 2.0 * (w.dqk + w.dv)
    return {"value": flops / (t_sel + t_att) / 1e12, "unit": "TFLOP/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{rows_done} of {w.n_q} query rows (all heads), seeded random; "
                      f"selection {t_sel:.2f}s + attention {t_att:.2f}s in fp64 numpy",
            "seconds": t_sel + t_att}


class _SubRows:
    """A view of a workload restricted to some rows (for effective_pairs)."""

    def __init__(self, w, rows):
        self.cu_seqlens, self.block_size, self.mode = w.cu_seqlens, w.block_size, w.mode
        self.q_seq, self.q_pos, self.hq = w.q_seq[rows], w.q_pos[rows], w.hq


def graph_step(torch, select, attend, args):
    """Captures one step (selection + attention, the same calls) into a HIP graph and
    times `steps` replays.  Every checked replay must reproduce the eager output and
    log-sum-exp bit for bit, with eager work and synchronizations in between."""
    ref_out, ref_lse = attend(select())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            attend(select())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        g_out, g_lse = attend(select())
    torch.cuda.synchronize()
    replays = 3
    for _ in range(replays):
        g.replay()
        torch.cuda.synchronize()
        if not (torch.equal(g_out, ref_out) and torch.equal(g_lse, ref_lse)):
            raise RuntimeError("graph replay differs from the eager step")
        attend(select())  # eager work between replays
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / args.steps, replays


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(each context-parallel rank's shard is independent once K/V are gathered). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import context_sparse_attention_amd as csa
    from csa_inputs import make_workload

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    w = make_workload(args.workload)
    dev = "cuda"

    def up(x):
        t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        return t.to(torch.bfloat16) if w.dtype == "bf16" else t

    q, k = up(w.q), up(w.k)
    v = k[..., : w.dv] if w.v_alias else up(w.v)
    lay = csa.Layout(w.q_pos, w.q_seq, w.cu_seqlens)
    if w.mode == "token":
        iq, ik, wt = up(w.iq), up(w.ik), torch.from_numpy(w.w).to(dev)
    out_dtype = q.dtype

    def select():
        if w.mode == "block":
            return csa.moba_gate_topk(q, k, lay, w.block_size, w.topk)
        return csa.dsa_indexer_topk(iq, ik, wt, lay, w.topk)

    mode = csa.CSA_SEL_BLOCK if w.mode == "block" else csa.CSA_SEL_TOKEN

    def attend(idx):
        return csa.sparse_attn_fwd_shard(q, k, v, lay, mode, idx, block_size=w.block_size,
                                         softmax_scale=w.scale, out_dtype=out_dtype)

    for _ in range(args.warmup):
        attend(select())
    torch.cuda.synchronize()
    idx_np = select().cpu().numpy()
    pairs = effective_pairs(w, idx_np)
    flops = pairs * 2.0 * (w.dqk + w.dv)
    sel_bytes = selection_bytes(w)

    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    csa.trace_begin(4 * args.steps + 8)
    torch.cuda.synchronize()
    # about 20 ms of HBM copies on the stream first, so that the host has queued
    # every step before the GPU reaches it: the traced kernel times then hold no
    # launch gaps.  Copies keep the clocks where the steps left them; a spin
    # kernel let them drop, and the first traced kernels ran up to 15% slower.
    fill = torch.empty((2, 1 << 28), dtype=torch.uint8, device="cuda")
    for _ in range(200):
        fill[1].copy_(fill[0])
    for s in range(args.steps):
        ev[s][0].record(stream)
        idx = select()
        ev[s][1].record(stream)
        attend(idx)
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    traced = csa.trace_collect()
    csa.trace_begin(0)
    # GPU time of the queued eager steps (the host clock would count the spin)
    eager_ms_per_step = ev[0][0].elapsed_time(ev[args.steps - 1][2]) / args.steps
    ms_per_step = eager_ms_per_step
    graph = None
    if not args.no_graph:
        graph_ms, replays = graph_step(torch, select, attend, args)
        ms_per_step = graph_ms
        graph = {"ms_per_step": graph_ms, "replays_checked": replays}
    sel_ms = [ev[s][0].elapsed_time(ev[s][1]) for s in range(args.steps)]
    att_ms = [ev[s][1].elapsed_time(ev[s][2]) for s in range(args.steps)]
    kern = {}
    for name, ms in traced:
        kern.setdefault(name, []).append(ms)

    cold = None
    if not args.no_cold:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        c_sel, c_att = [], []
        for s in range(max(5, min(args.steps, 10))):
            flush.fill_(s & 0xFF)  # 1 GiB write evicts the 256 MB MALL and the L2s
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            idx = select()
            e[1].record(stream)
            attend(idx)
            e[2].record(stream)
            torch.cuda.synchronize()
            c_sel.append(e[0].elapsed_time(e[1]))
            c_att.append(e[1].elapsed_time(e[2]))
        del flush
        cold = {"select_ms_median": float(np.median(c_sel)),
                "attention_ms_median": float(np.median(c_att)),
                "select_GBs": sel_bytes["total"] / (np.median(c_sel) * 1e-3) / 1e9,
                "attention_TFLOPs": flops / (np.median(c_att) * 1e-3) / 1e12}

    up_proj = None
    if w.mode == "token" and w.v_alias:
        # absorbed MLA: the value up-projection after the attention, on this step's
        # latent output and a synthetic per-head weight (128 output channels); not
        # part of the step, timed on its own over 20 launches
        from csa_inputs import up_projection_inputs
        o_lat = attend(select())[0]
        w_up = torch.from_numpy(up_projection_inputs(1, w.hq, w.dv, 128)[1]).to(dev)
        w_up = w_up.to(torch.bfloat16)
        for _ in range(3):
            csa.mla_v_up_proj(o_lat, w_up)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(20):
            csa.mla_v_up_proj(o_lat, w_up)
        e1.record(stream)
        torch.cuda.synchronize()
        up_ms = e0.elapsed_time(e1) / 20
        up_bytes = (o_lat.numel() + w_up.numel() + w.n_q * w.hq * 128) * 2
        up_proj = {"kernel": "k_mla_v_up", "ms": up_ms, "alg_bytes": up_bytes,
                   "GBs": up_bytes / (up_ms * 1e-3) / 1e9,
                   "frac_hbm": up_bytes / (up_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}

    att_med = float(np.median(att_ms))
    sel_med = float(np.median(sel_ms))
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    # dominant attention kernel and the algorithmic flops of one launch
    if "k_bm_attn" in kern:
        # full-block and own-block (causal) chunks are both computed there
        dom, dom_flops = "k_bm_attn", flops
    elif "k_tok_attn" in kern:
        dom, dom_flops = "k_tok_attn", flops
    else:
        dom, dom_flops = "k_attn_generic", flops
    dom_ms = float(np.mean(kern[dom])) if dom in kern else att_med
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    # dominant selection kernel
    if w.mode == "block":
        sk = "k_moba_gate_mfma" if "k_moba_gate_mfma" in kern else "k_moba_gate"
        esz = 2 if w.dtype == "bf16" else 4
        sk_work = w.n_q * w.hq * w.dqk * esz + w.n_q * w.hq * (w.topk + 1) * 4
        sk_unit, sk_peak = "GB/s", PEAK_HBM_GBS
    else:
        sk = "k_dsa_logits_mfma" if "k_dsa_logits_mfma" in kern else "k_dsa_logits"
        sk_work = sel_bytes["indexer_flops"]
        sk_unit, sk_peak = "TFLOP/s", peak
    sk_ms = float(np.mean(kern[sk])) if sk in kern else float("nan")
    sk_rate = sk_work / (sk_ms * 1e-3) / (1e9 if sk_unit == "GB/s" else 1e12)
    result = {
        "metric": METRIC,
        "value": flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) bf16 inputs of the workload's shapes)",
        "config": {"workload": w.name, "n_q": w.n_q, "n_kv": w.n_kv, "hq": w.hq,
                   "hkv": w.hkv, "dqk": w.dqk, "dv": w.dv, "mode": w.mode,
                   "block_size": w.block_size, "topk": w.topk,
                   "effective_pairs": pairs, "effective_gflop": flops / 1e9},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": measured_traffic(dom, w.name),
                     "kernel_ms": dom_ms, "kernel_gflop": dom_flops / 1e9},
        "stages": {"select_ms_median": sel_med, "attention_ms_median": att_med,
                   "attention_TFLOPs": flops / (att_med * 1e-3) / 1e12,
                   "attention_frac_peak": flops / (att_med * 1e-3) / 1e12 / peak,
                   "select_alg_bytes": sel_bytes["total"],
                   "select_GBs": sel_bytes["total"] / (sel_med * 1e-3) / 1e9,
                   "select_frac_hbm": sel_bytes["total"] / (sel_med * 1e-3) / 1e9 / PEAK_HBM_GBS,
                   "select_kernel": {"kernel": sk, "ms": sk_ms, "rate": sk_rate,
                                     "unit": sk_unit, "frac": sk_rate / sk_peak},
                   "kernels_ms": {k: float(np.mean(v)) for k, v in kern.items()},
                   "eager_ms_per_step": eager_ms_per_step, "graph": graph,
                   "cold": cold, "v_up_proj": up_proj},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
