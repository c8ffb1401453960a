"""Benchmark: one step = selection + sparse attention of one context-parallel shard.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step runs the whole hot path once over one synthetic batch already resident
in HBM: ``dsa_indexer_topk`` then ``sparse_attn_fwd_shard`` (token mode) for
the DSA workload, ``moba_gate_topk`` then ``sparse_attn_fwd_shard`` (block
mode) for the MoBA workloads.  The headline workload is the largest one that
fits one GPU, the DSA shard (absorbed MLA, 4096 queries at offset 8192 of a
16384-token stream, 128 query heads over one 576-wide latent key, indexer
64 x 128, top-2048 tokens; 2336.5 effective GFLOP per step).

Printed: one JSON line.  ``value`` is effective TFLOP/s of the headline step
(selected permitted query-key pairs x 2 x (Dqk + Dv) per second), timed over
K replays of the step captured as a HIP graph (the same library calls; every
checked replay reproduces the eager output bit for bit).  ``stages`` holds,
for the headline and for each of the other bf16 workloads (8K MHA, 32K GQA
zigzag, 64K packed THD), the step time (median, p10, p90 of per-step GPU
times), the call-level attention rate F / t(sparse_attn_fwd_shard) against
the bf16 peak, the dominant kernel's rate, and the selection stage's GB/s
against HBM.  ``roofline`` is the headline's dominant kernel; ``cpu_baseline``
the fp64 CPU oracle on the host's cores over a bounded share of the headline.
"""

import argparse
import json
import os
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective sparse-attn TFLOP/s per shard (+ gate/top-k HBM GB/s), % of roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
HEADLINE = "dsa_mla_16k"
OTHERS = ["moba_mha_8k", "moba_gqa_zigzag_32k", "moba_thd_64k"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=HEADLINE)
    p.add_argument("--stage-steps", type=int, default=20,
                   help="timed steps of each other workload's stage figures")
    p.add_argument("--no-stages", action="store_true",
                   help="measure the named workload only (no other workloads)")
    p.add_argument("--cpu-seconds", type=float, default=20.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-cold", action="store_true")
    p.add_argument("--no-backward", action="store_true",
                   help="skip the backward stage (sparse_attn_bwd_shard) of the headline")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain device-to-device copy of known size (the reference "
                        "for scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return p.parse_args()


# Source files of each kernel; the HBM traffic of a kernel, taken from counter
# runs, is reported only while these files are unchanged.
KERNEL_SOURCES = {
    "k_bm_attn": ["attn_block_mfma.hip"],
    "k_tok_attn": ["attn_token_mfma.hip", "mfma.hpp"],
    "k_tok_attn16": ["attn_token_mfma.hip"],
    "k_tok_attn16p": ["attn_token_mfma.hip"],
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


def permitted_bounds(cu, q_seq, q_pos):
    cu = np.asarray(cu, np.int64)
    seq = np.asarray(q_seq, np.int64)
    pos = np.asarray(q_pos, np.int64)
    ok = (seq >= 0) & (seq < len(cu) - 1)
    s = np.clip(seq, 0, len(cu) - 2)
    lo, end = cu[s], cu[s + 1]
    ok &= (pos >= lo) & (pos < end)
    return lo, pos, end, ok


def effective_pairs(mode, cu, q_seq, q_pos, hq, block_size, idx):
    """Selected permitted (query head, key) pairs of the given rows and index rows."""
    lo, pos, end, ok = permitted_bounds(cu, q_seq, q_pos)
    idx = np.asarray(idx, np.int64)
    if idx.ndim == 2:
        idx = idx[:, None, :]
    lo_, pos_, end_ = lo[:, None, None], pos[:, None, None], end[:, None, None]
    valid = ok[:, None, None] & (idx >= lo_) & (idx <= pos_)
    if mode == "block":
        valid &= ((idx - lo_) % block_size) == 0
        n = np.minimum(np.minimum(idx + block_size, end_), pos_ + 1) - idx
        pairs = int(np.where(valid, n, 0).sum())
    else:
        pairs = int(valid.sum())
    if idx.shape[1] == 1:
        pairs *= hq
    return pairs


def selection_bytes(w):
    """Algorithmic HBM bytes of the selection stage (read once, written once)."""
    lo, pos, end, ok = permitted_bounds(w.cu_seqlens, w.q_seq, w.q_pos)
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


# ------------------------------------------------------------------------------
# CPU baseline: the fp64 oracle over the host's cores (worker processes)
# ------------------------------------------------------------------------------

_CPU = {}


def _cpu_init(folder, names):
    global _CPU
    _CPU = {n: np.asarray(np.load(os.path.join(folder, n + ".npy"), mmap_mode="r"))
            for n in names}


def _cpu_rows(args):
    """Selection and attention of some rows by the oracle; (pairs, t_sel, t_att)."""
    import oracle
    rows, p = args
    A = _CPU
    rows = np.asarray(rows)
    q, q_pos, q_seq = A["q"][rows], A["q_pos"][rows], A["q_seq"][rows]
    t0 = time.perf_counter()
    if p["mode"] == "block":
        gate = oracle.gate_scores(q, A["k"], q_pos, q_seq, A["cu"], p["block_size"])
        idx = oracle.select_blocks(gate, p["topk"])
    else:
        idx, _, _ = oracle.indexer_topk(A["iq"][rows], A["ik"], A["w"][rows], q_pos, q_seq,
                                        A["cu"], p["topk"])
        idx = idx[:, None, :]
    t1 = time.perf_counter()
    v = A["k"][..., :p["dv"]] if p["v_alias"] else A["v"]
    oracle.shard_forward(q, A["k"], v, q_pos, q_seq, A["cu"], p["mode"], idx, p["scale"],
                         p["block_size"])
    t2 = time.perf_counter()
    pairs = effective_pairs(p["mode"], A["cu"], q_seq, q_pos, q.shape[1], p["block_size"], idx)
    return pairs, t1 - t0, t2 - t1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, seconds):
    """The fp64 oracle (selection + attention) on chunks of rows in worker
    processes, one per affinity core up to 16 (the host share of a one-GPU job;
    one BLAS thread each), until about ``seconds`` of wall time have passed;
    effective TFLOP/s of the rows done."""
    import multiprocessing as mp
    import shutil
    cores = min(16, len(os.sched_getaffinity(0)))
    folder = tempfile.mkdtemp(prefix="csa_cpu_")
    arrays = dict(q=w.q, k=w.k, q_pos=w.q_pos, q_seq=w.q_seq, cu=w.cu_seqlens)
    if not w.v_alias:
        arrays["v"] = w.v
    if w.mode == "token":
        arrays.update(iq=w.iq, ik=w.ik, w=w.w)
    for n, a in arrays.items():
        np.save(os.path.join(folder, n + ".npy"), np.ascontiguousarray(a))
    params = dict(mode=w.mode, block_size=w.block_size, topk=w.topk, scale=w.scale,
                  dv=w.dv, v_alias=w.v_alias)
    order = np.random.default_rng(0).permutation(w.n_q)
    chunks = [np.sort(order[s:s + 8]).tolist() for s in range(0, w.n_q, 8)]
    saved = {v: os.environ.get(v) for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                              "MKL_NUM_THREADS")}
    for v in saved:
        os.environ[v] = "1"
    pool = mp.get_context("spawn").Pool(cores, initializer=_cpu_init,
                                        initargs=(folder, list(arrays)))
    for v, old in saved.items():
        if old is None:
            os.environ.pop(v, None)
        else:
            os.environ[v] = old
    try:
        pool.map(_cpu_rows, [(chunks[0], params)] * cores)  # warm-up: every worker loaded
        pairs = rows = 0
        t_sel = t_att = 0.0
        t_start = time.perf_counter()
        t_end = t_start
        for res, c in zip(pool.imap(_cpu_rows, [(c, params) for c in chunks]), chunks):
            pairs += res[0]
            t_sel += res[1]
            t_att += res[2]
            rows += len(c)
            t_end = time.perf_counter()
            if t_end - t_start > seconds:
                break
    finally:
        pool.terminate()
        pool.join()
        shutil.rmtree(folder, ignore_errors=True)
    wall = t_end - t_start
    flops = pairs * 2.0 * (w.dqk + w.dv)
    return {"value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{rows} of {w.n_q} query rows of {w.name} (all heads; seeded random "
                      f"chunks of 8 rows), indexer/gate selection + attention in fp64 numpy, "
                      f"{cores} worker processes with one BLAS thread each, {wall:.1f} s wall "
                      f"(selection {t_sel:.1f} + attention {t_att:.1f} core-seconds)",
            "seconds": wall}


# ------------------------------------------------------------------------------
# GPU measurement of one workload
# ------------------------------------------------------------------------------

def _q(xs, p):
    return float(np.percentile(np.asarray(xs, np.float64), p))


def backward_stage(torch, csa, w, q, k, v, lay, idx, mode, out_dtype, reps=1):
    """sparse_attn_bwd_shard after the forward on the step's selection: the mean time
    of `reps` calls (events around each call, after one untimed call), its kernels,
    and the algorithmic rate.  Algorithmic flops per selected pair: the logits
    recomputed (2 Dqk), dP (2 Dv), dV (2 Dv), dQ (2 Dqk) and dK (2 Dqk), priced
    against the bf16 dense MFMA peak for the matrix-core kernels and against the
    fp32 vector peak for the vector-ALU ones."""
    out, lse = csa.sparse_attn_fwd_shard(q, k, v, lay, mode, idx, block_size=w.block_size,
                                         softmax_scale=w.scale, out_dtype=out_dtype)
    dout = torch.randn(out.shape, generator=torch.Generator(device="cuda").manual_seed(1),
                       device="cuda", dtype=torch.float32).to(out_dtype)
    ws_bytes = csa.sparse_attn_bwd_shard_workspace_size(
        q, k, v, lay, mode, 1 if idx.dim() == 2 else idx.shape[1], idx.shape[-1], w.block_size)
    dq = torch.empty((w.n_q, w.hq, w.dqk), dtype=torch.float32, device="cuda")
    dk = torch.empty((w.n_kv, w.hkv, w.dqk), dtype=torch.float32, device="cuda")
    dv = torch.empty((w.n_kv, w.hkv, w.dv), dtype=torch.float32, device="cuda")

    def call():
        csa.sparse_attn_bwd_shard(q, k, v, lay, mode, idx, out, dout, lse,
                                  block_size=w.block_size, softmax_scale=w.scale, dq=dq, dk=dk,
                                  dv=dv)

    call()
    torch.cuda.synchronize()
    csa.trace_begin(8 * reps + 8)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for r in range(reps):
        call()
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    traced = csa.trace_collect()
    csa.trace_begin(0)
    ms = [ev[r].elapsed_time(ev[r + 1]) for r in range(reps)]
    kern = {}
    for name, t in traced:
        kern.setdefault(name, []).append(t)
    pairs = effective_pairs(w.mode, w.cu_seqlens, w.q_seq, w.q_pos, w.hq, w.block_size,
                            idx.cpu().numpy())
    flops = pairs * 2.0 * (3 * w.dqk + 2 * w.dv)
    mean = float(np.mean(ms))
    family = csa.sparse_attn_bwd_shard_kernel(q, k, v, lay, mode,
                                              1 if idx.dim() == 2 else idx.shape[1],
                                              idx.shape[-1], w.block_size)
    # the matrix-core kernels price against the bf16 dense peak, the vector-ALU
    # ones against the fp32 vector peak
    on_mfma = family in ("block_mfma", "token_mfma")
    peak = PEAK_BF16_TFLOPS if on_mfma else PEAK_FP32_TFLOPS
    return {"call": "sparse_attn_bwd_shard", "kernel_family": family, "ms": mean,
            "ms_min": float(np.min(ms)), "alg_gflop": flops / 1e9,
            "TFLOPs": flops / (mean * 1e-3) / 1e12,
            "bound": "mfma" if on_mfma else "alu", "peak": peak,
            "frac": flops / (mean * 1e-3) / 1e12 / peak,
            "kernels_ms": {k_: float(np.mean(v_)) for k_, v_ in kern.items()},
            "reps": reps}


def measure(torch, csa, w, steps, warmup, cold=True, up_proj=False, timed_steps=None,
            backward=False):
    """Everything measured on one workload; returns a dict (headline fields included)."""
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
    mode = csa.CSA_SEL_BLOCK if w.mode == "block" else csa.CSA_SEL_TOKEN

    def select():
        if w.mode == "block":
            return csa.moba_gate_topk(q, k, lay, w.block_size, w.topk)
        return csa.dsa_indexer_topk(iq, ik, wt, lay, w.topk)

    def attend(idx):
        return csa.sparse_attn_fwd_shard(q, k, v, lay, mode, idx, block_size=w.block_size,
                                         softmax_scale=w.scale, out_dtype=out_dtype)

    for _ in range(warmup):
        attend(select())
    torch.cuda.synchronize()
    idx_np = select().cpu().numpy()
    pairs = effective_pairs(w.mode, w.cu_seqlens, w.q_seq, w.q_pos, w.hq, w.block_size, idx_np)
    flops = pairs * 2.0 * (w.dqk + w.dv)
    sel_bytes = selection_bytes(w)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS

    # eager steps with event pairs around each call and the library's own trace
    # events around its kernels.  About 20 ms of HBM copies on the stream first,
    # so that the host has queued every step before the GPU reaches it (no
    # launch gaps inside the pairs); copies also keep the clocks up.
    stream = torch.cuda.current_stream()
    n_ev = max(steps, 10)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
    csa.trace_begin(8 * n_ev + 8)
    torch.cuda.synchronize()
    fill = torch.empty((2, 1 << 28), dtype=torch.uint8, device=dev)
    for _ in range(200):
        fill[1].copy_(fill[0])
    for s in range(n_ev):
        ev[s][0].record(stream)
        idx = select()
        ev[s][1].record(stream)
        attend(idx)
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    del fill
    traced = csa.trace_collect()
    csa.trace_begin(0)
    sel_ms = [ev[s][0].elapsed_time(ev[s][1]) for s in range(n_ev)]
    att_ms = [ev[s][1].elapsed_time(ev[s][2]) for s in range(n_ev)]
    eager_step = [ev[s][0].elapsed_time(ev[s][2]) for s in range(n_ev)]
    kern = {}
    for name, ms in traced:
        kern.setdefault(name, []).append(ms)

    # the step as a captured HIP graph: every checked replay must reproduce the
    # eager output and log-sum-exp bit for bit, with eager work in between
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
        attend(select())
        torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    # per-step GPU times of replays (events between replays) for the spread
    rev = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev + 1)]
    rev[0].record(stream)
    for s in range(n_ev):
        g.replay()
        rev[s + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = [rev[s].elapsed_time(rev[s + 1]) for s in range(n_ev)]
    # the timed region: exactly `timed_steps` replays between two synchronizations
    timed = timed_steps or steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(timed):
        g.replay()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / timed
    del g

    cold_res = None
    if cold:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        c_sel, c_att = [], []
        for s in range(5):
            flush.fill_(s & 0xFF)  # a 1 GiB write evicts the 256 MB MALL and the L2s
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
        cold_res = {"select_ms_median": _q(c_sel, 50), "attention_ms_median": _q(c_att, 50),
                    "select_GBs": sel_bytes["total"] / (_q(c_sel, 50) * 1e-3) / 1e9,
                    "attention_TFLOPs": flops / (_q(c_att, 50) * 1e-3) / 1e12}

    up_res = None
    if up_proj and w.mode == "token" and w.v_alias:
        # absorbed MLA: the value up-projection after the attention, on this
        # step's latent output and a synthetic per-head weight (128 output
        # channels); not part of the step, timed on its own over 20 launches
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
        up_res = {"kernel": "k_mla_v_up", "ms": up_ms, "alg_bytes": up_bytes,
                  "GBs": up_bytes / (up_ms * 1e-3) / 1e9,
                  "frac_hbm": up_bytes / (up_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}

    bwd_res = None
    if backward:
        bwd_res = backward_stage(torch, csa, w, q, k, v, lay, select(), mode, out_dtype)

    att_med, sel_med = _q(att_ms, 50), _q(sel_ms, 50)
    for dom in ("k_bm_attn", "k_tok_attn16p", "k_tok_attn16", "k_tok_attn", "k_attn_generic"):
        if dom in kern:
            break
    dom_ms = float(np.mean(kern[dom])) if dom in kern else att_med
    achieved = flops / (dom_ms * 1e-3) / 1e12
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
    sel_gbs = sel_bytes["total"] / (sel_med * 1e-3) / 1e9
    res = {
        "workload": w.name,
        "ms_per_step": ms_per_step,
        "step_ms": {"p10": _q(step_ms, 10), "median": _q(step_ms, 50), "p90": _q(step_ms, 90)},
        "TFLOPs": flops / (ms_per_step * 1e-3) / 1e12,
        "effective_pairs": pairs,
        "effective_gflop": flops / 1e9,
        "attention_call": {"ms_median": att_med, "ms_p10": _q(att_ms, 10),
                           "ms_p90": _q(att_ms, 90),
                           "TFLOPs": flops / (att_med * 1e-3) / 1e12,
                           "frac_peak": flops / (att_med * 1e-3) / 1e12 / peak},
        "attention_kernel": {"kernel": dom, "ms": dom_ms, "TFLOPs": achieved,
                             "frac_peak": achieved / peak,
                             "traffic": measured_traffic(dom, w.name)},
        "select_call": {"ms_median": sel_med, "ms_p10": _q(sel_ms, 10),
                        "ms_p90": _q(sel_ms, 90), "alg_bytes": sel_bytes["total"],
                        "GBs": sel_gbs, "frac_hbm": sel_gbs / PEAK_HBM_GBS,
                        # the block selection is bound by HBM; the token indexer's
                        # call by its MFMA logits (flops / call time / bf16 peak)
                        "bound": "hbm" if w.mode == "block" else "mfma",
                        "frac": (sel_gbs / PEAK_HBM_GBS if w.mode == "block" else
                                 sel_bytes["indexer_flops"] / (sel_med * 1e-3) / 1e12 / peak)},
        "select_kernel": {"kernel": sk, "ms": sk_ms, "rate": sk_rate, "unit": sk_unit,
                          "frac": sk_rate / sk_peak},
        "kernels_ms": {k_: float(np.mean(v_)) for k_, v_ in kern.items()},
        "eager_ms_per_step": _q(eager_step, 50),
        "graph_replays_checked": replays,
        "cold": cold_res,
        "v_up_proj": up_res,
        "backward": bwd_res,
        "peak": peak,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
    }
    if w.mode == "token":
        res["select_kernel_dsa_select"] = {
            "kernel": "k_dsa_select_reg",
            "ms": float(np.mean(kern["k_dsa_select_reg"])) if "k_dsa_select_reg" in kern
            else None}
        if "k_dsa_select_reg" in kern:
            ms_ = res["select_kernel_dsa_select"]["ms"]
            res["select_kernel_dsa_select"]["GBs"] = sel_bytes["total"] / (ms_ * 1e-3) / 1e9
            res["select_kernel_dsa_select"]["frac_hbm"] = \
                res["select_kernel_dsa_select"]["GBs"] / PEAK_HBM_GBS
    return res


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

    # the other workloads first (their stage figures), so that the headline's
    # timed steps also run on a warm GPU
    stages = {}
    if not args.no_stages:
        for name in OTHERS:
            if name == args.workload:
                continue
            wo = make_workload(name)
            stages[name] = measure(torch, csa, wo, args.stage_steps, max(args.warmup, 50),
                                   cold=False)
            print(f"[stage] {name}: {stages[name]['ms_per_step']:.4f} ms/step", file=sys.stderr,
                  flush=True)
            del wo
            torch.cuda.empty_cache()

    w = make_workload(args.workload)
    head = measure(torch, csa, w, args.steps, args.warmup, cold=not args.no_cold, up_proj=True,
                   timed_steps=args.steps, backward=not args.no_backward)
    stages[w.name] = head
    dom = head["attention_kernel"]
    result = {
        "metric": METRIC,
        "value": head["TFLOPs"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded N(0,1) bf16 inputs of the workload's shapes)",
        "config": {"workload": w.name, "n_q": w.n_q, "n_kv": w.n_kv, "hq": w.hq,
                   "hkv": w.hkv, "dqk": w.dqk, "dv": w.dv, "mode": w.mode,
                   "block_size": w.block_size, "topk": w.topk,
                   "effective_pairs": head["effective_pairs"],
                   "effective_gflop": head["effective_gflop"]},
        "roofline": {"kernel": dom["kernel"], "bound": "mfma", "achieved": dom["TFLOPs"],
                     "peak": head["peak"], "unit": "TFLOP/s", "frac": dom["frac_peak"],
                     "traffic": dom["traffic"], "kernel_ms": dom["ms"],
                     "kernel_gflop": head["effective_gflop"]},
        "stages": stages,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
