"""Full-size oracle checks spread over worker processes (test infrastructure).

The fp64 oracle is a per-row loop; at the named workloads' sizes one process
takes minutes.  ``OraclePool`` writes the workload's arrays (and the GPU's
results) once as .npy files, starts worker processes that memory-map them, and
runs a check on chunks of rows in each worker.  The checks compare the GPU's
results with the oracle row by row inside the worker and return only counts
and the worst errors, so nothing large crosses the process boundary.

This module imports numpy and the oracle only (no torch, no GPU library), so
the workers never touch the GPU.  Workers are started with the "spawn" method
(a fresh interpreter, not a fork of a process that may hold GPU state), each
with one BLAS thread.

Index outputs follow the margin criterion stated in ``classify_row``; attention
outputs are compared with the oracle evaluated on the GPU's own selection.
"""

import multiprocessing as mp
import os
import shutil
import tempfile

import numpy as np

import oracle

REL_MARGIN = 1e-3

_A = {}  # worker side: name -> memory-mapped array


def n_workers():
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    # the GPU machines allot 16 cores to a one-GPU job
    return max(1, min(16, cores))


def classify_row(scores, gpu_set, ora_set, k):
    """Compare one selection with the margin criterion.

    scores: oracle candidate scores (float64) indexed like the candidate ids in
    gpu_set / ora_set (sets of candidate positions 0..n-1).  The GPU must keep
    exactly min(k, n) candidates; where the oracle's k-th vs (k+1)-th margin
    exceeds 1e-3 relative (ties to the lower index) the sets must be equal;
    otherwise they may differ only inside the +-1e-3 band around the k-th score.
    Returns "exact", "near_tie_ok" or a failure string.
    """
    n = len(scores)
    kept = min(k, n)
    if len(gpu_set) != kept:
        return f"fail: {len(gpu_set)} kept, {kept} expected"
    if gpu_set == ora_set:
        return "exact"
    if n <= k:
        return "fail: short history must take every candidate"
    srt = np.sort(scores)[::-1]
    sk, sk1 = srt[k - 1], srt[k]
    denom = max(abs(sk), abs(sk1))
    rel = (sk - sk1) / denom if denom > 0 else 0.0
    if rel > REL_MARGIN:
        return f"fail: margin {rel:.2e} but selections differ"
    band = REL_MARGIN * abs(sk)
    for j in gpu_set ^ ora_set:
        if abs(scores[j] - sk) > band:
            return f"fail: candidate {j} (score {scores[j]:.6g}) outside the tie band"
    return "near_tie_ok"


# ------------------------------------------------------------------------------
# worker side
# ------------------------------------------------------------------------------

def _init(folder, names):
    global _A
    # plain ndarray views of the maps (memmap objects are slow to index)
    _A = {n: np.asarray(np.load(os.path.join(folder, n + ".npy"), mmap_mode="r"))
          for n in names}


def _attn_check(args):
    """Oracle attention on the GPU's selection for some rows against GPU outputs.

    ``p["targets"]`` lists (output name, lse name, tolerance) triples: several
    GPU outputs of the same selection (e.g. fp32 and bf16 output) are compared
    with one oracle evaluation.  Returns per target the worst absolute output
    and lse errors, the count of checked (row, head) pairs and of pairs without
    keys, and the first failures.
    """
    rows, p = args
    A = _A
    # keys and values are stored head-major (see OraclePool); the oracle reads
    # them through [token, head, dim] views
    k = A["k_hm"].transpose(1, 0, 2)
    v = A["v_hm"].transpose(1, 0, 2)
    ref, ref_lse = oracle.shard_forward(A["q"], k, v, A["q_pos"], A["q_seq"], A["cu"],
                                        p["mode"], A["idx"], p["scale"], p["block_size"],
                                        rows=rows)
    fin = np.isfinite(ref_lse)
    results = []
    for out_name, lse_name, tol in p["targets"]:
        got = np.asarray(A[out_name][rows], np.float64)
        got_lse = np.asarray(A[lse_name][rows], np.float64)
        res = {"pairs": int(got.shape[0] * got.shape[1]), "max_err": 0.0,
               "max_lse_err": 0.0, "no_key_pairs": int((~fin).sum()), "fails": []}
        results.append(res)
        if not np.isfinite(got).all():
            bad = np.argwhere(~np.isfinite(got))[0]
            res["fails"].append(f"{out_name}: row {rows[bad[0]]} head {bad[1]}: "
                                "non-finite output")
            continue
        if np.isnan(got_lse).any():
            bad = np.argwhere(np.isnan(got_lse))[0]
            res["fails"].append(f"{lse_name}: row {rows[bad[0]]} head {bad[1]}: NaN lse")
            continue
        err = np.abs(got - ref)
        res["max_err"] = float(err.max()) if err.size else 0.0
        if res["max_err"] > tol:
            worst = np.unravel_index(int(np.argmax(err)), err.shape)
            res["fails"].append(f"{out_name}: row {rows[worst[0]]} head {worst[1]} col "
                                f"{worst[2]}: |err| {res['max_err']:.3e} > {tol}")
        if not (np.isfinite(got_lse) == fin).all():
            bad = np.argwhere(np.isfinite(got_lse) != fin)[0]
            res["fails"].append(f"{lse_name}: row {rows[bad[0]]} head {bad[1]}: "
                                "lse finiteness differs")
        elif fin.any():
            res["max_lse_err"] = float(np.abs(got_lse[fin] - ref_lse[fin]).max())
            lse_tol = max(tol, 1e-4)
            if res["max_lse_err"] > lse_tol:
                res["fails"].append(f"{lse_name}: lse error {res['max_lse_err']:.3e} > "
                                    f"{lse_tol}")
        if (~fin).any() and ((got[~fin] != 0).any() or not np.isneginf(got_lse[~fin]).all()):
            res["fails"].append(f"{out_name}: a (row, head) without keys has a nonzero "
                                "output or a finite lse")
    return results


def _dsa_check(args):
    """Indexer rows: margin criterion on the GPU's indices, and the GPU's scores.

    The oracle's logits of each row are recomputed here; the GPU's selected
    logits must match them within ``p["score_rel"]`` of the sum of absolute
    terms sum_h w_h sum_d |iq_hd| |ik_jd| (which bounds fp32 rounding).
    """
    rows, p = args
    A = _A
    topk = p["topk"]
    counts = {"exact": 0, "near_tie_ok": 0, "no_keys": 0}
    fails = []
    max_score_err = 0.0
    for i in rows:
        gpu = np.asarray(A["idx"][i])
        gsc = np.asarray(A["score"][i], np.float64) if "score" in A else None
        iv = oracle.permitted_interval(int(A["q_pos"][i]), int(A["q_seq"][i]), A["cu"])
        if iv is None:
            if not (gpu == -1).all():
                fails.append(f"row {i}: no keys but selects")
            elif gsc is not None and not np.isneginf(gsc).all():
                fails.append(f"row {i}: no keys but scores are not -inf")
            counts["no_keys"] += 1
            continue
        lo, hi, _ = iv
        valid = gpu[gpu >= 0]
        if (gpu[len(valid):] != -1).any() or (np.diff(valid) <= 0).any():
            fails.append(f"row {i}: indices not ascending / -1 padded")
            continue
        if len(valid) and (valid[0] < lo or valid[-1] > hi):
            fails.append(f"row {i}: index outside [{lo}, {hi}]")
            continue
        L = oracle.indexer_logits_row(A["iq"][i], A["ik"], A["w"][i], lo, hi)
        ora = oracle.select_tokens_row(L, lo, topk)
        res = classify_row(L, set((valid - lo).tolist()), set((ora[ora >= 0] - lo).tolist()),
                           topk)
        if res.startswith("fail"):
            fails.append(f"row {i}: {res}")
            continue
        counts[res] += 1
        if gsc is not None:
            if not np.isneginf(gsc[len(valid):]).all():
                fails.append(f"row {i}: padding scores are not -inf")
                continue
            absdot = np.abs(np.asarray(A["iq"][i], np.float64)) @ \
                np.abs(np.asarray(A["ik"][valid], np.float64)).T
            bound = p["score_rel"] * (np.asarray(A["w"][i], np.float64) @ absdot) + 1e-30
            e = np.abs(gsc[:len(valid)] - L[valid - lo])
            max_score_err = max(max_score_err, float(e.max()) if e.size else 0.0)
            if (e > bound).any():
                j = int(np.argmax(e / bound))
                fails.append(f"row {i} key {valid[j]}: score error {e[j]:.3e} > {bound[j]:.3e}")
    return {"counts": counts, "fails": fails[:5], "n_fail": len(fails),
            "max_score_err": max_score_err}


def _bwd_keys(args):
    """Oracle dk, dv of the keys [a, a + n) of key head g, from the given rows
    (their query heads of group g only); float64 [n, D] partial sums."""
    rows, p = args
    A = _A
    g, a, n = p["g"], p["a"], p["n"]
    G = A["q"].shape[1] // A["k_hm"].shape[0]
    hs = slice(g * G, (g + 1) * G)
    k = A["k_hm"][g:g + 1].transpose(1, 0, 2)
    v = A["v_hm"][g:g + 1].transpose(1, 0, 2)
    _, dk, dv = oracle.shard_backward(A["q"][rows][:, hs], k, v, A["q_pos"][rows],
                                      A["q_seq"][rows], A["cu"], p["mode"],
                                      A["idx"][rows][:, hs], p["scale"], A["dout"][rows][:, hs],
                                      p["block_size"])
    return np.array(dk[a:a + n, 0]), np.array(dv[a:a + n, 0])


# ------------------------------------------------------------------------------
# parent side
# ------------------------------------------------------------------------------

def run_local(arrays, check, rows, params):
    """Runs one of the worker checks in this process (small cases)."""
    global _A
    saved = _A
    _A = {}
    for name, a in arrays.items():
        if name in ("k", "v"):
            a, name = np.asarray(a).transpose(1, 0, 2), name + "_hm"
        _A[name] = np.ascontiguousarray(a)
    try:
        return check((list(rows), params))
    finally:
        _A = saved


class OraclePool:
    """Worker processes over one set of arrays (context manager).

    ``arrays``: name -> numpy array.  The workers see them memory-mapped under
    the same names.  Arrays named ``k`` and ``v`` ([tokens, heads, dim]) are
    stored as ``k_hm`` / ``v_hm``: head-major (the same values; each head's keys
    are then contiguous, which is what the attention check reads slot by slot).
    """

    def __init__(self, arrays, processes=None):
        self.folder = tempfile.mkdtemp(prefix="csa_oracle_")
        names = []
        for name, a in arrays.items():
            if name in ("k", "v"):
                a = np.asarray(a).transpose(1, 0, 2)
                name += "_hm"
            np.save(os.path.join(self.folder, name + ".npy"), np.ascontiguousarray(a))
            names.append(name)
        self.processes = processes or n_workers()
        saved = {v: os.environ.get(v) for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                                  "MKL_NUM_THREADS")}
        try:
            for v in saved:
                os.environ[v] = "1"
            ctx = mp.get_context("spawn")
            self.pool = ctx.Pool(self.processes, initializer=_init,
                                 initargs=(self.folder, names))
        finally:
            for v, old in saved.items():
                if old is None:
                    os.environ.pop(v, None)
                else:
                    os.environ[v] = old

    def chunks(self, rows, per_worker=4):
        rows = np.asarray(list(rows), np.int64)
        n = max(1, min(len(rows), self.processes * per_worker))
        return [c.tolist() for c in np.array_split(rows, n) if len(c)]

    def attn_check(self, rows, params):
        """One summary dict per target of ``params["targets"]``."""
        parts = self.pool.map(_attn_check, [(c, params) for c in self.chunks(rows)])
        outs = []
        for t in range(len(params["targets"])):
            out = {"pairs": 0, "max_err": 0.0, "max_lse_err": 0.0, "no_key_pairs": 0,
                   "fails": []}
            for r in parts:
                r = r[t]
                out["pairs"] += r["pairs"]
                out["no_key_pairs"] += r["no_key_pairs"]
                out["max_err"] = max(out["max_err"], r["max_err"])
                out["max_lse_err"] = max(out["max_lse_err"], r["max_lse_err"])
                out["fails"] += r["fails"]
            outs.append(out)
        return outs

    def bwd_keys(self, rows, params):
        """(dk, dv) float64 of keys [a, a + n) of key head g (``params``: g, a, n,
        mode, scale, block_size) summed over ``rows``' contributions."""
        parts = self.pool.map(_bwd_keys, [(c, params) for c in self.chunks(rows, 1)])
        dk = sum(p[0] for p in parts)
        dv = sum(p[1] for p in parts)
        return dk, dv

    def dsa_check(self, rows, params):
        parts = self.pool.map(_dsa_check, [(c, params) for c in self.chunks(rows)])
        out = {"counts": {"exact": 0, "near_tie_ok": 0, "no_keys": 0}, "fails": [],
               "n_fail": 0, "max_score_err": 0.0}
        for r in parts:
            for k, v in r["counts"].items():
                out["counts"][k] += v
            out["fails"] += r["fails"]
            out["n_fail"] += r["n_fail"]
            out["max_score_err"] = max(out["max_score_err"], r["max_score_err"])
        return out

    def close(self):
        self.pool.terminate()
        self.pool.join()
        shutil.rmtree(self.folder, ignore_errors=True)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
