"""Selection accuracy of the key scan against exact top-k (measurement; not
on the decode path).

The pages measure a scan by the attention output it leads to, against exact
top-k attention (basis-choice section, the table of attention errors; the
same-GPU-time comparison with SparQ).  The formula is not printed; the
reading here: for each query head h with selected token set S (k tokens),

    o_S = sum_{i in S} softmax_S(q_h . k_i / sqrt(D)) v_i

over the unquantised keys and values, and

    error = ||o_S - o_S*|| / ||o_S*||,   recall = |S n S*| / k,

with S* the k largest exact scores q_h . k_i (ties to the lower index).  The
selection S comes from the library (pack, plan, fused scan + top-k through
the C ABI); exact scores and attention are plain float64 numpy definitions.

    python -m sparse_attention_key_amd.accuracy --workload qwen32k --pairs 4
"""
from __future__ import annotations

import argparse
import json
import sys
import time

import numpy as np

from . import fathom as F

PLAN_MODES = {"waterfill": F.PLAN_WATERFILL, "topr": F.PLAN_TOPR, "uniform": F.PLAN_UNIFORM}


def exact_scores(keys: np.ndarray, q: np.ndarray) -> np.ndarray:
    """keys [n][D], q [G][D] -> [G][n] float64 dot products."""
    return np.asarray(q, np.float64) @ np.asarray(keys, np.float64).T


def exact_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """[G][n] -> [G][k] indices by (score descending, index ascending)."""
    G, n = scores.shape
    out = np.empty((G, k), np.int64)
    idx = np.arange(n)
    for h in range(G):
        out[h] = np.lexsort((idx, -scores[h]))[:k]
    return out


def attention(q_h: np.ndarray, keys: np.ndarray, values: np.ndarray, sel) -> np.ndarray:
    """Softmax attention of one head over the rows `sel` (float64)."""
    sel = np.asarray(sel, np.int64)
    k = np.asarray(keys, np.float64)[sel]
    s = k @ np.asarray(q_h, np.float64) / np.sqrt(k.shape[1])
    s -= s.max()
    p = np.exp(s)
    p /= p.sum()
    return p @ np.asarray(values, np.float64)[sel]


def selection_metrics(q, keys, values, sel, ref):
    """Per head: (relative attention-output error, recall) of selection
    `sel` [G][k] against the reference selection `ref` [G][k]."""
    G = q.shape[0]
    err = np.empty(G)
    rec = np.empty(G)
    for h in range(G):
        o = attention(q[h], keys, values, sel[h])
        o_ref = attention(q[h], keys, values, ref[h])
        err[h] = np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref)
        rec[h] = len(np.intersect1d(sel[h], ref[h])) / len(ref[h])
    return err, rec


def parse_plan(spec: str):
    """'B48' -> waterfill 48, 'r16' -> top-r 16, 'u2' -> uniform depth 2."""
    kind, val = spec[0], int(spec[1:])
    return {"B": "waterfill", "r": "topr", "u": "uniform"}[kind], val


def evaluate(w, plans, pairs, basis="raw", n=None, device="cuda"):
    """Mean error and recall of each plan over `pairs` of workload `w`."""
    import torch

    import workloads as wl

    n = w.n if n is None else n
    P = len(pairs)
    keys = np.stack([wl.keys_host(w, p, n=n) for p in pairs])
    q = np.stack([wl.queries(w, p) for p in pairs])
    kd = torch.from_numpy(keys).to(device)
    if w.key_dtype == "bf16":
        kd = kd.to(torch.bfloat16)
    cal = torch.from_numpy(np.stack([wl.calibration_sample(w, p) for p in pairs])).to(device)
    cov, s2 = F.calib_covariance(cal, with_cov=basis == "klt")
    rot = None
    if basis == "klt":
        rot, s2 = F.calib_basis(cov)
    planes, scales = F.pack(kd, rot=rot)
    qd = torch.from_numpy(q).to(device)
    values = [wl.values_host(w, p, n=n) for p in pairs]
    refs = [exact_topk(exact_scores(keys[i], q[i]), w.k) for i in range(P)]
    out = {}
    for spec in plans:
        mode, val = parse_plan(spec)
        pl = F.plan(qd, s2, val, PLAN_MODES[mode], rot=rot)
        sel = F.scan_topk(planes, scales, n, pl, w.k).idx.cpu().numpy()
        errs, recs = [], []
        for i in range(P):
            e, r = selection_metrics(q[i], keys[i], values[i], sel[i], refs[i])
            errs.append(e)
            recs.append(r)
        depth = pl.depth.to(torch.int64)
        bits = float((depth.sum(1).double() + 16.0 * (depth > 0).sum(1).double() / 64.0).mean())
        out[spec] = {"error": float(np.mean(errs)), "recall": float(np.mean(recs)),
                     "bits_per_token": round(bits, 2)}
    return out


def main(argv=None):
    import workloads as wl

    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="qwen32k", choices=sorted(wl.WORKLOADS))
    ap.add_argument("--pairs", type=int, default=4, help="pairs sampled evenly across the workload")
    ap.add_argument("--n", type=int, default=None, help="tokens per pair (default: the workload's)")
    ap.add_argument("--plans", default="B32,B40,B48,B68,B92,B136,r16,r32,u2")
    ap.add_argument("--basis", default="raw", choices=["raw", "klt"])
    a = ap.parse_args(argv)
    w = wl.WORKLOADS[a.workload]
    pairs = sorted({int(p) for p in np.linspace(0, w.P - 1, a.pairs).round()})
    t0 = time.time()
    res = evaluate(w, a.plans.split(","), pairs, basis=a.basis, n=a.n)
    print(json.dumps({"workload": w.name, "n": a.n or w.n, "k": w.k, "basis": a.basis, "pairs": pairs,
                      "metric": "attention-output relative error and recall vs exact top-k",
                      "plans": res, "seconds": round(time.time() - t0, 1)}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
