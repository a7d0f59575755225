"""Oracle outputs for whole heads of the full-size workloads (test fixtures).

Calls only the CPU oracle (``oracle/``) on the seeded synthetic inputs of
``synth`` and stores its fp64 results rounded to fp32 (rounding error 2^-24
relative, far inside the parity tolerances), with a hash of the inputs the
results belong to:

* qwen3-8b-layer-kvzip+-32k: LSE of every repeat query of query heads 0-7
  (KV heads 0 and 1) and the KVzip+ max score of every context key of KV
  heads 0 and 1;
* kvpop-future-mass-causal-16k: LSE of every query of every head and the
  future-attention target (window 128) of every key of every head;
* qwen2.5-14b-layer-kvzip+-120k: LSE of every repeat query of query heads
  0-4 and the KVzip+ max score of every context key of KV head 0.

The oracle is exact row by row, so the work is split over processes by query
row ranges (LSE rows are independent; the max / sum over query rows of the
score passes is taken over the ranges' partial results).

    python tests/golden/fullsize/make_fixtures.py [--procs 8] [workload ...]
"""
from __future__ import annotations

import os

# one BLAS thread per worker process (set before numpy loads its BLAS)
os.environ.setdefault("OPENBLAS_NUM_THREADS", "1")
os.environ.setdefault("OMP_NUM_THREADS", "1")

import argparse
import hashlib
import multiprocessing as mp
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402
from synth.workloads import BY_NAME  # noqa: E402

# workload -> KV heads whose query heads and keys are covered
HEADS = {
    "qwen3-8b-layer-kvzip+-32k": [0, 1],
    "kvpop-future-mass-causal-16k": list(range(8)),
    "qwen2.5-14b-layer-kvzip+-120k": [0],
}

_D = {}  # the drawn inputs, shared with forked workers


def input_hash(d, kv_heads, G):
    """sha256 of the bf16 inputs (and fp32 weights) the fixture belongs to."""
    h = hashlib.sha256()
    g0, g1 = kv_heads[0] * G, (kv_heads[-1] + 1) * G
    for name in ("Q", "Kctx", "Kself", "vnorm", "hnorm"):
        if name not in d:
            continue
        x = d[name]
        if name == "Q":
            x = x[g0:g1]
        elif name in ("Kctx", "Kself", "vnorm"):
            x = x[kv_heads[0]:kv_heads[-1] + 1]
        h.update(name.encode())
        h.update(np.ascontiguousarray(x).tobytes())
    return h.hexdigest()


def _lse_job(args):
    g0, g1, rows = args
    d, r = _D["d"], _D["r"]
    G = r.Hq // r.Hkv
    h0, h1 = g0 // G, (g1 - 1) // G + 1
    Ks = d["Kself"][h0:h1] if "Kself" in d else None
    chunk = r.self_chunk if r.mask == "repeat" else 0
    out = oracle.lse(d["Q"][g0:g1], d["Kctx"][h0:h1], Ks, d["scale"], r.mask, chunk, rows=rows)
    return g0, rows, out


def _score_job(args):
    h, rows, lse_rows, window = args
    d, r = _D["d"], _D["r"]
    G = r.Hq // r.Hkv
    Q = d["Q"][h * G:(h + 1) * G, rows[0]:rows[-1] + 1]
    vn = d["vnorm"][h:h + 1] if "vnorm" in d else None
    hn = d["hnorm"][rows[0]:rows[-1] + 1] if "hnorm" in d else None
    if r.mask == "repeat":
        return h, oracle.max_scores(Q, d["Kctx"][h:h + 1], lse_rows, d["scale"], 1, vnorm=vn, hnorm=hn)[0]
    raise ValueError("future mass is computed over whole rows below")


def _sum_job(args):
    h, lse_h, window = args
    d, r = _D["d"], _D["r"]
    G = r.Hq // r.Hkv
    vn = d["vnorm"][h:h + 1] if "vnorm" in d else None
    hn = d["hnorm"] if "hnorm" in d else None
    return h, oracle.future_mass(d["Q"][h * G:(h + 1) * G], d["Kctx"][h:h + 1], lse_h, d["scale"], window, 1,
                                 vnorm=vn, hnorm=hn)[0]


def make(name, procs):
    wl = BY_NAME[name]
    r = wl.recipe
    G = r.Hq // r.Hkv
    heads = HEADS[name]
    t0 = time.time()
    d = synth.draw(r, wl.seed)
    _D["d"], _D["r"] = d, r
    g_lo, g_hi = heads[0] * G, (heads[-1] + 1) * G
    n_q = r.n_q
    # LSE: every query row of the covered query heads, split by row ranges
    step = max(256, -(-n_q // (procs * 2)) // 256 * 256)
    jobs = [(g, g + 1, np.arange(j0, min(j0 + step, n_q))) for g in range(g_lo, g_hi) for j0 in range(0, n_q, step)]
    lse = np.empty((g_hi - g_lo, n_q))
    ctx = mp.get_context("fork")
    with ctx.Pool(procs) as pool:
        for g0, rows, out in pool.imap_unordered(_lse_job, jobs):
            lse[g0 - g_lo, rows] = out[0]
        print(f"[{name}] lse done in {time.time() - t0:.0f} s", flush=True)
        scores = np.zeros((len(heads), r.n_ctx))
        if wl.score_mode == "sum":
            sjobs = [(h, lse[(h - heads[0]) * G:(h - heads[0] + 1) * G], wl.window) for h in heads]
            for h, t in pool.imap_unordered(_sum_job, sjobs):
                scores[h - heads[0]] = t
        else:
            sjobs = []
            for h in heads:
                gl = (h - heads[0]) * G
                for j0 in range(0, n_q, step):
                    rows = np.arange(j0, min(j0 + step, n_q))
                    sjobs.append((h, rows, lse[gl:gl + G, rows], wl.window))
            for h, s in pool.imap_unordered(_score_job, sjobs):
                scores[h - heads[0]] = np.maximum(scores[h - heads[0]], s)
    print(f"[{name}] scores done in {time.time() - t0:.0f} s", flush=True)
    out = os.path.join(HERE, f"{name}.npz")
    np.savez_compressed(out, lse=lse.astype(np.float32), scores=scores.astype(np.float32),
                        kv_heads=np.array(heads, dtype=np.int64), seed=np.int64(wl.seed),
                        input_sha256=np.array(input_hash(d, heads, G)))
    print(f"[{name}] wrote {out} ({os.path.getsize(out)} bytes)", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--procs", type=int, default=os.cpu_count() or 8)
    ap.add_argument("names", nargs="*", default=list(HEADS))
    a = ap.parse_args()
    for name in a.names:
        make(name, a.procs)


if __name__ == "__main__":
    main()
