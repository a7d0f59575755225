#!/usr/bin/env python3
"""Throughput of the scoring + eviction path on one MI355X.

Workload: one Qwen3-8B-shaped layer with a 32768-token context (Hq=32,
Hkv=8, D=128, bf16), KVzip+ scoring of the teacher-forced repeat in 16 chunks
of 2048 queries, then threshold eviction (tau = e^-6, window 128) with K/V
compaction. Inputs are seeded synthetic tensors, resident in HBM before the
timed region.

One step = kvscore_lse (all chunks in one call) + kvscore_max + kv_evict.
value = context keys scored per second over whole steps (Hkv * n_ctx / step).

Also reported: per-kernel times (HIP events on the launch stream); the
roofline of the step's dominant kernel, the LSE pass (TFLOP/s against the
bf16 MFMA peak, and against a dense bf16 GEMM timed in the same run), with
its exp2 rate; the score pass's TFLOP/s; eviction GB/s with cold caches
against HBM peak and against a plain device copy of the same bytes timed in
the same run; the CPU oracle timed on a bounded sample of the same workload
and on whole small layers; and (under "adjacent", timed after the step and
not part of it) the attention forward that also returns O, the value-norm
kernel that produces the vnorm input, decode attention of one new token per
query head over the cache this step compacted, and eviction with one
layer-wide top-k budget keeping as many rows as the step did.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--no-cpu-baseline]
    python bench.py --cpu-configs   # the oracle alone on whole layers (no GPU)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# v_exp_f32 issues at half rate: a wave64 instruction takes 8 cycles of a
# 16-lane SIMD, so 8 exp2 per cycle per SIMD; 256 CUs x 4 SIMDs at 2.4 GHz
PEAK_EXP2_PER_S = 256 * 4 * 8 * 2.4e9
METRIC = "keys scored/sec & score-pass TFLOP/s (MFMA util) at 32k ctx; evict GB/s"


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic(kernel_src: str, name: str):
    """HBM bytes per launch of a kernel from the counter runs kept in
    profiles/<name>, or None when the kernel source changed since they were
    taken."""
    p = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_sha256_16") != source_hash(kernel_src):
        return None
    return t.get("hbm_bytes_per_launch")


def host_cpu():
    """Cores this process may run on, the BLAS threads numpy uses, and the CPU model."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info

        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return cores, blas, model


def oracle_whole_layer(wl):
    """Wall seconds of the oracle over a whole workload: LSE, the score pass,
    then the selection and compaction of every keep fraction."""
    import oracle
    import synth

    r = wl.recipe
    d = synth.draw(r, wl.seed)
    t0 = time.perf_counter()
    if wl.score_mode == "sum":
        L = oracle.lse(d["Q"], d["Kctx"], None, d["scale"], "causal", 0)
        s = oracle.future_mass(d["Q"], d["Kctx"], L, d["scale"], wl.window, r.Hkv, vnorm=d.get("vnorm"),
                               hnorm=d.get("hnorm"))
    else:
        L = oracle.lse(d["Q"], d["Kctx"], d["Kself"], d["scale"], "repeat", r.self_chunk)
        s = oracle.max_scores(d["Q"], d["Kctx"], L, d["scale"], r.Hkv, vnorm=d.get("vnorm"), hnorm=d.get("hnorm"))
    sels = [dict(tau=wl.tau)] if wl.tau >= 0 else [dict(k=k) for k in wl.ks()]
    for sel in sels:
        kept = oracle.select(s, wl.window, **sel)
        oracle.compact(d["Kctx"], d["V"], kept)
    return time.perf_counter() - t0


def cpu_baseline(d, wl, n_heads_sample=1, n_chunks_sample=6, whole=()):
    """The oracle as it stands on a bounded sample: LSE + max score for one KV
    head's query heads over `n_chunks_sample` repeat chunks against the whole
    context, then selection + compaction of the full layer; scaled to the
    whole workload (an extrapolation, labelled as such). Also the oracle's
    wall time on the whole small layers in `whole`."""
    import oracle

    cores, blas, model = host_cpu()
    r = wl.recipe
    G, C = r.group, r.chunk
    hs = slice(0, n_heads_sample)
    gs = slice(0, n_heads_sample * G)
    qs = slice(0, n_chunks_sample * C)
    t0 = time.perf_counter()
    L = oracle.lse(d["Q"][gs, qs], d["Kctx"][hs], d["Kself"][hs, qs], d["scale"], "repeat", C)
    s = oracle.max_scores(d["Q"][gs, qs], d["Kctx"][hs], L, d["scale"], n_heads_sample,
                          vnorm=d["vnorm"][hs], hnorm=d["hnorm"][qs])
    t_score = time.perf_counter() - t0
    frac = (n_heads_sample / r.Hkv) * (n_chunks_sample * C / r.n_q)
    import synth

    sc = synth.evict_scores(wl.seed, r.Hkv, r.n_ctx)  # full-layer shape; selection cost is data-light
    t1 = time.perf_counter()
    kept = oracle.select(sc, wl.window, tau=wl.tau)
    oracle.compact(d["Kctx"], d["V"], kept)
    t_evict = time.perf_counter() - t1
    t_full = t_score / frac + t_evict
    out = {
        "value": r.Hkv * r.n_ctx / t_full,
        "unit": "keys/s",
        "cores": int(blas or cores),
        "kind": "oracle",
        "sample": (f"extrapolated: {n_heads_sample} KV head ({n_heads_sample * G} query heads) x {n_chunks_sample} "
                   f"of {r.n_q // C} repeat chunks against the full {r.n_ctx}-key context, LSE + max score "
                   f"({t_score:.1f} s, scaled x{1 / frac:.1f} = {t_score / frac:.0f} s for the layer); threshold "
                   f"selection + compaction of a whole layer's seeded scores ({t_evict:.2f} s)"),
        "host_cores": cores,
        "blas_threads": blas,
        "cpu_model": model,
        "layer_s_extrapolated": t_full,
    }
    if whole:
        out["whole_layer_s"] = {w.name: round(oracle_whole_layer(w), 3) for w in whole}
    return out


def cpu_configs(names):
    """--cpu-configs: the oracle alone on whole layers, one JSON line."""
    from synth.workloads import BY_NAME

    cores, blas, model = host_cpu()
    res = {}
    for n in names:
        _log(f"[cpu] oracle on the whole {n}")
        res[n] = round(oracle_whole_layer(BY_NAME[n]), 2)
        _log(f"[cpu] {n}: {res[n]} s")
    print(json.dumps({"kind": "oracle", "unit": "s per whole layer", "host_cores": cores, "blas_threads": blas,
                      "cpu_model": model, "whole_layer_s": res}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-adjacent", action="store_true",
                    help="skip the kernels timed after the step (attention forward with output)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (for scaling HBM byte counters)")
    ap.add_argument("--cpu-configs", nargs="*", default=None,
                    help="only time the CPU oracle on whole layers (default: the tiny, 2k and KVpop 16k layers)")
    ap.add_argument("--workload", default="qwen3-8b-layer-kvzip+-32k",
                    help="named synthetic layer (synth/workloads.py); the default is the 32k layer the "
                         "headline metric is quoted on")
    args = ap.parse_args()
    if args.cpu_configs is not None:
        cpu_configs(args.cpu_configs or ["tiny-kvzip-d64-256", "qwen2.5-1.5b-layer-kvzip+-2k",
                                         "kvpop-future-mass-causal-16k"])
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the scoring path shards by KV head "
              "with no communication, and this benchmark measures one GPU.", file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cache_eviction_lse_amd as kvs
    from kv_cache_eviction_lse_amd import accounting as acc
    import synth
    from synth.workloads import BY_NAME

    wl = BY_NAME[args.workload]
    sum_mode = wl.score_mode == "sum"

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        # a copy kernel of known size: 1 GiB read + 1 GiB written per dispatch
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30, "dispatches": 3}))
        return
    kvs.lib()  # fail loudly without the HIP library

    r = wl.recipe
    _log(f"[bench] drawing {wl.name}")
    t0 = time.perf_counter()
    d = synth.draw(r, wl.seed)
    _log(f"[bench] drawn in {time.perf_counter() - t0:.1f} s")

    def dev_bf16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()

    Q, K, V = dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), dev_bf16(d["V"])
    Ks = dev_bf16(d["Kself"]) if "Kself" in d else None
    vn = torch.from_numpy(d["vnorm"]).cuda() if "vnorm" in d else None
    hn = torch.from_numpy(d["hnorm"]).cuda() if "hnorm" in d else None
    scale = d["scale"]
    L = torch.empty((r.Hq, r.n_q), dtype=torch.float32, device="cuda")
    S = torch.empty((r.Hkv, r.n_ctx), dtype=torch.float32, device="cuda")
    sel = dict(tau=wl.tau) if wl.tau >= 0 else dict(k=wl.ks()[0])
    e = kvs.evict_desc(S, K, window=wl.window, **sel)
    cap = e.capacity
    outs = (torch.empty(cap, dtype=torch.int32, device="cuda"),
            torch.empty(r.Hkv + 1, dtype=torch.int64, device="cuda"),
            torch.empty((cap, r.D), dtype=torch.bfloat16, device="cuda"),
            torch.empty((cap, r.D), dtype=torch.bfloat16, device="cuda"))
    ws = torch.empty(max(kvs.evict_workspace_bytes(e), 256), dtype=torch.uint8, device="cuda")
    if args.no_cpu_baseline or sum_mode:
        del d["Q"]  # the host copy is needed only by the CPU baseline
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        if sum_mode:
            kvs.lse(Q, K, None, scale=scale, mask="causal", out=L)
        else:
            kvs.lse(Q, K, Ks, scale=scale, mask="repeat", chunk=r.chunk, out=L)
        if ev:
            ev[1].record(stream)
        if sum_mode:
            kvs.future_mass(Q, K, L, scale=scale, window=wl.window, vnorm=vn, hnorm=hn, out=S)
        else:
            kvs.max_scores(Q, K, L, scale=scale, vnorm=vn, hnorm=hn, out=S)
        if ev:
            ev[2].record(stream)
        kvs.evict(S, K, V, window=wl.window, workspace=ws, outputs=outs, **sel)
        if ev:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    per_step = {k: [a[i].elapsed_time(a[i + 1]) for a in evs] for i, k in enumerate(("lse", "score", "evict"))}
    t_lse = float(np.mean(per_step["lse"]))
    t_score = float(np.mean(per_step["score"]))
    t_evict = float(np.mean(per_step["evict"]))

    # Eviction with cold caches (not part of the step): before each
    # repetition a 512 MiB write pushes the scores and K/V out of L2 and the
    # Infinity Cache.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = []
    for i in range(10):
        flush.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kvs.evict(S, K, V, window=wl.window, workspace=ws, outputs=outs, **sel)
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))

    # Measured ceilings in the same run (not part of the step), from the
    # calibration kernels built beside the library:
    # * a plain copy of the eviction's byte volume (half read, half written)
    #   with 16-byte non-temporal accesses, the same cache flush before each
    #   repetition;
    # * MFMA chains alone at the LSE pass's occupancy (3 four-wave workgroups
    #   per CU), and the shader clock under that load.
    import ctypes

    from kv_cache_eviction_lse_amd import build as kbuild

    cal = ctypes.CDLL(kbuild.CALIB_LIB)
    cal.kvs_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    cal.kvs_calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    sptr = ctypes.c_void_p(stream.cuda_stream)
    offs_now = outs[1].cpu().numpy()
    ev_bytes_now = acc.evict_bytes(r.Hkv, r.n_ctx, int(offs_now[-1]), r.D)
    half = max(ev_bytes_now // 2 // 16 * 16, 16)
    csrc = torch.empty(half, dtype=torch.uint8, device="cuda").fill_(3)
    cdst = torch.empty_like(csrc)
    copy_ms = []
    for i in range(10):
        flush.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        assert cal.kvs_calib_copy(ctypes.c_void_p(csrc.data_ptr()), ctypes.c_void_p(cdst.data_ptr()), half, sptr) == 0
        e1.record(stream)
        torch.cuda.synchronize()
        copy_ms.append(e0.elapsed_time(e1))
    assert torch.equal(csrc[:4096], cdst[:4096])
    del csrc, cdst, flush
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    mf_blocks, mf_iters = 3 * n_cus, 2000
    sink = torch.empty(mf_blocks * 256, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    mf_ms = []
    for i in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        assert cal.kvs_calib_mfma(mf_iters, mf_blocks, ctypes.c_void_p(sink.data_ptr()),
                                  ctypes.c_void_p(clocks.data_ptr()), sptr) == 0
        e1.record(stream)
        torch.cuda.synchronize()
        if i:  # (the first run warms the clock)
            mf_ms.append(e0.elapsed_time(e1))
    cyc, ticks = (int(x) for x in clocks.cpu().tolist())
    clock_mhz = cyc * 100.0 / ticks if ticks > 0 else None  # real-time counter at 100 MHz
    mfma_tflops = mf_blocks * 4 * 2 * 8 * mf_iters * 32768 / (float(np.median(mf_ms)) * 1e-3) / 1e12
    copy_gbs = 2 * half / (float(np.median(copy_ms)) * 1e-3) / 1e9
    del sink, clocks

    # Adjacent kernels, timed after the step (not part of it): the attention
    # forward that returns O with the same LSE.
    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    adjacent = {}
    if not args.no_adjacent:
        Vs = dev_bf16(d["Vself"]) if "Vself" in d else None
        O = torch.empty_like(Q)
        L2 = torch.empty_like(L)
        if sum_mode:
            t_attn = timed(lambda: kvs.attention(Q, K, V, None, None, scale=scale, mask="causal", out=O, lse_out=L2))
        else:
            t_attn = timed(lambda: kvs.attention(Q, K, V, Ks, Vs, scale=scale, mask="repeat", chunk=r.chunk, out=O,
                                                 lse_out=L2))
        del O, L2, Vs
        if "WO" in d:
            WO = dev_bf16(d["WO"])
            vn_out = torch.empty((r.Hkv, r.n_ctx), dtype=torch.float32, device="cuda")
            t_vn = timed(lambda: kvs.value_norms(V, WO, out=vn_out))
            vn_flops = 2 * r.Hkv * r.n_ctx * r.D * d["WO"].shape[0]
            vn_tflops = vn_flops / (t_vn * 1e-3) / 1e12
            adjacent["value_norms"] = {"entry": "kvscore_vnorm", "ms": t_vn, "flops": vn_flops, "tflops": vn_tflops,
                                       "frac_of_bf16_peak": vn_tflops / PEAK_BF16_TFLOPS,
                                       "d_model": int(d["WO"].shape[0])}
            del WO, vn_out
        # decode over the cache this step compacted: one new token per query head
        Qd = Q[:, -1:, :].contiguous()
        dd = kvs.decode_desc(Qd, outs[2], r.Hkv, scale)
        dws = torch.empty(max(kvs.decode_workspace_bytes(dd), 16), dtype=torch.uint8, device="cuda")
        Od, Ld = torch.empty_like(Qd), torch.empty((r.Hq, 1), dtype=torch.float32, device="cuda")
        t_dec = timed(lambda: kvs.decode(Qd, outs[2], outs[3], outs[1], scale=scale, workspace=dws, out=Od, lse_out=Ld),
                      reps=20)
        del Qd, dws, Od, Ld
        # the same number of kept rows under one layer-wide top-k budget
        kept_now = int(outs[1][-1].item())
        w_eff = min(wl.window, r.n_ctx)
        k_layer = max(kept_now - r.Hkv * w_eff, 0)
        lay_outs = tuple(torch.empty_like(t) for t in outs)
        el = kvs.evict_desc(S, K, window=wl.window, k=k_layer, scope="layer")
        lws = torch.empty(max(kvs.evict_workspace_bytes(el), 256), dtype=torch.uint8, device="cuda")
        t_lay = timed(lambda: kvs.evict(S, K, V, window=wl.window, k=k_layer, scope="layer", workspace=lws,
                                        outputs=lay_outs), reps=20)
        lay_total = int(lay_outs[1][-1].item())
        del lay_outs, lws
        # threshold pruning as tokens arrive (threshold workloads): the layer's
        # context goes into a stream cache in one call, then decoding steps of
        # one token per head, then decode attention over the stream cache
        if wl.tau >= 0:
            n_steps = 32
            cap = r.n_ctx + n_steps
            # (a first bulk call into a throwaway cache loads the kernels)
            warm = kvs.StreamCache(r.Hkv, r.D, cap, window=wl.window, tau=wl.tau)
            warm.append(S, K, V)
            del warm
            sc = kvs.StreamCache(r.Hkv, r.D, cap, window=wl.window, tau=wl.tau)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            sc.append(S, K, V)
            e1.record(stream)
            torch.cuda.synchronize()
            t_bulk = e0.elapsed_time(e1)
            live_bulk = int(sc.head_len.sum().item())
            s_new, K_new, V_new = S[:, :n_steps].contiguous(), K[:, :n_steps], V[:, :n_steps]
            steps_in = [(s_new[:, i:i + 1], K_new[:, i:i + 1], V_new[:, i:i + 1]) for i in range(n_steps)]
            # queue GPU work first so the appends run back to back at GPU speed
            # (the host enqueues them while the GPU is busy)
            torch.cuda._sleep(20_000_000)
            e0.record(stream)
            for a in steps_in:
                sc.append(*a)
            e1.record(stream)
            torch.cuda.synchronize()
            t_step = e0.elapsed_time(e1) / n_steps
            Qd = Q[:, -1:, :].contiguous()
            flat = sc.K.view(-1, r.D)
            sd = kvs.decode_desc(Qd, flat, r.Hkv, scale, head_stride_rows=cap)
            sws = torch.empty(max(kvs.decode_workspace_bytes(sd), 16), dtype=torch.uint8, device="cuda")
            Od, Ld = torch.empty_like(Qd), torch.empty((r.Hq, 1), dtype=torch.float32, device="cuda")
            t_sdec = timed(lambda: sc.decode(Qd, scale=scale, workspace=sws, out=Od, lse_out=Ld), reps=20)
            live = int(sc.head_len.sum().item())
            adjacent["stream"] = {"entry": "kv_stream_append, kvscore_decode over its head regions",
                                  "bulk_tokens_per_head": r.n_ctx, "bulk_ms": t_bulk,
                                  "live_rows_after_bulk": live_bulk, "equals_evict_kept_rows": live_bulk == kept_now,
                                  "step_tokens_per_head": 1, "step_us": t_step * 1e3,
                                  "decode_ms": t_sdec, "decode_rows": live,
                                  "decode_gbs": live * 4 * r.D / (t_sdec * 1e-3) / 1e9}
            del sc, s_new, steps_in, Qd, sws, Od, Ld
    offs = outs[1].cpu().numpy()
    kept = np.diff(offs)
    kept_total = int(offs[-1])
    if sum_mode:
        score_flops = acc.flops(acc.sum_pairs(r.Hq, r.n_ctx, wl.window), r.D)
        lse_flops = acc.flops(acc.lse_pairs(r.Hq, r.n_ctx, r.n_q, "causal"), r.D)
    else:
        score_flops = acc.flops(acc.max_pairs(r.Hq, r.n_ctx, r.n_q), r.D)
        lse_flops = acc.flops(acc.lse_pairs(r.Hq, r.n_ctx, r.n_q, "repeat", r.self_chunk), r.D)
    ev_bytes = acc.evict_bytes(r.Hkv, r.n_ctx, kept_total, r.D)
    score_tflops = score_flops / (t_score * 1e-3) / 1e12
    lse_tflops = lse_flops / (t_lse * 1e-3) / 1e12
    evict_gbs = ev_bytes / (t_evict * 1e-3) / 1e9
    keys_per_s = r.Hkv * r.n_ctx / (ms_per_step * 1e-3)

    csrc_dir = os.path.join(ROOT, "kv_cache_eviction_lse_amd", "csrc")
    headline = wl is BY_NAME["qwen3-8b-layer-kvzip+-32k"]
    lse_traffic = stored_traffic(os.path.join(csrc_dir, "lse.hip"), "lse_qwen3-8b-32k_traffic.json") \
        if headline else None
    score_traffic = stored_traffic(os.path.join(csrc_dir, "score.hip"), "score_max_qwen3-8b-32k_traffic.json") \
        if headline else None
    lse_pairs = lse_flops / (2 * r.D)
    cold_ms = float(np.median(cold))
    cold_gbs = ev_bytes / (cold_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": keys_per_s,
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "Hq": r.Hq, "Hkv": r.Hkv, "head_dim": r.D, "n_ctx": r.n_ctx,
                   "n_q": r.n_q, "chunk": r.self_chunk, "mask": r.mask,
                   "selection": ({"tau": wl.tau} if wl.tau >= 0 else {"k": wl.ks()[0]}),
                   "window": wl.window, "parallelism": "single GPU"},
        # the step's dominant kernel: the LSE pass
        "roofline": {"bound": "mfma", "achieved": lse_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": lse_tflops / PEAK_BF16_TFLOPS, "traffic": lse_traffic,
                     "kernel": "LSE pass (kvscore_lse)",
                     "measured_peak": mfma_tflops, "frac_of_measured": lse_tflops / mfma_tflops},
        "kernels_ms": {"lse": t_lse, "score": t_score, "evict": t_evict},
        "kernels_ms_median": {k: float(np.median(v)) for k, v in per_step.items()},
        "kernels_ms_min": {k: float(np.min(v)) for k, v in per_step.items()},
        "lse_pass": {"tflops": lse_tflops, "frac_of_bf16_peak": lse_tflops / PEAK_BF16_TFLOPS, "flops": lse_flops,
                     "exp2_per_s": lse_pairs / (t_lse * 1e-3),
                     "exp2_frac_of_peak": lse_pairs / (t_lse * 1e-3) / PEAK_EXP2_PER_S},
        "score_pass": {"tflops": score_tflops, "flops": score_flops, "frac_of_bf16_peak": score_tflops / PEAK_BF16_TFLOPS,
                       "frac_of_measured": score_tflops / mfma_tflops, "traffic": score_traffic,
                       "kernel": "kvscore_futuremass" if sum_mode else "kvscore_max"},
        "ceilings": {"mfma_bf16_tflops": mfma_tflops, "clock_mhz_under_mfma": clock_mhz,
                     "copy_gbs_cold": copy_gbs, "copy_bytes": 2 * half,
                     "kernels": "kvs_calib_mfma (MFMA chains alone, 3 four-wave workgroups per CU), "
                                "kvs_calib_copy (16-byte non-temporal copy, caches flushed first)"},
        # HBM fraction from the cold-cache repetitions (scores, K and V pushed out
        # of L2 and the Infinity Cache first); the in-step (warm) rate beside it
        "evict": {"gbs": cold_gbs, "frac_of_hbm_peak": cold_gbs / PEAK_HBM_GBS,
                  "frac_of_copy": cold_gbs / copy_gbs, "bytes": ev_bytes,
                  "warm_gbs": evict_gbs, "warm_frac_of_hbm_peak": evict_gbs / PEAK_HBM_GBS,
                  "kept_per_head": kept.tolist(),
                  "compression_per_head": [round(acc.compression_ratio(int(x), r.n_ctx), 4) for x in kept],
                  "cold_caches": {"median_ms": float(np.median(cold)), "min_ms": float(np.min(cold)), "reps": len(cold),
                                  "gbs_median": ev_bytes / (float(np.median(cold)) * 1e-3) / 1e9}},
    }
    if not args.no_cpu_baseline and not sum_mode:
        _log("[bench] timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(d, wl, whole=(BY_NAME["tiny-kvzip-d64-256"],
                                                         BY_NAME["qwen2.5-1.5b-layer-kvzip+-2k"]))
    if not args.no_adjacent:
        attn_tflops = 2 * lse_flops / (t_attn * 1e-3) / 1e12
        attn_traffic = stored_traffic(os.path.join(csrc_dir, "attn.hip"), "attn_qwen3-8b-32k_traffic.json") \
            if wl.name == "qwen3-8b-layer-kvzip+-32k" else None
        adjacent["attention"] = {"entry": "kvscore_attention", "ms": t_attn, "flops": 2 * lse_flops,
                                 "tflops": attn_tflops, "frac_of_bf16_peak": attn_tflops / PEAK_BF16_TFLOPS,
                                 "traffic": attn_traffic}
        dec_bytes = kept_total * 2 * r.D * 2 + r.Hq * r.D * 2 * 2  # kept K and V rows, plus Q and O
        adjacent["decode"] = {"entry": "kvscore_decode", "ms": t_dec, "queries_per_head": 1, "rows": kept_total,
                              "bytes": dec_bytes, "gbs": dec_bytes / (t_dec * 1e-3) / 1e9,
                              "frac_of_hbm_peak": dec_bytes / (t_dec * 1e-3) / 1e9 / PEAK_HBM_GBS}
        lay_bytes = acc.evict_bytes(r.Hkv, r.n_ctx, lay_total, r.D)
        adjacent["evict_layer_budget"] = {"entry": "kv_evict (scope layer)", "ms": t_lay, "k": k_layer,
                                          "kept_rows": lay_total, "bytes": lay_bytes,
                                          "gbs": lay_bytes / (t_lay * 1e-3) / 1e9,
                                          "frac_of_hbm_peak": lay_bytes / (t_lay * 1e-3) / 1e9 / PEAK_HBM_GBS}
        out["adjacent"] = adjacent
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
