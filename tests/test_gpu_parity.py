"""GPU path against the CPU oracle, element by element, on seeded inputs small
enough for the oracle (several tiles, ragged tails, odd GQA groups, D = 64
and 128, chunk edges, degenerate cases). Every call goes through the C ABI."""
import numpy as np
import pytest

import oracle
import synth
from synth.workloads import TINY_KVZIP, QWEN25_1P5B_2K

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_eviction_lse_amd as kvs  # noqa: E402
from gpu_util import (check_kept, check_lse, check_rows, check_scores, dev_bf16, dev_f32, host,  # noqa: E402
                      host_bits, kept_from_gpu, say)


def _draw(seed, **kw):
    return synth.draw(synth.Recipe(**kw), seed)


def _gpu_lse(d, mask, chunk):
    r = d["recipe"]
    Ks = dev_bf16(d["Kself"]) if mask == "repeat" else None
    out = kvs.lse(dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), Ks, scale=d["scale"], mask=mask, chunk=chunk)
    torch.cuda.synchronize()
    return host(out)


LSE_CASES = [
    # name, recipe kwargs, mask, chunk
    ("repeat-g2-d64", dict(Hq=4, Hkv=2, D=64, n_ctx=256, n_q=256, scale=1.0, q_prescale=0.125), "repeat", 256),
    ("repeat-g5-ragged-chunks", dict(Hq=10, Hkv=2, D=128, n_ctx=1000, n_q=700, lowrank_rank=8,
                                      lowrank_scale=2.0), "repeat", 300),
    ("repeat-g6-chunk1", dict(Hq=6, Hkv=1, D=128, n_ctx=77, n_q=130), "repeat", 1),
    ("repeat-no-context", dict(Hq=4, Hkv=1, D=64, n_ctx=0, n_q=200), "repeat", 64),
    ("repeat-one-query", dict(Hq=8, Hkv=8, D=128, n_ctx=513, n_q=1), "repeat", 1),
    ("repeat-chunk-gt-nq", dict(Hq=3, Hkv=3, D=128, n_ctx=40, n_q=97), "repeat", 4096),
    ("causal-g6-ragged", dict(Hq=6, Hkv=1, D=128, n_ctx=777, n_q=777, mask="causal"), "causal", 0),
    ("causal-g4-sinks-d64", dict(Hq=8, Hkv=2, D=64, n_ctx=1000, n_q=1000, mask="causal", sinks=4), "causal", 0),
    ("causal-tiny", dict(Hq=2, Hkv=1, D=128, n_ctx=3, n_q=3, mask="causal"), "causal", 0),
    # the cases above have fewer workgroups than CUs, so they take the pass's
    # key-split form; these two are large enough (256 workgroups of 8
    # subtiles) for the form that shares key tiles through LDS
    ("repeat-lds-form-ragged", dict(Hq=32, Hkv=8, D=128, n_ctx=700, n_q=2048, lowrank_rank=8,
                                    lowrank_scale=2.0), "repeat", 1000),
    ("causal-lds-form", dict(Hq=32, Hkv=8, D=128, n_ctx=2048, n_q=2048, mask="causal", sinks=4), "causal", 0),
    # LDS form with every tile count from 1 up (8 query heads per KV head: a
    # workgroup serves one 32-position block, so block b sees b + 1 key
    # tiles), for both head dims; and three tiles per workgroup with a
    # partial context tile (20 context keys, chunks of 32)
    ("causal-lds-form-g8", dict(Hq=64, Hkv=8, D=128, n_ctx=1024, n_q=1024, mask="causal"), "causal", 0),
    ("causal-lds-form-g8-d64", dict(Hq=64, Hkv=8, D=64, n_ctx=1024, n_q=1024, mask="causal"), "causal", 0),
    ("repeat-lds-form-short-context", dict(Hq=32, Hkv=8, D=128, n_ctx=20, n_q=2048), "repeat", 32),
]


@pytest.mark.parametrize("name,kw,mask,chunk", LSE_CASES, ids=[c[0] for c in LSE_CASES])
def test_lse_parity(name, kw, mask, chunk):
    kw = dict(kw)
    kw.setdefault("mask", mask)
    kw["chunk"] = chunk
    d = _draw(101, **kw)
    say(f"[lse] {name}")
    g = _gpu_lse(d, mask, chunk)
    ref = oracle.lse(d["Q"], d["Kctx"], d.get("Kself"), d["scale"], mask, chunk)
    check_lse(g, ref, name)


def test_lse_long_context_does_not_drift():
    """~3000 key tiles per query: the running sum must not pick up a per-tile
    rescaling error (the error stays far below the 1e-3 parity bar)."""
    r = synth.Recipe(Hq=4, Hkv=1, D=128, n_ctx=100000, n_q=64, chunk=64, lowrank_rank=8, lowrank_scale=2.0)
    d = synth.draw(r, 111)
    say("[lse] long-context drift")
    g = _gpu_lse(d, "repeat", 64)
    ref = oracle.lse(d["Q"], d["Kctx"], d["Kself"], d["scale"], "repeat", 64)
    err = check_lse(g, ref, "long-context")
    assert err <= 1e-4, f"LSE error {err:.2e} grows with context length"


MAX_CASES = [
    ("tiny-kvzip", TINY_KVZIP.recipe, False),
    ("g5-ragged-weighted", synth.Recipe(Hq=10, Hkv=2, D=128, n_ctx=1000, n_q=700, chunk=300, lowrank_rank=8,
                                        lowrank_scale=2.0, value_norms=True), True),
    ("g6-d64-weighted", synth.Recipe(Hq=6, Hkv=1, D=64, n_ctx=1537, n_q=333, chunk=128, value_norms=True,
                                     d_hidden=384), True),
    ("mha-single-query", synth.Recipe(Hq=2, Hkv=2, D=128, n_ctx=100, n_q=1, chunk=1), False),
]


@pytest.mark.parametrize("name,recipe,weighted", MAX_CASES, ids=[c[0] for c in MAX_CASES])
def test_max_score_parity(name, recipe, weighted):
    d = synth.draw(recipe, 202)
    say(f"[max] {name}")
    Q, K, Ks = dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), dev_bf16(d["Kself"])
    chunk = recipe.self_chunk
    L = kvs.lse(Q, K, Ks, scale=d["scale"], mask="repeat", chunk=chunk)
    vn = dev_f32(d["vnorm"]) if weighted else None
    hn = dev_f32(d["hnorm"]) if weighted else None
    s = kvs.max_scores(Q, K, L, scale=d["scale"], vnorm=vn, hnorm=hn)
    torch.cuda.synchronize()
    ref_L = oracle.lse(d["Q"], d["Kctx"], d["Kself"], d["scale"], "repeat", chunk)
    check_lse(host(L), ref_L, name)
    ref = oracle.max_scores(d["Q"], d["Kctx"], ref_L, d["scale"], recipe.Hkv,
                            vnorm=d.get("vnorm") if weighted else None, hnorm=d.get("hnorm") if weighted else None)
    check_scores(host(s), ref, name)


def test_max_score_given_lse_input():
    """The score pass alone, on a stand-in normaliser that no attention produced."""
    r = synth.Recipe(Hq=8, Hkv=2, D=128, n_ctx=700, n_q=900, chunk=900, lowrank_rank=8, lowrank_scale=2.0,
                     value_norms=True)
    d = synth.draw(r, 303)
    lse_in = synth.lse_values(303, r.Hq, r.n_q, 6.0, 9.0)
    say("[max] given-lse")
    s = kvs.max_scores(dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), dev_f32(lse_in), scale=d["scale"],
                       vnorm=dev_f32(d["vnorm"]), hnorm=dev_f32(d["hnorm"]))
    torch.cuda.synchronize()
    ref = oracle.max_scores(d["Q"], d["Kctx"], lse_in, d["scale"], r.Hkv, vnorm=d["vnorm"], hnorm=d["hnorm"])
    check_scores(host(s), ref, "given-lse")


@pytest.mark.parametrize("D", [128, 64])
def test_max_score_long_context_form(D):
    """Enough 768-key blocks (>= 4 rounds of workgroups) for the score pass's
    long-context form (3 resident key subtiles per wave, 64-row query tiles),
    with a ragged last key block and a ragged query tile, on a stand-in
    normaliser."""
    r = synth.Recipe(Hq=64, Hkv=64, D=D, n_ctx=12289, n_q=100, chunk=100)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert -(-r.n_ctx // 768) * r.Hkv >= 4 * cus, "sized for the long-context form on this GPU"
    d = synth.draw(r, 305)
    lse_in = synth.lse_values(305, r.Hq, r.n_q, 6.0, 9.0)
    hn = synth.lse_values(306, 1, r.n_q, 1.0, 3.0)[0].astype(np.float32)
    say(f"[max] long-context form D={D}")
    s = kvs.max_scores(dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), dev_f32(lse_in), scale=d["scale"], hnorm=dev_f32(hn))
    torch.cuda.synchronize()
    ref = oracle.max_scores(d["Q"], d["Kctx"], lse_in, d["scale"], r.Hkv, hnorm=hn)
    check_scores(host(s), ref, f"long-context D={D}")


def test_max_score_accumulate_over_chunks_equals_one_call():
    r = synth.Recipe(Hq=8, Hkv=2, D=128, n_ctx=600, n_q=1000, chunk=400, value_norms=True)
    d = synth.draw(r, 404)
    Q, K, Ks = dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), dev_bf16(d["Kself"])
    L = kvs.lse(Q, K, Ks, scale=d["scale"], mask="repeat", chunk=400)
    vn, hn = dev_f32(d["vnorm"]), dev_f32(d["hnorm"])
    say("[max] accumulate")
    one = kvs.max_scores(Q, K, L, scale=d["scale"], vnorm=vn, hnorm=hn)
    acc = torch.zeros_like(one)
    for c0 in range(0, 1000, 400):
        c1 = min(c0 + 400, 1000)
        kvs.max_scores(Q[:, c0:c1], K, L[:, c0:c1].contiguous(), scale=d["scale"], vnorm=vn,
                       hnorm=hn[c0:c1].contiguous(), out=acc, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(one, acc)


def test_max_score_no_queries_gives_zero():
    r = synth.Recipe(Hq=4, Hkv=2, D=128, n_ctx=300, n_q=0, chunk=1)
    d = synth.draw(r, 505)
    Q = torch.empty((4, 0, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full((2, 300), 7.0, device="cuda")
    kvs.max_scores(Q, dev_bf16(d["Kctx"]), torch.empty((4, 0), device="cuda"), scale=d["scale"], out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


SUM_CASES = [
    ("g4-w128-sinks", synth.Recipe(Hq=8, Hkv=2, D=128, n_ctx=1500, n_q=1500, mask="causal", sinks=4), 128, False),
    ("g5-w0-weighted", synth.Recipe(Hq=5, Hkv=1, D=128, n_ctx=1100, n_q=1100, mask="causal", value_norms=True,
                                    d_hidden=640), 0, True),
    ("g2-d64-w37", synth.Recipe(Hq=4, Hkv=2, D=64, n_ctx=2100, n_q=2100, mask="causal"), 37, False),
    ("window-covers-all", synth.Recipe(Hq=4, Hkv=2, D=128, n_ctx=300, n_q=300, mask="causal"), 300, False),
    ("short", synth.Recipe(Hq=2, Hkv=1, D=128, n_ctx=5, n_q=5, mask="causal"), 1, False),
]


@pytest.mark.parametrize("name,recipe,window,weighted", SUM_CASES, ids=[c[0] for c in SUM_CASES])
def test_future_mass_parity(name, recipe, window, weighted):
    d = synth.draw(recipe, 606)
    say(f"[sum] {name}")
    Q, K = dev_bf16(d["Q"]), dev_bf16(d["Kctx"])
    L = kvs.lse(Q, K, None, scale=d["scale"], mask="causal")
    vn = dev_f32(d["vnorm"]) if weighted else None
    hn = dev_f32(d["hnorm"]) if weighted else None
    t = kvs.future_mass(Q, K, L, scale=d["scale"], window=window, vnorm=vn, hnorm=hn)
    torch.cuda.synchronize()
    ref_L = oracle.lse(d["Q"], d["Kctx"], None, d["scale"], "causal", 0)
    check_lse(host(L), ref_L, name)
    ref = oracle.future_mass(d["Q"], d["Kctx"], ref_L, d["scale"], window, recipe.Hkv,
                             vnorm=d.get("vnorm") if weighted else None, hnorm=d.get("hnorm") if weighted else None)
    check_scores(host(t), ref, name)
    if window >= recipe.n_ctx:
        assert np.all(host(t) == 0)


def test_future_mass_conserves_mass_at_window_zero():
    r = synth.Recipe(Hq=8, Hkv=2, D=128, n_ctx=3000, n_q=3000, mask="causal", sinks=4)
    d = synth.draw(r, 707)
    Q, K = dev_bf16(d["Q"]), dev_bf16(d["Kctx"])
    L = kvs.lse(Q, K, None, scale=d["scale"], mask="causal")
    t = kvs.future_mass(Q, K, L, scale=d["scale"], window=0)
    tot = host(t).astype(np.float64).sum(axis=1)
    assert np.allclose(tot, 4 * 3000, rtol=1e-4)


def test_future_mass_sentinel_window_gives_zero():
    """A window far past T (a sentinel such as 2**62) is the same as T: every
    key is still inside it, so every target is 0 (and no row before the
    first is ever read)."""
    r = synth.Recipe(Hq=8, Hkv=2, D=128, n_ctx=3000, n_q=3000, mask="causal")
    d = synth.draw(r, 709)
    Q, K = dev_bf16(d["Q"]), dev_bf16(d["Kctx"])
    L = kvs.lse(Q, K, None, scale=d["scale"], mask="causal")
    for w in (2 ** 62, 2 ** 63 - 1, 3000, 2999):
        say(f"[sum] window {w}")
        t = kvs.future_mass(Q, K, L, scale=d["scale"], window=w)
        torch.cuda.synchronize()
        ht = host(t)
        if w >= 3000:
            assert np.all(ht == 0), w
        else:
            # only key 0 leaves the window (query 2999 counts it)
            assert np.all(ht[:, 1:] == 0) and np.all(ht[:, 0] > 0), w


def test_future_mass_is_deterministic():
    """Few key blocks: the query rows of each block pair are split in two and
    added atomically; repeated calls must still give identical bits."""
    r = synth.Recipe(Hq=8, Hkv=2, D=128, n_ctx=4100, n_q=4100, mask="causal", value_norms=True)
    d = synth.draw(r, 708)
    Q, K = dev_bf16(d["Q"]), dev_bf16(d["Kctx"])
    L = kvs.lse(Q, K, None, scale=d["scale"], mask="causal")
    vn, hn = dev_f32(d["vnorm"]), dev_f32(d["hnorm"])
    say("[sum] deterministic")
    outs = [kvs.future_mass(Q, K, L, scale=d["scale"], window=128, vnorm=vn, hnorm=hn) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(outs[0].view(torch.int32), o.view(torch.int32))


# ---------------------------------------------------------------- eviction

def _evict_case(seed, Hkv, n, D, **kw):
    s = synth.evict_scores(seed, Hkv, n, tie_frac=0.1, zero_frac=0.02)
    K = synth.normal_bf16(seed, 90, (Hkv, n, D))
    V = synth.normal_bf16(seed, 91, (Hkv, n, D))
    return s, K, V


EVICT_CASES = [
    # name, Hkv, n, D, window, k, tau
    ("topk-multiblock", 3, 5000, 128, 128, 1000, None),
    ("topk-one-block", 2, 700, 64, 32, 64, None),
    ("topk-k0", 2, 3000, 128, 16, 0, None),
    ("topk-keep-all", 2, 3000, 128, 16, 5000, None),
    ("topk-window-covers", 1, 100, 128, 200, 10, None),
    ("topk-k-equals-cand-minus-1", 2, 2049, 128, 1, 2047, None),
    ("topk-no-window", 8, 4096, 128, 0, 1024, None),
    ("tau", 4, 9000, 128, 128, None, float(np.exp(-6.0))),
    ("tau-zero", 2, 3000, 64, 8, None, 0.0),
    ("tau-inf", 2, 3000, 128, 8, None, float("inf")),
    ("empty", 2, 0, 128, 8, 5, None),
    # grid path: thresholds, layer budgets and heads past the long-head
    # path; per-head top-k with at most 16384 candidates per head: one
    # workgroup per head selects in LDS; above that, the long-head path
    ("many-heads-topk", 4097, 100, 64, 10, 30, None),
    ("many-heads-tau", 300, 700, 64, 16, None, float(np.exp(-6.0))),
    ("long-heads-topk", 2, 140000, 64, 128, 35000, None),
    ("topk-head-path-largest", 3, 16384 + 64, 128, 64, 4000, None),
    ("topk-grid-path-smallest", 3, 16385 + 64, 64, 64, 4000, None),
    ("topk-head-path-top1", 2, 16384, 128, 0, 1, None),
    ("topk-head-path-k-cand-minus-1", 2, 16384, 64, 0, 16383, None),
    ("keep-all-head-path", 3, 9000, 64, 16, 20000, None),
    ("window-only-head-path", 3, 9000, 64, 16, 0, None),
    # window keys spanning many wave segments, candidates ending on a segment
    # edge (16 segments of 64 * ceil(n / 1024) positions), one candidate
    ("topk-head-wide-window", 2, 10000, 64, 9000, 300, None),
    ("topk-head-segment-edge", 2, 4096 + 100, 128, 100, 1000, None),
    ("topk-head-one-candidate", 2, 129, 128, 128, 1, None),
    # the per-head path splits a head's output rows over one workgroup per
    # 128 rows (at most 64, and at most about 512 workgroups in all): rows
    # on an exact multiple of 128, one row past it, the cap for many heads
    # (70 heads: 8 workgroups each), and window rows split over workgroups
    ("topk-head-rows-256", 2, 1000, 128, 0, 256, None),
    ("topk-head-rows-257", 2, 1000, 64, 0, 257, None),
    ("topk-head-70-heads", 70, 3000, 64, 40, 2900, None),
    ("topk-head-window-split", 1, 2000, 128, 300, 1, None),
    # small outputs: several key blocks per head with few kept rows, and
    # threshold mode on a short layer (its capacity is every token)
    ("topk-write-copies-rows", 4, 5000, 64, 8, 20, None),
    ("tau-write-copies-rows", 2, 100, 64, 4, None, float(np.exp(-6.0))),
    ("long-heads-tau", 2, 140000, 64, 128, None, float(np.exp(-6.0))),
    # long-head path (per-head top-k, 16384 < candidates <= 524288): candidates
    # ending off a 4-key boundary, a wide window, top-1 and k = candidates - 1,
    # a head count that is not a multiple of 8, the largest such head and
    # one past it (grid path)
    ("long-topk-ragged-tail", 3, 70001, 128, 0, 20000, None),
    ("long-topk-wide-window", 2, 40000, 64, 20000, 10000, None),
    ("long-topk-top1", 2, 30000, 64, 5, 1, None),
    ("long-topk-cand-minus-1", 2, 30000, 64, 5, 29994, None),
    ("long-topk-12-heads", 12, 20000, 128, 64, 5000, None),
    ("long-topk-largest", 1, 524288 + 128, 64, 128, 100000, None),
    ("long-topk-past-largest", 1, 524289 + 128, 64, 128, 100000, None),
]


def _tie_heavy_scores(kind, Hkv, n, seed):
    rng = np.random.default_rng(seed)
    if kind == "constant":  # every candidate ties: lowest positions win
        return np.full((Hkv, n), 0.25, dtype=np.float32)
    if kind == "three-values":  # huge buckets at the k-th key
        return rng.choice(np.array([0.1, 0.2, 0.3], dtype=np.float32), size=(Hkv, n))
    if kind == "one-octave":  # every key shares the top 11 bits, many share 16
        return (0.5 + 0.5 * rng.random((Hkv, n))).astype(np.float32)
    if kind == "nan-heavy":  # half NaN, NaN ranks below every number
        s = rng.random((Hkv, n)).astype(np.float32)
        s[:, ::2] = np.nan
        return s
    if kind == "signed":  # negative and positive scores, -0 and +0
        s = rng.standard_normal((Hkv, n)).astype(np.float32)
        s[:, ::7] = -0.0
        s[:, 3::7] = 0.0
        return s
    raise ValueError(kind)


TIE_CASES = [
    # kind, Hkv, n, D, window, k (tau for threshold mode)
    ("constant", 2, 40000, 64, 64, 10000, None),
    ("constant", 2, 3000, 64, 8, None, 0.25),
    ("constant", 3, 1000, 128, 0, 200, None),  # ties across the 128-row split of the per-head path
    ("three-values", 3, 50000, 64, 100, 20000, None),
    ("one-octave", 2, 120000, 64, 128, 30000, None),
    ("one-octave", 2, 9000, 128, 16, 4000, None),
    ("nan-heavy", 2, 20000, 64, 32, 15000, None),
    ("nan-heavy", 2, 20000, 64, 32, None, 0.5),
    ("signed", 2, 70000, 64, 0, 35000, None),
    ("signed", 2, 70000, 64, 10, None, -0.0),
]


@pytest.mark.parametrize("kind,Hkv,n,D,window,k,tau", TIE_CASES,
                         ids=[f"{c[0]}-{'topk' if c[5] is not None else 'tau'}-{c[2]}" for c in TIE_CASES])
def test_evict_tie_heavy(kind, Hkv, n, D, window, k, tau):
    """Scores whose k-th key shares its top bits with very many others (the
    k-th key's 16-bit bucket overflows the LDS stash, or everything ties),
    NaN-heavy and signed scores: exactly the oracle's selection."""
    s = _tie_heavy_scores(kind, Hkv, n, 77)
    K = synth.normal_bf16(78, 90, (Hkv, n, D))
    V = synth.normal_bf16(78, 91, (Hkv, n, D))
    say(f"[evict] tie-heavy {kind} Hkv={Hkv} n={n} k={k} tau={tau}")
    kept, offs, Ko, Vo = kvs.evict(dev_f32(s), dev_bf16(K), dev_bf16(V), window=window, k=k, tau=tau)
    torch.cuda.synchronize()
    _check_evict_exact(kind, s, K, V, window, k, tau, kept, offs, Ko, Vo)


def _evict_special_scores(s):
    if s.shape[1] > 10:
        s[0, 3] = np.nan
        s[-1, 5] = -0.0
        s[-1, 6] = 0.0
        s[0, 7] = np.inf


def _check_evict_exact(name, s, K, V, window, k, tau, kept, offs, Ko, Vo):
    offs = host(offs)
    ref = oracle.select(s, window, k=k, tau=tau)
    gk = kept_from_gpu(host(kept), offs)
    for h in range(s.shape[0]):
        assert np.array_equal(gk[h], ref[h]), f"{name}: head {h} differs"
    Kr, Vr, offr = oracle.compact(K, V, ref)
    assert np.array_equal(offs, offr), f"{name}: head offsets differ"
    total = int(offs[-1])
    assert np.array_equal(host_bits(Ko)[:total], Kr) and np.array_equal(host_bits(Vo)[:total], Vr), \
        f"{name}: compacted rows differ"


@pytest.mark.parametrize("name,Hkv,n,D,window,k,tau", EVICT_CASES, ids=[c[0] for c in EVICT_CASES])
def test_evict_parity(name, Hkv, n, D, window, k, tau):
    s, K, V = _evict_case(808, Hkv, n, D)
    _evict_special_scores(s)
    say(f"[evict] {name}")
    kept, offs, Ko, Vo = kvs.evict(dev_f32(s), dev_bf16(K), dev_bf16(V), window=window, k=k, tau=tau)
    torch.cuda.synchronize()
    _check_evict_exact(name, s, K, V, window, k, tau, kept, offs, Ko, Vo)


def test_evict_long_head_strided_scores():
    """Long-head top-k reading its scores through a head stride that is not a
    multiple of 4 from a base that is not 16-byte aligned (element loads
    instead of 16-byte loads): exactly the oracle's selection."""
    Hkv, n, D, window, k = 3, 30001, 64, 17, 9000
    s, K, V = _evict_case(831, Hkv, n, D)
    _evict_special_scores(s)
    wide = np.zeros((Hkv, n + 2), dtype=np.float32)
    wide[:, 1:n + 1] = s
    sd = dev_f32(wide)[:, 1:n + 1]
    assert sd.stride(0) % 4 != 0 and sd.data_ptr() % 16 != 0
    say("[evict] long-head strided scores")
    kept, offs, Ko, Vo = kvs.evict(sd, dev_bf16(K), dev_bf16(V), window=window, k=k)
    torch.cuda.synchronize()
    _check_evict_exact("long-head-strided", s, K, V, window, k, None, kept, offs, Ko, Vo)


def test_evict_reuses_one_workspace():
    """One workspace (left uninitialised) through a sequence of calls of
    every mode and of different shapes (more blocks, then fewer): each call
    matches the oracle, whatever the calls before left in the workspace."""
    seq = [
        ("tau", 4, 9000, 128, 128, None, float(np.exp(-6.0))),
        ("tau-again", 4, 9000, 128, 128, None, float(np.exp(-6.0))),
        ("topk", 3, 5000, 128, 128, 1000, None),
        ("tau-more-blocks", 8, 20000, 64, 64, None, float(np.exp(-5.0))),
        ("window-only", 2, 3000, 128, 16, 0, None),
        ("tau-fewer-blocks", 2, 700, 128, 16, None, float(np.exp(-6.0))),
        ("keep-all", 3, 2000, 128, 16, 10 ** 6, None),
        ("long-topk", 2, 40000, 64, 64, 9000, None),
        ("long-topk-shorter", 2, 20000, 128, 64, 3000, None),
        ("tau-last", 4, 9000, 128, 128, None, float(np.exp(-7.0))),
    ]
    cases = []
    for i, (name, Hkv, n, D, window, k, tau) in enumerate(seq):
        s, K, V = _evict_case(820 + i, Hkv, n, D)
        _evict_special_scores(s)
        sd, Kd, Vd = dev_f32(s), dev_bf16(K), dev_bf16(V)
        cases.append((name, s, K, V, sd, Kd, Vd, window, k, tau))
    nbytes = max(kvs.evict_workspace_bytes(kvs.evict_desc(c[4], c[5], window=c[7], k=c[8], tau=c[9]))
                 for c in cases)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    for name, s, K, V, sd, Kd, Vd, window, k, tau in cases:
        say(f"[evict-reuse] {name}")
        kept, offs, Ko, Vo = kvs.evict(sd, Kd, Vd, window=window, k=k, tau=tau, workspace=ws)
        torch.cuda.synchronize()
        _check_evict_exact(name, s, K, V, window, k, tau, kept, offs, Ko, Vo)


def _sweep_case(i):
    """Seeded random eviction case i: shape, window, mode (per-head top-k,
    threshold or one layer budget) and score law (log-normal with ties and
    zeros, one octave, three values)."""
    rng = np.random.default_rng(5150 + i)
    Hkv = int(rng.integers(1, 13))
    n = int(np.exp(rng.uniform(0.0, np.log(20000.0))))
    n = min(n, 120000 // Hkv)
    D = int(rng.choice([64, 128]))
    window = int(rng.integers(0, n + 11)) if rng.random() < 0.3 else int(rng.integers(0, min(n, 512) + 1))
    mode = str(rng.choice(["topk", "topk", "tau", "layer"]))
    law = str(rng.choice(["lognormal", "lognormal", "octave", "three"]))
    if law == "lognormal":
        sc = synth.evict_scores(6000 + i, Hkv, n, tie_frac=float(rng.uniform(0, 0.3)), zero_frac=0.02)
    elif law == "octave":
        sc = (0.5 + 0.5 * rng.random((Hkv, n))).astype(np.float32)
    else:
        sc = rng.choice(np.array([0.1, 0.2, 0.3], dtype=np.float32), size=(Hkv, n))
    cand = max(n - window, 0)
    k = tau = None
    if mode == "tau":
        tau = float(np.quantile(sc, rng.uniform(0, 1))) if sc.size else 0.5
    elif mode == "layer":
        k = int(rng.integers(0, Hkv * cand + 2))
    else:
        k = int(rng.integers(0, cand + 2))
    return Hkv, n, D, window, mode, law, sc, k, tau


@pytest.mark.parametrize("i", range(40))
def test_evict_random_sweep(i):
    """Forty seeded random layers through both eviction paths and all modes:
    exactly the oracle's selection and compaction."""
    Hkv, n, D, window, mode, law, sc, k, tau = _sweep_case(i)
    K = synth.normal_bf16(7000 + i, 90, (Hkv, n, D))
    V = synth.normal_bf16(7000 + i, 91, (Hkv, n, D))
    name = f"sweep-{i} Hkv={Hkv} n={n} D={D} w={window} {mode} {law} k={k} tau={tau}"
    say(f"[evict] {name}")
    scope = "layer" if mode == "layer" else "head"
    kept, offs, Ko, Vo = kvs.evict(dev_f32(sc), dev_bf16(K), dev_bf16(V), window=window, k=k, tau=tau, scope=scope)
    torch.cuda.synchronize()
    offs = host(offs)
    ref = oracle.select(sc, window, k=k, tau=tau, scope=scope)
    gk = kept_from_gpu(host(kept), offs)
    for h in range(Hkv):
        assert np.array_equal(gk[h], ref[h]), f"{name}: head {h} differs"
    Kr, Vr, offr = oracle.compact(K, V, ref)
    assert np.array_equal(offs, offr), f"{name}: offsets differ"
    total = int(offs[-1])
    assert np.array_equal(host_bits(Ko)[:total], Kr) and np.array_equal(host_bits(Vo)[:total], Vr), name


def _long_sweep_case(i):
    """Seeded random per-head top-k layer i with 16,385-200,000 candidates per
    head (the long-head path): 1-12 heads, D = 64/128, windows up to 2048,
    k from 1 to all but one candidate, and log-normal (with ties and zeros),
    one-octave, three-valued or rounded-normal scores (the latter two give
    first-digit bins too large for the key list)."""
    rng = np.random.default_rng(9150 + i)
    Hkv = int(rng.integers(1, 13))
    n = int(np.exp(rng.uniform(np.log(16500.0), np.log(200000.0))))
    n = min(n, 600000 // Hkv)
    D = int(rng.choice([64, 128]))
    window = int(rng.integers(0, 2049))
    cand = n - window
    if cand <= 16384:
        window, cand = 0, n
    k = int(rng.integers(1, cand))
    law = str(rng.choice(["lognormal", "lognormal", "octave", "three", "rounded"]))
    if law == "lognormal":
        sc = synth.evict_scores(9600 + i, Hkv, n, tie_frac=float(rng.uniform(0, 0.3)), zero_frac=0.02)
    elif law == "octave":
        sc = (0.5 + 0.5 * rng.random((Hkv, n))).astype(np.float32)
    elif law == "three":
        sc = rng.choice(np.array([0.1, 0.2, 0.3], dtype=np.float32), size=(Hkv, n))
    else:
        sc = np.round(rng.standard_normal((Hkv, n)), 2).astype(np.float32)
    return Hkv, n, D, window, law, sc, k


@pytest.mark.parametrize("i", range(16))
def test_evict_long_head_sweep(i):
    """Sixteen seeded random layers through the long-head top-k path: exactly
    the oracle's selection and compaction."""
    Hkv, n, D, window, law, sc, k = _long_sweep_case(i)
    K = synth.normal_bf16(9700 + i, 90, (Hkv, n, D))
    V = synth.normal_bf16(9700 + i, 91, (Hkv, n, D))
    name = f"long-sweep-{i} Hkv={Hkv} n={n} D={D} w={window} {law} k={k}"
    say(f"[evict] {name}")
    kept, offs, Ko, Vo = kvs.evict(dev_f32(sc), dev_bf16(K), dev_bf16(V), window=window, k=k)
    torch.cuda.synchronize()
    _check_evict_exact(name, sc, K, V, window, k, None, kept, offs, Ko, Vo)


LAYER_CASES = [
    # name, Hkv, n, D, window, k (one budget for the layer), identical heads
    ("layer-multiblock", 4, 5000, 128, 128, 3000, False),
    ("layer-identical-heads-ties", 5, 3000, 64, 16, 2501, True),
    ("layer-k0", 3, 2000, 128, 32, 0, False),
    ("layer-keep-all", 3, 2000, 128, 32, 10 ** 6, False),
    ("layer-many-heads", 300, 700, 64, 16, 50000, False),
    ("layer-long-heads", 2, 140000, 64, 128, 70001, False),
]


@pytest.mark.parametrize("name,Hkv,n,D,window,k,same", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_evict_layer_budget_parity(name, Hkv, n, D, window, k, same):
    """One top-k budget over all heads' candidates (ties: lower head, then
    lower position), exactly as the oracle ranks them."""
    s, K, V = _evict_case(810, Hkv, n, D)
    if same:
        s[:] = s[0]
    s[0, 3] = np.nan
    s[-1, 5] = -0.0
    s[-1, 6] = 0.0
    s[0, 7] = np.inf
    say(f"[evict-layer] {name}")
    kept, offs, Ko, Vo = kvs.evict(dev_f32(s), dev_bf16(K), dev_bf16(V), window=window, k=k, scope="layer")
    torch.cuda.synchronize()
    offs = host(offs)
    ref = oracle.select(s, window, k=k, scope="layer")
    gk = kept_from_gpu(host(kept), offs)
    for h in range(Hkv):
        assert np.array_equal(gk[h], ref[h]), f"{name}: head {h} differs"
    Kr, Vr, offr = oracle.compact(K, V, ref)
    assert np.array_equal(offs, offr)
    total = int(offs[-1])
    assert np.array_equal(host_bits(Ko)[:total], Kr) and np.array_equal(host_bits(Vo)[:total], Vr)


def test_evict_strided_inputs():
    """Scores with a padded head stride; K/V views with padded token rows."""
    Hkv, n, D = 2, 3000, 128
    s, K, V = _evict_case(909, Hkv, n, D)
    s_pad = np.zeros((Hkv, n + 100), dtype=np.float32)
    s_pad[:, :n] = s
    Kp = np.zeros((Hkv, n, D + 64), dtype=np.uint16)
    Vp = np.zeros((Hkv, n, D + 64), dtype=np.uint16)
    Kp[:, :, :D], Vp[:, :, :D] = K, V
    sd = dev_f32(s_pad)[:, :n]
    Kd, Vd = dev_bf16(Kp)[:, :, :D], dev_bf16(Vp)[:, :, :D]
    kept, offs, Ko, Vo = kvs.evict(sd, Kd, Vd, window=64, k=500)
    torch.cuda.synchronize()
    ref = oracle.select(s, 64, k=500)
    gk = kept_from_gpu(host(kept), host(offs))
    for h in range(Hkv):
        assert np.array_equal(gk[h], ref[h])
    check_rows(K, V, gk, host_bits(Ko), host_bits(Vo), host(offs), "strided")


# ---------------------------------------------------------------- end to end

@pytest.mark.parametrize("wl", [TINY_KVZIP, QWEN25_1P5B_2K], ids=lambda w: w.name)
def test_workload_end_to_end(wl):
    r = wl.recipe
    d = synth.draw(r, wl.seed)
    say(f"[e2e] {wl.name}")
    Q, K, Ks, V = dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), dev_bf16(d["Kself"]), dev_bf16(d["V"])
    L = kvs.lse(Q, K, Ks, scale=d["scale"], mask="repeat", chunk=r.self_chunk)
    vn = dev_f32(d["vnorm"]) if r.value_norms else None
    hn = dev_f32(d["hnorm"]) if r.value_norms else None
    s = kvs.max_scores(Q, K, L, scale=d["scale"], vnorm=vn, hnorm=hn)
    ref_L = oracle.lse(d["Q"], d["Kctx"], d["Kself"], d["scale"], "repeat", r.self_chunk)
    check_lse(host(L), ref_L, wl.name)
    ref_s = oracle.max_scores(d["Q"], d["Kctx"], ref_L, d["scale"], r.Hkv, vnorm=d.get("vnorm"),
                              hnorm=d.get("hnorm"))
    check_scores(host(s), ref_s, wl.name)
    for k in wl.ks():
        kept, offs, Ko, Vo = kvs.evict(s, K, V, window=wl.window, k=k)
        torch.cuda.synchronize()
        gk = kept_from_gpu(host(kept), host(offs))
        ref_k = oracle.select(ref_s, wl.window, k=k)
        check_kept(gk, ref_k, ref_s, k=k, window=wl.window, what=f"{wl.name} k={k}")
        check_rows(d["Kctx"], d["V"], gk, host_bits(Ko), host_bits(Vo), host(offs), wl.name)


def test_pipeline_is_deterministic():
    r = QWEN25_1P5B_2K.recipe
    d = synth.draw(r, 1)
    Q, K, Ks, V = dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), dev_bf16(d["Kself"]), dev_bf16(d["V"])
    vn, hn = dev_f32(d["vnorm"]), dev_f32(d["hnorm"])
    outs = []
    for _ in range(2):
        L = kvs.lse(Q, K, Ks, scale=d["scale"], mask="repeat", chunk=r.self_chunk)
        s = kvs.max_scores(Q, K, L, scale=d["scale"], vnorm=vn, hnorm=hn)
        kept, offs, Ko, Vo = kvs.evict(s, K, V, window=128, k=1024)
        outs.append([x.clone() for x in (L, s, kept, offs, Ko, Vo)])
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("selection", ["topk", "tau"])
def test_step_replays_from_a_hip_graph(selection):
    """LSE + max score + eviction (top-k, or threshold) captured once in a
    HIP graph (no allocation, no host sync inside) and replayed three times,
    with eager work between the replays: every replay equals the eager step
    bit for bit."""
    wl = QWEN25_1P5B_2K
    r = wl.recipe
    d = synth.draw(r, wl.seed)
    Q, K, Ks, V = dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), dev_bf16(d["Kself"]), dev_bf16(d["V"])
    vn, hn = dev_f32(d["vnorm"]), dev_f32(d["hnorm"])
    k, tau = (wl.ks()[1], None) if selection == "topk" else (None, float(np.exp(-6.0)))
    L = torch.empty((r.Hq, r.n_q), dtype=torch.float32, device="cuda")
    S = torch.empty((r.Hkv, r.n_ctx), dtype=torch.float32, device="cuda")
    e = kvs.evict_desc(S, K, window=wl.window, k=k, tau=tau)
    ws = torch.empty(max(kvs.evict_workspace_bytes(e), 256), dtype=torch.uint8, device="cuda")
    outs = (torch.empty(e.capacity, dtype=torch.int32, device="cuda"),
            torch.empty(r.Hkv + 1, dtype=torch.int64, device="cuda"),
            torch.empty((e.capacity, r.D), dtype=torch.bfloat16, device="cuda"),
            torch.empty((e.capacity, r.D), dtype=torch.bfloat16, device="cuda"))

    def step():
        kvs.lse(Q, K, Ks, scale=d["scale"], mask="repeat", chunk=r.chunk, out=L)
        kvs.max_scores(Q, K, L, scale=d["scale"], vnorm=vn, hnorm=hn, out=S)
        kvs.evict(S, K, V, window=wl.window, k=k, tau=tau, workspace=ws, outputs=outs)

    say(f"[graph] {selection}: eager step")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (L, S, *outs)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("[graph] capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (L, S, *outs):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("lse", "scores", "kept", "offsets", "K_out", "V_out"), (L, S, *outs), ref):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.bfloat16 else a.view(torch.int16),
                               b.view(torch.uint8) if b.dtype != torch.bfloat16 else b.view(torch.int16)), \
                f"replay {rep}: {name} differs"
