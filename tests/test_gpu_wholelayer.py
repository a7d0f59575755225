"""Whole heads of the full-size layers against the oracle, in the launch
configuration the benchmark times.

The oracle's fp64 results for whole heads (every query row of their query
heads, every key of their KV heads) are stored under tests/golden/fullsize,
written by the committed script there, which calls only the oracle; each
fixture carries a hash of the seeded inputs it belongs to. The GPU runs the
whole layer; its LSE rows, scores and kept sets of the stored heads are
compared element by element:
* LSE: |gpu - ref| <= 1e-3;
* scores / future mass: relative <= 5e-3 where ref >= 1e-6, else <= 1e-8;
* kept sets: equal up to keys within 5e-3 of the k-th score or tau; rows
  bit-exact; counts exact in top-k mode.
"""
import hashlib
import os

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import BY_NAME, KVPOP_CAUSAL_16K, QWEN25_1P5B_2K, QWEN25_14B_120K, QWEN3_8B_32K

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_eviction_lse_amd as kvs  # noqa: E402
from gpu_util import (check_kept, check_lse, check_rows, check_scores, dev_bf16, dev_f32, host,  # noqa: E402
                      host_bits, kept_from_gpu, say)

FIXTURES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fullsize")


def _fixture(name):
    path = os.path.join(FIXTURES, f"{name}.npz")
    if not os.path.exists(path):
        pytest.fail(f"missing fixture {path} (tests/golden/fullsize/make_fixtures.py writes it)")
    return np.load(path)


def _input_hash(d, kv_heads, G):
    """sha256 of the inputs the fixture belongs to (as make_fixtures.py takes it)."""
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


def _check_selection(wl, d, s_gpu, ref_scores, heads, K, V, k=None, tau=None):
    """GPU eviction of the GPU's scores: the stored heads' kept sets against
    the oracle's selection on the oracle's scores (exempt band 5e-3)."""
    kept, offs, Ko, Vo = kvs.evict(s_gpu, K, V, window=wl.window, k=k, tau=tau)
    torch.cuda.synchronize()
    offs = host(offs)
    gk = kept_from_gpu(host(kept), offs)
    ref = oracle.select(ref_scores.astype(np.float64), wl.window, k=k, tau=tau)
    check_kept([gk[h] for h in heads], ref, ref_scores.astype(np.float64), k=k, tau=tau, window=wl.window,
               what=f"{wl.name} kept")
    check_rows(d["Kctx"], d["V"], gk, host_bits(Ko), host_bits(Vo), offs, wl.name)
    return offs


@pytest.mark.parametrize("wl", [QWEN3_8B_32K, QWEN25_14B_120K], ids=lambda w: w.name)
def test_repeat_layer_whole_heads(wl):
    r = wl.recipe
    fx = _fixture(wl.name)
    heads = [int(h) for h in fx["kv_heads"]]
    G = r.Hq // r.Hkv
    say(f"[whole] {wl.name}: drawing")
    d = synth.draw(r, wl.seed)
    assert str(fx["input_sha256"]) == _input_hash(d, heads, G), "inputs differ from the fixture's"
    Q, K, Ks, V = dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), dev_bf16(d["Kself"]), dev_bf16(d["V"])
    vn, hn = dev_f32(d["vnorm"]), dev_f32(d["hnorm"])
    say(f"[whole] {wl.name}: gpu lse + max score (all heads)")
    L = kvs.lse(Q, K, Ks, scale=d["scale"], mask="repeat", chunk=r.chunk)
    s = kvs.max_scores(Q, K, L, scale=d["scale"], vnorm=vn, hnorm=hn)
    torch.cuda.synchronize()
    g0, g1 = heads[0] * G, (heads[-1] + 1) * G
    e_lse = check_lse(host(L)[g0:g1], fx["lse"].astype(np.float64), f"{wl.name} lse, query heads {g0}-{g1 - 1}")
    ref_s = fx["scores"].astype(np.float64)
    e_s = check_scores(host(s)[heads], ref_s, f"{wl.name} scores, KV heads {heads}")
    say(f"[whole] {wl.name}: lse max err {e_lse:.2e}, score max rel err {e_s:.2e} over "
        f"{(g1 - g0) * r.n_q} rows and {len(heads) * r.n_ctx} keys")
    sel = dict(tau=wl.tau) if wl.tau >= 0 else dict(k=wl.ks()[0])
    offs = _check_selection(wl, d, s, ref_s, heads, K, V, **sel)
    if "k" in sel:
        assert np.all(np.diff(offs) == sel["k"] + wl.window)


def test_kvpop_layer_every_row_and_key():
    wl = KVPOP_CAUSAL_16K
    r = wl.recipe
    fx = _fixture(wl.name)
    heads = [int(h) for h in fx["kv_heads"]]
    assert heads == list(range(r.Hkv))
    say(f"[whole] {wl.name}: drawing")
    d = synth.draw(r, wl.seed)
    assert str(fx["input_sha256"]) == _input_hash(d, heads, r.Hq // r.Hkv), "inputs differ from the fixture's"
    Q, K, V = dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), dev_bf16(d["V"])
    L = kvs.lse(Q, K, None, scale=d["scale"], mask="causal")
    t = kvs.future_mass(Q, K, L, scale=d["scale"], window=wl.window)
    torch.cuda.synchronize()
    check_lse(host(L), fx["lse"].astype(np.float64), "kvpop lse, every row")
    ref_t = fx["scores"].astype(np.float64)
    check_scores(host(t), ref_t, "kvpop future mass, every key")
    for k in wl.ks():
        offs = _check_selection(wl, d, t, ref_t, heads, K, V, k=k)
        assert np.all(np.diff(offs) == k + wl.window)


def test_future_mass_multi_pair_32k():
    """Causal 32k layer with 8 KV heads: enough key-block pairs that every
    workgroup takes two whole pairs with no query split (the form the 16k
    layer does not reach). The oracle's future mass given the GPU's LSE on
    sampled keys, the LSE on sampled rows, and at window 0 the total mass of
    each head equals G * T (each softmax row sums to one)."""
    r = synth.Recipe(Hq=16, Hkv=8, D=128, n_ctx=32768, n_q=32768, mask="causal", sinks=4)
    d = synth.draw(r, 909)
    Q, K = dev_bf16(d["Q"]), dev_bf16(d["Kctx"])
    L = kvs.lse(Q, K, None, scale=d["scale"], mask="causal")
    t = kvs.future_mass(Q, K, L, scale=d["scale"], window=128)
    t0 = kvs.future_mass(Q, K, L, scale=d["scale"], window=0)
    torch.cuda.synchronize()
    tot = host(t0).astype(np.float64).sum(axis=1)
    assert np.allclose(tot, r.group * r.n_ctx, rtol=1e-4), tot
    rows = np.unique(np.r_[0:4, 16380:16388, r.n_q - 4:r.n_q])
    check_lse(host(L)[:, rows], oracle.lse(d["Q"], d["Kctx"], None, d["scale"], "causal", 0, rows=rows),
              "32k causal lse rows")
    u = synth.u64(909, 78, 40)
    keys = np.unique(np.r_[[int(x % np.uint64(r.n_ctx - 128)) for x in u], 0, 511, 512, r.n_ctx - 129])
    ref = oracle.future_mass(d["Q"], d["Kctx"], host(L).astype(np.float64), d["scale"], 128, r.Hkv, keys=keys)
    check_scores(host(t)[:, keys], ref, "32k future mass, sampled keys, GPU LSE given")
    assert np.all(host(t)[:, r.n_ctx - 128:] == 0)


def test_value_norms_feed_the_max_score():
    """kvscore_vnorm's output as kvscore_max's vnorm input, on the 1.5B-shaped
    2k layer, against the oracle's value norms fed to the oracle's score."""
    wl = QWEN25_1P5B_2K
    r = wl.recipe
    d = synth.draw(r, wl.seed)
    Q, K, Ks, V, WO = (dev_bf16(d[x]) for x in ("Q", "Kctx", "Kself", "V", "WO"))
    hn = dev_f32(d["hnorm"])
    vn = kvs.value_norms(V, WO)
    L = kvs.lse(Q, K, Ks, scale=d["scale"], mask="repeat", chunk=r.self_chunk)
    s = kvs.max_scores(Q, K, L, scale=d["scale"], vnorm=vn, hnorm=hn)
    torch.cuda.synchronize()
    ref_vn = oracle.value_norms(d["V"], d["WO"], r.Hkv)
    ref_L = oracle.lse(d["Q"], d["Kctx"], d["Kself"], d["scale"], "repeat", r.self_chunk)
    ref_s = oracle.max_scores(d["Q"], d["Kctx"], ref_L, d["scale"], r.Hkv, vnorm=ref_vn, hnorm=d["hnorm"])
    check_lse(host(L), ref_L, "2k lse")
    check_scores(host(s), ref_s, "2k KVzip+ score with GPU value norms")
    for k in wl.ks():
        kept, offs, Ko, Vo = kvs.evict(s, K, V, window=wl.window, k=k)
        torch.cuda.synchronize()
        gk = kept_from_gpu(host(kept), host(offs))
        check_kept(gk, oracle.select(ref_s, wl.window, k=k), ref_s, k=k, window=wl.window, what=f"2k keep {k}")
