"""Full-size workloads in the launch configuration the benchmark times.

The oracle cannot afford a whole 32k-120k layer, so at full size:
* LSE: sampled query rows (first and last rows of the first and last chunks)
  against the oracle restricted to those rows;
* score pass: run on a stand-in normaliser (seeded uniform values, not from
  any attention) so that the oracle can evaluate sampled keys one by one;
* eviction: seeded full-size scores with ties, compared exactly;
* the GPU's own pipeline: properties that hold at any size (scores bounded
  by vnorm / min hnorm, window kept, threshold respected, rows bit-exact, and
  for the future mass with window 0, total mass = G * T);
* attention forward: sampled query rows against the oracle restricted to
  those rows; decode: over the cache that eviction of seeded scores leaves
  (identical to the oracle's), every query head against the oracle;
* layer-wide budget: seeded full-size scores, compared exactly.
"""
import numpy as np
import pytest

import oracle
import synth
from synth.workloads import KVPOP_CAUSAL_16K, QWEN3_8B_32K, QWEN25_14B_120K

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_eviction_lse_amd as kvs  # noqa: E402
from gpu_util import (bf16_abs, bf16_to_f64, check_attn_out, check_kept, check_lse, check_rows,  # noqa: E402
                      check_scores, dev_bf16, dev_f32, host, host_bits, kept_from_gpu, say)

SAMPLE_KEYS = 48


def _sample_rows(n_q, chunk):
    last_c0 = ((n_q - 1) // chunk) * chunk
    rows = list(range(0, 6)) + list(range(chunk - 6, chunk)) + list(range(last_c0, last_c0 + 6)) + \
        list(range(n_q - 6, n_q))
    return np.unique(np.array(rows, dtype=np.int64))


def _sample_keys(seed, n, window):
    u = synth.u64(seed, 77, SAMPLE_KEYS)
    keys = set(int(x % np.uint64(n)) for x in u) | {0, 1, n - window - 1, n - window, n - 1}
    return np.array(sorted(k for k in keys if 0 <= k < n), dtype=np.int64)


def _repeat_layer(wl, lse_range, kth_check):
    r = wl.recipe
    say(f"[full] {wl.name}: drawing")
    d = synth.draw(r, wl.seed)
    Q, K, Ks, V = dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), dev_bf16(d["Kself"]), dev_bf16(d["V"])
    vn, hn = dev_f32(d["vnorm"]), dev_f32(d["hnorm"])
    say(f"[full] {wl.name}: gpu lse + max")
    L = kvs.lse(Q, K, Ks, scale=d["scale"], mask="repeat", chunk=r.chunk)
    s = kvs.max_scores(Q, K, L, scale=d["scale"], vnorm=vn, hnorm=hn)
    torch.cuda.synchronize()

    # LSE on sampled rows
    rows = _sample_rows(r.n_q, r.chunk)
    ref_rows = oracle.lse(d["Q"], d["Kctx"], d["Kself"], d["scale"], "repeat", r.chunk, rows=rows)
    check_lse(host(L)[:, rows], ref_rows, f"{wl.name} lse rows")

    # the pipeline's own scores: 0 < s_i <= vnorm_i / min_j hnorm_j
    sg = host(s)
    bound = d["vnorm"].astype(np.float64) / d["hnorm"].astype(np.float64).min()
    assert np.all(sg > 0) and np.all(sg <= bound * (1 + 1e-3))

    # score pass on a stand-in normaliser, sampled keys
    say(f"[full] {wl.name}: score pass on stand-in lse")
    lse_in = synth.lse_values(wl.seed + 100, r.Hq, r.n_q, *lse_range)
    s2 = kvs.max_scores(Q, K, dev_f32(lse_in), scale=d["scale"], vnorm=vn, hnorm=hn)
    torch.cuda.synchronize()
    keys = _sample_keys(wl.seed, r.n_ctx, wl.window)
    ref_s = oracle.max_scores(d["Q"], d["Kctx"], lse_in, d["scale"], r.Hkv, vnorm=d["vnorm"], hnorm=d["hnorm"],
                              keys=keys)
    check_scores(host(s2)[:, keys], ref_s, f"{wl.name} sampled keys")
    return d, s, K, V, kth_check


def _evict_on_seeded_scores(wl, d, K, V, k=None, tau=None):
    r = wl.recipe
    sc = synth.evict_scores(wl.seed + 200, r.Hkv, r.n_ctx, tie_frac=0.05, zero_frac=0.01)
    kept, offs, Ko, Vo = kvs.evict(dev_f32(sc), K, V, window=wl.window, k=k, tau=tau)
    torch.cuda.synchronize()
    ref = oracle.select(sc, wl.window, k=k, tau=tau)
    gk = kept_from_gpu(host(kept), host(offs))
    for h in range(r.Hkv):
        assert np.array_equal(gk[h], ref[h]), f"{wl.name}: seeded-score selection differs on head {h}"
    check_rows(d["Kctx"], d["V"], gk, host_bits(Ko), host_bits(Vo), host(offs), wl.name)


def _evict_properties(wl, d, s, K, V, k=None, tau=None):
    """Selection on the GPU's own scores: window kept, the rule respected."""
    r = wl.recipe
    kept, offs, Ko, Vo = kvs.evict(s, K, V, window=wl.window, k=k, tau=tau)
    torch.cuda.synchronize()
    sg = host(s)
    gk = kept_from_gpu(host(kept), host(offs))
    n, w = r.n_ctx, min(wl.window, r.n_ctx)
    for h in range(r.Hkv):
        idx = gk[h]
        assert np.all(np.diff(idx) > 0)
        assert set(range(n - w, n)) <= set(idx.tolist())
        cand = idx[idx < n - w]
        dropped = np.setdiff1d(np.arange(n - w), cand)
        if tau is not None:
            assert np.all(sg[h, cand] >= np.float32(tau)) and np.all(sg[h, dropped] < np.float32(tau))
        else:
            assert cand.size == min(k, n - w)
            if cand.size and dropped.size:
                assert sg[h, cand].min() >= sg[h, dropped].max()
    check_rows(d["Kctx"], d["V"], gk, host_bits(Ko), host_bits(Vo), host(offs), wl.name)
    return host(offs)


def test_qwen3_8b_32k_threshold():
    wl = QWEN3_8B_32K
    d, s, K, V, _ = _repeat_layer(wl, (10.0, 14.0), None)
    offs = _evict_properties(wl, d, s, K, V, tau=wl.tau)
    kept = np.diff(offs)
    say(f"[full] {wl.name}: kept per head {kept.tolist()} "
        f"(compression {[round(1 - x / wl.recipe.n_ctx, 3) for x in kept]})")
    _evict_on_seeded_scores(wl, d, K, V, tau=wl.tau)


def test_qwen25_14b_120k_topk():
    wl = QWEN25_14B_120K
    d, s, K, V, _ = _repeat_layer(wl, (12.0, 16.0), None)
    k = wl.ks()[0]
    offs = _evict_properties(wl, d, s, K, V, k=k)
    assert np.all(np.diff(offs) == k + wl.window)
    _evict_on_seeded_scores(wl, d, K, V, k=k)


def test_kvpop_causal_16k():
    wl = KVPOP_CAUSAL_16K
    r = wl.recipe
    say(f"[full] {wl.name}: drawing")
    d = synth.draw(r, wl.seed)
    Q, K, V = dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), dev_bf16(d["V"])
    L = kvs.lse(Q, K, None, scale=d["scale"], mask="causal")
    t = kvs.future_mass(Q, K, L, scale=d["scale"], window=wl.window)
    t0 = kvs.future_mass(Q, K, L, scale=d["scale"], window=0)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0:6, 5000:5006, r.n_q - 6:r.n_q])
    ref_rows = oracle.lse(d["Q"], d["Kctx"], None, d["scale"], "causal", 0, rows=rows)
    check_lse(host(L)[:, rows], ref_rows, "kvpop lse rows")
    # window 0: every softmax row sums to one, so each head's targets add to G*T
    tot = host(t0).astype(np.float64).sum(axis=1)
    assert np.allclose(tot, r.group * r.n_ctx, rtol=1e-4), tot
    tg = host(t)
    assert np.all(tg[:, r.n_ctx - wl.window:] == 0)
    # sum pass on a stand-in normaliser, sampled keys
    lse_in = synth.lse_values(wl.seed + 100, r.Hq, r.n_q, 5.0, 10.0)
    t2 = kvs.future_mass(Q, K, dev_f32(lse_in), scale=d["scale"], window=wl.window)
    torch.cuda.synchronize()
    keys = _sample_keys(wl.seed, r.n_ctx, wl.window)
    ref_t = oracle.future_mass(d["Q"], d["Kctx"], lse_in, d["scale"], wl.window, r.Hkv, keys=keys)
    check_scores(host(t2)[:, keys], ref_t, "kvpop sampled keys")
    for k in wl.ks():
        offs = _evict_properties(wl, d, t, K, V, k=k)
        assert np.all(np.diff(offs) == k + wl.window)
        _evict_on_seeded_scores(wl, d, K, V, k=k)


def _attention_rows(wl, d, Q, K, V, Ks, Vs, rows, mask, chunk):
    O, L = kvs.attention(Q, K, V, Ks, Vs, scale=d["scale"], mask=mask, chunk=chunk)
    torch.cuda.synchronize()
    args = (d["Q"], d["Kctx"], d.get("Kself"))
    ref_O, ref_L = oracle.attention(*args, d["V"], d.get("Vself"), d["scale"], mask, chunk, rows=rows)
    ref_abs, _ = oracle.attention(*args, bf16_abs(d["V"]), bf16_abs(d["Vself"]) if "Vself" in d else None,
                                  d["scale"], mask, chunk, rows=rows)
    check_lse(host(L)[:, rows], ref_L, f"{wl.name} attention lse rows")
    check_attn_out(host_bits(O)[:, rows], ref_O, ref_abs, f"{wl.name} attention rows")


def test_qwen3_8b_32k_attention_and_decode():
    wl = QWEN3_8B_32K
    r = wl.recipe
    say(f"[full] {wl.name}: drawing (attention, decode)")
    d = synth.draw(r, wl.seed)
    Q, K, V = dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), dev_bf16(d["V"])
    Ks, Vs = dev_bf16(d["Kself"]), dev_bf16(d["Vself"])
    say(f"[full] {wl.name}: attention on sampled rows")
    _attention_rows(wl, d, Q, K, V, Ks, Vs, _sample_rows(r.n_q, r.chunk), "repeat", r.chunk)
    # decode: one new token per query head over the cache eviction leaves
    say(f"[full] {wl.name}: evict seeded scores, then decode")
    sc = synth.evict_scores(wl.seed + 300, r.Hkv, r.n_ctx, tie_frac=0.05, zero_frac=0.01)
    kept, offs, Ko, Vo = kvs.evict(dev_f32(sc), K, V, window=wl.window, tau=wl.tau)
    Qd_bits = np.ascontiguousarray(d["Q"][:, -1:, :])
    Od, Ld = kvs.decode(dev_bf16(Qd_bits), Ko, Vo, offs, scale=d["scale"])
    torch.cuda.synchronize()
    ref_kept = oracle.select(sc, wl.window, tau=wl.tau)
    Kc, Vc, ref_offs = oracle.compact(d["Kctx"], d["V"], ref_kept)
    assert np.array_equal(host(offs), ref_offs)
    ref_O, ref_L = oracle.decode_attention(Qd_bits, Kc, Vc, ref_offs, d["scale"])
    ref_abs, _ = oracle.decode_attention(Qd_bits, Kc, bf16_abs(Vc), ref_offs, d["scale"])
    check_lse(host(Ld), ref_L, "32k decode lse")
    g = bf16_to_f64(host_bits(Od))
    tol = 2.0 ** -8 * np.abs(ref_O) + 2.0 ** -12 * ref_abs
    assert np.all(np.abs(g - ref_O) <= tol), "32k decode O"


def test_kvpop_causal_16k_attention():
    wl = KVPOP_CAUSAL_16K
    r = wl.recipe
    say(f"[full] {wl.name}: drawing (attention)")
    d = synth.draw(r, wl.seed)
    rows = np.unique(np.r_[0:6, 5000:5006, r.n_q - 6:r.n_q])
    _attention_rows(wl, d, dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), dev_bf16(d["V"]), None, None, rows, "causal", 0)


def test_qwen25_14b_120k_layer_budget():
    """One top-k budget over the 8 heads of the 120k layer (25 % of all
    candidates), on seeded scores with ties, compared exactly."""
    wl = QWEN25_14B_120K
    r = wl.recipe
    say(f"[full] {wl.name}: layer budget on seeded scores")
    sc = synth.evict_scores(wl.seed + 400, r.Hkv, r.n_ctx, tie_frac=0.05, zero_frac=0.01)
    sc[3] = sc[1]  # two heads with identical scores: ties across heads at every level
    K = synth.normal_bf16(wl.seed, 500, (r.Hkv, r.n_ctx, r.D))
    V = synth.normal_bf16(wl.seed, 501, (r.Hkv, r.n_ctx, r.D))
    k = wl.ks()[0] * r.Hkv
    kept, offs, Ko, Vo = kvs.evict(dev_f32(sc), dev_bf16(K), dev_bf16(V), window=wl.window, k=k, scope="layer")
    torch.cuda.synchronize()
    ref = oracle.select(sc, wl.window, k=k, scope="layer")
    gk = kept_from_gpu(host(kept), host(offs))
    for h in range(r.Hkv):
        assert np.array_equal(gk[h], ref[h]), f"layer budget: head {h} differs"
    assert int(host(offs)[-1]) == k + r.Hkv * wl.window
    check_rows(K, V, gk, host_bits(Ko), host_bits(Vo), host(offs), "120k layer budget")

