"""Decode attention over the compacted per-head cache (kvscore_decode) against
the CPU oracle through the C ABI: ragged and empty heads, D = 64 and 128,
several query groups per head, wave chunks of 32, 64 and 128 rows (chosen
by the cache's size), 4 and 8 queries per wave, clamped offsets, and the
full pipeline
kv_evict -> kvscore_decode against oracle select -> compact -> decode.

Tolerance: scores (bf16 products summed in fp32 on the matrix cores),
exponentials and sums are fp32 (chunks of at most 128 rows, then a merge
over chunks), so the summation error stays far below 2^-12 of
sum_r a_r |v_r|; O is rounded once to bf16 (2^-8 |O|):
    |O_gpu - O_ref| <= 2^-8 |O_ref| + 2^-12 sum_r a_r |v_r|,  |LSE err| <= 1e-3,
and a head with no rows gives exactly O = 0, LSE = -inf.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_eviction_lse_amd as kvs  # noqa: E402
from gpu_util import bf16_abs, bf16_to_f64, check_lse, dev_bf16, host, host_bits, say  # noqa: E402


def _check(O_bits, L, Q, Kc, Vc, offs, scale, what):
    ref_O, ref_L = oracle.decode_attention(Q, Kc, Vc, offs, scale)
    ref_abs, _ = oracle.decode_attention(Q, Kc, bf16_abs(Vc), offs, scale)
    g = bf16_to_f64(O_bits)
    empty = np.isneginf(ref_L)
    assert np.all(np.isneginf(L[empty])) and np.all(g[empty] == 0), f"{what}: empty heads"
    check_lse(L[~empty], ref_L[~empty], what)
    err = np.abs(g - ref_O)
    tol = 2.0 ** -8 * np.abs(ref_O) + 2.0 ** -12 * ref_abs
    assert np.all(err <= tol), f"{what}: O err/tol {np.max(err / np.maximum(tol, 1e-300)):.2f}"


def _case(seed, Hq, Hkv, D, counts, n_q):
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    Q = synth.normal_bf16(seed, 1, (Hq, n_q, D))
    Kc = synth.normal_bf16(seed, 2, (int(offs[-1]), D))
    Vc = synth.normal_bf16(seed, 3, (int(offs[-1]), D))
    return Q, Kc, Vc, offs


CASES = [
    # name, Hq, Hkv, D, rows per head, n_q
    ("d64-ragged-and-empty-head", 6, 3, 64, [300, 0, 517], 2),
    ("d128-g4-chunk-edges", 16, 4, 128, [1, 128, 129, 3000], 1),
    ("g5-three-tokens-two-query-groups", 10, 2, 128, [700, 45], 3),
    ("mha-one-row", 4, 4, 128, [1, 2, 3, 4], 1),
    # the wave-chunk size follows the cache: 32 rows below 98,304 rows of
    # cache, 64 below 196,608, else 128; 4 or 8 queries per wave
    ("d128-32-row-chunks-many", 16, 4, 128, [9000, 33, 32, 7000], 1),
    ("g5-8q-32-row-chunks", 10, 2, 128, [6000, 4001], 1),
    ("d128-4q-64-row-chunks", 8, 2, 128, [60000, 40001], 1),
    ("d64-8q-64-row-chunks", 8, 2, 64, [50000, 48305], 2),
    ("d128-8q-128-row-chunks", 10, 2, 128, [120000, 76609], 1),
    ("d64-4q-128-row-chunks", 4, 2, 64, [100000, 100001], 1),
    # heads are located 64 at a time (one per lane): 70 heads span two such
    # groups, with empty heads on both sides of the group edge
    ("d64-70-heads-two-lane-groups", 140, 70, 64,
     [(37 * k) % 211 if k not in (0, 5, 63, 64, 69) else 0 for k in range(70)], 1),
]


@pytest.mark.parametrize("name,Hq,Hkv,D,counts,n_q", CASES, ids=[c[0] for c in CASES])
def test_decode_parity(name, Hq, Hkv, D, counts, n_q):
    Q, Kc, Vc, offs = _case(111, Hq, Hkv, D, counts, n_q)
    say(f"[decode] {name}")
    O, L = kvs.decode(dev_bf16(Q), dev_bf16(Kc), dev_bf16(Vc), torch.from_numpy(offs).cuda(), scale=0.09)
    torch.cuda.synchronize()
    _check(host_bits(O), host(L), Q, Kc, Vc, offs, 0.09, name)


def test_decode_is_deterministic():
    """Two calls give bit-identical O and LSE (fixed-order merges, no atomics)."""
    Q, Kc, Vc, offs = _case(119, 10, 2, 128, [60000, 40001], 1)
    args = (dev_bf16(Q), dev_bf16(Kc), dev_bf16(Vc), torch.from_numpy(offs).cuda())
    say("[decode] determinism")
    O1, L1 = kvs.decode(*args, scale=0.09)
    O2, L2 = kvs.decode(*args, scale=0.09)
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16)) and torch.equal(L1, L2)


def test_decode_clamps_offsets():
    """Offsets past the cache or decreasing are clamped to [0, capacity] and made monotone."""
    Q, Kc, Vc, offs = _case(113, 4, 2, 128, [200, 300], 1)
    bad = np.array([0, 200, 10 ** 9], dtype=np.int64)  # last head runs past the cache: 300 rows used
    say("[decode] clamped offsets")
    O, L = kvs.decode(dev_bf16(Q), dev_bf16(Kc), dev_bf16(Vc), torch.from_numpy(bad).cuda(), scale=0.09)
    torch.cuda.synchronize()
    _check(host_bits(O), host(L), Q, Kc, Vc, offs, 0.09, "clamped")


def test_decode_clamps_offsets_across_lane_groups():
    """Negative, decreasing and too-large offsets over 70 heads (two groups of
    64 heads): clamped to [0, capacity], then a running max, as one sequence."""
    counts = [(53 * k) % 97 for k in range(70)]
    Q, Kc, Vc, offs = _case(117, 70, 70, 128, counts, 1)
    cap = int(offs[-1])
    bad = offs.copy()
    bad[3] = -50                 # negative: clamped to 0, then the running max
    bad[40] = bad[38]            # decreasing into head 39's range
    bad[64] = bad[60] - 7        # across the lane-group edge
    bad[66] = cap + 10 ** 6      # past the cache: clamped to capacity, later heads empty
    eff = np.maximum.accumulate(np.clip(bad, 0, cap))
    say("[decode] clamped offsets across lane groups")
    O, L = kvs.decode(dev_bf16(Q), dev_bf16(Kc), dev_bf16(Vc), torch.from_numpy(bad).cuda(), scale=0.09)
    torch.cuda.synchronize()
    _check(host_bits(O), host(L), Q, Kc, Vc, eff, 0.09, "clamped across lane groups")


def test_evict_then_decode_pipeline():
    """kv_evict (top-k + window) followed by kvscore_decode equals the oracle's
    select -> compact -> decode on the same scores."""
    Hkv, n, D, G = 4, 3000, 128, 4
    scores = synth.evict_scores(115, Hkv, n)
    K = synth.normal_bf16(115, 1, (Hkv, n, D))
    V = synth.normal_bf16(115, 2, (Hkv, n, D))
    Q = synth.normal_bf16(115, 3, (Hkv * G, 1, D))
    say("[decode] evict -> decode")
    S, Kd, Vd = torch.from_numpy(scores).cuda(), dev_bf16(K), dev_bf16(V)
    kept_idx, offs, K_out, V_out = kvs.evict(S, Kd, Vd, window=128, k=700)
    O, L = kvs.decode(dev_bf16(Q), K_out, V_out, offs, scale=0.0883883)
    torch.cuda.synchronize()
    kept = oracle.select(scores, 128, k=700)
    Kc, Vc, ref_offs = oracle.compact(K, V, kept)
    assert np.array_equal(host(offs), ref_offs)
    _check(host_bits(O), host(L), Q, Kc, Vc, ref_offs, 0.0883883, "pipeline")
