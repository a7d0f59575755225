"""Threshold pruning as tokens arrive (kv_stream_append) against the CPU
oracle through the C ABI: after every call the device state (window ring
rows, kept rows, their positions, the ring's scores, head_len) must equal the
oracle's token-by-token simulation bit for bit; decode attention over the
stream cache (kvscore_decode with a head stride) must equal the oracle's
decode over the same live rows.

Cases cover one token per call across the window edge, bulk calls longer
than the window (tokens that enter and leave in one call), more leaving
tokens than one pass of the kernel decides, bulk calls split over several
workgroups per head, w = 0 and w = 1, a stream that never fills its window,
many heads, D = 64 and 128, and scores that are NaN, +inf or exactly tau.
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
from gpu_util import bf16_abs, bf16_to_f64, check_lse, dev_bf16, dev_f32, host, host_bits, say  # noqa: E402

TAU = 0.25


def _stream(seed, Hkv, T, D):
    rng = np.random.default_rng(seed)
    s = rng.normal(size=(Hkv, T)).astype(np.float32)
    s[0, min(2, T - 1)] = np.nan
    s[-1, min(4, T - 1)] = np.inf
    s[:, 6::11] = TAU  # exactly the threshold: kept
    K = synth.normal_bf16(seed, 70, (Hkv, T, D))
    V = synth.normal_bf16(seed, 71, (Hkv, T, D))
    return s, K, V


def _check_state(cache, s, K, V, w, n, slots, kept, what):
    Hkv, C, D = cache.K.shape
    Kc, Vc, pos = host_bits(cache.K), host_bits(cache.V), host(cache.pos)
    hl, ws = host(cache.head_len), host(cache.win_scores)
    for h in range(Hkv):
        nwin = min(n, w)
        assert hl[h] == nwin + kept[h].size, f"{what}: head {h} head_len {hl[h]}"
        rows = [(r, int(slots[h][r])) for r in range(nwin)] + [(w + i, int(p)) for i, p in enumerate(kept[h])]
        for r, p in rows:
            assert pos[h, r] == p, f"{what}: head {h} row {r} holds position {pos[h, r]}, expected {p}"
        idx = np.array([r for r, _ in rows], dtype=np.int64)
        src = np.array([p for _, p in rows], dtype=np.int64)
        assert np.array_equal(Kc[h, idx], K[h, src]) and np.array_equal(Vc[h, idx], V[h, src]), \
            f"{what}: head {h} rows differ"
        for r in range(nwin):
            a, b = ws[h, r], s[h, slots[h][r]]
            assert a == b or (np.isnan(a) and np.isnan(b)), f"{what}: head {h} window score {r}"


CASES = [
    # name, Hkv, D, w, steps
    ("one-token-calls-across-the-window", 3, 128, 16, [1] * 40 + [5, 1, 1]),
    ("bulk-longer-than-window-then-steps", 2, 64, 8, [100, 1, 1, 3, 50]),
    ("bulk-several-passes", 2, 128, 16, [700, 1, 600]),
    ("window-zero", 2, 128, 0, [3, 1, 10, 1]),
    ("window-one", 4, 64, 1, [1, 2, 1, 7]),
    ("window-never-filled", 2, 128, 64, [5, 10, 1]),
    ("many-heads", 40, 64, 4, [3, 1, 20, 1]),
    # bulk calls split over workgroups of 1024 leaving tokens (ring tokens
    # leave in the first chunk)
    ("bulk-multi-block-after-a-partial-ring", 2, 128, 16, [5, 10000, 1, 3]),
    ("bulk-multi-block-full-ring-d64", 3, 64, 128, [300, 9000, 2]),
    # the widest window a split bulk call allows (w = 1024): its 1024 ring
    # tokens are exactly the first chunk, the call's 1100 leaving tokens two chunks
    ("bulk-two-chunks-widest-window", 2, 128, 1024, [1500, 1100, 1]),
]


@pytest.mark.parametrize("name,Hkv,D,w,steps", CASES, ids=[c[0] for c in CASES])
def test_stream_matches_oracle(name, Hkv, D, w, steps):
    T = sum(steps)
    s, K, V = _stream(500 + len(name), Hkv, T, D)
    cache = kvs.StreamCache(Hkv, D, max(w, T) + 3, window=w, tau=TAU)
    states = oracle.stream_states(s, w, TAU, steps)
    n0 = 0
    for i, (m, (n, slots, kept)) in enumerate(zip(steps, states)):
        if i % 8 == 0 or i == len(steps) - 1:
            say(f"[stream] {name}: call {i}, {m} tokens")
        cache.append(dev_f32(s[:, n0:n0 + m]), dev_bf16(K[:, n0:n0 + m]), dev_bf16(V[:, n0:n0 + m]))
        n0 += m
        torch.cuda.synchronize()
        _check_state(cache, s, K, V, w, n, slots, kept, f"{name} call {i}")


def test_stream_strided_inputs():
    """New tokens given as views with padded token rows and a padded score row."""
    Hkv, D, w, steps = 2, 128, 4, [3, 9, 1]
    T = sum(steps)
    s, K, V = _stream(611, Hkv, T, D)
    cache = kvs.StreamCache(Hkv, D, T, window=w, tau=TAU)
    n0 = 0
    for m, (n, slots, kept) in zip(steps, oracle.stream_states(s, w, TAU, steps)):
        sp = np.zeros((Hkv, m + 5), dtype=np.float32)
        sp[:, :m] = s[:, n0:n0 + m]
        Kp = np.zeros((Hkv, m, D + 64), dtype=np.uint16)
        Vp = np.zeros((Hkv, m, D + 64), dtype=np.uint16)
        Kp[:, :, :D], Vp[:, :, :D] = K[:, n0:n0 + m], V[:, n0:n0 + m]
        say(f"[stream] strided call of {m}")
        cache.append(dev_f32(sp)[:, :m], dev_bf16(Kp)[:, :, :D], dev_bf16(Vp)[:, :, :D])
        n0 += m
        torch.cuda.synchronize()
        _check_state(cache, s, K, V, w, n, slots, kept, f"strided n={n}")


@pytest.mark.parametrize("D,G,n_q", [(128, 4, 1), (64, 5, 3)])
def test_stream_decode_matches_oracle(D, G, n_q):
    """Decode over the stream cache (head stride = capacity, head_len as the
    live rows) equals the oracle's decode over the same rows; tolerance as
    for the compacted cache: |dO| <= 2^-8 |O| + 2^-12 sum_r a_r |v_r|."""
    Hkv, w, steps = 3, 32, [300, 1, 1, 2, 40]
    T = sum(steps)
    s, K, V = _stream(620 + D, Hkv, T, D)
    cache = kvs.StreamCache(Hkv, D, T + 10, window=w, tau=TAU)
    n0 = 0
    for m in steps:
        cache.append(dev_f32(s[:, n0:n0 + m]), dev_bf16(K[:, n0:n0 + m]), dev_bf16(V[:, n0:n0 + m]))
        n0 += m
    n, slots, kept = oracle.stream_states(s, w, TAU, steps)[-1]
    live = [np.concatenate([slots[h][slots[h] >= 0], kept[h]]) for h in range(Hkv)]
    Kc, Vc, offs = oracle.compact(K, V, live)
    Q = synth.normal_bf16(621, 1, (Hkv * G, n_q, D))
    say(f"[stream-decode] D={D} G={G} n_q={n_q}")
    O, L = cache.decode(dev_bf16(Q), scale=0.09)
    torch.cuda.synchronize()
    ref_O, ref_L = oracle.decode_attention(Q, Kc, Vc, offs, 0.09)
    ref_abs, _ = oracle.decode_attention(Q, Kc, bf16_abs(Vc), offs, 0.09)
    check_lse(host(L), ref_L, "stream decode")
    err = np.abs(bf16_to_f64(host_bits(O)) - ref_O)
    tol = 2.0 ** -8 * np.abs(ref_O) + 2.0 ** -12 * ref_abs
    assert np.all(err <= tol), f"O err/tol {np.max(err / np.maximum(tol, 1e-300)):.2f}"


def test_stream_clamps_a_corrupt_head_len():
    """A head_len far outside what the state allows (huge, negative) is
    clamped: the call writes only inside each head's region (guard rows past
    the last region keep their pattern) and leaves head_len in [0, capacity]."""
    Hkv, D, C, w, G = 2, 128, 64, 8, 512
    s, K, V = _stream(630, Hkv, 40, D)
    cache = kvs.StreamCache(Hkv, D, C, window=w, tau=TAU)
    cache.append(dev_f32(s[:, :20]), dev_bf16(K[:, :20]), dev_bf16(V[:, :20]))
    # the same state in tensors with guard rows after the last region
    Kg = torch.full((Hkv * C + G, D), 3.0, dtype=torch.bfloat16, device="cuda")
    Vg = torch.full((Hkv * C + G, D), 3.0, dtype=torch.bfloat16, device="cuda")
    Pg = torch.full((Hkv * C + G,), -7, dtype=torch.int32, device="cuda")
    Kg[:Hkv * C] = cache.K.view(-1, D)
    Vg[:Hkv * C] = cache.V.view(-1, D)
    Pg[:Hkv * C] = cache.pos.view(-1)
    cache.K, cache.V, cache.pos = Kg[:Hkv * C].view(Hkv, C, D), Vg[:Hkv * C].view(Hkv, C, D), Pg[:Hkv * C].view(Hkv, C)
    cache.head_len.copy_(torch.tensor([1 << 40, -5], dtype=torch.int64))
    say("[stream] corrupt head_len")
    cache.append(dev_f32(s[:, 20:40]), dev_bf16(K[:, 20:40]), dev_bf16(V[:, 20:40]))
    torch.cuda.synchronize()
    hl = host(cache.head_len)
    assert np.all((hl >= 0) & (hl <= C))
    assert np.all(host(Kg[Hkv * C:].float()) == 3.0) and np.all(host(Vg[Hkv * C:].float()) == 3.0)
    assert np.all(host(Pg[Hkv * C:]) == -7)
