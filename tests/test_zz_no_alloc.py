"""kv_evict_noalloc (eviction with the library's fixed scratch instead of a
caller workspace) against kv_evict on the same inputs, through the C ABI:
two calls in a row, the second on a smaller layer, so the scratch holds the
first call's intermediates when the second starts. Outputs must be
identical bit for bit (indices, offsets, rows)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_eviction_lse_amd as kvs  # noqa: E402
from gpu_util import dev_bf16, dev_f32, say  # noqa: E402


def _layer(seed, Hkv, n, D):
    s = synth.evict_scores(seed, Hkv, n, tie_frac=0.1, zero_frac=0.02)
    K = synth.normal_bf16(seed, 90, (Hkv, n, D))
    V = synth.normal_bf16(seed, 91, (Hkv, n, D))
    return dev_f32(s), dev_bf16(K), dev_bf16(V)


def _outs(e):
    cap = max(e.capacity, 1)
    return (torch.full((cap,), -7, dtype=torch.int32, device="cuda"),
            torch.full((e.n_kvheads + 1,), -7, dtype=torch.int64, device="cuda"),
            torch.zeros((cap, e.head_dim), dtype=torch.bfloat16, device="cuda"),
            torch.zeros((cap, e.head_dim), dtype=torch.bfloat16, device="cuda"))


def _same(a, b, what):
    ka, oa, Ka, Va = a
    kb, ob, Kb, Vb = b
    assert torch.equal(oa, ob), f"{what}: offsets"
    tot = int(oa[-1].item())
    assert torch.equal(ka[:tot], kb[:tot]), f"{what}: kept indices"
    assert torch.equal(Ka[:tot].view(torch.int16), Kb[:tot].view(torch.int16)), f"{what}: K rows"
    assert torch.equal(Va[:tot].view(torch.int16), Vb[:tot].view(torch.int16)), f"{what}: V rows"
    return tot


# (name, first layer (Hkv, n, D), second, smaller layer, selection)
SEQUENCES = [
    ("topk-grid-then-lds", (8, 40000, 128), (4, 9000, 64), dict(k=3000)),
    ("topk-lds-then-smaller", (8, 16000, 128), (2, 5000, 128), dict(k=700)),
    ("tau", (8, 32768, 128), (3, 3000, 64), dict(tau=0.2)),
    ("layer-budget", (8, 30000, 128), (2, 20000, 128), dict(k=50000, scope="layer")),
]


@pytest.mark.parametrize("name,first,second,sel", SEQUENCES, ids=[s[0] for s in SEQUENCES])
def test_noalloc_equals_evict_on_two_calls(name, first, second, sel):
    for i, (Hkv, n, D) in enumerate((first, second)):
        say(f"[noalloc] {name} call {i}: Hkv={Hkv} n={n} D={D} {sel}")
        s, K, V = _layer(300 + i, Hkv, n, D)
        e = kvs.evict_desc(s, K, window=128, **sel)
        assert kvs.evict_workspace_bytes(e) <= kvs.EVICT_NOALLOC_MAX_WORKSPACE
        ref = kvs.evict(s, K, V, window=128, outputs=_outs(e), **sel)
        got = kvs.evict_noalloc(s, K, V, window=128, outputs=_outs(e), **sel)
        torch.cuda.synchronize()
        tot = _same(got, ref, f"{name} call {i}")
        assert tot > 0


def test_noalloc_long_heads_past_its_scratch_take_the_grid_selection():
    """Per-head top-k on 20 KV heads of 120,000 tokens: kv_evict's long-head
    kernels need more workspace than the scratch holds, so kv_evict_noalloc
    selects with the grid's histogram passes instead. Both are exact: the
    outputs must still be identical, on two calls in a row (the second on a
    smaller layer that takes the long-head kernels inside the scratch)."""
    for i, (Hkv, n) in enumerate(((20, 120000), (4, 30000))):
        say(f"[noalloc] long heads call {i}: Hkv={Hkv} n={n}")
        g = torch.Generator(device="cuda")
        g.manual_seed(500 + i)
        s = torch.rand((Hkv, n), device="cuda", generator=g)
        K = torch.randn((Hkv, n, 64), device="cuda", generator=g).to(torch.bfloat16)
        V = torch.randn((Hkv, n, 64), device="cuda", generator=g).to(torch.bfloat16)
        e = kvs.evict_desc(s, K, window=128, k=n // 4)
        assert (kvs.evict_workspace_bytes(e) > kvs.EVICT_NOALLOC_MAX_WORKSPACE) == (i == 0)
        ref = kvs.evict(s, K, V, window=128, k=n // 4, outputs=_outs(e))
        got = kvs.evict_noalloc(s, K, V, window=128, k=n // 4, outputs=_outs(e))
        torch.cuda.synchronize()
        assert _same(got, ref, f"long heads call {i}") == Hkv * (n // 4 + 128)
        del s, K, V, ref, got


def test_noalloc_rejects_layers_past_its_scratch():
    Hkv, n = 300, 1000  # threshold mode: the grid path, 24 KiB of histograms per head
    s = torch.zeros((Hkv, n), dtype=torch.float32, device="cuda")
    K = torch.zeros((Hkv, n, 64), dtype=torch.bfloat16, device="cuda")
    e = kvs.evict_desc(s, K, window=8, tau=0.5)
    assert kvs.evict_workspace_bytes(e) > kvs.EVICT_NOALLOC_MAX_WORKSPACE
    with pytest.raises(kvs.KvsError) as ei:
        kvs.evict_noalloc(s, K, K, window=8, tau=0.5, outputs=_outs(e))
    assert ei.value.status == kvs.KVS_EWORKSPACE


def test_noalloc_in_a_fresh_order_after_evict_calls():
    """The same as above with the entry points called in the other order
    (the scratch first meets a call after ordinary kv_evict calls ran)."""
    for i, (Hkv, n, D, k) in enumerate(((4, 20000, 128, 5000), (2, 300, 128, 20))):
        s, K, V = _layer(400 + i, Hkv, n, D)
        e = kvs.evict_desc(s, K, window=16, k=k)
        got = kvs.evict_noalloc(s, K, V, window=16, k=k, outputs=_outs(e))
        ref = kvs.evict(s, K, V, window=16, k=k, outputs=_outs(e))
        torch.cuda.synchronize()
        _same(got, ref, f"reverse call {i}")
