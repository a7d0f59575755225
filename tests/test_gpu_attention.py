"""Attention forward (O and LSE) against the CPU oracle through the C ABI:
repeat and causal visibility, D = 64 and 128, GQA groups of 1 to 6, ragged
chunks and tails, no context, one query, and a long context."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_eviction_lse_amd as kvs  # noqa: E402
from gpu_util import bf16_abs, check_attn_out, check_lse, dev_bf16, host, host_bits, say  # noqa: E402


def _run(d, mask, chunk):
    Q, K, V = dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), dev_bf16(d["V"])
    Ks = dev_bf16(d["Kself"]) if mask == "repeat" else None
    Vs = dev_bf16(d["Vself"]) if mask == "repeat" else None
    O, L = kvs.attention(Q, K, V, Ks, Vs, scale=d["scale"], mask=mask, chunk=chunk)
    torch.cuda.synchronize()
    return host_bits(O), host(L)


def _ref(d, mask, chunk, rows=None):
    args = (d["Q"], d["Kctx"], d.get("Kself"))
    O, L = oracle.attention(*args, d["V"], d.get("Vself"), d["scale"], mask, chunk, rows=rows)
    Oa, _ = oracle.attention(*args, bf16_abs(d["V"]), bf16_abs(d["Vself"]) if "Vself" in d else None,
                             d["scale"], mask, chunk, rows=rows)
    return O, L, Oa


CASES = [
    # name, recipe kwargs, mask, chunk
    ("repeat-g2-d64", dict(Hq=4, Hkv=2, D=64, n_ctx=256, n_q=256, q_prescale=0.125, scale=1.0), "repeat", 256),
    ("repeat-g5-ragged-chunks-peaky", dict(Hq=10, Hkv=2, D=128, n_ctx=1000, n_q=700, lowrank_rank=8,
                                           lowrank_scale=2.0), "repeat", 300),
    ("repeat-g6-chunk1", dict(Hq=6, Hkv=1, D=128, n_ctx=77, n_q=130), "repeat", 1),
    ("repeat-no-context", dict(Hq=4, Hkv=1, D=64, n_ctx=0, n_q=200), "repeat", 64),
    ("repeat-one-query", dict(Hq=8, Hkv=8, D=128, n_ctx=513, n_q=1), "repeat", 1),
    ("causal-g6-ragged", dict(Hq=6, Hkv=1, D=128, n_ctx=777, n_q=777, mask="causal"), "causal", 0),
    ("causal-g4-sinks-d64", dict(Hq=8, Hkv=2, D=64, n_ctx=1000, n_q=1000, mask="causal", sinks=4), "causal", 0),
    ("causal-tiny", dict(Hq=2, Hkv=1, D=128, n_ctx=3, n_q=3, mask="causal"), "causal", 0),
    # key tiles go through LDS 4 to a stage; workgroups hold 12 query
    # subtiles: one whole stage of context tiles, a stage plus one tile, and a
    # last workgroup with 3 of its 12 subtiles filled
    ("repeat-one-stage", dict(Hq=4, Hkv=1, D=128, n_ctx=128, n_q=70), "repeat", 64),
    ("repeat-stage-plus-one-g3", dict(Hq=3, Hkv=1, D=64, n_ctx=160, n_q=132), "repeat", 40),
    ("causal-five-tiles-g5", dict(Hq=5, Hkv=1, D=128, n_ctx=129, n_q=129, mask="causal"), "causal", 0),
]


@pytest.mark.parametrize("name,kw,mask,chunk", CASES, ids=[c[0] for c in CASES])
def test_attention_parity(name, kw, mask, chunk):
    kw = dict(kw)
    kw.setdefault("mask", mask)
    kw["chunk"] = chunk
    d = synth.draw(synth.Recipe(**kw), 901)
    say(f"[attn] {name}")
    O, L = _run(d, mask, chunk)
    ref_O, ref_L, ref_abs = _ref(d, mask, chunk)
    check_lse(L, ref_L, name)
    check_attn_out(O, ref_O, ref_abs, name)


def test_attention_long_context_sampled_rows():
    """20k context keys, peaky queries: the shared offset and the fp32 sums
    hold over 600+ key tiles (rows sampled for the oracle)."""
    r = synth.Recipe(Hq=8, Hkv=2, D=128, n_ctx=20000, n_q=512, chunk=256, lowrank_rank=8, lowrank_scale=2.0)
    d = synth.draw(r, 903)
    say("[attn] long context")
    O, L = _run(d, "repeat", 256)
    rows = np.array([0, 1, 31, 32, 255, 256, 300, 511])
    ref_O, ref_L, ref_abs = _ref(d, "repeat", 256, rows=rows)
    check_lse(L[:, rows], ref_L, "long-context")
    check_attn_out(O[:, rows], ref_O, ref_abs, "long-context")


def test_attention_lse_matches_the_lse_pass():
    """The attention kernel's LSE and kvscore_lse agree to the LSE bar."""
    r = synth.Recipe(Hq=8, Hkv=2, D=128, n_ctx=3000, n_q=1024, chunk=512, lowrank_rank=8, lowrank_scale=2.0)
    d = synth.draw(r, 905)
    Q, K, Ks = dev_bf16(d["Q"]), dev_bf16(d["Kctx"]), dev_bf16(d["Kself"])
    say("[attn] lse vs lse pass")
    _, L_attn = kvs.attention(Q, K, dev_bf16(d["V"]), Ks, dev_bf16(d["Vself"]), scale=d["scale"], mask="repeat",
                              chunk=512)
    L_pass = kvs.lse(Q, K, Ks, scale=d["scale"], mask="repeat", chunk=512)
    torch.cuda.synchronize()
    assert float((L_attn - L_pass).abs().max()) <= 1e-3
