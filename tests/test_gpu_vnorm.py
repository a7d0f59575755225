"""Value norms ||W_O v_i|| (kvscore_vnorm) against the CPU oracle through the
C ABI: D = 64 and 128, ragged key blocks and feature tiles, padded strides,
empty inputs, and sampled keys of the 32k layer's shape.

Tolerance (fp32 sums of exact bf16 products): each output feature y_f is a
D-term fp32 sum, so |dy_f| <= (D + 2) u sum_d |w_fd v_d|; the lane-wise sum
of d_model / 2 squares adds (d_model / 2 + 8) u relative. With
A = || |W_h| |v_i| || (the oracle's value for |W|, |V|):
    |gpu - ref| <= (d_model / 2 + 8) u ref + (D + 2) u A,   u = 2^-24.
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
from gpu_util import bf16_abs, dev_bf16, host, say  # noqa: E402

U = 2.0 ** -24


def _check(gpu, V, W, Hkv, what):
    ref = oracle.value_norms(V, W, Hkv)
    A = oracle.value_norms(bf16_abs(V), bf16_abs(W), Hkv)
    D, d_model = V.shape[2], W.shape[0]
    tol = (d_model / 2 + 8) * U * ref + (D + 2) * U * A
    err = np.abs(gpu.astype(np.float64) - ref)
    assert np.all(np.isfinite(gpu)), what
    assert np.all(err <= tol), f"{what}: worst err/tol {np.max(err / np.maximum(tol, 1e-300)):.2f}"


CASES = [
    # name, Hkv, n, D, d_model
    ("cfg1-shape-ragged-keys", 2, 1000, 128, 1536),
    ("d64-ragged-features", 3, 33, 64, 100),
    ("one-key", 1, 1, 128, 64),
    ("features-below-one-tile", 2, 600, 128, 40),
    ("ragged-last-feature-tile", 2, 700, 128, 200),  # tiles of 128 features: 128 + 72
]


@pytest.mark.parametrize("name,Hkv,n,D,d_model", CASES, ids=[c[0] for c in CASES])
def test_vnorm_parity(name, Hkv, n, D, d_model):
    V = synth.normal_bf16(71, 1, (Hkv, n, D))
    W = synth.normal_bf16(71, 2, (d_model, Hkv * D), std=0.02)
    say(f"[vnorm] {name}")
    g = kvs.value_norms(dev_bf16(V), dev_bf16(W))
    torch.cuda.synchronize()
    _check(host(g), V, W, Hkv, name)


def test_vnorm_padded_strides():
    Hkv, n, D, d_model = 2, 700, 128, 512
    V = synth.normal_bf16(73, 1, (Hkv, n, D))
    W = synth.normal_bf16(73, 2, (d_model, Hkv * D), std=0.02)
    Vp = torch.zeros((Hkv, n + 5, D + 64), dtype=torch.bfloat16, device="cuda")
    Vp[:, :n, :D] = dev_bf16(V)
    Wp = torch.zeros((d_model, Hkv * D + 16), dtype=torch.bfloat16, device="cuda")
    Wp[:, :Hkv * D] = dev_bf16(W)
    say("[vnorm] padded strides")
    g = kvs.value_norms(Vp[:, :n, :D], Wp[:, :Hkv * D])
    torch.cuda.synchronize()
    _check(host(g), V, W, Hkv, "padded")


def test_vnorm_empty_inputs():
    V = dev_bf16(synth.normal_bf16(75, 1, (2, 300, 128)))
    W0 = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    out = torch.full((2, 300), 7.0, device="cuda")
    kvs.value_norms(V, W0, out=out)
    g = kvs.value_norms(torch.empty((2, 0, 128), dtype=torch.bfloat16, device="cuda"),
                        dev_bf16(synth.normal_bf16(75, 2, (64, 256))))
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0 and g.numel() == 0


def test_vnorm_32k_layer_sampled_keys():
    """Qwen3-8B shape: 8 KV heads x 32768 keys, d_model 4096; keys sampled for the oracle."""
    Hkv, n, D, d_model = 8, 32768, 128, 4096
    V = synth.normal_bf16(77, 1, (Hkv, n, D))
    W = synth.normal_bf16(77, 2, (d_model, Hkv * D), std=0.02)
    say("[vnorm] 32k layer")
    g = host(kvs.value_norms(dev_bf16(V), dev_bf16(W)))
    keys = np.unique(np.concatenate([np.arange(0, n, 997), [0, 1, 511, 512, n - 1]]))
    _check(g[:, keys], np.ascontiguousarray(V[:, keys]), W, Hkv, "32k")
