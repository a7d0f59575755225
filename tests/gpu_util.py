"""Helpers shared by the GPU tests: device copies and the parity checks.

Tolerances (fp32 kernels against the fp64 oracle):
  LSE: |gpu - ref| <= 1e-3
  scores: |gpu - ref| / ref <= 5e-3 where ref >= 1e-6, else |gpu - ref| <= 1e-8
  kept sets: identical, except keys whose oracle score is within 5e-3 (relative)
  of the k-th score or of tau; compacted rows are bit copies.
  attention output O (bf16): |gpu - ref| <= 2^-8 |ref| + 2^-7 sum_i a_ji |v_id|.
    The probabilities enter the value product rounded to bf16 (relative error
    <= 2^-8 each, so <= 2^-8 sum a|v| in total), fp32 accumulation adds far
    less than another 2^-8 sum a|v|, and the final rounding of O to bf16 is
    <= 2^-8 |O|. sum_i a_ji |v_id| is the oracle's output for |V|.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

LSE_ATOL = 1e-3
SCORE_RTOL = 5e-3
SCORE_FLOOR = 1e-6
SCORE_ATOL = 1e-8


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def check_lse(gpu: np.ndarray, ref: np.ndarray, what=""):
    err = np.abs(gpu.astype(np.float64) - ref)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite LSE"
    assert err.max() <= LSE_ATOL, f"{what}: LSE max abs err {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}"
    return float(err.max())


def check_scores(gpu: np.ndarray, ref: np.ndarray, what=""):
    g = gpu.astype(np.float64)
    big = ref >= SCORE_FLOOR
    rel = np.abs(g - ref)[big] / ref[big]
    small = np.abs(g - ref)[~big]
    assert np.all(np.isfinite(g)), f"{what}: non-finite score"
    if rel.size:
        assert rel.max() <= SCORE_RTOL, f"{what}: score max rel err {rel.max():.3e}"
    if small.size:
        assert small.max() <= SCORE_ATOL, f"{what}: small-score max abs err {small.max():.3e}"
    return float(rel.max()) if rel.size else 0.0


def kept_from_gpu(kept_idx: np.ndarray, offs: np.ndarray):
    return [kept_idx[offs[h]:offs[h + 1]].astype(np.int64) for h in range(offs.size - 1)]


def check_kept(gpu_kept, ref_kept, ref_scores, *, k=None, tau=None, window=0, what=""):
    """Kept sets equal up to the exemption band; every GPU list strictly ascending."""
    for h, (g, r) in enumerate(zip(gpu_kept, ref_kept)):
        assert np.all(np.diff(g) > 0), f"{what}: head {h} not ascending"
        n = ref_scores.shape[1]
        w = min(window, n)
        if k is not None:
            assert g.size == r.size, f"{what}: head {h} kept {g.size} != {r.size}"
        diff = np.setxor1d(g, r)
        if diff.size == 0:
            continue
        assert np.all(diff < n - w), f"{what}: window key differs"
        s = ref_scores[h]
        if k is not None:
            cand = s[: n - w]
            kk = min(k, cand.size)
            kth = np.sort(cand)[::-1][kk - 1]
            band = np.abs(s[diff] - kth) <= SCORE_RTOL * kth
        else:
            band = np.abs(s[diff] - tau) <= SCORE_RTOL * tau
        assert np.all(band), f"{what}: head {h}: {int((~band).sum())} differing keys outside the band"


def check_rows(K_bits, V_bits, gpu_kept, K_out, V_out, offs, what=""):
    for h, idx in enumerate(gpu_kept):
        a, b = offs[h], offs[h + 1]
        assert np.array_equal(K_out[a:b], K_bits[h, idx]), f"{what}: K rows differ on head {h}"
        assert np.array_equal(V_out[a:b], V_bits[h, idx]), f"{what}: V rows differ on head {h}"


def bf16_abs(bits: np.ndarray) -> np.ndarray:
    """|x| of bf16 bit patterns (clears the sign bit; exact)."""
    return (np.asarray(bits, dtype=np.uint16) & np.uint16(0x7FFF)).astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def check_attn_out(gpu_bits: np.ndarray, ref: np.ndarray, ref_abs: np.ndarray, what=""):
    """O parity: gpu_bits bf16 [.., D]; ref = oracle O; ref_abs = oracle O for |V|."""
    g = bf16_to_f64(gpu_bits)
    assert np.all(np.isfinite(g)), f"{what}: non-finite O"
    err = np.abs(g - ref)
    tol = 2.0 ** -8 * np.abs(ref) + 2.0 ** -7 * ref_abs
    ratio = err / np.maximum(tol, 1e-30)
    assert np.all(err <= tol), (f"{what}: O error {err.max():.3e} exceeds its bound "
                                f"(worst ratio {ratio.max():.2f} at {np.unravel_index(ratio.argmax(), ratio.shape)})")
    return float(ratio.max())

