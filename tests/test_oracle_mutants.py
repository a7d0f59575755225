"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin catches each. A mutant is the oracle's source with one edit, loaded
as a separate module and swapped in for the ``oracle`` package's functions."""
import inspect
import types

import pytest

import oracle
import oracle.reference as ref
import pins

MUTANTS = {
    "gqa-mapping-modulo": ("return g // G", "return g % G"),
    "self-diagonal-excluded": ("self_pos[None, :] <= rows[:, None]", "self_pos[None, :] < rows[:, None]"),
    "self-keys-dropped": ("return np.concatenate([l_ctx, l_self], axis=1)", "return l_ctx"),
    "causal-diagonal-excluded": ("np.where(keys[None, :] <= rows[:, None], l, -np.inf)",
                                 "np.where(keys[None, :] < rows[:, None], l, -np.inf)"),
    "ctx-logit-unscaled": ("l_ctx = scale * (q_rows @ Kctx_h.T)", "l_ctx = (q_rows @ Kctx_h.T)"),
    "lse-max-term-dropped": ("for j in blk]] = M[:, 0] + np.log(", "for j in blk]] = np.log("),
    "window-edge-exclusive": ("keys[None, :] + window <= rows[:, None]", "keys[None, :] + window < rows[:, None]"),
    "max-hnorm-dropped": ("w = a * vn[h][None, :] / hn[j0:j1, None]\n            s[h]",
                          "w = a * vn[h][None, :]\n            s[h]"),
    "max-vnorm-dropped": ("w = a * vn[h][None, :] / hn[j0:j1, None]\n            s[h]",
                          "w = a / hn[j0:j1, None]\n            s[h]"),
    "max-lse-sign": ("a = np.exp(scale * (Qf[g, j0:j1] @ Kc[h].T) - lse_in[g, j0:j1, None])",
                     "a = np.exp(scale * (Qf[g, j0:j1] @ Kc[h].T) + lse_in[g, j0:j1, None])"),
    "max-overwrites": ("s[h] = np.maximum(s[h], w.max(axis=0))", "s[h] = w.max(axis=0)"),
    "max-key-axis": ("s[h] = np.maximum(s[h], w.max(axis=0))", "s[h] = np.maximum(s[h], w.max(axis=1).max())"),
    "sum-group-overwrites": ("t[h] += w.sum(axis=0)", "t[h] = w.sum(axis=0)"),
    "sum-hnorm-multiplies": ("a * vn[h][None, :] / hn[j0:j1, None], 0.0)", "a * vn[h][None, :] * hn[j0:j1, None], 0.0)"),
    "attn-unnormalised": ("O[g, cols] = (E / tot) @ vals", "O[g, cols] = E @ vals"),
    "attn-self-values-reversed": ("vals = np.concatenate([Vc[h], Vs[h][c0:c1]], axis=0)",
                                  "vals = np.concatenate([Vc[h], Vs[h][c0:c1][::-1]], axis=0)"),
    "attn-causal-value-head": ("if mask == REPEAT else Vc[h]", "if mask == REPEAT else Vc[(h + 1) % Hkv]"),
    "attn-lse-max-dropped": ("L_out[g, cols] = M[:, 0] + np.log(tot[:, 0])", "L_out[g, cols] = np.log(tot[:, 0])"),
    "vnorm-next-head-block": ("W_h = Wf[:, h * D:(h + 1) * D]", "W_h = Wf[:, ((h + 1) % Hkv) * D:((h + 1) % Hkv + 1) * D]"),
    "vnorm-no-sqrt": ("out[h, i0:i1] = np.sqrt((Y * Y).sum(axis=1))", "out[h, i0:i1] = (Y * Y).sum(axis=1)"),
    "vnorm-l1-norm": ("out[h, i0:i1] = np.sqrt((Y * Y).sum(axis=1))", "out[h, i0:i1] = np.abs(Y).sum(axis=1)"),
    "decode-next-head-rows": ("r0, r1 = int(offs[h]), int(offs[h + 1])",
                              "r0, r1 = int(offs[(h + 1) % Hkv]), int(offs[(h + 1) % Hkv + 1])"),
    "decode-unnormalised": ("O[g] = (E / tot) @ Vf[r0:r1]", "O[g] = E @ Vf[r0:r1]"),
    "decode-last-row-dropped": ("L = scale * (Qf[g] @ Kf[r0:r1].T)", "r1 = max(r0 + 1, r1 - 1)\n        L = scale * (Qf[g] @ Kf[r0:r1].T)"),
    "layer-ties-head-descending": ("order = np.lexsort((pos, heads, neg, is_nan))",
                                   "order = np.lexsort((pos, -heads, neg, is_nan))"),
    "layer-scope-per-head-k": ("kk = min(max(int(k), 0), vals.size)", "kk = min(max(int(k), 0), n - w)"),
    "window-not-kept": ("keep[n - w:] = True", "pass"),
    "threshold-strict": ("keep[cand] |= s[cand] >= float(np.float32(tau))", "keep[cand] |= s[cand] > float(np.float32(tau))"),
    "ties-higher-index-first": ("order = np.lexsort((cand, neg, is_nan))", "order = np.lexsort((-cand, neg, is_nan))"),
    "topk-ascending": ("neg = np.where(is_nan, 0.0, -s[cand])", "neg = np.where(is_nan, 0.0, s[cand])"),
    "compact-reversed": ("K_out[offsets[h]:offsets[h + 1]] = K[h, idx]", "K_out[offsets[h]:offsets[h + 1]] = K[h, idx[::-1]]"),
    "stream-leaves-late": ("q = p - w  # the token that has just left", "q = p - w - 1  # the token that has just left"),
    "stream-strict": ("if q >= 0 and s[h, q] >= tau32:", "if q >= 0 and s[h, q] > tau32:"),
    "stream-slot-offset": ("slot_pos[h, p % w] = p", "slot_pos[h, (p + 1) % w] = p"),
    "compact-offsets-shifted": ("offsets = np.concatenate([[0], np.cumsum(counts)])",
                                "offsets = np.concatenate([np.cumsum(counts), [0]])"),
}

EXPORTED = ["lse", "attention", "attention_weights", "max_scores", "future_mass", "decode_attention", "value_norms", "select", "compact",
            "stream_states",
            "visible_logits", "kv_head_of", "outside_window"]


def _mutant_module(old, new):
    src = inspect.getsource(ref)
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(name, monkeypatch):
    mod = _mutant_module(*MUTANTS[name])
    for attr in EXPORTED:
        monkeypatch.setattr(oracle, attr, getattr(mod, attr))
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except Exception as e:  # an assertion or an error raised by the mutant
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutant {name}"


def test_unmutated_oracle_passes_all_pins():
    for pin in pins.ALL_PINS:
        pin()
