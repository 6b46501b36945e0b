"""Plant one mistake at a time in a copy of the oracle; some pin must catch each.

Mistakes are planted on the CPU in a private copy of the oracle's source text
(the real module is untouched). A mutant that every pin accepts would mean
the pins cannot tell that mistake from the definition.
"""
import os
import types

import pytest

from tests import oracle_pins as pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
SRC = os.path.join(ORACLE_DIR, "attention.py")
PROLOGUE_SRC = os.path.join(ORACLE_DIR, "prologue.py")
LINEAR_SRC = os.path.join(ORACLE_DIR, "linear_attention.py")

MUTANTS = {
    "gqa_modulo_mapping": ("g = h // grp", "g = h % hkv"),
    "causal_top_left": ("off = (lk - lq) if offset is None else int(offset)",
                        "off = 0 if offset is None else int(offset)"),
    "causal_diagonal_masked": ("vis &= j <= (i_pos[:, None] + off)", "vis &= j < (i_pos[:, None] + off)"),
    "causal_offset_ignored": ("off = (lk - lq) if offset is None else int(offset)", "off = lk - lq"),
    "causal_offset_sign": ("off = (lk - lq) if offset is None else int(offset)",
                           "off = (lk - lq) if offset is None else -int(offset)"),
    "scale_dropped": ("s = scale * (q_rows @ k_seq.T)", "s = (q_rows @ k_seq.T)"),
    "lse_without_max": ("lse[has] = m[has] + np.log(l_sum[has])", "lse[has] = np.log(l_sum[has])"),
    "lse_log2": ("lse[has] = m[has] + np.log(l_sum[has])", "lse[has] = m[has] + np.log2(l_sum[has])"),
    "v_rows_reversed": ("o = (e @ v_seq)", "o = (e @ v_seq[::-1])"),
    "head_row_swap": ("out[rows, h, :] = o_h", "out[rows, (h + 1) % hq, :] = o_h"),
    "merge_unnormalised": ("np.exp(lse - np.where(live, lse_m, 0.0)[None, :])", "np.exp(lse - safe_max[None, :])"),
    "merge_min_not_max": ("lse_max = lse.max(axis=0)", "lse_max = lse.min(axis=0)"),
    "merge_lse_no_log": ("lse_m = np.where(live, safe_max + np.log(np.where(live, ssum, 1.0)), -np.inf)",
                         "lse_m = np.where(live, safe_max + np.where(live, ssum, 1.0), -np.inf)"),
    "chunk_drops_key": ("return (c * lk) // sp, ((c + 1) * lk) // sp", "return (c * lk) // sp, max((c * lk) // sp, ((c + 1) * lk) // sp - 1)"),
    "gather_first_token": ("idx = cu[1:] - 1", "idx = cu[:-1]"),
    "paged_page_slot_swapped": ("cache[table[b, j // page_size], j % page_size]",
                                "cache[table[b, j % page_size], j // page_size]"),
    "paged_next_page": ("cache[table[b, j // page_size], j % page_size]",
                        "cache[table[b, (j + 1) // page_size], j % page_size]"),
    "paged_table_row_of_b0": ("cache[table[b, j // page_size], j % page_size]",
                              "cache[table[0, j // page_size], j % page_size]"),
    "paged_drops_last_key": ("j = np.arange(int(used[b]), dtype=np.int64)",
                             "j = np.arange(max(int(used[b]) - 1, 0), dtype=np.int64)"),
}


PROLOGUE_MUTANTS = {
    "rotate_half_sign": ("np.concatenate([-x[..., h:], x[..., :h]], axis=-1)",
                         "np.concatenate([x[..., h:], -x[..., :h]], axis=-1)"),
    "rotate_half_no_swap": ("np.concatenate([-x[..., h:], x[..., :h]], axis=-1)",
                            "np.concatenate([-x[..., :h], x[..., h:]], axis=-1)"),
    "cos_sin_swapped": ("return x * c + rotate_half(x) * s", "return x * s + rotate_half(x) * c"),
    "rms_sum_not_mean": ("np.mean(x * x, axis=-1, keepdims=True)", "np.sum(x * x, axis=-1, keepdims=True)"),
    "rms_eps_outside_sqrt": ("x / np.sqrt(var + eps)", "x / (np.sqrt(var) + eps)"),
    "rms_weight_dropped": ("* np.asarray(weight, dtype=np.float64)", "* 1.0"),
    "k_takes_q_weight": ("rotary(rms_norm(k, k_weight, eps), cos, sin)", "rotary(rms_norm(k, q_weight, eps), cos, sin)"),
}


GDN_MUTANTS = {
    "decay_after_correction": ("s = np.exp(g[t, h]) * s\n                u = beta[t, h] * (v[t, h] - s.T @ k[t, hk])",
                               "u = beta[t, h] * (v[t, h] - s.T @ k[t, hk])\n                s = np.exp(g[t, h]) * s"),
    "beta_dropped": ("u = beta[t, h] * (v[t, h] - s.T @ k[t, hk])", "u = (v[t, h] - s.T @ k[t, hk])"),
    "delta_sign": ("u = beta[t, h] * (v[t, h] - s.T @ k[t, hk])", "u = beta[t, h] * (v[t, h] + s.T @ k[t, hk])"),
    "read_before_write": ("s = s + np.outer(k[t, hk], u)\n                out[t, h] = scale * (s.T @ q[t, hk])",
                          "out[t, h] = scale * (s.T @ q[t, hk])\n                s = s + np.outer(k[t, hk], u)"),
    "write_with_query": ("s = s + np.outer(k[t, hk], u)", "s = s + np.outer(q[t, hk], u)"),
    "head_map_modulo": ("hk = h // rep", "hk = h % hqk"),
    "state_not_reset": ("s = (np.zeros((dk, dv)) if initial_state is None", "s = (s if (b > 0 and initial_state is None) else np.zeros((dk, dv)) if initial_state is None"),
}


def _mutant_module(old, new, path=SRC):
    with open(path) as fh:
        src = fh.read()
    assert src.count(old) == 1, f"mutation site not found exactly once: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), path + " (mutant)", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant_module(*MUTANTS[name])
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            caught.append((check.__name__, type(exc).__name__))
    assert caught, f"no pin catches mutant {name}"


def test_unmutated_copy_passes():
    mod = _mutant_module("import numpy as np", "import numpy as np")
    for check in pins.ALL_CHECKS:
        check(mod)


@pytest.mark.parametrize("name", sorted(PROLOGUE_MUTANTS))
def test_prologue_mutant_is_caught(name):
    mod = _mutant_module(*PROLOGUE_MUTANTS[name], path=PROLOGUE_SRC)
    caught = []
    for check in pins.PROLOGUE_CHECKS:
        try:
            check(mod)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            caught.append((check.__name__, type(exc).__name__))
    assert caught, f"no pin catches prologue mutant {name}"


def test_unmutated_prologue_passes():
    mod = _mutant_module("import numpy as np", "import numpy as np", path=PROLOGUE_SRC)
    for check in pins.PROLOGUE_CHECKS:
        check(mod)


@pytest.mark.parametrize("name", sorted(GDN_MUTANTS))
def test_gated_delta_mutant_is_caught(name):
    mod = _mutant_module(*GDN_MUTANTS[name], path=LINEAR_SRC)
    caught = []
    for check in pins.GDN_CHECKS:
        try:
            check(mod)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            caught.append((check.__name__, type(exc).__name__))
    assert caught, f"no pin catches gated delta mutant {name}"
