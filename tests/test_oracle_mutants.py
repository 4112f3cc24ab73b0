"""Planted mistakes: every plausible slip in the oracle must be caught by a pin (CPU).

Each mutant is a textual change to a copy of an oracle module's source,
executed in a fresh namespace; the real oracle files are never touched.
"""
import importlib
import os
import types

import pytest

import test_oracle
import test_oracle_bwd
import test_oracle_tiles

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def _mutant(module_file, old, new, extra_globals=None):
    with open(os.path.join(ORACLE_DIR, module_file), encoding="utf-8") as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__.update(extra_globals or {})
    code = compile(src.replace("from .attention import dense_mask", "from oracle.attention import dense_mask"),
                   module_file, "exec")
    exec(code, mod.__dict__)
    return mod


def _caught(pins, fn):
    for pin in pins:
        try:
            pin(fn)
        except Exception:          # a failed assertion or a crash both expose the mutant
            return True
    return False


ATTN_MUTANTS = {
    "exclusive_end": ("(j[None, :] <= e[k][:, None])", "(j[None, :] < e[k][:, None])"),
    "exclusive_start": ("(j[None, :] >= s[k][:, None])", "(j[None, :] > s[k][:, None])"),
    "union_keeps_last_range": ("        M |= (j[None, :]", "        M = (j[None, :]"),
    "union_as_intersection": ("    M = np.zeros((s.shape[1], N), dtype=bool)\n    for k in range(s.shape[0]):\n        M |= ",
                              "    M = np.ones((s.shape[1], N), dtype=bool)\n    for k in range(s.shape[0]):\n        M &= "),
    "dropped_scale": ("S = scale64 * (qh @ kh.T)", "S = (qh @ kh.T)"),
    "scale_squared": ("S = scale64 * (qh @ kh.T)", "S = scale64 * scale64 * (qh @ kh.T)"),
    "lse_without_max": ("m[ok] + np.log(l[ok])", "np.log(l[ok])"),
    "unnormalised": ("num[ok] / l[ok][:, None]", "num[ok]"),
    "k_for_v": ("vh = np.asarray(v[b, h][support]", "vh = np.asarray(k[b, h][support]"),
    "mask_ignored": ("S = np.where(Ms, S, -np.inf)", "S = S"),
    "off_by_one_row": ("qh = np.asarray(q[b, h][rr]", "qh = np.asarray(q[b, h][np.maximum(rr - 1, 0)]"),
    "log2_lse": ("m[ok] + np.log(l[ok])", "m[ok] + np.log2(l[ok])"),
}


@pytest.mark.parametrize("name", sorted(ATTN_MUTANTS))
def test_attention_mutant_is_caught(name):
    old, new = ATTN_MUTANTS[name]
    mod = _mutant("attention.py", old, new)
    assert _caught(test_oracle.ALL_PINS, mod.attention), f"mutant {name} survived every pin"


TILE_MUTANTS = {
    "skip_left_inclusive": ("if khi < min_s or klo > max_e:", "if khi <= min_s or klo > max_e:"),
    "skip_right_inclusive": ("if khi < min_s or klo > max_e:", "if khi < min_s or klo >= max_e:"),
    "no_right_skip": ("if khi < min_s or klo > max_e:", "if khi < min_s:"),
    "khi_exclusive": ("khi = min(klo + Bc, N) - 1\n            if khi < min_s", "khi = min(klo + Bc, N)\n            if khi < min_s"),
    "full_swapped_bounds": ("elif klo >= max_s and khi <= min_e:", "elif klo >= min_s and khi <= max_e:"),
    "full_start_only": ("elif klo >= max_s and khi <= min_e:", "elif klo >= max_s:"),
    "page_literal_skip": ("if khi < min_s or klo > max_e:", "if khi + 1 <= s[rows[-1]]:"),
    "rows_not_clipped": ("rows = range(t * Br, min(t * Br + Br, N))", "rows = range(t * Br, min(t * Br + Br, N - 1))"),
}


@pytest.mark.parametrize("name", sorted(TILE_MUTANTS))
def test_tile_mutant_is_caught(name):
    import oracle
    old, new = TILE_MUTANTS[name]
    mod = _mutant("tiles.py", old, new, {"dense_mask": oracle.dense_mask})
    assert _caught(test_oracle_tiles.ALL_PINS, mod.classes_minmax), f"mutant {name} survived every pin"


MULTI_TILE_MUTANTS = {
    "skip_if_any_range_skips": ("        out = np.where((out == SKIP) & (tab != SKIP), PARTIAL, out)\n    for tab in per_k:\n        out = np.where(tab == FULL, FULL, out)",
                                "        out = np.where((out == SKIP) & (tab != SKIP), PARTIAL, out)\n    out = np.where(np.any([t == SKIP for t in per_k], axis=0), SKIP, out)\n    for tab in per_k:\n        out = np.where(tab == FULL, FULL, out)"),
    "full_ignored": ("        out = np.where(tab == FULL, FULL, out)", "        out = out"),
    "first_range_only": ("range(s_all.shape[0])]", "range(1)]"),
}


@pytest.mark.parametrize("name", sorted(MULTI_TILE_MUTANTS))
def test_multi_tile_mutant_is_caught(name):
    import oracle
    old, new = MULTI_TILE_MUTANTS[name]
    mod = _mutant("tiles.py", old, new, {"dense_mask": oracle.dense_mask})
    assert _caught(test_oracle_tiles.MULTI_PINS, mod.classes_minmax_multi), f"mutant {name} survived every pin"


BWD_MUTANTS = {
    "no_row_correction": ("dS = P * (dP - Dr[:, None])", "dS = P * dP"),
    "row_correction_sign": ("dS = P * (dP - Dr[:, None])", "dS = P * (dP + Dr[:, None])"),
    "row_correction_from_dP": ("Dr = (P * dP).sum(axis=1)", "Dr = dP.sum(axis=1)"),
    "dq_without_scale": ("dQ[b, h][rr] = scale64 * (dS @ kh)", "dQ[b, h][rr] = (dS @ kh)"),
    "dk_without_scale": ("dK[b, h][support] += scale64 * (dS.T @ qh)", "dK[b, h][support] += (dS.T @ qh)"),
    "dq_with_v": ("dQ[b, h][rr] = scale64 * (dS @ kh)", "dQ[b, h][rr] = scale64 * (dS @ vh)"),
    "dv_from_dS": ("dV[b, h][support] += P.T @ doh", "dV[b, h][support] += dS.T @ doh"),
    "unnormalised_P": ("P[attended] = p[attended] / l[attended][:, None]", "P[attended] = p[attended]"),
    "mask_ignored": ("S = np.where(Ms, S, -np.inf)", "S = S"),
    "dP_with_k": ("dP = doh @ vh.T", "dP = doh @ kh.T"),
    "dk_overwritten": ("dK[b, h][support] += scale64", "dK[b, h][support] = scale64"),
    "dv_overwritten": ("dV[b, h][support] += P.T", "dV[b, h][support] = P.T"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name):
    old, new = BWD_MUTANTS[name]
    mod = _mutant("backward.py", old, new)
    assert _caught(test_oracle_bwd.ALL_BWD_PINS, mod.attention_bwd), f"mutant {name} survived every pin"


NONSKIP_MUTANTS = {
    "skip_left_inclusive": ("(khi[None, :] < min_s[:, None])", "(khi[None, :] <= min_s[:, None])"),
    "skip_right_inclusive": ("(klo[None, :] > max_e[:, None])", "(klo[None, :] >= max_e[:, None])"),
    "no_right_skip": ("skip = (khi[None, :] < min_s[:, None]) | (klo[None, :] > max_e[:, None])",
                      "skip = (khi[None, :] < min_s[:, None])"),
    "khi_exclusive": ("khi = np.minimum(klo + Bc, N) - 1", "khi = np.minimum(klo + Bc, N)"),
    "largest_start": ("s[t * Br:min(t * Br + Br, N)].min()", "s[t * Br:min(t * Br + Br, N)].max()"),
    "rows_not_clipped": ("e[t * Br:min(t * Br + Br, N)].max()", "e[t * Br:min(t * Br + Br - 1, N)].max()"),
}


@pytest.mark.parametrize("name", sorted(NONSKIP_MUTANTS))
def test_nonskip_mutant_is_caught(name):
    import oracle
    old, new = NONSKIP_MUTANTS[name]
    mod = _mutant("tiles.py", old, new, {"dense_mask": oracle.dense_mask})
    assert _caught(test_oracle_tiles.NONSKIP_PINS, mod.nonskip_counts), f"mutant {name} survived every pin"
