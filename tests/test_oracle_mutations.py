"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch them.

Each mutant replaces one oracle function with a subtly wrong variant; at least
one pin from tests/test_oracle_pins.py must then fail.
"""
import numpy as np
import pytest

import oracle.mla_oracle as om
import tests.test_oracle_pins as pins

PIN_TESTS = [
    pins.test_rms_norm_matches_torch_rms_norm,
    pins.test_rope_identity_norm_and_complex_form,
    pins.test_rope_scores_depend_on_relative_position_only,
    pins.test_index_build_hand_worked_fixture,
    pins.test_weight_orientation_and_row_layout_one_hot,
    pins.test_wq_b_columns_are_head_major_nope_then_rope,
    lambda: pins.test_absorbed_path_equals_explicit_wkv_b_mha(10),
    pins.test_absorbed_path_equals_explicit_mha_on_tiny_workload,
    pins.test_dense_selection_matches_torch_sdpa,
    pins.test_single_valid_entry_and_all_masked,
    pins.test_self_row_is_read_after_write,
    pins.test_zero_scale_averages_the_multiset,
    pins.test_permutation_invariance,
    pins.test_doubling_every_entry_changes_nothing_but_one_duplicate_does,
    pins.test_masked_rows_are_never_read,
    pins.test_cache_write_row_and_locality,
    pins.test_bf16_round_matches_torch_conversion,
    pins.test_index_build_multi_token_fixture,
    pins.test_multi_token_batch_equals_successive_single_token_steps,
]


def _rope_sign(x, cos, sin):
    x = np.asarray(x, dtype=np.float64)
    y = np.empty_like(x)
    y[..., 0::2] = x[..., 0::2] * cos + x[..., 1::2] * sin
    y[..., 1::2] = -x[..., 0::2] * sin + x[..., 1::2] * cos
    return y


def _rope_half(x, cos, sin):
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def _rms_eps_outside(x, g, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * np.asarray(g).reshape(-1)


def _rms_no_gamma(x, g, eps):
    return _ORIG["rms_norm"](x, np.ones_like(np.asarray(g)), eps)


def _resolve_strict(g, position, bt, bs):
    return -1 if (g < 0 or g >= position) else int(bt[g // bs]) * bs + g % bs


def _resolve_swapped(g, position, bt, bs):
    return -1 if (g < 0 or g > position) else int(bt[g % bs]) * bs + g // bs


def _resolve_table_first(g, position, bt, bs):
    phys = int(bt[g // bs])  # dereferences the table before masking
    return -1 if (g < 0 or g > position) else phys * bs + g % bs


def _core_dedup(q_lat, q_pe, keys, scale, r):
    if keys.shape[0]:
        keys = np.unique(keys, axis=0)
    return _ORIG["attention_core"](q_lat, q_pe, keys, scale, r)


def _core_no_rope_scale(q_lat, q_pe, keys, scale, r):
    nh = q_lat.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((nh, r))
    s = scale * (q_lat @ keys[:, :r].T) + q_pe @ keys[:, r:].T
    p = np.exp(s - s.max(1, keepdims=True))
    return p @ keys[:, :r] / p.sum(1, keepdims=True)


def _core_value_includes_rope(q_lat, q_pe, keys, scale, r):
    nh = q_lat.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((nh, r))
    s = scale * (q_lat @ keys[:, :r].T + q_pe @ keys[:, r:].T)
    p = np.exp(s - s.max(1, keepdims=True))
    return p @ keys[:, -r:] / p.sum(1, keepdims=True)


def _oproj_transposed_heads(o_lat, out_absorb_w, o_proj_w):
    nh, dv, r = out_absorb_w.shape
    o_v = np.stack([out_absorb_w[h] @ o_lat[h] for h in range(nh)])
    return o_v.T.reshape(-1) @ o_proj_w  # dim-major instead of head-major concat


def _ff_row_swapped(x_t, w, cos_t, sin_t, n_heads, dn, dr, r, eps):
    q_lat, q_pe, q_nope, row = _ORIG["front_fold"](x_t, w, cos_t, sin_t, n_heads, dn, dr, r, eps)
    return q_lat, q_pe, q_nope, np.concatenate([row[r:], row[:r]])


def _ff_heads_split(x_t, w, cos_t, sin_t, n_heads, dn, dr, r, eps):
    # all heads' nope first, then all rope (not head-major)
    xh = om.rms_norm(x_t, w["input_norm_w"], eps)
    c_q = om.rms_norm(xh @ w["wq_a"], w["q_norm_w"], eps)
    q = c_q @ w["wq_b"]
    q_nope = q[: n_heads * dn].reshape(n_heads, dn)
    q_pe = om.rope_interleaved(q[n_heads * dn:].reshape(n_heads, dr), cos_t, sin_t)
    kv = xh @ w["wkv_a"]
    row = np.concatenate([om.rms_norm(kv[:r], w["kv_norm_w"], eps), om.rope_interleaved(kv[r:], cos_t, sin_t)])
    q_lat = np.stack([q_nope[h] @ w["q_absorb_w"][h] for h in range(n_heads)])
    return q_lat, q_pe, q_nope, row


def _gather_ignores_this_steps_rows(rows_t, written, read_rows, kv_row):
    return _ORIG["gather_keys"](rows_t, {}, read_rows, kv_row)


def _bf16_truncate(x):
    x = np.asarray(x, dtype=np.float64).astype(np.float32)
    b = x.view(np.uint32) & np.uint32(0xFFFF0000)
    return b.view(np.float32).astype(np.float64)


_ORIG = {k: getattr(om, k) for k in ("rms_norm", "rope_interleaved", "resolve_row", "attention_core",
                                     "output_projection", "front_fold", "bf16_round", "gather_keys")}

MUTANTS = {
    "rope_sign": ("rope_interleaved", _rope_sign),
    "rope_rotate_half": ("rope_interleaved", _rope_half),
    "rms_eps_outside_root": ("rms_norm", _rms_eps_outside),
    "rms_gamma_dropped": ("rms_norm", _rms_no_gamma),
    "mask_excludes_own_position": ("resolve_row", _resolve_strict),
    "block_offset_swapped": ("resolve_row", _resolve_swapped),
    "table_read_before_mask": ("resolve_row", _resolve_table_first),
    "duplicates_deduplicated": ("attention_core", _core_dedup),
    "scale_missing_on_rope_term": ("attention_core", _core_no_rope_scale),
    "value_includes_rope_part": ("attention_core", _core_value_includes_rope),
    "heads_concat_dim_major": ("output_projection", _oproj_transposed_heads),
    "cache_row_rope_first": ("front_fold", _ff_row_swapped),
    "wq_b_not_head_major": ("front_fold", _ff_heads_split),
    "bf16_truncation": ("bf16_round", _bf16_truncate),
    "rows_written_this_step_invisible": ("gather_keys", _gather_ignores_this_steps_rows),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    fn_name, fn = MUTANTS[name]
    monkeypatch.setattr(om, fn_name, fn)
    import oracle

    monkeypatch.setattr(oracle, fn_name, fn)
    caught = []
    for t in PIN_TESTS:
        try:
            t()
        except Exception:  # an assertion, or an out-of-range table read
            caught.append(getattr(t, "__name__", "lambda"))
    assert caught, f"mutant {name} survived every pin"
