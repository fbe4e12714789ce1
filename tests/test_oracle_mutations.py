"""Plant plausible mistakes in copies of the oracle (on the CPU) and require
that at least one pin catches each.  This shows the pins are strong enough to
trust the oracle: a dropped term, a wrong sign or index, a transposed operand
or a wrong head mapping all fail."""

import inspect
import types

import pytest

import oracle.tree_attention_oracle as orc_src
from oracle_pins import ALL_PINS

MUTATIONS = {
    "mask_excludes_self": ("            j = i\n            while j != -1:",
                           "            j = int(p[b, i])\n            while j != -1:"),
    "mask_transposed": ("visible[:, L:] = anc[b]", "visible[:, L:] = anc[b].T"),
    "mask_bit_word": ("out[b, i, j // 64] |=", "out[b, i, 0] |="),
    "mask_bit_shift": ("np.uint64(j % 64)", "np.uint64(j % 63)"),
    "scale_dropped": ("s = scale * (q[b, :, h, :] @ keys.T)", "s = (q[b, :, h, :] @ keys.T)"),
    "lse_drops_max": ("lse = (m + np.log(z))[:, 0]", "lse = np.log(z)[:, 0]"),
    "o_not_normalised": ("o = (e @ vals) / z", "o = (e @ vals)"),
    "gqa_interleaved": ("for h in range(g * G, (g + 1) * G):\n                s = scale * (q[b, :, h, :] @ keys.T)\n                o[b, :, h, :]",
                        "for h in range(g, Hq, Hkv):\n                s = scale * (q[b, :, h, :] @ keys.T)\n                o[b, :, h, :]"),
    "keys_tree_first": ("keys = np.concatenate([kp[off[b]:off[b + 1], g, :], kt[b, :, g, :]])",
                        "keys = np.concatenate([kt[b, :, g, :], kp[off[b]:off[b + 1], g, :]])"),
    "values_from_keys": ("vals = np.concatenate([vp[off[b]:off[b + 1], g, :], vt[b, :, g, :]])",
                         "vals = np.concatenate([kp[off[b]:off[b + 1], g, :], vt[b, :, g, :]])"),
    "prefix_from_start": ("keys = np.concatenate([kp[off[b]:off[b + 1], g, :]",
                          "keys = np.concatenate([kp[0:off[b + 1] - off[b], g, :]"),
    "parent_allows_self": ("if not (-1 <= int(p[b, i]) <= i - 1):", "if not (-1 <= int(p[b, i]) <= i):"),
    "merge_unnormalised": ("o = sum((w[k] / z)[..., None]", "o = sum((w[k])[..., None]"),
    "merge_lse_no_max": ("lse = m + np.log(z)\n", "lse = np.log(z)\n"),
    "prefix_attn_wrong_head": ("            keys = kp[off[b]:off[b + 1], h // G, :]", "            keys = kp[off[b]:off[b + 1], h % Hkv, :]"),
    "prefix_attn_values_from_keys": ("            vals = vp[off[b]:off[b + 1], h // G, :]", "            vals = kp[off[b]:off[b + 1], h // G, :]"),
    "prefix_attn_scale_dropped": ("            s = (q[b, :, h, :] @ keys.T) * scale          # [T, L_b]", "            s = (q[b, :, h, :] @ keys.T)          # [T, L_b]"),
    "commit_wrong_source": ("            kc[d + j] = kt[b, int(acc[b, j])]", "            kc[d + j] = kt[b, j]"),
    "commit_off_by_one": ("        ok = 0 <= n <= T and 0 <= d and d + n <= rows", "        ok = 0 <= n <= T and 0 <= d and d + n < rows"),
    "commit_values_from_keys": ("            vc[d + j] = vt[b, int(acc[b, j])]", "            vc[d + j] = kt[b, int(acc[b, j])]"),
    "rope_position_off_by_one": ("            rot = np.exp(1j * (L + depth[b, i] - 1) * theta)", "            rot = np.exp(1j * (L + depth[b, i]) * theta)"),
    "rope_adjacent_pairs": ("                z = (x[:, :half] + 1j * x[:, half:]) * rot", "                z = (x[:, 0::2] + 1j * x[:, 1::2]) * rot"),
    "rope_theta_exponent": ("    theta = np.power(float(base), -2.0 * np.arange(half) / D)", "    theta = np.power(float(base), -1.0 * np.arange(half) / D)"),
    "rope_q_only_for_k": ("            for x in (q[b, i], kt[b, i]):", "            for x in (q[b, i],):"),
    "round_ties_away": ("    return np.ldexp(np.rint(m * 256.0) / 256.0, e)", "    return np.ldexp(np.floor(m * 256.0 + 0.5) / 256.0, e)"),
    "window_off_by_one": ("(kpos[None, :] > qpos[:, None] - window)", "(kpos[None, :] >= qpos[:, None] - window)"),
    "window_tree_position": ("kpos = np.concatenate([np.arange(L), L + depth[b] - 1])", "kpos = np.concatenate([np.arange(L), L + depth[b]])"),
    "window_ignores_branch": ("        visible = on_branch & in_window\n", "        visible = in_window\n"),
    "window_values_from_keys": ("            vals = np.concatenate([vc[off[b]:off[b + 1], g, :], vt[b, :, g, :]])", "            vals = np.concatenate([kc[off[b]:off[b + 1], g, :], vt[b, :, g, :]])"),
    "strided_head_offset": ("            out[r, g, :] = flat[start + g * D: start + g * D + D]", "            out[r, g, :] = flat[start + g: start + g + D]"),
    "strided_row_start": ("        start = r * row_stride", "        start = r * Hkv * D"),
    "paged_row_from_page_index": ("            rows.append(pages[page, j % page_size])", "            rows.append(pages[page, j // page_size])"),
    "paged_wrong_page_slot": ("            page = int(bt[b, j // page_size])", "            page = int(bt[b, j % page_size])"),
    "rows_wrong_head": ("        g = h // G\n        if (b, g) not in cache:", "        g = h % Hkv\n        if (b, g) not in cache:"),
}


def _mutant(name):
    src = inspect.getsource(orc_src)
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation {name} does not apply uniquely"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:  # AssertionError, or a crash caused by the mistake
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
