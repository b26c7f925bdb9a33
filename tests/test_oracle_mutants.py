"""Plant plausible mistakes in copies of the oracle (CPU only) and check that
every one of them is caught by at least one pin."""

import os
import types

import pytest

import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "attention.py")

MUTANTS = {
    "causal_top_left": ("admissible &= j <= (L - int(q_len) + i)", "admissible &= j <= i"),
    "causal_off_by_one": ("admissible &= j <= (L - int(q_len) + i)",
                          "admissible &= j < (L - int(q_len) + i)"),
    "scale_dropped": ("scores = scale * (Qrows @", "scores = (Qrows @"),
    "scale_squared": ("scores = scale * (Qrows @", "scores = scale * scale * (Qrows @"),
    "no_normalisation": ("/ safe[:, None]", "/ 1.0"),
    "max_sign_flipped": ("np.exp(scores - m[:, None])", "np.exp(m[:, None] - scores)"),
    "gather_block_index": ("phys = np.asarray(block_table_row)[j // B]",
                           "phys = np.asarray(block_table_row)[j % B]"),
    "gather_slot_index": ("cache[phys, j % B]", "cache[phys, j // B % B]"),
    "gqa_wrong_kv_head": ("K[:, g, :], V[:, g, :], q_len, L[s],",
                          "K[:, (g + 1) % Hkv, :], V[:, g, :], q_len, L[s],"),
    "k_v_swapped": ("K[:, g, :], V[:, g, :], q_len, L[s],",
                    "V[:, g, :], K[:, g, :], q_len, L[s],"),
    "row_token_map": ("positions = np.repeat(np.arange(q_len), G)",
                      "positions = np.tile(np.arange(q_len), G)"),
    "q_rows_transposed": ("Qrows = np.asarray(q[t0:t1, heads, :], dtype=np.float64).reshape(q_len * G, d)",
                          "Qrows = np.asarray(q[t0:t1, heads, :], dtype=np.float64).transpose(1, 0, 2).reshape(q_len * G, d)"),
    "lse_missing_log_term": ("lse = np.where(has_key, m + np.log(safe), -np.inf)",
                             "lse = np.where(has_key, m, -np.inf)"),
    "merge_max_not_sum": ("wsum = w.sum(axis=0)", "wsum = w.max(axis=0)"),
    "merge_unweighted": ("merged = (w[..., None] * outs).sum(axis=0)",
                         "merged = outs.sum(axis=0) * w.mean(axis=0)[..., None]"),
    "rows_api_wrong_position": ("tokens[sel] - cu[s], K[:, g, :]", "tokens[sel] - cu[s] - 1, K[:, g, :]"),
    "fp8_bias_8": ("np.ldexp(1.0 + m / 8.0, e - 7)", "np.ldexp(1.0 + m / 8.0, e - 8)"),
    "fp8_no_subnormals": ("np.where(e == 0, np.ldexp(m / 8.0, -6),", "np.where(e == 0, 0.0 * m,"),
    "fp8_scale_not_applied": ("return decode_e4m3fn(codes) * float(np.float32(scale))",
                              "return decode_e4m3fn(codes)"),
    "fp8_ties_away": ("(above == below) & (idx % 2 == 0)", "(above == below)"),
    "fp8_overflow_to_nan": ("code = np.where(a >= 464.0, 0x7E, code)",
                            "code = np.where(a >= 464.0, 0x7F, code)"),
    "cache_write_slot_swap": ("blk, pos = slot // B, slot % B", "blk, pos = slot % B, slot // B"),
}


def load_mutant(old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text.replace(old, new), "oracle_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = load_mutant(*MUTANTS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"mutant {name} passed every pin"
