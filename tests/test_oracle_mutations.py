"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin catches each; this shows the pins constrain every step of the oracle."""
import numpy as np
import pytest

import oracle.dequant
import oracle.dot
import oracle.i2s
import oracle.norm
import oracle.t3
import oracle.quant
import oracle.ternary
import pins

MUTATIONS = {
    "quant_round_half_up": (oracle.quant, "_round_half_even", lambda v: np.floor(v + 0.5)),
    "quant_round_truncate": (oracle.quant, "_round_half_even", np.trunc),
    "quant_scale_128": (oracle.quant, "QMAX", 128),
    "quant_signed_max": (oracle.quant, "_row_absmax", lambda x: np.max(x, axis=1)),
    "quant_tensor_first_row_max": (oracle.quant, "_tensor_absmax",
                                   lambda x: np.float32(np.max(np.abs(x[0])))),
    "quant_tensor_signed_max": (oracle.quant, "_tensor_absmax", lambda x: np.float32(np.max(x))),
    "token_sums_of_magnitudes": (oracle.quant, "_row_total", lambda q: np.abs(q).sum(axis=1)),
    "token_sums_drop_last_k": (oracle.quant, "_row_total", lambda q: q[:, :-1].sum(axis=1)),
    "norm_sum_not_mean": (oracle.norm, "_mean_square", lambda h: oracle.norm._exact_sum_squares(h)),
    "norm_residual_half_up": (oracle.norm, "_bf16_rne_from_f32",
                              lambda v: ((np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
                                          + 0x8000) >> 16).astype(np.uint16)),
    "norm_mean_over_k_minus_1": (oracle.norm, "_mean_square",
                                 lambda h: oracle.norm._exact_sum_squares(h) / (h.shape[0] - 1)),
    "t3_digits_reversed": (oracle.t3, "POW3", oracle.t3.POW3[::-1].copy()),
    "t3_encode_floor": (oracle.t3, "_encode", lambda v: (256 * v) // 243),
    "t3_bytes_sequential": (oracle.t3, "_planes",
                            lambda w: w.reshape(w.shape[0], -1, 16, 5).transpose(0, 1, 3, 2)),
    "ternary_ge_threshold": (oracle.ternary, "_above", lambda w, t: w >= t),
    "ternary_threshold_0.7": (oracle.ternary, "THRESHOLD_FRACTION", 0.7),
    "ternary_fp32_sum": (oracle.ternary, "_exact_abs_sum",
                         lambda w: float(np.sum(np.abs(w), dtype=np.float32))),
    "ternary_signed_mean": (oracle.ternary, "_exact_abs_sum",
                            lambda w: abs(float(np.sum(w.astype(np.float64))))),
    "pack_swap_codes": (oracle.i2s, "CODE_POS", 0b10),
    "pack_bit_order_reversed": (oracle.i2s, "_field_shift", lambda j: 2 * (3 - j)),
    "pack_plain_byte_order": (oracle.i2s, "GROUP", 4),
    "dot_missing_transpose": (oracle.dot, "_as_columns", lambda w: w.astype(np.int64)),
    "dot_drops_last_k": (oracle.dot, "_as_columns",
                         lambda w: np.concatenate([w[:, :-1], 0 * w[:, -1:]], axis=1)
                         .astype(np.int64).T),
    "dequant_drops_d": (oracle.dequant, "_scale_product",
                        lambda g, d: float(np.float32(g)) * np.ones(np.shape(d))),
    "bf16_ties_away": (oracle.dequant, "_tie_up", lambda lo_odd: np.ones_like(lo_odd)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    mod, attr, value = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, value)
    if name == "pack_swap_codes":
        monkeypatch.setattr(mod, "CODE_NEG", 0b01)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except Exception:   # AssertionError, or the oracle raising on its own check
            caught.append(pin.__name__)
    assert caught, f"mutation {name} passed every pin"
