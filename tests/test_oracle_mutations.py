"""Plant plausible mistakes in the oracle (on the CPU) and check that the
pins in test_oracle_pins.py catch each one."""

import numpy as np
import pytest

import oracle
import oracle.nf4_oracle as core
import test_oracle_pins as pins


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(core, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _fails(test_fn):
    with pytest.raises(AssertionError):
        test_fn()


def test_swapped_nibble_order_is_caught(monkeypatch):
    def bad(codes):
        c = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
        if c.size % 2:
            c = np.concatenate([c, np.array([7], np.uint8)])
        return (c[1::2] | (c[0::2] << 4)).astype(np.uint8)
    _patch(monkeypatch, "pack_nibbles", bad)
    _fails(pins.test_pack_layout_by_hand_and_odd_tail)


def test_dropped_lora_scale_is_caught(monkeypatch):
    def bad(x, w, a, b, s):
        t = x @ a.T
        return x @ w.T + t @ b.T, t
    _patch(monkeypatch, "forward_f64", bad)
    _fails(pins.test_forward_equals_triple_loop)


def test_wrong_sign_in_backward_is_caught(monkeypatch):
    def bad(dy, x, w, a, b, s, t=None):
        t = x @ a.T if t is None else t
        g = dy @ b
        return dy @ w - s * (g @ a), s * (g.T @ x), s * (dy.T @ t)
    _patch(monkeypatch, "backward_f64", bad)
    _fails(pins.test_backward_matches_finite_differences)


def test_missing_scale_on_adapter_grad_is_caught(monkeypatch):
    def bad(dy, x, w, a, b, s, t=None):
        t = x @ a.T if t is None else t
        g = dy @ b
        return dy @ w + s * (g @ a), g.T @ x, s * (dy.T @ t)
    _patch(monkeypatch, "backward_f64", bad)
    _fails(pins.test_backward_matches_finite_differences)


def test_ties_to_upper_code_is_caught(monkeypatch):
    real_t = core.nf4_thresholds

    def bad_codes(w, absmax):
        flat = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
        c = absmax[np.arange(flat.size) // 64]
        n = np.where(c != 0, flat / np.where(c != 0, c, 1), 0).astype(np.float32)
        return (n[:, None] >= real_t()[None, :]).sum(1).astype(np.uint8)
    _patch(monkeypatch, "nf4_codes", bad_codes)
    _fails(pins.test_ties_at_thresholds_go_to_lower_code)


def test_round_half_up_in_dq_is_caught(monkeypatch):
    def bad(absmax):
        c = np.asarray(absmax, np.float32)
        ng = -(-c.size // 256)
        q = np.zeros(c.size, np.uint8)
        d = np.zeros(ng, np.float32)
        for g in range(ng):
            seg = c[256 * g: 256 * g + 256]
            if seg.max() == 0:
                continue
            d[g] = np.float32(seg.max()) / np.float32(255)
            q[256 * g: 256 * g + 256] = np.minimum(np.floor(seg / d[g] + np.float32(0.5)), 255)
        return q, d
    _patch(monkeypatch, "double_quantize", bad)
    _fails(pins.test_dq_rint_half_even_and_clamp_by_hand)


def test_swapped_level_split_is_caught(monkeypatch):
    import statistics
    inv = statistics.NormalDist().inv_cdf
    dl = pins.DELTA

    def bad():
        pos = [inv(dl + (0.5 - dl) * i / 7.0) for i in range(7)]
        neg = [-inv(dl + (0.5 - dl) * i / 8.0) for i in range(8)]
        v = sorted(pos + neg + [0.0])
        return (np.array(v) / max(v)).astype(np.float32)
    monkeypatch.setattr(pins, "L", bad())
    _fails(pins.test_levels_shape_order_and_anchor_values)


def test_truncating_bf16_is_caught(monkeypatch):
    def bad(x):
        return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    _patch(monkeypatch, "bf16_rne_bits", bad)
    _fails(pins.test_bf16_rne_matches_torch_cast)


def test_dq_without_rounding_cprime_is_caught(monkeypatch):
    # dequantizing with the fp32 block constant instead of q*d breaks the
    # decoded value of the absmax element
    real = core.nf4_dequantize

    def bad(packed, q, d, numel):
        lv = core.nf4_levels()
        codes = core.unpack_nibbles(packed, numel)
        blk = np.arange(numel) // 64
        cprime = (q.astype(np.float32) + np.float32(0.5))[blk] * d[blk // 256]
        return core.bf16_rne_bits(lv[codes] * cprime)
    _patch(monkeypatch, "nf4_dequantize", bad)
    _fails(pins.test_absmax_element_decodes_to_plus_minus_cprime)


def test_merge_rounding_through_fp32_is_caught(monkeypatch):
    import test_oracle_merge_pins as mpins

    def bad(v):       # rounds twice: float64 -> fp32 -> bf16
        return core.bf16_rne_bits(np.asarray(v, dtype=np.float64).astype(np.float32))
    _patch(monkeypatch, "bf16_rne_from_f64", bad)
    _fails(mpins.test_rne_from_f64_ties_and_near_ties)


def test_merge_without_scale_is_caught(monkeypatch):
    import test_oracle_merge_pins as mpins

    def bad(w_bits, a_bits, b_bits, s):
        w, a, b = (core.bf16_bits_to_f64(t) for t in (w_bits, a_bits, b_bits))
        v = w + b @ a
        return core.bf16_rne_from_f64(v), v
    _patch(monkeypatch, "merge_f64", bad)
    _fails(mpins.test_merge_rank_one_by_hand)


# --- codec variants -------------------------------------------------------

import oracle.codec_variants as cvm  # noqa: E402
import test_oracle_variant_pins as vpins  # noqa: E402


def test_fp4_table_without_subnormal_is_caught(monkeypatch):
    # exponent field 0 read as a normal number: 0.5 becomes 1.0, 0 becomes 0.5
    def bad():
        vals = []
        for b in range(16):
            s = -1.0 if b & 8 else 1.0
            e, m = (b >> 1) & 3, b & 1
            vals.append(s * 2.0 ** (e - 1) * (1.0 + 0.5 * m))
        vals = sorted(vals)
        return (np.array(vals) / max(vals)).astype(np.float32)
    monkeypatch.setattr(cvm, "fp4_levels", bad)
    _fails(vpins.test_fp4_table_is_e2m1_over_its_max)


def test_int4_scaled_by_eight_is_caught(monkeypatch):
    monkeypatch.setattr(cvm, "int4_levels",
                        lambda: ((np.arange(16) - 8) / 8.0).astype(np.float32))
    _fails(vpins.test_int4_codes_are_the_absmax_integer_quantizer)


def test_centered_mean_not_added_back_is_caught(monkeypatch):
    real = cvm.block_constants

    def bad(consts, gscale, gmean, nb, dq):
        if dq == cvm.DQ_CENTERED:
            return real(consts, gscale, np.zeros_like(gmean), nb, dq)
        return real(consts, gscale, gmean, nb, dq)
    monkeypatch.setattr(cvm, "block_constants", bad)
    _fails(vpins.test_centered_dq_bounds_and_extremes)


def test_centered_unsigned_step_is_caught(monkeypatch):
    real = cvm.centered_quantize

    def bad(absmax):
        q, d, mu = real(absmax)
        return q, (d * np.float32(127.0 / 255.0)).astype(np.float32), mu
    monkeypatch.setattr(cvm, "centered_quantize", bad)
    _fails(vpins.test_centered_dq_bounds_and_extremes)


def test_centered_fused_decode_is_caught(monkeypatch):
    def bad(consts, gscale, gmean, nb, dq):
        blk = np.arange(nb)
        v = (np.asarray(consts, np.int8).astype(np.float64) * gscale[blk // 256].astype(np.float64)
             + gmean[blk // 256].astype(np.float64))
        return v.astype(np.float32)
    monkeypatch.setattr(cvm, "block_constants", bad)
    _fails(vpins.test_centered_decode_rounds_twice)


def test_left_to_right_group_sum_is_caught(monkeypatch):
    def bad(x):
        s = np.float32(0)
        for v in np.asarray(x, np.float32):
            s = np.float32(s + v)
        return s
    monkeypatch.setattr(cvm, "pairwise_sum_f32", bad)
    _fails(vpins.test_pairwise_sum_pairs_adjacent_values)


# --- 8-bit AdamW ----------------------------------------------------------

import oracle.adamw8 as awm  # noqa: E402
import test_oracle_adamw_pins as apins  # noqa: E402


def test_missing_bias_correction_is_caught(monkeypatch):
    real = awm.HParams.constants

    def bad(self, step):
        k = real(self, step)
        k["bc1"] = np.float32(1.0)
        k["bc2"] = np.float32(1.0)
        return k
    monkeypatch.setattr(awm.HParams, "constants", bad)
    _fails(apins.test_adamw_f32_matches_torch_adamw)


def test_weight_decay_through_the_gradient_is_caught(monkeypatch):
    # Adam with L2 in the gradient (not decoupled)
    real = awm.adamw_step_f32

    def bad(p32, g, m, v, hp, step):
        g = (np.asarray(g, np.float32) + np.float32(hp.weight_decay) * p32).astype(np.float32)
        hp2 = awm.HParams(hp.lr, hp.beta1, hp.beta2, hp.eps, 0.0, hp.grad_scale)
        return real(p32, g, m, v, hp2, step)
    monkeypatch.setattr(awm, "adamw_step_f32", bad)
    _fails(apins.test_adamw_f32_matches_torch_adamw)


def test_e4m3_bias_eight_is_caught(monkeypatch):
    def bad(code):
        c = np.asarray(code, dtype=np.uint8).astype(np.int64)
        sign = np.where(c & 0x80, -1.0, 1.0)
        e, m = (c >> 3) & 0xF, c & 7
        mag = np.where(e == 0, m * 2.0 ** -10, (1.0 + m / 8.0) * np.exp2(e - 8.0))
        return sign * mag
    monkeypatch.setattr(awm, "e4m3_value", bad)
    _fails(apins.test_e4m3_decode_matches_torch)


def test_e4m3_truncation_is_caught(monkeypatch):
    real = awm.e4m3_encode

    def bad(x):
        x = np.asarray(x, np.float32)
        # shave the magnitude so ties and upper halves round down
        return real((x * np.float32(1 - 2 ** -5)).astype(np.float32))
    monkeypatch.setattr(awm, "e4m3_encode", bad)
    _fails(apins.test_e4m3_encode_matches_torch)


def test_state_scale_by_127_is_caught(monkeypatch):
    monkeypatch.setattr(awm, "E4M3_MAX", 127.0)
    _fails(apins.test_state_block_maps_its_absmax_to_448)


def test_eps_inside_the_sqrt_is_caught(monkeypatch):
    def bad(p32, m, v, k):
        den = np.sqrt((v * k["bc2"] + k["eps"]).astype(np.float32)).astype(np.float32)
        u = ((m * k["bc1"]).astype(np.float32) / den).astype(np.float32)
        return ((p32 * k["decay"]).astype(np.float32)
                - (k["lr"] * u).astype(np.float32)).astype(np.float32)
    monkeypatch.setattr(awm, "param_update_f32", bad)
    _fails(apins.test_adamw_f32_matches_torch_adamw)


# --- LoRA dropout -----------------------------------------------------------

import oracle.dropout as drm  # noqa: E402
import test_oracle_dropout_pins as dpins  # noqa: E402


def test_philox_without_key_bump_is_caught(monkeypatch):
    monkeypatch.setattr(drm, "PHILOX_W0", 0)
    monkeypatch.setattr(drm, "PHILOX_W1", 0)
    _fails(dpins.test_philox_known_answers)


def test_dropout_without_rescale_is_caught(monkeypatch):
    monkeypatch.setattr(drm, "keep_scale", lambda p: np.float32(1.0))
    _fails(dpins.test_inverted_dropout_is_unbiased)


def test_unmasked_dx_is_caught(monkeypatch):
    real = drm.backward_f64

    def bad(dy, x, xd, w, a, b, s, mask_scale, t):
        return real(dy, x, xd, w, a, b, s, np.ones_like(mask_scale), t)
    monkeypatch.setattr(drm, "backward_f64", bad)
    _fails(dpins.test_backward_matches_autograd_of_the_dropout_forward)


def test_da_from_undropped_x_is_caught(monkeypatch):
    real = drm.backward_f64

    def bad(dy, x, xd, w, a, b, s, mask_scale, t):
        return real(dy, x, x, w, a, b, s, mask_scale, t)
    monkeypatch.setattr(drm, "backward_f64", bad)
    _fails(dpins.test_backward_matches_autograd_of_the_dropout_forward)
