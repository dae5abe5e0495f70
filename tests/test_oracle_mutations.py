"""Planted mistakes in the oracle (CPU only): each must be caught by a pin.

Every mutant replaces one definitional helper of ``oracle.attention`` with a
plausible bug (a wrong index, a dropped term, a swapped operand, a shifted
mask) and the pins of ``oracle_pins`` are run against it; at least one must
fail.  The mistakes are planted in the oracle on the CPU only.
"""

import numpy as np
import pytest

import oracle.attention as oa
from tests import oracle_pins

_real_gather = oa.gather_request_kv
_real_merge = oa.merge_partials
_real_fp8 = oa.fp8_e4m3_bits_to_f64


def _fp8_bias8(bits):
    # the exponent bias of the other FP8 convention (8 instead of 7)
    return _real_fp8(bits) * 0.5


def _gather_v_scale_on_k(batch, r, kv_len, tokens=None):
    k, v = _real_gather(batch, r, kv_len, tokens)
    if batch.get("kv_dtype") == "fp8_e4m3":
        ks = np.asarray(batch["k_scale"], np.float64)
        vs = np.asarray(batch["v_scale"], np.float64)
        k = k / ks[None, :, None] * vs[None, :, None]
    return k, v


def _gather_scales_other_head(batch, r, kv_len, tokens=None):
    k, v = _real_gather(batch, r, kv_len, tokens)
    if batch.get("kv_dtype") == "fp8_e4m3":
        ks = np.asarray(batch["k_scale"], np.float64)
        k = k / ks[None, :, None] * ks[::-1][None, :, None]
    return k, v


def _swap_kv(batch, r, kv_len, tokens=None):
    k, v = _real_gather(batch, r, kv_len, tokens)
    return v, k


def _merge_no_norm(parts):
    o, l = _real_merge(parts)
    # forgets to renormalise: weights exp(LSE_s - max) instead of - LSE
    lses = np.stack([p[1] for p in parts])
    m = np.max(lses, axis=0)
    m = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lses - m[None])
    os_ = np.stack([p[0] for p in parts])
    return np.sum(w[..., None] * os_, axis=0), l


MUTANTS = {
    "gqa_interleaved": ("kv_head_of", lambda h, hq, hkv: h % hkv),
    "mask_excludes_diagonal": ("visible_key_count",
                               lambda pos, kv, causal: min(pos, kv) if causal else kv),
    "mask_one_future_key": ("visible_key_count",
                            lambda pos, kv, causal: min(pos + 2, kv) if causal else kv),
    "top_left_alignment": ("_row_positions",
                           lambda qo, kv: np.arange(0, qo, dtype=np.int64)),
    "no_scale": ("_scores", lambda q, k, s: q @ k.T),
    "scale_squared": ("_scores", lambda q, k, s: s * s * (q @ k.T)),
    "transposed_scores": ("_scores",
                          lambda q, k, s: s * (q @ k.T) if q.shape[0] != k.shape[0]
                          else s * (q @ k.T).T),
    "lse_drops_max": ("_lse", lambda m, l: np.log(l)),
    "lse_log2": ("_lse", lambda m, l: m + np.log2(l)),
    "bf16_wrong_shift": ("bf16_bits_to_f64",
                         lambda b: (np.asarray(b).astype(np.uint32) << np.uint32(15))
                         .view(np.float32).astype(np.float64)),
    "kv_swapped": ("gather_request_kv", _swap_kv),
    "merge_unnormalised": ("merge_partials", _merge_no_norm),
    "fp8_bias8": ("fp8_e4m3_bits_to_f64", _fp8_bias8),
    "fp8_v_scale_on_k": ("gather_request_kv", _gather_v_scale_on_k),
    "fp8_scales_other_head": ("gather_request_kv", _gather_scales_other_head),
    # a chunk's first row handed to the request before it
    "sample_row_to_previous_request": (
        "_request_of_row", lambda offs, g: int(np.searchsorted(offs, g, side="left") - 1)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oa, attr, fn)
    import oracle
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, TypeError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
