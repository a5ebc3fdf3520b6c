"""Host-side checks of the seeded input generators (no GPU): the outlier
recipe is placed as documented (second half of each segment, same channels
in Q and K), the device generator is deterministic per seed, and the
alternative recipes change only what they say."""
import numpy as np
import torch

from bit_quantized_attention_rope3d_amd import inputs


def _outlier_set(w, seed):
    return {(h, c) for h, sel in enumerate(inputs.outlier_channels(w, np.random.default_rng(seed)))
            for c, _ in sel}


def test_outliers_in_second_half_of_segments():
    w = inputs.small(heads=4)
    offs = np.cumsum((0,) + tuple(w.seg))
    for h, c in _outlier_set(w, 3):
        s = int(np.searchsorted(offs, c, side="right")) - 1
        assert offs[s] + w.seg[s] // 2 <= c < offs[s + 1], (h, c)


def test_generate_device_deterministic_and_mirrored():
    w = inputs.small(heads=3)
    q1, k1, v1 = inputs.generate_device(w, 5, "cpu")
    q2, k2, v2 = inputs.generate_device(w, 5, "cpu")
    assert torch.equal(q1, q2) and torch.equal(k1, k2) and torch.equal(v1, v2)
    q3, _, _ = inputs.generate_device(w, 6, "cpu")
    assert not torch.equal(q1, q3)
    assert q1.dtype == torch.bfloat16 and q1.shape == (1, w.tokens, 3, w.head_dim)
    # The multiplied channels stand out in both Q and K, and nowhere else.
    big_q = q1.float().abs().amax(dim=(0, 1)) > 8.0
    big_k = k1.float().abs().amax(dim=(0, 1)) > 8.0
    want = torch.zeros_like(big_q)
    for h, c in _outlier_set(w, 5):
        want[h, c] = True
    assert torch.equal(big_q, want) and torch.equal(big_k, want)
    assert v1.float().abs().max() < 8.0


def test_input_recipes():
    w = inputs.get("wan720")
    assert inputs.with_inputs(w, "recipe") == w
    assert inputs.with_inputs(w, "plain").outliers_per_segment == (0, 0, 0)
    assert inputs.with_inputs(w, "mild").outlier_scale == (3.0, 5.0)
    t = inputs.with_inputs(w, "student_t3")
    assert t.outlier_dist == "student_t3" and t.outlier_segments == (1, 2)
    assert _outlier_set(inputs.with_inputs(inputs.small(), "plain"), 0) == set()
    try:
        inputs.with_inputs(w, "other")
    except ValueError:
        pass
    else:
        raise AssertionError("unknown recipe accepted")
