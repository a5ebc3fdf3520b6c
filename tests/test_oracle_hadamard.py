"""Pins of the oracle's V-side Hadamard.

Page: RotateAttention review, summary and reproducibility notes: a standard
Hadamard transform is fused offline into V.  Reading: V rows are multiplied
by the orthonormal Walsh-Hadamard matrix H = H_D / sqrt(D) before their
per-channel INT4 quantization, and the output rows by H again (H is symmetric
and its own inverse), so the operator still computes attention(Q, K, V).
Checked against scipy's Hadamard matrix, the algebra of H, and closed forms.
"""
import numpy as np
import pytest
from scipy.linalg import hadamard

from oracle import ref_fp64 as ref


@pytest.mark.parametrize("D", [64, 128])
def test_fwht_is_the_sylvester_hadamard_matrix(ora, D):
    x = np.random.default_rng(D).standard_normal((7, D)).astype(np.float32)
    want = x.astype(np.float64) @ (hadamard(D) / np.sqrt(D))
    got = ora.fwht(x).astype(np.float64)
    # log2(D) rounded adds and one rounded multiply per element
    assert np.abs(got - want).max() <= 1e-5 * np.abs(x).max()
    e = np.zeros((2, D), np.float32)
    e[0, 0] = 1.0
    e[1, 1] = 1.0
    h = ora.fwht(e)
    assert np.allclose(h[0], 1.0 / np.sqrt(D), rtol=1e-7)
    assert np.allclose(h[1], (1.0 / np.sqrt(D)) * np.where(np.arange(D) % 2 == 0, 1.0, -1.0), rtol=1e-7)


def test_fwht_is_orthogonal_and_self_inverse(ora):
    x = np.random.default_rng(1).standard_normal((50, 128)).astype(np.float32)
    y = ora.fwht(x)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-5)
    assert np.abs(ora.fwht(y) - x).max() <= 1e-5 * np.abs(x).max()


def test_attention_is_invariant_in_exact_arithmetic():
    """softmax(Q K^T) (V H) H = softmax(Q K^T) V: the transform changes only
    what is quantized, not what is computed."""
    rng = np.random.default_rng(2)
    N, D = 90, 64
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    H = hadamard(D) / np.sqrt(D)
    a = ref.attention(q[None, :, None], k[None, :, None], v[None, :, None])[0, :, 0]
    b = ref.attention(q[None, :, None], k[None, :, None], (v @ H)[None, :, None])[0, :, 0] @ H
    assert np.abs(a - b).max() < 1e-12


def test_zero_queries_give_rotated_back_channel_means(ora):
    """Q = 0: every key gets the same weight, so the output is the mean of the
    dequantized rows of V H, times H."""
    rng = np.random.default_rng(3)
    grid, seg = (1, 4, 25), (24, 20, 20)
    N, H_, D = 100, 2, 64
    q = np.zeros((1, N, H_, D), np.float32)
    k = rng.standard_normal((1, N, H_, D)).astype(np.float32)
    v = rng.standard_normal((1, N, H_, D)).astype(np.float32)
    pro = ora.prologue(q, k, v, grid, seg, 10000.0, 2, v_hadamard=True)
    o = ora.attention_full(pro, v_hadamard=True)
    Hm = hadamard(D) / np.sqrt(D)
    for h in range(H_):
        mean_rot = pro["s_v"][0, h].astype(np.float64) * pro["v_codes"][0, h].astype(np.float64).mean(axis=0)
        assert np.allclose(o[0, :, h, :], (mean_rot @ Hm)[None, :], rtol=1e-10, atol=1e-12)
    # and the codes are those of V H, not of V
    vc_plain, _ = ora.quant_v(v)
    vc_rot, _ = ora.quant_v(ora.fwht(v))
    assert np.array_equal(pro["v_codes"], vc_rot) and not np.array_equal(vc_rot, vc_plain)


def test_hadamard_path_close_to_full_precision(ora):
    rng = np.random.default_rng(4)
    grid, seg = (2, 5, 12), (24, 20, 20)
    N, H_, D = 120, 2, 64
    q = rng.standard_normal((1, N, H_, D)).astype(np.float32)
    k = rng.standard_normal((1, N, H_, D)).astype(np.float32)
    v = rng.standard_normal((1, N, H_, D)).astype(np.float32)
    pro = ora.prologue(q, k, v, grid, seg, 10000.0, 2, v_hadamard=True)
    o = ora.attention_full(pro, v_hadamard=True)
    want = ref.reference_output(q, k, v, grid, seg)
    cos = (o * want).sum() / np.sqrt((o * o).sum() * (want * want).sum())
    assert cos > 0.9
