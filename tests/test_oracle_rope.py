"""Pins of the oracle's 3D RoPE and RoPE-aware rotations.

Page: RotateAttention review -- Sec. 3 / Fig. 2 (head dims split into frame,
height and width segments, each rotated by its own axis), Sec. 4.1 / Fig. 3
(Interleaved rotation on adjacent dims, which folds into the RoPE angles;
Half rotation of dim i with dim i + L/2 inside a segment of length L; orthogonal
blocks keep (QR)(KR)^T = QK^T; the SVD argument for why only orthogonal R
keeps Q and K ranges balanced).
"""
import numpy as np
import pytest

from oracle import ref_fp64 as ref

GRID = (3, 4, 5)
SEG = (24, 20, 20)
D = sum(SEG)


def _x(seed, n=60, h=2):
    return np.random.default_rng(seed).standard_normal((1, n, h, D)).astype(np.float32)


@pytest.mark.parametrize("rot", [0, 1, 2])
def test_tables_within_one_ulp_of_fp64(ora, rot):
    for npos, L in ((21, 44), (45, 42), (80, 56), (4, 20)):
        cs, sn = ora.rope_table(npos, L, 10000.0, rot)
        p = np.arange(npos)[:, None]
        j = np.arange(L // 2)[None, :]
        ang = p * 10000.0 ** (-2.0 * j / L) + (np.pi / 4 if rot == 1 else 0.0)
        assert np.max(np.abs(cs - np.cos(ang))) <= 2.0 ** -24
        assert np.max(np.abs(sn - np.sin(ang))) <= 2.0 ** -24


@pytest.mark.parametrize("rot", [0, 1, 2])
def test_oracle_rotation_matches_fp64_reference(ora, rot):
    x = _x(1)
    y = ora.rope_rotate(x, GRID, SEG, 10000.0, rot)
    want = ref.rope_rotate(x.astype(np.float64), GRID, SEG, 10000.0, rot)
    scale = np.max(np.abs(x))
    assert np.max(np.abs(y - want)) <= 4e-7 * scale * 4


def test_pair_norms_preserved():
    x = _x(2).astype(np.float64)
    y = ref.rope3d(x, GRID, SEG)
    n_in = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n_out = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-13, atol=1e-13)


def test_scores_depend_only_on_relative_position():
    q = _x(3).astype(np.float64)
    k = _x(4).astype(np.float64)
    s0 = np.einsum("bnhd,bmhd->bhnm", ref.rope3d(q, GRID, SEG), ref.rope3d(k, GRID, SEG))
    off = (7, 2, 11)
    s1 = np.einsum("bnhd,bmhd->bhnm", ref.rope3d(q, GRID, SEG, offset=off),
                   ref.rope3d(k, GRID, SEG, offset=off))
    assert np.allclose(s0, s1, rtol=1e-11, atol=1e-10)


def test_single_axis_grid_is_textbook_1d_rope():
    """F = H = 1: frame/height segments see position 0 (identity) and the width
    segment is the RoFormer rotation by pos * theta^(-2j/L)."""
    W = 9
    x = np.random.default_rng(6).standard_normal((1, W, 1, D))
    y = ref.rope3d(x, (1, 1, W), SEG)
    L = SEG[2]
    off = SEG[0] + SEG[1]
    want = x.copy()
    for n in range(W):
        for j in range(L // 2):
            th = n * 10000.0 ** (-2.0 * j / L)
            M = np.array([[np.cos(th), -np.sin(th)], [np.sin(th), np.cos(th)]])
            want[0, n, 0, off + 2 * j:off + 2 * j + 2] = M @ x[0, n, 0, off + 2 * j:off + 2 * j + 2]
    assert np.allclose(y, want, atol=1e-13)


@pytest.mark.parametrize("rot", [1, 2])
def test_rotations_orthogonal_and_score_preserving(rot):
    R = ref.rotation_matrix(SEG, rot)
    assert np.allclose(R.T @ R, np.eye(D), atol=1e-15)
    q = np.random.default_rng(7).standard_normal((50, D))
    k = np.random.default_rng(8).standard_normal((60, D))
    assert np.allclose((q @ R.T) @ (k @ R.T).T, q @ k.T, atol=1e-12)


def test_half_block_is_h2_involution():
    R = ref.rotation_matrix(SEG, 2)
    assert np.allclose(R @ R, np.eye(D), atol=1e-15)
    h2 = R[np.ix_([0, SEG[0] // 2], [0, SEG[0] // 2])]
    assert np.allclose(h2, np.array([[1, 1], [1, -1]]) / np.sqrt(2))


def test_interleaved_block_commutes_with_rope_pairs():
    """R(pi/4) commutes with every pair rotation R(theta), so applying it after
    RoPE equals RoPE with the angle shifted by pi/4 (merged tables)."""
    def rot2(t):
        return np.array([[np.cos(t), -np.sin(t)], [np.sin(t), np.cos(t)]])
    B = ref.rotation_matrix((2, 2, 2), 1)[:2, :2]
    assert np.allclose(B, rot2(np.pi / 4))
    for t in np.linspace(-3, 3, 13):
        assert np.allclose(B @ rot2(t), rot2(t) @ B, atol=1e-15)
        assert np.allclose(B @ rot2(t), rot2(t + np.pi / 4), atol=1e-15)
    # H2 (a reflection) would not commute: H2 R(t) = R(-t) H2.
    H2 = np.array([[1, 1], [1, -1]]) / np.sqrt(2)
    assert not np.allclose(H2 @ rot2(0.3), rot2(0.3) @ H2)


def test_merged_interleaved_equals_rope_then_rotation(ora):
    x = _x(9)
    merged = ora.rope_rotate(x, GRID, SEG, 10000.0, 1)
    explicit = ref.rope3d(x.astype(np.float64), GRID, SEG) @ ref.rotation_matrix(SEG, 1).T
    assert np.max(np.abs(merged - explicit)) <= 2e-6 * np.max(np.abs(x))


def test_non_orthogonal_rotation_unbalances_q_and_k():
    """SVD argument: with R = diag(sigma), K must take R^-T to keep QK^T; the
    amax ratios move in opposite directions, which simultaneous INT4 of Q and
    K cannot absorb.  Orthogonal R keeps both amaxes comparable."""
    rng = np.random.default_rng(10)
    q = rng.standard_normal((256, D))
    k = rng.standard_normal((256, D))
    R = np.diag(np.full(D, 4.0))
    qr, kr = q @ R.T, k @ np.linalg.inv(R)
    assert np.allclose(qr @ kr.T, q @ k.T, atol=1e-10)
    ratio_q = np.abs(qr).max() / np.abs(q).max()
    ratio_k = np.abs(kr).max() / np.abs(k).max()
    assert ratio_q > 3.9 and ratio_k < 0.26
    Ro = ref.rotation_matrix(SEG, 2)
    assert 0.6 < np.abs(q @ Ro.T).max() / np.abs(q).max() < 1.5


def test_half_rotation_spreads_a_segment_outlier():
    """A channel outlier in the second half of a segment is split over the
    pair (i - L/2, i) by H2, lowering the segment amax by about sqrt(2)."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((512, D)) * 0.1
    c = SEG[0] // 2 + 3
    x[:, c] = 20.0 * np.sign(rng.standard_normal(512))
    y = x @ ref.rotation_matrix(SEG, 2).T
    assert np.abs(y).max() < np.abs(x).max() / np.sqrt(2) * 1.05


# ---- full rotation (rot = 3) -----------------------------------------------
# Figs. 4-6 compare against a full rotation of all D dimensions; reading: the
# orthonormal Walsh-Hadamard matrix applied to the RoPE'd head row.

def test_full_rotation_is_hadamard_times_rope(ora):
    from scipy.linalg import hadamard
    rng = np.random.default_rng(21)
    grid, seg = (2, 3, 5), (24, 20, 20)
    x = rng.standard_normal((1, 30, 2, 64)).astype(np.float32)
    y0 = ora.rope_rotate(x, grid, seg, 10000.0, 0).astype(np.float64)
    y3 = ora.rope_rotate(x, grid, seg, 10000.0, 3).astype(np.float64)
    want = y0 @ (hadamard(64) / np.sqrt(64))
    assert np.abs(y3 - want).max() <= 1e-5 * np.abs(y0).max()
    # orthogonal: norms and all scores q.k are kept (fp32 rounding aside)
    assert np.allclose(np.linalg.norm(y3, axis=-1), np.linalg.norm(y0, axis=-1), rtol=1e-5)
    s0 = np.einsum("bnhd,bmhd->bhnm", y0, y0)
    s3 = np.einsum("bnhd,bmhd->bhnm", y3, y3)
    assert np.abs(s3 - s0).max() <= 1e-4 * np.abs(s0).max()


def test_full_rotation_spreads_any_channel_outlier(ora):
    """One large channel anywhere in the row ends up as equal magnitudes in
    every channel (unlike Half, which only pairs inside its segment)."""
    x = np.zeros((1, 1, 1, 128), np.float32)
    x[0, 0, 0, 77] = 100.0          # position 0: RoPE leaves the row as is
    y = ora.rope_rotate(x, (1, 1, 1), (44, 42, 42), 10000.0, 3)
    assert np.allclose(np.abs(y), 100.0 / np.sqrt(128), rtol=1e-6)
    yh = ora.rope_rotate(x, (1, 1, 1), (44, 42, 42), 10000.0, 2)
    assert np.count_nonzero(yh) == 2
