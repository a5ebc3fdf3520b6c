"""The P-map byte table the INT4 kernels use, as the host builds it (no GPU
needed), checked cell by cell against the oracle's thresholds.

RotateAttention review, Sec. 4.2 and free-parameter ledger: u = round(P p)
with p = 2^d (P = 15, or 7 for the symmetric baseline), so u = #{k : x <= X_k}
for x = -d and X_k = -T_k, the oracle's thresholds (pinned in
test_oracle_pmap.py).  The table holds one byte per exponent cell j =
rint(4096 x) (ties to even), stored in reverse at address top - j; every
cell whose x all share one u holds e4m3(u), and the cell of an X_k that also
holds values above X_k is marked 0x80 | k, its record holding X_k / 8 for the
kernels' exact compare.  The GPU test test_pmap_exhaustive runs the kernels'
lookup on every binary32 d of the live range; this one checks the table
itself on the host."""
import numpy as np
import pytest

from bit_quantized_attention_rope3d_amd import api

ENTRIES = 20112


def e4m3_value(b):
    b = np.asarray(b, np.int64)
    e, m = b >> 3, b & 7
    return np.where(b == 0, 0.0, (1.0 + m / 8.0) * np.exp2(e - 7.0))


def cell_bounds(j):
    """Smallest and largest binary32 x >= 0 with rint(4096 x) = j (ties to
    even); (j -+ 0.5) / 4096 is exact in binary32."""
    j = np.asarray(j, np.int64)
    lo = ((j - 0.5) / 4096.0).astype(np.float32)
    hi = ((j + 0.5) / 4096.0).astype(np.float32)
    odd = (j & 1) == 1
    lo = np.where(odd, np.nextafter(lo, np.float32(np.inf)), lo)
    hi = np.where(odd, np.nextafter(hi, np.float32(-np.inf)), hi)
    lo = np.maximum(lo, np.float32(0.0))
    assert np.all(np.rint(lo.astype(np.float64) * 4096.0) == j)
    assert np.all(np.rint(hi.astype(np.float64) * 4096.0) == j)
    return lo, hi


def u_of(x, X):
    """u = #{k : x <= X_k}, in binary32 (both sides exact)."""
    return (x[:, None].astype(np.float32) <= X[None, :]).sum(axis=1)


@pytest.mark.parametrize("p_mode", [0, 1])
def test_host_table_matches_threshold_count(ora, p_mode):
    tab, top = api.pmap_table(p_mode)
    X = (-ora.pmap_thresholds(p_mode)).astype(np.float32)
    P = X.size
    assert P == (15 if p_mode == 0 else 7)
    assert top % 2 == 0 and 0 < top < ENTRIES
    a = np.arange(top + 1)
    j = top - a
    lo, hi = cell_bounds(j)
    u_lo, u_hi = u_of(lo, X), u_of(hi, X)
    ent = tab[: top + 1].astype(np.int64)
    marked = (ent & 0x80) != 0
    # Unmarked cells: one u over the whole cell, stored as its e4m3 byte.
    # Address 0 stands for every x from cell top on (the kernels clamp the
    # address at 0): u = 0 there.
    assert ent[0] == 0 and u_lo[0] == 0
    um = ~marked
    assert np.array_equal(u_lo[um], u_hi[um])
    assert np.array_equal(e4m3_value(ent[um]), u_lo[um].astype(np.float64))
    # Marked cells: the cell of X_k holding values above X_k.
    k = ent[marked] & 0x0F
    assert np.all(k < P)
    assert np.all(lo[marked] <= X[k]) and np.all(X[k] < hi[marked])
    assert np.array_equal(u_lo[marked], k + 1) and np.array_equal(u_hi[marked], k)
    # Every X_k whose cell holds values above it is marked, and only those.
    jk = np.rint(X.astype(np.float64) * 4096.0).astype(np.int64)
    _, hik = cell_bounds(jk)
    want = {int(kk) for kk in range(P) if X[kk] < hik[kk]}
    assert set(int(v) for v in k) == want
    # Entries past top are zero; records hold X_k / 8 and the two codes.
    assert not np.any(tab[top + 1: ENTRIES])
    rec = tab[ENTRIES:].reshape(16, 8)
    thr = rec[:, :4].copy().view(np.float32)[:, 0]
    assert np.array_equal(thr[:P], X * np.float32(0.125)) and not np.any(thr[P:])
    assert np.array_equal(e4m3_value(rec[:P, 4]), np.arange(float(P)))
    assert np.array_equal(e4m3_value(rec[:P, 5]), np.arange(1.0, P + 1.0))
    assert not np.any(rec[P:])


def test_host_table_rejects_bad_arguments():
    from bit_quantized_attention_rope3d_amd import native
    import ctypes
    L = native.lib()
    buf = np.zeros(20240, np.uint8)
    top = ctypes.c_int32(0)
    ptr = buf.ctypes.data_as(ctypes.c_void_p)
    assert L.ra_pmap_table(2, ptr, buf.size, ctypes.byref(top)) == 1
    assert L.ra_pmap_table(0, ptr, buf.size - 1, ctypes.byref(top)) == 1
    assert L.ra_pmap_table(0, None, buf.size, ctypes.byref(top)) == 1
    assert L.ra_pmap_table(0, ptr, buf.size, None) == 1
