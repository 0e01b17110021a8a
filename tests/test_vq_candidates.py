"""Host-side candidate lists of the 2-bit nearest-codeword search
(nsnq_vq_candidates; technical summary sec. 3, "Vector Quantization").  The
lists restrict the search and must never drop the nearest codeword of a point
in their orthant box, so they are pinned against (1) an independent linear
programme (scipy's HiGHS) deciding, codeword by codeword, whether its Voronoi
cell meets the box, and (2) brute-force nearest codewords of many points of
each box, including faces, corners and points near cell boundaries.  No GPU is
needed: the table is built on the host."""
import numpy as np
import pytest
import torch
from scipy.optimize import linprog

import oracle
from kv_cache_bit_amd import nsnq, synth

BOX = 12.0


@pytest.fixture(scope="module")
def cb2():
    x = synth.randn_samples(5, 1 << 14, 4).numpy()
    _, cb, _ = oracle.kmeans(x, 256, 15)
    return cb


def _table(cb):
    p = nsnq.params(2, 128)
    table, tiles = nsnq.nsnq_vq_candidates(p, torch.from_numpy(cb.view(np.float16)))
    return table.numpy(), tiles


def _lists(tab):
    return [sorted(set(tab[o].tolist())) for o in range(16)]


def _gap_lp(C, k, o):
    """min over x in box O of max_j (|x - c_k|^2 - |x - c_j|^2), by scipy."""
    sg = np.array([-1.0 if (o >> i) & 1 else 1.0 for i in range(4)])
    j = np.arange(len(C)) != k
    n2 = (C * C).sum(1)
    A = np.hstack([2 * (C[j] - C[k]), -np.ones((j.sum(), 1))])  # 2 x.(c_j - c_k) - t <= n2_j - n2_k
    b = n2[j] - n2[k]
    bounds = [(0, BOX) if s > 0 else (-BOX, 0) for s in sg] + [(None, None)]
    res = linprog(np.r_[np.zeros(4), 1.0], A_ub=A, b_ub=b, bounds=bounds, method="highs")
    assert res.status == 0
    return res.fun


def test_table_layout(cb2):
    tab, span = _table(cb2)
    assert tab.shape == (16, 128)
    lists = _lists(tab)
    longest = max(len(l) for l in lists)
    assert span == (longest + 15) // 16 * 16 and 16 <= span <= 128
    for o in range(16):
        n = len(lists[o])
        assert np.array_equal(tab[o, :n], np.array(lists[o], np.uint8)), "ascending, no repeats before the pad"
        assert np.all(tab[o, n:] == tab[o, n - 1]), "padded with the last entry"
    # the 16 boxes cover the space: every codeword is on some list
    assert set().union(*map(set, lists)) == set(range(256))


def test_lists_match_an_independent_lp(cb2):
    tab, _ = _table(cb2)
    lists = _lists(tab)
    C = oracle.f16_to_f64(cb2)
    for o in (0, 5, 10, 15):
        on = set(lists[o])
        for k in range(256):
            g = _gap_lp(C, k, o)
            if g <= -1e-7:
                assert k in on, (o, k, g)
            elif g >= 1e-7:
                assert k not in on, (o, k, g)


def test_brute_force_nearest_is_always_listed(cb2):
    tab, _ = _table(cb2)
    lists = [np.zeros(256, bool) for _ in range(16)]
    for o in range(16):
        lists[o][tab[o]] = True
    C = oracle.f16_to_f64(cb2)
    rng = np.random.default_rng(11)
    pts = [rng.standard_normal((20000, 4)) * s for s in (0.3, 1.0, 2.0, 5.0)]
    pts.append(rng.uniform(-BOX, BOX, (20000, 4)))
    # faces and corners of the boxes: some elements exactly 0 or +-12
    f = rng.standard_normal((20000, 4))
    f[rng.random((20000, 4)) < 0.4] = 0.0
    pts.append(f)
    pts.append(rng.choice([-BOX, 0.0, BOX], (2000, 4)))
    # points close to a boundary between two codewords
    a, b = rng.integers(0, 256, 4000), rng.integers(0, 256, 4000)
    pts.append(0.5 * (C[a] + C[b]) + 1e-9 * rng.standard_normal((4000, 4)))
    u = np.concatenate(pts)
    d = ((u[:, None, :] - C[None, :, :]) ** 2).sum(-1)
    near = np.argmin(d, axis=1)
    # the nearest codeword is listed for the box of u; a zero element sits on
    # the face of two boxes, and both lists must hold it
    L = np.stack(lists)
    neg = (u < 0).astype(np.int64)
    box = (neg << np.arange(4)).sum(1)
    zero = (u == 0).any(1)
    assert L[box[~zero], near[~zero]].all()
    for i in np.flatnonzero(zero):
        boxes = {int(box[i])}
        for e in np.flatnonzero(u[i] == 0):
            boxes |= {bx | (1 << e) for bx in boxes}
        for bx in boxes:
            assert L[bx, near[i]], (u[i], near[i], bx)


def test_unsupported_and_invalid(cb2):
    with pytest.raises(nsnq.NsnqError):
        nsnq.nsnq_vq_candidates(nsnq.params(1, 128), torch.zeros(256, 8, dtype=torch.float16).view(-1)[:1024])
    bad = cb2.copy()
    bad[3, 1] = 0x7C00  # +inf
    with pytest.raises(nsnq.NsnqError):
        _table(bad)


def test_params_carry_the_table(cb2):
    p = nsnq.with_candidates(nsnq.params(2, 64), torch.from_numpy(cb2.view(np.float16)))
    assert p.vq_span in (64, 80, 96) and p.vq_candidates
    assert p._cand_ref.numel() == 2048
