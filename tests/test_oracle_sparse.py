"""Pins of the oracle's sparse gradient encoder and decoder (CPU)."""
import numpy as np
import pytest

import oracle


def _synthetic(seed, V=3, cap=40, n_owner=200, density=0.35):
    rng = np.random.default_rng(seed)
    vis_count = rng.integers(0, cap + 1, size=V)
    vis_count[0] = cap  # a full view
    vis_ids = np.full((V, cap), -7, np.int32)
    per_view = []
    for v in range(V):
        n = int(vis_count[v])
        vis_ids[v, :n] = np.sort(rng.choice(n_owner, size=n, replace=False))
        R = rng.standard_normal((n, 9)).astype(np.float32)
        zero = rng.random(n) > density
        R[zero] = 0.0
        # partial zeros stay records; negative zeros alone do not
        if n > 3:
            R[1, :] = 0.0
            R[1, 4] = 1e-30
            R[2, :] = -0.0
        per_view.append(R)
    return vis_count, vis_ids, per_view, n_owner


def _dense_scatter(vis_count, vis_ids, per_view, n_owner):
    V = len(per_view)
    dense = np.zeros((V, n_owner, 9))
    for v in range(V):
        for s in range(int(vis_count[v])):
            dense[v, vis_ids[v, s]] = per_view[v][s]
    return dense


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_round_trip_equals_dense_scatter(seed):
    vis_count, vis_ids, per_view, n_owner = _synthetic(seed)
    enc = oracle.grad_encode(vis_count, vis_ids, per_view)
    out = oracle.grad_decode(enc["view_offset"], enc["keys"], enc["records"], np.zeros((len(per_view), n_owner, 9)))
    assert np.array_equal(out, _dense_scatter(vis_count, vis_ids, per_view, n_owner))


def test_counts_and_order_from_an_explicit_loop():
    vis_count, vis_ids, per_view, n_owner = _synthetic(5)
    enc = oracle.grad_encode(vis_count, vis_ids, per_view)
    off = [0]
    for v, R in enumerate(per_view):
        kept = [s for s in range(R.shape[0]) if any(float(c) != 0.0 for c in R[s])]
        off.append(off[-1] + len(kept))
        seg = slice(int(enc["view_offset"][v]), int(enc["view_offset"][v + 1]))
        assert list(enc["keys"][seg]) == [int(vis_ids[v, s]) for s in kept]
        assert np.array_equal(enc["records"][seg], R[kept])
    assert list(enc["view_offset"]) == off


def test_nan_is_kept_negative_zero_is_dropped():
    R = np.zeros((4, 9), np.float32)
    R[0, 3] = np.nan
    R[1, :] = -0.0
    R[2, 8] = -1.0
    enc = oracle.grad_encode([4], np.arange(4, dtype=np.int32)[None], [R])
    assert list(enc["keys"]) == [0, 2]
    assert np.isnan(enc["records"][0, 3])


def test_all_zero_gives_no_records():
    enc = oracle.grad_encode([5, 0], np.zeros((2, 5), np.int32), [np.zeros((5, 9)), np.zeros((0, 9))])
    assert enc["keys"].size == 0 and list(enc["view_offset"]) == [0, 0, 0]


def test_streams_accumulate_and_foreign_keys_are_skipped():
    vis_count, vis_ids, a, n_owner = _synthetic(7)
    _, _, b, _ = _synthetic(8)
    b = [B[:int(vis_count[v])] if B.shape[0] >= int(vis_count[v]) else
         np.vstack([B, np.ones((int(vis_count[v]) - B.shape[0], 9))]) for v, B in enumerate(b)]
    ea, eb = oracle.grad_encode(vis_count, vis_ids, a), oracle.grad_encode(vis_count, vis_ids, b)
    own = oracle.grad_decode(ea["view_offset"], ea["keys"], ea["records"], np.zeros((len(a), n_owner, 9)))
    own = oracle.grad_decode(eb["view_offset"], eb["keys"], eb["records"], own)
    expect = _dense_scatter(vis_count, vis_ids, a, n_owner) + _dense_scatter(vis_count, vis_ids, b, n_owner)
    assert np.allclose(own, expect, rtol=0, atol=0)
    # a key past the owner range changes nothing
    keys = ea["keys"].copy()
    if keys.size:
        keys[0] = n_owner + 3
        out = oracle.grad_decode(ea["view_offset"], keys, ea["records"], np.zeros((len(a), n_owner, 9)))
        ref = oracle.grad_decode(ea["view_offset"], ea["keys"], ea["records"], np.zeros((len(a), n_owner, 9)))
        v0 = int(np.searchsorted(ea["view_offset"], 0, side="right") - 1)
        ref[v0, ea["keys"][0]] = 0.0
        assert np.array_equal(out, ref)
