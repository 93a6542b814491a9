"""The parity check itself, on the CPU: fabricated index lists at thresholds
that sit on (or within 1e-7 of) a CDF cell edge.  Only the neighbouring
token across that edge may be accepted; any other token is a hard mismatch
(key design 1: J_m = F^-1(T_m); a threshold within rounding of an edge may
fall on either side of it, and nowhere else)."""
import numpy as np

import oracle as O
import parity


def _problem(logits, T):
    """One head, head dim 1, scale 1, q = 1: the scores are `logits`."""
    n = len(logits)
    q = np.ones((1, 1, 1), np.float32)
    k = np.asarray(logits, np.float32).reshape(1, 1, n, 1)
    v = np.arange(n, dtype=np.float32).reshape(1, 1, n, 1)
    prob = O.Problem(1, 1, 1, 1, n, q_dtype="f32", kv_dtype="f32", scale=1.0, tile_len=T)
    return prob, q, k, v


def _prop_report(prob, q, k, v, S, U, gpu_idx):
    u = np.array([U], np.float32)
    r = O.santa_prop(prob, q, k, v, S, u)
    rep = parity.index_report(np.array([gpu_idx], np.int32), r["idx"], r["delta"],
                              lambda tok: O.prop_cells(prob, q, k, S, u, tok))
    return r["idx"][0].tolist(), rep


def test_exact_ties_accept_only_the_neighbour():
    """Uniform four tokens, S = 2, U = 1/4: the thresholds 1/4 and 3/4 lie
    exactly on F(0) and F(2).  The oracle takes (1, 3); (0, 2) are the
    neighbours across those edges; tokens two cells away are wrong."""
    prob, q, k, v = _problem([0.0, 0.0, 0.0, 0.0], T=64)
    want, rep = _prop_report(prob, q, k, v, 2, 0.25, [1, 3])
    assert want == [1, 3] and rep["mismatch"] == 0
    _, rep = _prop_report(prob, q, k, v, 2, 0.25, [0, 2])
    assert rep["exempt"] == 2 and rep["hard"] == 0
    for bad in ([3, 3], [2, 3], [1, 0], [1, 1]):
        _, rep = _prop_report(prob, q, k, v, 2, 0.25, bad)
        assert rep["hard"] >= 1, (bad, rep)


def test_near_edge_accepts_neighbour_rejects_far_token():
    """Thresholds 6e-8 above the edges F(0) = 1/4 and F(2) = 3/4: the token
    below each edge is still within 1e-6 of its threshold; a token two cells
    away, or outside the request, is not."""
    prob, q, k, v = _problem([0.0, 0.0, 0.0, 0.0], T=64)
    U = float(np.float32(0.25) + np.float32(2.0 ** -24))
    want, rep = _prop_report(prob, q, k, v, 2, U, [1, 3])
    assert want == [1, 3] and rep["mismatch"] == 0 and rep["near_edges"] == 2
    _, rep = _prop_report(prob, q, k, v, 2, U, [0, 2])
    assert rep["exempt"] == 2 and rep["hard"] == 0
    assert 0 < rep["max_exempt_cell_distance"] < 1e-7
    for bad in ([2, 3], [1, 1], [1, 4], [-1, 3]):
        _, rep = _prop_report(prob, q, k, v, 2, U, bad)
        assert rep["hard"] == 1, (bad, rep)


def test_zero_mass_tokens_between():
    """F = (1/2, 1/2, 1/2, 1): tokens 1 and 2 have empty cells at 1/2.  At the
    threshold 1/2 the oracle takes token 3; tokens 0, 1 and 2 end exactly at
    that edge (distance 0), so each is accepted there; the same token at a
    threshold away from any edge is not."""
    prob, q, k, v = _problem([0.0, -1000.0, -1000.0, 0.0], T=64)
    want, rep = _prop_report(prob, q, k, v, 2, 0.0, [0, 3])
    assert want == [0, 3] and rep["mismatch"] == 0
    for alt in (0, 1, 2):
        _, rep = _prop_report(prob, q, k, v, 2, 0.0, [0, alt])
        assert rep["exempt"] == 1 and rep["hard"] == 0, alt
    # U = 1/8: the thresholds 1/8 and 5/8 lie 1/8 or more from every edge
    _, rep = _prop_report(prob, q, k, v, 2, 0.125, [1, 3])
    assert rep["hard"] == 1


def test_flash_uses_the_tile_cdf():
    """Flash on w = (1, 3 | 2, 2), T = 2, S = 4, U = 1/8: u_f = 1/4 puts tile
    0's first threshold on its local edge 1/4.  The other token of tile 0 is
    accepted there; a token of tile 1 is not (its cell is in another tile),
    and within tile 1 a token whose local cell is a quarter away is hard."""
    w = np.array([1.0, 3.0, 2.0, 2.0])
    prob, q, k, v = _problem(np.log(w), T=2)
    S, u = 4, np.array([0.125], np.float32)
    r = O.santa_flash(prob, q, k, v, S, u)
    oi = r["idx"][0].tolist()
    assert oi[2:] == [2, 3] and oi[0] in (0, 1) and oi[1] == 1

    def rep_of(idx):
        return parity.index_report(np.array([idx], np.int32), r["idx"], r["delta"],
                                   lambda tok: O.flash_cells(prob, q, k, S, u, tok))

    assert rep_of(oi)["mismatch"] == 0
    rep = rep_of([1 - oi[0]] + oi[1:])
    assert rep["exempt"] == 1 and rep["hard"] == 0
    assert rep_of([2] + oi[1:])["hard"] == 1          # right local position, wrong tile
    assert rep_of(oi[:3] + [2])["hard"] == 1          # local threshold 3/4 vs token 2's cell [0, 1/2)


def test_cell_distance_undefined_cells_are_infinite():
    d = parity.cell_distance([0.5, 0.5, 0.5], [0.5, np.nan, 0.0], [0.75, 1.0, 0.5])
    assert d[0] == 0.0 and np.isinf(d[1]) and d[2] == 0.0
