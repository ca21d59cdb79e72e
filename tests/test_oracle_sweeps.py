"""Randomised shape sweeps of the oracle's ranking and selection steps against
brute force (CPU only).

Hypothesis draws tiny shapes and contents (derandomised, so every run checks
the same cases); each case is compared with an O(n^2) enumeration written
from the rule itself, not from the oracle's vectorised code:
  * top-k selection ([P1] section 二: 8 of 384 by score): repeatedly take the
    best remaining score, the lower index on ties, -0.0 equal to +0.0;
  * send slots (one fixed pool per destination, capped): an assignment's
    rank is the number of earlier (token, k-slot) assignments to the same
    destination;
  * receive slots (one fixed row block per local expert, capped): a row's
    rank is the number of earlier (source, slot) rows of the same expert;
  * capacities: the ceiling of factor x balanced load, in exact rationals;
  * whole layers on tiny shapes: every token against the dense MoE formula
    with the assignments that survive both caps (found by enumeration).
"""

from fractions import Fraction
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import moe_oracle as O

SWEEP = settings(max_examples=150, deadline=None, derandomize=True)


def _topk_by_enumeration(row, k):
    taken = []
    for _ in range(k):
        best = None
        for e in range(len(row)):
            if e not in taken and (best is None or row[e] > row[best]):
                best = e
        taken.append(best)
    return taken


@SWEEP
@given(st.data())
def test_select_topk_sweep(data):
    E = data.draw(st.integers(1, 40), label="E")
    k = data.draw(st.integers(1, min(8, E)), label="k")
    T = data.draw(st.integers(1, 6), label="T")
    vals = data.draw(st.lists(st.sampled_from([-2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 3.0]),
                              min_size=T * E, max_size=T * E), label="logits")
    logits = np.array(vals, dtype=np.float32).reshape(T, E)
    idx, w = O.select_topk(logits, k)
    for t in range(T):
        want = _topk_by_enumeration([float(v) for v in logits[t]], k)
        assert list(idx[t]) == want
        sel = np.array([logits[t, e] for e in want], dtype=np.float64)
        p = np.exp(sel - sel.max())
        np.testing.assert_allclose(w[t], p / p.sum(), rtol=1e-6, atol=0)


def _send_by_enumeration(idx, X, cap):
    T, k = idx.shape
    flat = [(t, i) for t in range(T) for i in range(k)]
    slot = -np.ones((T, k), dtype=np.int64)
    for (t, i) in flat:
        d = idx[t, i] // X
        earlier = sum(1 for (t2, i2) in flat if (t2, i2) < (t, i) and idx[t2, i2] // X == d)
        if earlier < cap:
            slot[t, i] = d * cap + earlier
    return slot


@SWEEP
@given(st.data())
def test_send_slots_sweep(data):
    R = data.draw(st.integers(1, 5), label="R")
    X = data.draw(st.integers(1, 4), label="X")
    k = data.draw(st.integers(1, min(4, R * X)), label="k")
    T = data.draw(st.integers(0, 12), label="T")
    cap = data.draw(st.integers(1, max(1, T * k)), label="cap")
    rows = [data.draw(st.permutations(range(R * X)), label=f"row{t}")[:k] for t in range(T)]
    idx = np.array(rows, dtype=np.int64).reshape(T, k)
    s = O.send_slots(idx, X, R, cap)
    assert np.array_equal(s["slot_of"], _send_by_enumeration(idx, X, cap))
    demand = np.bincount((idx // X).reshape(-1), minlength=R) if T else np.zeros(R, dtype=np.int64)
    assert np.array_equal(s["demand"], demand)
    assert np.array_equal(s["send_count"], np.minimum(demand, cap))
    assert s["send_dropped"] == int(np.maximum(demand - cap, 0).sum())


def _recv_by_enumeration(ids, r, X, rcap):
    n_src, cap = ids.shape
    order = [(s, sl) for s in range(n_src) for sl in range(cap)]
    rows = [[] for _ in range(X)]
    for (s, sl) in order:
        e = ids[s, sl]
        if e < 0:
            continue
        j = e - X * r
        earlier = sum(1 for (s2, sl2) in order if (s2, sl2) < (s, sl) and ids[s2, sl2] == e)
        if earlier < rcap:
            rows[j].append(s * cap + sl)
    return rows


@SWEEP
@given(st.data())
def test_recv_slots_sweep(data):
    n_src = data.draw(st.integers(1, 5), label="n_src")
    cap = data.draw(st.integers(1, 8), label="cap")
    X = data.draw(st.integers(1, 4), label="X")
    r = data.draw(st.integers(0, 3), label="my_rank")
    rcap = data.draw(st.integers(1, n_src * cap), label="rcap")
    cells = data.draw(st.lists(st.integers(-1, X - 1), min_size=n_src * cap, max_size=n_src * cap), label="ids")
    ids = np.array([c if c < 0 else X * r + c for c in cells], dtype=np.int32).reshape(n_src, cap)
    rv = O.recv_slots(ids, r, X, rcap)
    want = _recv_by_enumeration(ids, r, X, rcap)
    for j in range(X):
        n = int(rv["count"][j])
        assert list(rv["row_src"][j, :n]) == want[j] and np.all(rv["row_src"][j, n:] == -1)
        arrivals = int(np.sum(ids == X * r + j))
        assert rv["arrivals"][j] == arrivals and rv["recv_dropped"][j] == max(0, arrivals - rcap)


@SWEEP
@given(T=st.integers(0, 5000), k=st.integers(1, 32), R=st.integers(1, 1024), Xr=st.integers(1, 64),
       num=st.integers(100, 400), den=st.sampled_from([100, 1000]))
def test_capacities_sweep(T, k, R, Xr, num, den):
    E = R * Xr
    assert O.send_capacity(T, k, R, num, den) == math.ceil(Fraction(num, den) * Fraction(T * k, R))
    assert O.recv_capacity(T, k, R, E, num, den) == math.ceil(Fraction(num, den) * Fraction(R * T * k, E))


def _sweep_shape(R, X, W, k, T, S, sn, rn, act="f32"):
    from dataclasses import replace
    from workload import configs
    return replace(configs.get("mini_f32"), name="sweep", tokens=T, d_model=6, latent=8, n_experts=R * X, top_k=k,
                   n_ranks=R, waves=W, expert_hidden=4, shared_experts=S, shared_hidden=4,
                   send_num=sn, send_den=100, recv_num=rn, recv_den=100, act=act)


@settings(max_examples=60, deadline=None, derandomize=True)
@given(st.data())
def test_layer_sweep_against_textbook_tokens(data):
    """Whole oracle layers on tiny random shapes (ranks, experts per rank,
    waves, top-k, shared experts, both capacity factors; fp32 or bf16
    activations with their rounding points), every token of
    every rank against the dense MoE formula written out per token: the
    routed terms that survive both caps, found by enumeration, weights not
    renormalised, plus the shared path ([P1] sections 二 and 四).  The drop
    ledger equals the enumerated counts."""
    from test_oracle_pins import _brute_kept, _textbook_token
    from workload import gen
    R = data.draw(st.integers(1, 4), label="R")
    X = data.draw(st.integers(1, 3), label="X")
    E = R * X
    W = data.draw(st.sampled_from([w for w in range(1, X + 1) if X % w == 0]), label="waves")
    k = data.draw(st.integers(1, min(4, E)), label="k")
    T = data.draw(st.integers(1, 10), label="T")
    S = data.draw(st.integers(0, 2), label="S")
    sn = data.draw(st.integers(20, 150), label="send %")
    rn = data.draw(st.integers(20, 150), label="recv %")
    act = data.draw(st.sampled_from(["f32", "bf16"]), label="act")
    sh = _sweep_shape(R, X, W, k, T, S, sn, rn, act)
    inp = gen.generate(sh, seed=data.draw(st.integers(0, 10**6), label="seed"))
    res = O.layer_all_ranks(sh, inp)
    idx = [res["dispatch"][s]["idx"] for s in range(R)]
    send_kept, recv_kept = _brute_kept(idx, X, R, res["send_cap"], res["recv_cap"])
    for s in range(R):
        d = res["dispatch"][s]
        for t in range(T):
            ref = _textbook_token(sh, inp, s, t, d["idx"][t], d["w"][t], kept=recv_kept[s, t])
            np.testing.assert_allclose(res["out"][s]["out_exact"][t], ref, rtol=1e-9, atol=1e-12)
    assert int(res["ledger"]["send_dropped"].sum()) == int((~send_kept).sum())
    assert int(res["ledger"]["recv_dropped"].sum()) == int((send_kept & ~recv_kept).sum())
    assert res["ledger"]["kept"] == int(recv_kept.sum()) and res["ledger"]["total"] == R * T * k


def test_layer_with_an_empty_batch():
    """T = 0 on every rank: empty outputs, nothing kept or dropped."""
    from workload import gen
    sh = _sweep_shape(3, 2, 2, 2, 0, 1, 110, 115)
    res = O.layer_all_ranks(sh, gen.generate(sh, seed=3))
    assert all(res["out"][s]["out_exact"].shape == (0, sh.d_model) for s in range(sh.n_ranks))
    assert res["ledger"]["kept"] == 0 and res["ledger"]["total"] == 0
    assert not res["ledger"]["send_dropped"].any() and not res["ledger"]["recv_dropped"].any()


def test_layer_sweep_catches_planted_mistakes(monkeypatch):
    """Each mistake planted in the oracle makes the layer sweep fail."""
    good_send, good_recv, good_ret, good_comb = O.send_slots, O.recv_slots, O.expert_returns, O.combine

    def send_kslot_major(idx, X, R, cap):  # ranks in (k-slot, token) order
        r = good_send(np.ascontiguousarray(idx.T), X, R, cap)
        return dict(r, slot_of=np.ascontiguousarray(r["slot_of"].T))

    def recv_slot_major(pool_ids, my_rank, X, recv_cap):  # rows visited slot by slot across sources
        r = good_recv(np.ascontiguousarray(pool_ids.T), my_rank, X, recv_cap)
        n_src, cap = pool_ids.shape
        pos = r["row_src"]
        src_of = np.where(pos >= 0, (pos % n_src) * cap + pos // n_src, -1)
        return dict(r, row_src=src_of, row_rank=r["row_rank"].T, row_expert=r["row_expert"].T)

    def leaky_returns(pool_rows, recv, w13, w2, hidden, act):  # rows past recv_cap return expert outputs
        X = len(recv["count"])
        je, rk = recv["row_expert"].reshape(-1), recv["row_rank"].reshape(-1)
        row_src = np.full((X, max(int(recv["arrivals"].max()), 1)), -1, dtype=np.int64)
        for j in range(X):
            pos = np.flatnonzero(je == j)
            row_src[j, rk[pos]] = pos
        return good_ret(pool_rows, dict(recv, count=recv["arrivals"], row_src=row_src), w13, w2, hidden, act)

    def renormalised(ret, slot_of, w, cap, act):  # weights renormalised over the assignments kept at send
        kept = np.where(slot_of >= 0, w, 0.0)
        sums = kept.sum(axis=1, keepdims=True)
        return good_comb(ret, slot_of, np.where(sums > 0, kept / np.where(sums > 0, sums, 1), 0.0), cap, act)

    for name, fn in (("send_slots", send_kslot_major), ("recv_slots", recv_slot_major),
                     ("expert_returns", leaky_returns), ("combine", renormalised)):
        monkeypatch.setattr(O, name, fn)
        with pytest.raises(AssertionError):
            test_layer_sweep_against_textbook_tokens()
        monkeypatch.undo()
    test_layer_sweep_against_textbook_tokens()  # and passes again
