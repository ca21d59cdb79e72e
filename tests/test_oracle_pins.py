"""Pins of the CPU oracle against facts it does not compute itself.

Each check is independent of the oracle's own code path: library routines
(torch's bfloat16 conversion, a full softmax), exact integer arithmetic,
closed forms, the pages' constants, O(n^2) brute force on tiny inputs, and
the textbook MoE formula evaluated token by token.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from workload import configs, gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ formats


def test_round_bf16_matches_torch_on_f32_values():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        # exact halfway points between neighbouring bf16 values
        ((rng.integers(0, 2 ** 16, 4000, dtype=np.uint32) << 16) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0], dtype=np.float32),
    ])
    v = v[np.isfinite(v)]
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_round_bf16_direct_from_f64_has_no_double_rounding():
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: ties go to the even significand (1.0)
    assert O.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    # midpoint of 1 + 2^-7 (odd) and 1 + 2^-6 (even) goes up
    assert O.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    # just above the midpoint: float32 would first round to the midpoint and then to 1.0
    v = 1 + 2.0 ** -8 + 2.0 ** -40
    assert np.float32(v) == np.float32(1 + 2.0 ** -8)
    assert O.round_bf16(np.array([v]))[0] == 1 + 2.0 ** -7
    assert O.round_bf16(np.array([-v]))[0] == -(1 + 2.0 ** -7)


# --------------------------------------------------------------- capacities


def test_capacities_against_the_pages_constants():
    c = json.load(open(os.path.join(GOLDEN, "pages_constants.json")))
    T4k = 2 * c["pretrain_context"]["value"]      # 8192 tokens per rank
    k, R, E = c["top_k"]["value"], c["ep_ranks"]["value"], c["routed_experts"]["value"]
    sn, sd = c["send_capacity_factor"]["num"], c["send_capacity_factor"]["den"]
    rn, rd = c["recv_capacity_factor"]["num"], c["recv_capacity_factor"]["den"]
    assert E // R == c["experts_per_rank"]["value"]
    # exact rationals: ceil(1.10 * 8192 * 8 / 64) and ceil(1.15 * 64 * 8192 * 8 / 384)
    assert O.send_capacity(T4k, k, R, sn, sd) == math.ceil(Fraction(110, 100) * T4k * k / R) == 1127
    assert O.recv_capacity(T4k, k, R, E, rn, rd) == math.ceil(Fraction(115, 100) * R * T4k * k / E) == 12562
    assert O.send_capacity(65536, k, R, sn, sd) == 9012
    assert O.recv_capacity(65536, k, R, E, rn, rd) == 100489
    # the tiny fp32 workload: 4 ranks x 6 experts, top-2, 256 tokens per rank
    assert O.send_capacity(256, 2, 4) == 141
    assert O.recv_capacity(256, 2, 4, 24) == 99


def test_capacities_at_other_factors():
    # the factor multiplies the balanced load and the product is rounded up:
    # closed forms at the 4K shape (T*k/R = 1024 rows per pool, R*T*k/E = 10922.67 per expert)
    T, k, R, E = 8192, 8, 64, 384
    assert O.send_capacity(T, k, R, 1, 1) == 1024
    assert O.send_capacity(T, k, R, 125, 100) == 1280
    assert O.send_capacity(T, k, R, 3, 2) == 1536
    assert O.recv_capacity(T, k, R, E, 1, 1) == 10923          # ceil(32768 / 3)
    assert O.recv_capacity(T, k, R, E, 130, 100) == 14200      # ceil(1.3 * 32768 / 3) = ceil(14199.47)
    assert O.recv_capacity(T, k, R, E, 2, 1) == 21846          # ceil(65536 / 3)
    for num, den in [(1, 1), (11, 10), (7, 5), (999, 1000)]:
        for n in (1, 3, 50, 4097):
            assert O.send_capacity(n, 1, 1, num, den) == math.ceil(Fraction(num, den) * n)


def test_capacity_is_exact_where_float_ceil_is_not():
    # 1.10 * 50 is 55.000000000000007 in binary floating point
    assert math.ceil(1.10 * 50) == 56
    assert O.send_capacity(50, 1, 1) == 55
    bad = 0
    for n in range(1, 5000):
        exact = math.ceil(Fraction(110, 100) * n)
        assert O.send_capacity(n, 1, 1) == exact
        bad += math.ceil(1.10 * n) != exact
    assert bad > 0


# ------------------------------------------------------------------ routing


def _brute_topk(row, k):
    """Repeatedly take the best remaining (value, lowest index) -- O(k*E)."""
    taken = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in taken:
                continue
            if best is None or v > row[best]:
                best = e
        taken.append(best)
    return taken


def test_select_topk_brute_force_with_many_ties():
    rng = np.random.default_rng(2)
    for E, k in [(24, 2), (48, 4), (384, 8)]:
        logits = rng.integers(-3, 4, size=(64, E)).astype(np.float32)   # heavy ties
        logits[0, :] = 0.0
        logits[1, ::2] = -0.0                                           # -0 == +0
        idx, _ = O.select_topk(logits, k)
        for t in range(logits.shape[0]):
            assert list(idx[t]) == _brute_topk(list(logits[t]), k)


def test_select_weights_closed_form_and_full_softmax():
    l = np.full((1, 10), -50.0, dtype=np.float32)
    l[0, 3], l[0, 7], l[0, 1] = np.log(4.0), np.log(2.0), 0.0
    idx, w = O.select_topk(l, 3)
    assert list(idx[0]) == [3, 7, 1]
    np.testing.assert_allclose(w[0], [4 / 7, 2 / 7, 1 / 7], rtol=1e-6)
    # equals the full softmax renormalised over the chosen k
    rng = np.random.default_rng(3)
    l = rng.standard_normal((200, 384)).astype(np.float32) * 2
    idx, w = O.select_topk(l, 8)
    p = np.exp(l.astype(np.float64))
    p /= p.sum(axis=1, keepdims=True)
    q = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, q / q.sum(axis=1, keepdims=True), atol=1e-7)
    assert np.all(np.diff(w, axis=1) <= 0) and np.all(w >= 0)


def test_router_logits_exact_on_the_grid():
    sh = configs.get(2)
    inp = gen.generate(configs.with_tokens(sh, 8), seed=5, grid=True, with_foreign=False)
    l = O.router_logits(inp["x"], inp["w_router"])
    x = gen.to_f32(inp["x"]).astype(np.float64)
    w = gen.to_f32(inp["w_router"]).astype(np.float64)
    # integer numerators: x = a/4, w = b * 2^-s
    s = int(np.round(-np.log2(np.min(np.abs(w[w != 0])))))
    a = np.rint(x * 4).astype(np.int64)
    b = np.rint(w * 2.0 ** s).astype(np.int64)
    assert np.array_equal(a / 4.0, x) and np.array_equal(b * 2.0 ** -s, w)
    for t in range(8):
        for e in (0, 17, 383):
            exact = Fraction(int(np.dot(a[t], b[e])), 4 * 2 ** s)
            assert Fraction(float(l[t, e])) == exact


def test_grid_sums_are_exact_in_fp32_in_any_order():
    """What lets the GPU's logits be compared bit for bit on the exact grid:
    at d_model 6144 every partial sum of grid products is an integer multiple
    of 2^-(s+2) below 2^24 units, so float32 addition in any order (natural,
    reversed, shuffled, or in 16- and 64-long blocks summed in another order,
    as a matrix core does) gives the exact value; and grid values are stored
    in bf16 without rounding."""
    sh = configs.get(2)  # the router's shape: d_model 6144, 384 experts
    inp = gen.generate(configs.with_tokens(sh, 4), seed=6, grid=True, with_foreign=False)
    x = gen.to_f32(inp["x"])
    w = gen.to_f32(inp["w_router"])
    s = int(np.round(-np.log2(np.min(np.abs(w[w != 0])))))
    a = np.rint(x.astype(np.float64) * 4).astype(np.int64)
    b = np.rint(w.astype(np.float64) * 2.0 ** s).astype(np.int64)
    # bf16 storage round-trips every grid value (at most 8 significant bits)
    assert np.array_equal(gen.to_f32(gen._store(x, "bf16")), x) and np.array_equal(gen.to_f32(gen._store(w, "bf16")), w)
    rng = np.random.default_rng(3)
    for t in range(2):
        for e in (0, 191, 383):
            exact = np.float64(int(np.dot(a[t], b[e]))) / 2.0 ** (s + 2)
            prod = x[t] * w[e]  # float32 products, exact here
            orders = [np.arange(prod.size), np.arange(prod.size)[::-1], rng.permutation(prod.size)]
            for o in orders:
                acc = np.float32(0)
                for v in prod[o]:
                    acc = np.float32(acc + v)
                assert np.float64(acc) == exact
            for blk in (16, 64):
                parts = [np.float32(0)] * (prod.size // blk)
                for i in range(prod.size // blk):
                    p = np.float32(0)
                    for v in prod[i * blk:(i + 1) * blk]:
                        p = np.float32(p + v)
                    parts[i] = p
                acc = np.float32(0)
                for i in rng.permutation(len(parts)):
                    acc = np.float32(acc + parts[i])
                assert np.float64(acc) == exact


def test_router_bias_rows():
    x = np.zeros((10, 4), dtype=np.float32)
    w = np.zeros((3, 4), dtype=np.float32)
    bias = np.array([[1, 0, 0], [0, 2, 0], [0, 0, 3]], dtype=np.float32)
    l = O.router_logits(x, w, bias, bias_row_tokens=4)
    assert l[0].tolist() == [1, 0, 0] and l[3].tolist() == [1, 0, 0]
    assert l[4].tolist() == [0, 2, 0] and l[9].tolist() == [0, 0, 3]
    l = O.router_logits(x, w, bias[1:2], 0)
    assert np.all(l == np.array([0, 2, 0], dtype=np.float32))


# ----------------------------------------------------------------- dispatch


def _brute_send(idx, X, R, cap):
    T, k = idx.shape
    slot = -np.ones((T, k), dtype=np.int64)
    for t in range(T):
        for i in range(k):
            d = idx[t, i] // X
            earlier = sum(1 for t2 in range(T) for i2 in range(k)
                          if (t2, i2) < (t, i) and idx[t2, i2] // X == d)
            if earlier < cap:
                slot[t, i] = d * cap + earlier
    return slot


def test_send_slots_brute_force():
    rng = np.random.default_rng(4)
    for T, k, X, R, cap in [(30, 2, 2, 3, 9), (25, 3, 3, 4, 6), (40, 4, 6, 2, 50)]:
        idx = np.stack([rng.choice(X * R, k, replace=False) for _ in range(T)])
        s = O.send_slots(idx, X, R, cap)
        assert np.array_equal(s["slot_of"], _brute_send(idx, X, R, cap))
        assert s["send_count"].sum() + s["send_dropped"] == T * k
        assert np.all(s["send_count"] <= cap)


def test_send_closed_form_all_logits_equal():
    # W_r = 0: every token picks experts 0..7 with weights 1/8; rank 0 hosts 0..5, rank 1 hosts 6..7
    T, k, E, R = 8192, 8, 384, 64
    X = E // R
    cap = O.send_capacity(T, k, R)
    idx, w = O.select_topk(np.zeros((T, E), dtype=np.float32), k)
    assert np.all(idx == np.arange(8)) and np.all(w == np.float32(1 / 8))
    s = O.send_slots(idx, X, R, cap)
    assert s["send_count"][0] == s["send_count"][1] == 1127 and s["send_count"][2:].sum() == 0
    assert s["send_dropped"] == T * k - 2 * 1127 == 63282
    kept = s["slot_of"] >= 0
    # destination 0: tokens 0..186 fully, token 187 for k = 0..4
    assert kept[:187, :6].all() and kept[187, :5].all() and not kept[187, 5] and not kept[188:, :6].any()
    # destination 1: tokens 0..562 (k = 6, 7), token 563 for k = 6
    assert kept[:563, 6:].all() and kept[563, 6] and not kept[563, 7] and not kept[564:, 6:].any()


def test_pack_ids_and_rows():
    rng = np.random.default_rng(5)
    T, k, X, R, cap, L = 50, 3, 2, 4, 20, 5
    idx = np.stack([rng.choice(X * R, k, replace=False) for _ in range(T)])
    z = rng.standard_normal((T, L))
    s = O.send_slots(idx, X, R, cap)
    ids, rows = O.pack_pools(idx, s["slot_of"], R, cap, z)
    for t in range(T):
        for i in range(k):
            sl = s["slot_of"][t, i]
            if sl >= 0:
                d, r = divmod(sl, cap)
                assert ids[d, r] == idx[t, i] and np.array_equal(rows[d, r], z[t])
    for d in range(R):
        n = s["send_count"][d]
        assert np.all(ids[d, :n] // X == d) and np.all(ids[d, n:] == -1)


# ------------------------------------------------------------------ receive


def _brute_recv(pool_ids, r, X, rcap):
    n_src, cap = pool_ids.shape
    rows = [[] for _ in range(X)]
    arrivals = [0] * X
    for s in range(n_src):
        for sl in range(cap):
            e = pool_ids[s, sl]
            if e < 0:
                continue
            j = e - X * r
            if arrivals[j] < rcap:
                rows[j].append(s * cap + sl)
            arrivals[j] += 1
    return rows, arrivals


def test_recv_slots_brute_force():
    rng = np.random.default_rng(6)
    for n_src, cap, X, r, rcap in [(4, 10, 3, 1, 7), (6, 12, 6, 2, 9), (3, 30, 2, 0, 100)]:
        ids = np.full((n_src, cap), -1, dtype=np.int32)
        for s in range(n_src):
            n = rng.integers(0, cap + 1)
            ids[s, :n] = X * r + rng.integers(0, X, n)
            ids[s, rng.random(cap) < 0.1] = -1          # holes anywhere
        rv = O.recv_slots(ids, r, X, rcap)
        rows, arr = _brute_recv(ids, r, X, rcap)
        for j in range(X):
            n = rv["count"][j]
            assert list(rv["row_src"][j, :n]) == rows[j] and np.all(rv["row_src"][j, n:] == -1)
            assert rv["arrivals"][j] == arr[j] and rv["recv_dropped"][j] == max(0, arr[j] - rcap)


def test_recv_rejects_a_row_for_another_rank():
    ids = np.array([[0, 1, 7, -1]], dtype=np.int32)   # expert 7 lives on rank 1 for X = 6
    with pytest.raises(AssertionError):
        O.recv_slots(ids, 0, 6, 10)


def test_waves_partition_the_local_experts():
    assert O.wave_experts(6, 3) == [[0, 1], [2, 3], [4, 5]]
    assert O.wave_experts(6, 2) == [[0, 1, 2], [3, 4, 5]]


# ------------------------------------------------------------ whole layer


def _textbook_token(shape, inp, s, t, idx, w, kept=None):
    """Dense MoE formula for one token, fp64, with the layer's rounding points.
    ``kept[i]`` False leaves assignment i out of the routed sum (dropped at
    either side: it contributes nothing and the other weights stay as they
    are); None keeps all k (no capacities)."""
    act, H, HS = shape.act, shape.expert_hidden, shape.shared_hidden
    x = gen.to_f32(inp["x"][s][t]).astype(np.float64)
    Wd = gen.to_f32(inp["w_down"]).astype(np.float64)
    z = O.round_act(np.array([sum(x[q] * Wd[m, q] for q in range(x.size)) for m in range(Wd.shape[0])]), act)
    c = np.zeros(shape.latent)
    for i in range(shape.top_k):
        if kept is not None and not kept[i]:
            continue
        e = idx[i]
        W1 = gen.to_f32(inp["w13"][e][:H]).astype(np.float64)
        W3 = gen.to_f32(inp["w13"][e][H:]).astype(np.float64)
        W2 = gen.to_f32(inp["w2"][e]).astype(np.float64)
        a, b = W1.dot(z), W3.dot(z)
        h = O.round_act(a / (1 + np.exp(-a)) * b, act)
        c += float(w[i]) * O.round_act(W2.dot(h), act)
    c = O.round_act(c, act)
    out = gen.to_f32(inp["w_up"]).astype(np.float64).dot(c)
    for j in range(shape.shared_experts):
        W = gen.to_f32(inp["ws13"][j]).astype(np.float64)
        a, b = W[:HS].dot(x), W[HS:].dot(x)
        h = O.round_act(a / (1 + np.exp(-a)) * b, act)
        out += gen.to_f32(inp["ws2"][j]).astype(np.float64).dot(h)
    return out


def test_no_drop_limit_equals_textbook_moe():
    from dataclasses import replace
    sh = replace(configs.get("mini_f32"), send_num=100000, recv_num=100000)
    inp = gen.generate(sh, seed=7)
    res = O.layer_all_ranks(sh, inp)
    assert res["ledger"]["send_dropped"].sum() == 0 and res["ledger"]["recv_dropped"].sum() == 0
    rng = np.random.default_rng(0)
    for s in range(sh.n_ranks):
        d = res["dispatch"][s]
        for t in rng.choice(sh.tokens, 6, replace=False):
            ref = _textbook_token(sh, inp, s, t, d["idx"][t], d["w"][t])
            np.testing.assert_allclose(res["out"][s]["out_exact"][t], ref, rtol=1e-9, atol=1e-12)


def test_no_shared_experts_is_the_routed_textbook_layer():
    """S = 0 (a layer without the always-on shared experts): the output is the
    routed term alone, the textbook MoE evaluated token by token."""
    from dataclasses import replace
    sh = replace(configs.get("mini_f32"), shared_experts=0, send_num=100000, recv_num=100000)
    inp = gen.generate(sh, seed=9)
    res = O.layer_all_ranks(sh, inp)
    rng = np.random.default_rng(1)
    for s in range(sh.n_ranks):
        d = res["dispatch"][s]
        assert res["out"][s]["hs"].shape == (sh.tokens, 0)
        for t in rng.choice(sh.tokens, 6, replace=False):
            ref = _textbook_token(sh, inp, s, t, d["idx"][t], d["w"][t])
            np.testing.assert_allclose(res["out"][s]["out_exact"][t], ref, rtol=1e-9, atol=1e-12)


def test_a_fully_dropped_token_gets_the_shared_path_only():
    from dataclasses import replace
    sh = replace(configs.get("mini_f32"), send_num=1, send_den=100)   # tiny send pools
    inp = gen.generate(sh, seed=8)
    res = O.layer_all_ranks(sh, inp)
    hit = 0
    for s in range(sh.n_ranks):
        d = res["dispatch"][s]
        dropped = np.all(d["slot_of"] < 0, axis=1)
        for t in np.flatnonzero(dropped)[:5]:
            hit += 1
            x = gen.to_f32(inp["x"][s][t]).astype(np.float64)
            ref = np.zeros(sh.d_model)
            for j in range(sh.shared_experts):
                W = gen.to_f32(inp["ws13"][j]).astype(np.float64)
                a, b = W[:sh.shared_hidden] @ x, W[sh.shared_hidden:] @ x
                ref += gen.to_f32(inp["ws2"][j]).astype(np.float64) @ O.round_act(a / (1 + np.exp(-a)) * b, sh.act)
            np.testing.assert_allclose(res["out"][s]["out_exact"][t], ref, rtol=1e-12, atol=1e-12)
    assert hit > 0


def _brute_kept(idx_by_src, X, R, scap, rcap):
    """Kept flag of every assignment of every source, by enumeration.

    Send side: (t, i) is kept iff fewer than scap earlier assignments of its
    source (in (t, i) order) go to the same destination; its slot is that
    count.  Receive side: rank r visits sources in order and slots in order;
    a row is kept iff fewer than rcap earlier visited rows carry an expert of
    the same local index.  Returns (send_kept, recv_kept) as [R][T][k] bools."""
    n_src = len(idx_by_src)
    T, k = idx_by_src[0].shape
    slot = np.full((n_src, T, k), -1, dtype=np.int64)
    for s in range(n_src):
        used = [0] * R
        for t in range(T):
            for i in range(k):
                d = int(idx_by_src[s][t, i]) // X
                if used[d] < scap:
                    slot[s, t, i] = used[d]
                used[d] += 1
    recv_kept = np.zeros((n_src, T, k), dtype=bool)
    for r in range(R):
        seen = [0] * X
        for s in range(n_src):
            # the rows of pool (s -> r) in slot order
            rows = sorted((slot[s, t, i], t, i) for t in range(T) for i in range(k)
                          if slot[s, t, i] >= 0 and int(idx_by_src[s][t, i]) // X == r)
            for _, t, i in rows:
                j = int(idx_by_src[s][t, i]) - X * r
                recv_kept[s, t, i] = seen[j] < rcap
                seen[j] += 1
    return slot >= 0, recv_kept


def _recv_drop_case(seed=12):
    """mini_f32 with send pools no token overfills and a receive cap of 0.7 of
    the balanced load, so that only the receive cap drops."""
    from dataclasses import replace
    sh = replace(configs.get("mini_f32"), send_num=100000, recv_num=70)
    return sh, gen.generate(sh, seed=seed)


def test_receive_dropped_assignment_contributes_nothing():
    """[P1 section 四]: a dropped assignment is not a dropped token.  Per token,
    by brute force: with a receive cap that binds, every token gets exactly its
    routed terms that survive both caps (weights not renormalised) plus the
    shared path; the returned row of a receive-dropped assignment is zero."""
    sh, inp = _recv_drop_case()
    res = O.layer_all_ranks(sh, inp)
    scap, rcap = res["send_cap"], res["recv_cap"]
    X, R = sh.local_experts, sh.n_ranks
    idx = [res["dispatch"][s]["idx"] for s in range(R)]
    send_kept, recv_kept = _brute_kept(idx, X, R, scap, rcap)
    assert send_kept.all(), "the send pools are sized so that nothing drops at send"
    assert (~recv_kept).sum() > 20, "the receive cap must bind"
    checked = 0
    for s in range(R):
        d = res["dispatch"][s]
        hit = np.flatnonzero(~recv_kept[s].all(axis=1))
        for t in hit[:8]:
            ref = _textbook_token(sh, inp, s, t, d["idx"][t], d["w"][t], kept=recv_kept[s, t])
            np.testing.assert_allclose(res["out"][s]["out_exact"][t], ref, rtol=1e-9, atol=1e-12)
            checked += 1
            for i in np.flatnonzero(~recv_kept[s, t]):
                dest, sl = divmod(int(d["slot_of"][t, i]), scap)
                assert not np.any(res["ret"][dest][s, sl]), "a receive-dropped row returned nonzero values"
        # and a token that lost nothing is the plain textbook token
        whole = np.flatnonzero(recv_kept[s].all(axis=1))
        t = whole[0]
        ref = _textbook_token(sh, inp, s, t, d["idx"][t], d["w"][t])
        np.testing.assert_allclose(res["out"][s]["out_exact"][t], ref, rtol=1e-9, atol=1e-12)
    assert checked >= 2 * R


def _brute_wave_buffer(pool_ids, pool_rows, my_rank, X, experts, rcap):
    """Wave buffer by a plain walk over (source, slot): row q of expert j is the
    q-th row (q < rcap) that carries expert X*my_rank + j."""
    n_src, cap, L = pool_rows.shape
    buf = np.zeros((len(experts), rcap, L))
    for a, j in enumerate(experts):
        q = 0
        for s in range(n_src):
            for sl in range(cap):
                if pool_ids[s, sl] == X * my_rank + j:
                    if q < rcap:
                        buf[a, q] = pool_rows[s, sl]
                    q += 1
    return buf


def test_wave_buffer_by_enumeration():
    """[P1 section 二]: each wave holds its experts' received rows in buffers of
    one shape; rows in arrival order, at most recv_cap per expert."""
    sh, inp = _recv_drop_case(seed=13)
    res = O.layer_all_ranks(sh, inp)
    scap, rcap, X, R = res["send_cap"], res["recv_cap"], sh.local_experts, sh.n_ranks
    assert res["ledger"]["recv_dropped"].sum() > 0
    shapes = set()
    for r in range(R):
        pool_ids = np.stack([res["dispatch"][s]["pool_ids"][r] for s in range(R)])
        pool_rows = np.stack([res["dispatch"][s]["pool_rows"][r] for s in range(R)])
        for experts in O.wave_experts(X, sh.waves):
            got = O.wave_buffer(pool_rows, res["recv"][r], experts, rcap)
            want = _brute_wave_buffer(pool_ids, pool_rows, r, X, experts, rcap)
            assert np.array_equal(got, want)
            shapes.add(got.shape)
    assert len(shapes) == 1, "every wave buffer has the same shape"


def test_expert_permutation_invariance_without_drops():
    from dataclasses import replace
    sh = replace(configs.get("mini_f32"), send_num=100000, recv_num=100000)
    inp = gen.generate(sh, seed=9)
    res = O.layer_all_ranks(sh, inp)
    perm = np.random.default_rng(1).permutation(sh.n_experts)
    inp2 = dict(inp)
    inp2["w_router"] = inp["w_router"][perm]
    inp2["w13"] = inp["w13"][perm]
    inp2["w2"] = inp["w2"][perm]
    res2 = O.layer_all_ranks(sh, inp2)
    for s in range(sh.n_ranks):
        np.testing.assert_allclose(res2["out"][s]["out_exact"], res["out"][s]["out_exact"], rtol=1e-6, atol=1e-9)


@pytest.mark.parametrize("name", ["cfg1", "mini_bf16_skew", "mini_bf16_seg"])
def test_ledger_invariants(name):
    sh = configs.get(1) if name == "cfg1" else configs.get(name)
    inp = gen.generate(sh, seed=0)
    res = O.layer_all_ranks(sh, inp)
    led = res["ledger"]
    assert led["kept"] + led["send_dropped"].sum() + led["recv_dropped"].sum() == led["total"]
    scap, rcap = res["send_cap"], res["recv_cap"]
    for s in range(sh.n_ranks):
        d = res["dispatch"][s]
        assert np.all(d["send_count"] <= scap) and d["send_count"].sum() + d["send_dropped"] == sh.tokens * sh.top_k
        kept = d["slot_of"][d["slot_of"] >= 0]
        assert len(np.unique(kept)) == kept.size                  # slot_of is injective
        np.testing.assert_allclose(d["w"].astype(np.float64).sum(axis=1), 1.0, atol=4 * 2.0 ** -23)
    for r in range(sh.n_ranks):
        rv = res["recv"][r]
        assert np.all(rv["count"] <= rcap)
        assert np.array_equal(rv["arrivals"], rv["count"] + rv["recv_dropped"])
        # a returned row is a zero row exactly where the row was dropped at receive
        # or the slot is empty; every kept row carries an expert output (nonzero
        # for these inputs: a zero output row would need every hidden value zero)
        ret = res["ret"][r].reshape(-1, sh.latent)
        zero = ~np.any(ret != 0, axis=1)
        rank, expert = rv["row_rank"].reshape(-1), rv["row_expert"].reshape(-1)
        kept_row = (expert >= 0) & (rank < rcap)
        assert np.array_equal(zero, ~kept_row), f"rank {r}: zero returned rows != rows not kept"
    # both caps bind in these workloads
    assert led["send_dropped"].sum() > 0 and led["recv_dropped"].sum() > 0


def test_one_rank_layer_matches_all_rank_emulation():
    """The one-rank share equals the same rank inside a full emulation when the
    other ranks' pools and returns are taken from that emulation."""
    sh = configs.get("mini_bf16")
    inp = gen.generate(sh, seed=3)
    full = O.layer_all_ranks(sh, inp)
    r = 2
    from dataclasses import replace
    one_sh = replace(sh, emulate_all_ranks=False)
    scap = full["send_cap"]
    one = dict(x=inp["x"][r], w_router=inp["w_router"], w_down=inp["w_down"], bias=None,
               bias_row_tokens=0, receiver=r, w13=inp["w13"][r * 6:(r + 1) * 6],
               w2=inp["w2"][r * 6:(r + 1) * 6], w_up=inp["w_up"], ws13=inp["ws13"], ws2=inp["ws2"])
    one["foreign_ids"] = np.stack([full["dispatch"][s]["pool_ids"][r] for s in range(sh.n_ranks)])
    rows = np.stack([full["dispatch"][s]["pool_rows"][r] for s in range(sh.n_ranks)])
    one["foreign_rows"] = rows.astype(np.float32)
    one["foreign_ret"] = np.stack([full["ret"][d][r] for d in range(sh.n_ranks)]).astype(np.float32)
    res = O.layer_one_rank(one_sh, one)
    assert np.array_equal(res["recv"]["row_src"], full["recv"][r]["row_src"])
    np.testing.assert_array_equal(res["out"], full["out"][r]["out"])
    assert scap == res["send_cap"]


def test_routed_source_pools_match_all_rank_emulation():
    """The pools other ranks send to the measured rank, made by routing their
    own tokens (one-rank workloads), are exactly the pools those ranks send in
    the all-rank emulation of the same seed; the per-rank token draws agree."""
    from dataclasses import replace
    sh = configs.get("mini_bf16_skew")
    full_inp = gen.generate(sh, seed=7, grid=True)
    full = O.layer_all_ranks(sh, full_inp)
    one_sh = replace(sh, emulate_all_ranks=False, foreign="routed")
    scap, _ = O.capacities(one_sh)
    inp = gen.generate(one_sh, seed=7, grid=True, send_cap=scap)
    r = inp["receiver"]
    assert r == 0 and np.array_equal(inp["x"], full_inp["x"][r])
    for s in range(sh.n_ranks):
        assert np.array_equal(inp["sources"](s), full_inp["x"][s])
    ids, rows, tok = O.routed_source_pools(one_sh, inp, with_rows=True)
    for s in range(sh.n_ranks):
        if s == r:
            assert np.all(ids[s] == -1) and np.all(tok[s] == -1)
            continue
        d = full["dispatch"][s]
        assert np.array_equal(ids[s], d["pool_ids"][r])
        assert np.array_equal(rows[s], d["pool_rows"][r])
        kept = ids[s] >= 0
        assert np.all((tok[s] >= 0) == kept)
        # the token of every filled slot really chose that expert
        assert all(ids[s][q] in d["idx"][tok[s][q]] for q in np.flatnonzero(kept))
        assert all(r * sh.local_experts <= ids[s][q] < (r + 1) * sh.local_experts for q in np.flatnonzero(kept))
    # and the one-rank receive of those pools equals rank r's receive in the emulation
    inp["foreign_ids"] = ids
    res = O.layer_one_rank(one_sh, inp, with_floats=False)
    assert np.array_equal(res["recv"]["row_src"], full["recv"][r]["row_src"])
    assert np.array_equal(res["recv"]["recv_dropped"], full["recv"][r]["recv_dropped"])


# ------------------------------------------------------- planted mistakes


def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle and check that a pin fails."""
    rng = np.random.default_rng(10)
    idx = np.stack([rng.choice(12, 3, replace=False) for _ in range(30)])

    # 1. send ranks in (k-slot, token) order instead of (token, k-slot)
    good = O.send_slots(idx, 3, 4, 7)["slot_of"]
    bad = O.send_slots(idx.T.copy(), 3, 4, 7)["slot_of"].T
    assert not np.array_equal(bad, _brute_send(idx, 3, 4, 7))
    assert np.array_equal(good, _brute_send(idx, 3, 4, 7))

    # 2. tie-break by higher index
    l = rng.integers(-2, 3, size=(20, 24)).astype(np.float32)
    bad_idx = (23 - np.argsort(-l[:, ::-1], axis=1, kind="stable")[:, :4])
    assert any(list(bad_idx[t]) != _brute_topk(list(l[t]), 4) for t in range(20))

    # 3. gate and up swapped: the textbook pin sees it
    from dataclasses import replace
    sh = replace(configs.get("mini_f32"), send_num=100000, recv_num=100000)
    inp = gen.generate(sh, seed=11)
    orig = O.swiglu_hidden

    def swapped(inp_, w13, hidden, act):
        return orig(inp_, np.concatenate([w13[hidden:], w13[:hidden]]), hidden, act)

    monkeypatch.setattr(O, "swiglu_hidden", swapped)
    res = O.layer_all_ranks(sh, inp)
    d = res["dispatch"][0]
    ref = _textbook_token(sh, inp, 0, 0, d["idx"][0], d["w"][0])
    assert not np.allclose(res["out"][0]["out_exact"][0], ref, rtol=1e-6)
    monkeypatch.setattr(O, "swiglu_hidden", orig)

    # 4. combine forgets the routing weight
    orig_c = O.combine

    def unweighted(ret, slot_of, w, cap, act):
        return orig_c(ret, slot_of, np.ones_like(w), cap, act)

    monkeypatch.setattr(O, "combine", unweighted)
    res = O.layer_all_ranks(sh, inp)
    assert not np.allclose(res["out"][0]["out_exact"][0], ref, rtol=1e-6)
    monkeypatch.setattr(O, "combine", orig_c)

    # 5. rows past recv_cap return expert outputs instead of zero rows
    orig_r = O.expert_returns

    def leaky(pool_rows, recv, w13, w2, hidden, act):
        X = len(recv["count"])
        je, rk = recv["row_expert"].reshape(-1), recv["row_rank"].reshape(-1)
        row_src = np.full((X, max(int(recv["arrivals"].max()), 1)), -1, dtype=np.int64)
        for j in range(X):
            pos = np.flatnonzero(je == j)
            row_src[j, rk[pos]] = pos
        return orig_r(pool_rows, dict(recv, count=recv["arrivals"], row_src=row_src), w13, w2, hidden, act)

    monkeypatch.setattr(O, "expert_returns", leaky)
    with pytest.raises(AssertionError):
        test_receive_dropped_assignment_contributes_nothing()
    monkeypatch.setattr(O, "expert_returns", orig_r)

    # 6. receive ranking slot-major instead of source-major
    orig_s = O.recv_slots

    def slot_major(pool_ids, my_rank, X, recv_cap):
        r = orig_s(np.ascontiguousarray(pool_ids.T), my_rank, X, recv_cap)
        n_src, cap = pool_ids.shape
        pos = r["row_src"]
        src_of = np.where(pos >= 0, (pos % n_src) * cap + pos // n_src, -1)
        return dict(r, row_src=src_of, row_rank=r["row_rank"].T, row_expert=r["row_expert"].T)

    monkeypatch.setattr(O, "recv_slots", slot_major)
    with pytest.raises(AssertionError):
        test_wave_buffer_by_enumeration()
    monkeypatch.setattr(O, "recv_slots", orig_s)
