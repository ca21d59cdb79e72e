"""CPU oracle of the fixed-pool, three-wave MoE expert layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
CPU-baseline leg of the benchmark may import this module.  It shares no code
with the GPU path (no kernels, no headers, no helpers); the only common code
is the seeded input generator in ``workload``.

Plain, slow, obviously correct: numpy in float64, a library matmul as the only
primitive, one function per step of the layer, each citing the passage it
follows.  Sources (Marin 535B-A23B):
  [P1] "Marin 开始公开训练 535B 参数 MoE 模型" (lamjinlab blog), section 二
       "稀疏模型如何组织" and section 四 "长上下文取决于解决词元丢弃问题";
  [P2] "535B大模型"直播"训练三个月：代码、数据、Loss全公开…" (huxiu / AI前线),
       sections "535B并不意味着每次都要运行535B参数" and
       "训练MoE，难点不只是把模型切到更多GPU上".
Where the pages are silent the reading taken is stated at the function; every
such reading is listed together with the others in the design notes.

Number formats: ``act`` is "bf16" or "f32".  Every value handed from one step
to the next is rounded to ``act`` (round to nearest, ties to even); inside a
step the oracle accumulates in float64.  Router logits and routing weights
are float32.
"""

import numpy as np

from workload.gen import to_f32


# ===================================================================== formats


def round_bf16(v):
    """Nearest bfloat16 value (8 significant bits), ties to even, as float64.

    Rounds the float64 input directly (no detour through float32, so there is
    no double rounding).  Subnormal bf16 values use the fixed quantum 2**-133.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                  # v = m * 2**e with 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)         # quantum of the 8-bit significand
    r = np.ldexp(np.rint(np.ldexp(v, -q)), q)   # np.rint: half to even
    r[np.abs(r) > 3.3895313892515355e38] = np.inf * np.sign(r[np.abs(r) > 3.3895313892515355e38])
    return r


def round_f32(v):
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_act(v, act):
    return round_bf16(v) if act == "bf16" else round_f32(v)


def f64(a):
    """Generator storage (bf16 bits or float32) -> float64 values."""
    return to_f32(a).astype(np.float64)


# ================================================================== capacities


def send_capacity(T, k, R, num=110, den=100):
    """Rows of each fixed per-destination send pool.

    [P1 §二]: each sender keeps one fixed pool per destination GPU, and a send
    capacity factor of 1.10 caps what one source sends to one destination.
    Reading: the factor multiplies the balanced load T*k/R of one pool and the
    product is rounded up, in exact integer arithmetic.
    """
    return -(-(num * T * k) // (den * R))


def recv_capacity(T, k, R, E, num=115, den=100):
    """Rows each local expert accepts on the receive side.

    [P1 §二]: a receive capacity factor of 1.15 caps the rows assigned to one
    local expert.  Reading: the factor multiplies the balanced (static) load
    R*T*k/E of one expert, rounded up in exact integer arithmetic.
    """
    return -(-(num * R * T * k) // (den * E))


# ===================================================================== routing


def router_logits(x, w_router, bias=None, bias_row_tokens=0):
    """Router scores l = x . W_r^T (+ bias), accumulated in float64, stored float32.

    [P1 §二]: every block has a router over 384 routed experts.  The bias is a
    workload feature (per-expert skew, or per-segment boosts every
    ``bias_row_tokens`` tokens); it is added before selection.
    """
    X = f64(x)
    l = X @ f64(w_router).T
    if bias is not None:
        b = np.asarray(bias, dtype=np.float64)
        if bias_row_tokens:
            l = l + b[np.arange(X.shape[0]) // bias_row_tokens]
        else:
            l = l + b[0][None, :]
    return l.astype(np.float32)


def select_topk(logits, k):
    """Top-k experts per token and their renormalised softmax weights.

    [P1 §二]: the router picks 8 experts for every token.  Readings: selection
    on the float32 logits; the k chosen experts listed by descending score,
    equal scores ordered by lower expert index (-0.0 equals +0.0); weights are
    the softmax restricted to the k chosen scores,
    w_i = exp(l_i - l_0) / sum_j exp(l_j - l_0), which equals the full softmax
    renormalised over the k (the common denominator cancels).
    """
    l32 = np.asarray(logits, dtype=np.float32)
    assert np.all(np.isfinite(l32))
    order = np.argsort(-l32, axis=1, kind="stable")   # stable: lower index first on ties
    idx = order[:, :k].astype(np.int32)
    top = np.take_along_axis(l32, idx, axis=1).astype(np.float64)
    e = np.exp(top - top[:, :1])
    w = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx, w


def down_project(x, w_down, act):
    """Latent z = x . W_d^T (6144 -> 3072), rounded to the activation type.

    [P1 §二]: a latent projection compresses the routed activations from 6,144
    to 3,072 values before they cross GPUs, halving the all-to-all width.
    """
    return round_act(f64(x) @ f64(w_down).T, act)


# ==================================================================== dispatch


def send_slots(idx, X, R, send_cap):
    """Slot of every assignment in its destination's fixed pool.

    [P1 §二]: one fixed pool per destination GPU (6 routed experts per GPU),
    capped by the send capacity; anything over the cap is dropped and counted.
    Readings: expert e lives on rank e // X; assignments (t, i) are ranked
    within their destination in (token, k-slot) order; the first send_cap
    keep their rank as slot.

    Returns slot_of [T][k] (dest*send_cap + slot, or -1 if dropped),
    demand [R] (assignments per destination), send_count [R] (kept rows),
    send_dropped (total dropped).
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    dest = (idx // X).reshape(-1)                # lexicographic (t, i) order
    order = np.argsort(dest, kind="stable")      # keeps (t, i) order inside a dest
    demand = np.bincount(dest, minlength=R)
    first = np.concatenate([[0], np.cumsum(demand)[:-1]])
    rank = np.empty_like(dest)
    rank[order] = np.arange(dest.size) - first[dest[order]]
    kept = rank < send_cap
    slot_of = np.where(kept, dest * send_cap + rank, -1).reshape(T, k).astype(np.int32)
    send_count = np.minimum(demand, send_cap).astype(np.int64)
    return {"slot_of": slot_of, "demand": demand.astype(np.int64),
            "send_count": send_count, "send_dropped": int((~kept).sum())}


def pack_pools(idx, slot_of, R, send_cap, z=None):
    """Fill the fixed send pools: row = latent of the token, tagged with the expert id.

    [P1 §二]: the expert identifier is packed into the activation payload, so
    no token counts or routing metadata are exchanged.  Empty slots carry the
    id -1 (reading).  Returns ids [R][send_cap] int32 and, if z is given,
    rows [R][send_cap][L] (float64; empty rows are 0, their content is
    unspecified on the GPU path).
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    ids = np.full(R * send_cap, -1, dtype=np.int32)
    flat_slot = slot_of.reshape(-1)
    keep = flat_slot >= 0
    ids[flat_slot[keep]] = idx.reshape(-1)[keep]
    rows = None
    if z is not None:
        rows = np.zeros((R * send_cap, z.shape[1]), dtype=np.float64)
        tok = np.repeat(np.arange(T), k)[keep]
        rows[flat_slot[keep]] = z[tok]
        rows = rows.reshape(R, send_cap, z.shape[1])
    return ids.reshape(R, send_cap), rows


# ===================================================================== receive


def recv_slots(pool_ids, my_rank, X, recv_cap):
    """Place the rows arriving at one rank into its local experts' fixed rows.

    [P1 §二]: the receive capacity factor caps the rows assigned to one local
    expert; rows over it are dropped and reported separately from send drops.
    Readings: the receiver sees pools in source order and slots in order
    (src-major, which is token-index-then-k-slot order for globally numbered
    tokens); row (src, slot) with id e goes to local expert e - X*my_rank;
    its rank among earlier rows of that expert decides whether it fits.

    pool_ids: [R_src][send_cap] ids received from every source.
    Returns row_src [X][recv_cap] (src*send_cap + slot, -1 past the count),
    count [X], arrivals [X], recv_dropped [X], row_rank [R_src][send_cap]
    (-1 for empty slots), row_expert [R_src][send_cap] (-1 for empty slots).
    """
    ids = np.asarray(pool_ids, dtype=np.int64)
    n_src, cap = ids.shape
    flat = ids.reshape(-1)
    valid = flat >= 0
    assert np.all(flat[valid] // X == my_rank), "a row reached a rank that does not host its expert"
    j = np.where(valid, flat - X * my_rank, X)   # X = bucket of empty slots
    order = np.argsort(j, kind="stable")
    arrivals_all = np.bincount(j, minlength=X + 1)
    first = np.concatenate([[0], np.cumsum(arrivals_all)[:-1]])
    rank = np.empty_like(flat)
    rank[order] = np.arange(flat.size) - first[j[order]]
    rank = np.where(valid, rank, -1)
    arrivals = arrivals_all[:X].astype(np.int64)
    count = np.minimum(arrivals, recv_cap)
    row_src = np.full((X, recv_cap), -1, dtype=np.int32)
    kept = valid & (rank < recv_cap)
    pos = np.flatnonzero(kept)
    row_src[j[pos], rank[pos]] = pos
    return {"row_src": row_src, "count": count, "arrivals": arrivals,
            "recv_dropped": (arrivals - count).astype(np.int64),
            "row_rank": rank.reshape(n_src, cap).astype(np.int32),
            "row_expert": np.where(valid, j, -1).reshape(n_src, cap).astype(np.int32)}


def wave_experts(X, W):
    """Local experts of each receive wave.

    [P1 §二]: the transfer runs in three consecutive waves with identical array
    shapes, so only part of the receive pool is live at a time.  Reading: wave
    w serves the local experts w*X/W .. (w+1)*X/W - 1 (experts {2w, 2w+1} for
    6 experts in 3 waves), each in a buffer of recv_cap rows.
    """
    assert X % W == 0
    g = X // W
    return [list(range(w * g, (w + 1) * g)) for w in range(W)]


def wave_buffer(pool_rows, recv, experts, recv_cap):
    """Equal-shape wave buffer [len(experts)][recv_cap][L] (unused rows 0)."""
    n_src, cap, L = pool_rows.shape
    flat = pool_rows.reshape(n_src * cap, L)
    buf = np.zeros((len(experts), recv_cap, L))
    for a, j in enumerate(experts):
        n = recv["count"][j]
        buf[a, :n] = flat[recv["row_src"][j, :n]]
    return buf


# ===================================================================== experts


def silu(a):
    return a / (1.0 + np.exp(-a))


def swiglu_hidden(inp, w13, hidden, act):
    """h = act(silu(inp . W_gate^T) * (inp . W_up^T)); w13 rows: gate then up.

    [P2, "535B并不意味着…"]: routed and shared experts are FFNs of reduced width.
    Reading: SwiGLU experts; w13 holds the gate rows then the up rows.
    """
    W = f64(w13)
    a = inp @ W[:hidden].T
    b = inp @ W[hidden:].T
    return round_act(silu(a) * b, act)


def expert_ffn(z_rows, w13, w2, hidden, act):
    """One routed expert on its rows: y = act(h . W2^T), h as in swiglu_hidden."""
    h = swiglu_hidden(z_rows, w13, hidden, act)
    return round_act(h @ f64(w2).T, act)


def expert_returns(pool_rows, recv, w13_local, w2_local, hidden, act):
    """Rows the receiver sends back, indexed like its incoming pools.

    [P2, "训练MoE，难点…"]: after the experts run, results travel back to where
    the tokens came from.  Readings: ret[src][slot] = expert output for a kept
    row; a row dropped at receive gets a zero row (it contributes nothing,
    [P1 §四]: a dropped assignment is not a dropped token); empty slots stay 0.
    Returns ret [R_src][send_cap][L] and a mask of defined rows.
    """
    n_src, cap, L = pool_rows.shape
    flat = pool_rows.reshape(n_src * cap, L)
    ret = np.zeros((n_src * cap, L))
    for j in range(len(recv["count"])):
        n = recv["count"][j]
        rows = recv["row_src"][j, :n]
        if n:
            ret[rows] = expert_ffn(flat[rows], w13_local[j], w2_local[j], hidden, act)
    defined = (recv["row_expert"] >= 0).reshape(-1)
    return ret.reshape(n_src, cap, L), defined.reshape(n_src, cap)


# ===================================================================== combine


def combine(ret_from_dest, slot_of, w, send_cap, act):
    """c_t = act(sum_i w_ti * returned_row(t, i)) in latent space, i ascending.

    [P1 §二]: the routed output is projected back to model width before it
    merges with the shared path; [P1 §四]: the 8 routed experts add to the
    shared path, so a dropped assignment contributes nothing.  Readings: the
    weighted sum is taken in the 3,072-wide latent space (one up-projection
    afterwards, equal by linearity); dropped assignments (slot -1) add 0; the
    weights are not renormalised after drops.
    ret_from_dest: [R_dst][send_cap][L], rows returned by each destination.
    """
    n_dst, cap, L = ret_from_dest.shape
    flat = ret_from_dest.reshape(n_dst * cap, L)
    T, k = slot_of.shape
    c = np.zeros((T, L))
    w64 = np.asarray(w, dtype=np.float64)
    for i in range(k):
        s = slot_of[:, i]
        m = s >= 0
        c[m] += w64[m, i, None] * flat[s[m]]
    return round_act(c, act)


def shared_hidden(x, ws13, shared_hidden_width, act):
    """Hidden activations of the always-on shared experts: [T][S*HS].

    [P1 §二]: 2 shared experts stay local and process every token, outside
    the routed path.  Reading: SwiGLU experts on the 6,144-wide input.  With
    no shared experts (S = 0) the hidden rows are empty and the shared term
    of the output is zero.
    """
    X = f64(x)
    if ws13.shape[0] == 0:
        return np.zeros((X.shape[0], 0))
    return np.concatenate([swiglu_hidden(X, ws13[j], shared_hidden_width, act)
                           for j in range(ws13.shape[0])], axis=1)


def layer_output(c, hs, w_up, ws2, act):
    """out = act(c . U^T + sum_j hs_j . Ws2_j^T); also returns the unrounded value.

    [P1 §二]: the routed output is projected back to model width (3,072 ->
    6,144) and then merged with the shared-expert path.  Reading: the merge
    is a plain sum; no residual (it is outside the MoE branch).
    """
    S = ws2.shape[0]
    HS = ws2.shape[2]
    exact = c @ f64(w_up).T
    for j in range(S):
        exact = exact + hs[:, j * HS:(j + 1) * HS] @ f64(ws2[j]).T
    return round_act(exact, act), exact


# ================================================================ whole layer


def _dims(shape):
    return dict(T=shape.tokens, D=shape.d_model, L=shape.latent, E=shape.n_experts,
                k=shape.top_k, R=shape.n_ranks, X=shape.local_experts, W=shape.waves,
                H=shape.expert_hidden, S=shape.shared_experts, HS=shape.shared_hidden,
                act=shape.act)


def capacities(shape):
    return (send_capacity(shape.tokens, shape.top_k, shape.n_ranks, shape.send_num, shape.send_den),
            recv_capacity(shape.tokens, shape.top_k, shape.n_ranks, shape.n_experts,
                          shape.recv_num, shape.recv_den))


def dispatch(shape, x, w_router, w_down, bias=None, bias_row_tokens=0, with_rows=True):
    """Route + pack for one source rank."""
    d = _dims(shape)
    scap, _ = capacities(shape)
    logits = router_logits(x, w_router, bias, bias_row_tokens)
    idx, w = select_topk(logits, d["k"])
    z = down_project(x, w_down, d["act"]) if with_rows else None
    s = send_slots(idx, d["X"], d["R"], scap)
    ids, rows = pack_pools(idx, s["slot_of"], d["R"], scap, z)
    return dict(logits=logits, idx=idx, w=w, z=z, pool_ids=ids, pool_rows=rows, **s)


def layer_all_ranks(shape, inp):
    """Every rank of the EP domain emulated on the host (small workloads).

    Returns per-rank dispatch results, per-receiver receive results and
    returned rows, per-source outputs, and the drop ledger.
    """
    d = _dims(shape)
    R, X, H, HS, act = d["R"], d["X"], d["H"], d["HS"], d["act"]
    scap, rcap = capacities(shape)
    bias = inp["bias"]
    disp = []
    for s in range(R):
        b = None if bias is None else (bias[s] if bias.ndim == 3 else bias)
        disp.append(dispatch(shape, inp["x"][s], inp["w_router"], inp["w_down"], b,
                             inp["bias_row_tokens"]))
    recvs, rets = [], []
    for r in range(R):
        pool_ids = np.stack([disp[s]["pool_ids"][r] for s in range(R)])
        pool_rows = np.stack([disp[s]["pool_rows"][r] for s in range(R)])
        rv = recv_slots(pool_ids, r, X, rcap)
        ret, _ = expert_returns(pool_rows, rv, inp["w13"][r * X:(r + 1) * X],
                                inp["w2"][r * X:(r + 1) * X], H, act)
        recvs.append(rv)
        rets.append(ret)
    outs = []
    for s in range(R):
        ret_from_dest = np.stack([rets[dd][s] for dd in range(R)])
        c = combine(ret_from_dest, disp[s]["slot_of"], disp[s]["w"], scap, act)
        hs = shared_hidden(inp["x"][s], inp["ws13"], HS, act)
        out, exact = layer_output(c, hs, inp["w_up"], inp["ws2"], act)
        outs.append(dict(c=c, hs=hs, out=out, out_exact=exact))
    ledger = drop_ledger(shape, disp, recvs)
    return dict(dispatch=disp, recv=recvs, ret=rets, out=outs, ledger=ledger,
                send_cap=scap, recv_cap=rcap)


def drop_ledger(shape, disp, recvs):
    """Send drops and receive drops, counted apart ([P1 §二]: reported separately)."""
    R, T, k = shape.n_ranks, shape.tokens, shape.top_k
    send_dropped = np.array([dd["send_dropped"] for dd in disp], dtype=np.int64)
    recv_dropped = np.array([rv["recv_dropped"].sum() for rv in recvs], dtype=np.int64)
    kept = int(sum(rv["count"].sum() for rv in recvs))
    return dict(send_dropped=send_dropped, recv_dropped=recv_dropped, kept=kept,
                total=R * T * k)


def routed_source_pools(shape, inp, with_rows=True):
    """Pools that every other rank sends to the measured rank, by routing that
    rank's own tokens through the same router.

    [P1 §二]: each rank routes its tokens and keeps one fixed pool per
    destination; the measured rank receives pool `receiver` of every source.
    inp["sources"](s) gives source s's tokens; the measured rank's own pool is
    left empty here (it comes from the rank's own dispatch).
    Returns ids [R][send_cap] int32, rows [R][send_cap][L] (float64, zeros
    where empty; None unless with_rows) and tok [R][send_cap] int32: the
    source token whose latent fills each slot (-1 for empty slots).
    """
    d = _dims(shape)
    R, X, L = d["R"], d["X"], d["L"]
    scap, _ = capacities(shape)
    r = inp["receiver"]
    ids = np.full((R, scap), -1, dtype=np.int32)
    tok = np.full((R, scap), -1, dtype=np.int32)
    rows = np.zeros((R, scap, L)) if with_rows else None
    for s in range(R):
        if s == r:
            continue
        xs = inp["sources"](s)
        logits = router_logits(xs, inp["w_router"], inp["bias"], inp["bias_row_tokens"])
        idx, _ = select_topk(logits, d["k"])
        sl = send_slots(idx, X, R, scap)
        pid, _ = pack_pools(idx, sl["slot_of"], R, scap)
        ids[s] = pid[r]
        flat = sl["slot_of"].reshape(-1)
        mine = (flat >= r * scap) & (flat < (r + 1) * scap)
        slots = flat[mine] - r * scap
        tokens = np.repeat(np.arange(xs.shape[0]), d["k"])[mine]
        tok[s, slots] = tokens
        if with_rows and slots.size:
            rows[s, slots] = down_project(xs[tokens], inp["w_down"], d["act"])
    return ids, rows, tok


def layer_one_rank(shape, inp, with_floats=True):
    """One rank's share: its own tokens, plus pools/returns of the other ranks as inputs.

    The receiver r = inp["receiver"] receives its own pool r (from its own
    dispatch) and the pools of every other source (inp["foreign_ids"] and,
    for the float path, inp["foreign_rows"]: drawn by the workload, or
    computed with routed_source_pools); its combine reads the rows it
    computed for itself and the rows every other destination returned
    (inp["foreign_ret"]).
    """
    d = _dims(shape)
    R, X, H, HS, act = d["R"], d["X"], d["H"], d["HS"], d["act"]
    scap, rcap = capacities(shape)
    r = inp["receiver"]
    disp = dispatch(shape, inp["x"], inp["w_router"], inp["w_down"], inp["bias"],
                    inp["bias_row_tokens"], with_rows=with_floats)
    pool_ids = inp["foreign_ids"].copy()
    pool_ids[r] = disp["pool_ids"][r]
    rv = recv_slots(pool_ids, r, X, rcap)
    res = dict(dispatch=disp, recv=rv, pool_ids=pool_ids, send_cap=scap, recv_cap=rcap)
    if not with_floats or shape.layer != "full":
        return res
    pool_rows = f64(inp["foreign_rows"])
    pool_rows[r] = disp["pool_rows"][r]
    ret, defined = expert_returns(pool_rows, rv, inp["w13"], inp["w2"], H, act)
    ret_from_dest = f64(inp["foreign_ret"])
    ret_from_dest[r] = ret[r]
    c = combine(ret_from_dest, disp["slot_of"], disp["w"], scap, act)
    hs = shared_hidden(inp["x"], inp["ws13"], HS, act)
    out, exact = layer_output(c, hs, inp["w_up"], inp["ws2"], act)
    res.update(ret=ret, ret_defined=defined, c=c, hs=hs, out=out, out_exact=exact)
    return res
