"""Seeded synthetic inputs for the fixed-pool, three-wave MoE layer.

This module draws random numbers and lays them out; it computes nothing of
the layer itself (no routing, no capacities, no ranks, no products).  Both
the CPU oracle and the GPU path take their inputs from here, so neither has
to trust the other's input preparation.

Value recipe (the pages print no data; the shapes are those of the Marin
535B-A23B expert layer, "Marin 开始公开训练 535B 参数 MoE 模型", section 二):

* activations x ~ N(0, 1); every weight matrix ~ N(0, 1/fan_in);
* values are made exactly representable in the storage type by truncating
  the low mantissa bits (bf16 storage) -- a way of drawing bf16 numbers, not
  a rounding step of the layer;
* exact-grid mode (``grid=True``): x = a/4 with integer |a| <= 8 and router /
  down-projection weights = b * 2**-s with integer |b| <= 255, so that every
  partial sum of x . w is an integer multiple of 2**-(s+2) below 2**24 units
  in magnitude for d_model <= 8192: every float32 summation order then gives
  the exact value and routing cannot depend on the order of accumulation;
* router bias "zipf": b_e = c * (1 + pi(e))**-s for a seeded permutation pi,
  standardised to the requested population std;
* router bias "segments": each run of ``segment_tokens`` tokens adds
  ``segment_boost`` to the logits of ``segment_hot`` experts drawn per segment
  without replacement.

For one-rank workloads (configs 2-5) the measured rank needs the pools the
other ranks send it.  With ``shape.foreign == "routed"`` (configs 2-4) every
rank s has its own seeded tokens (``source_tokens``), the very draw that an
emulation of all ranks would use, and the consumers route them through the
same router themselves; this module only draws them.  With
``shape.foreign == "drawn"`` (config 5) the pools are drawn directly from a
model of the arrivals of segment-correlated routing (``foreign_pools``).  The
rows the other ranks return for the measured rank's own tokens are drawn in
both cases (``foreign_returns``).
"""

import numpy as np
from concurrent.futures import ThreadPoolExecutor

from .configs import Shape

# ---------------------------------------------------------------- storage


def f32_to_bf16_bits_trunc(a):
    """uint16 bf16 bit patterns of float32 values, low 16 bits dropped."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b):
    """float32 values of uint16 bf16 bit patterns (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_f32(a):
    """Storage array (uint16 bf16 bits or float32) -> float32 values."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a)
    return np.asarray(a, dtype=np.float32)


def _store(vals_f32, act):
    if act == "bf16":
        return f32_to_bf16_bits_trunc(vals_f32)
    return np.ascontiguousarray(vals_f32, dtype=np.float32)


# ---------------------------------------------------------------- drawing

_NAMES = ["x", "w_router", "w_down", "w13", "w2", "w_up", "ws13", "ws2",
          "bias", "foreign_pools", "foreign_rows", "foreign_returns", "receiver"]


class _Seeds:
    """One independent child seed per (tensor, part)."""

    def __init__(self, seed):
        root = np.random.SeedSequence([int(seed), 0x4D6F45])
        kids = root.spawn(len(_NAMES))
        self._kids = dict(zip(_NAMES, kids))

    def rng(self, name, part=0):
        ss = self._kids[name]
        return np.random.default_rng(np.random.SeedSequence(
            entropy=ss.entropy, spawn_key=ss.spawn_key + (int(part),)))


def _normal(rng, shape, std):
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def _normal_parts(seeds, name, n_parts, part_shape, std, act, threads=8):
    """Draw n_parts independent N(0, std^2) blocks in parallel, stacked."""
    out_dtype = np.uint16 if act == "bf16" else np.float32
    out = np.empty((n_parts,) + tuple(part_shape), dtype=out_dtype)

    def one(p):
        out[p] = _store(_normal(seeds.rng(name, p), part_shape, std), act)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, range(n_parts)))
    return out


def _grid_x(rng, shape):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(4.0)
    np.rint(a, out=a)
    np.clip(a, -8, 8, out=a)
    a *= np.float32(0.25)
    return a


def _grid_w(rng, shape, fan_in):
    # scale 2**-s chosen so that the integer numerators have rms about 50
    s = int(np.round(np.log2(50.0 * np.sqrt(fan_in))))
    b = np.clip(np.rint(rng.standard_normal(size=shape) * (2.0 ** s) / np.sqrt(fan_in)), -255, 255)
    return (b * 2.0 ** -s).astype(np.float32)


def grid_sum_bound_ok(shape):
    """Static bound of the exact-grid construction: max |a| * max |b| * D < 2**24."""
    return 8 * 255 * shape.d_model < 2 ** 24


# ---------------------------------------------------------------- biases


def _zipf_bias(rng, E, s, std):
    perm = rng.permutation(E)
    b = (1.0 + perm.astype(np.float64)) ** (-s)
    b = (b - b.mean()) / b.std() * std
    return b.astype(np.float32)


def _segment_bias(rng, T, E, seg_tokens, hot, boost):
    nseg = -(-T // seg_tokens)
    bias = np.zeros((nseg, E), dtype=np.float32)
    for g in range(nseg):
        bias[g, rng.choice(E, size=hot, replace=False)] = np.float32(boost)
    return bias


# ---------------------------------------------------------------- inputs


def source_tokens(shape: Shape, seed, s, grid=False):
    """Tokens [T][D] (storage type) of rank s: the same draw for every caller."""
    sd = _Seeds(seed)
    T, D = shape.tokens, shape.d_model
    if grid:
        return _store(_grid_x(sd.rng("x", s), (T, D)), shape.act)
    return _store(_normal(sd.rng("x", s), (T, D), 1.0), shape.act)



def generate(shape: Shape, seed=0, grid=False, send_cap=None, with_foreign=True):
    """All inputs of one workload as numpy arrays (float32 or uint16 bf16 bits).

    Keys (sizes use the symbols of configs.Shape, X = local experts):
      x          [R][T][D] if shape.emulate_all_ranks else [T][D]
      w_router   [E][D]      router weights
      w_down     [L][D]      latent down-projection
      w13        [E or X][2H][L]  expert gate rows 0..H-1, up rows H..2H-1
      w2         [E or X][L][H]   expert down rows
      w_up       [D][L]      up-projection
      ws13       [S][2HS][D] shared expert gate/up rows
      ws2        [S][D][HS]  shared expert down rows
      bias       None, [1][E] (zipf) or [nseg][E] (segments), float32
      bias_row_tokens  tokens per bias row (0 = one row for all tokens)
      receiver   measured rank (one-rank workloads)
      sources    (foreign == "routed") function s -> tokens [T][D] of rank s;
                 x is sources(receiver)
      foreign_ids, foreign_rows     (foreign == "drawn") pools the other ranks
                                    send to the receiver
      foreign_ret                   rows the other ranks return to the receiver
    For one-rank workloads ``send_cap`` (rows per pool) must be given when
    ``with_foreign`` is true; it is an input here, not derived.
    """
    sd = _Seeds(seed)
    R, T, D, L, E = shape.n_ranks, shape.tokens, shape.d_model, shape.latent, shape.n_experts
    H, S, HS, X = shape.expert_hidden, shape.shared_experts, shape.shared_hidden, shape.local_experts
    act = shape.act
    full = shape.layer == "full"
    out = {}

    # router and down projection
    if grid:
        out["w_router"] = _store(_grid_w(sd.rng("w_router"), (E, D), D), act)
        out["w_down"] = _store(_grid_w(sd.rng("w_down"), (L, D), D), act)
    else:
        out["w_router"] = _store(_normal(sd.rng("w_router"), (E, D), D ** -0.5), act)
        out["w_down"] = _normal_parts(sd, "w_down", 1, (L, D), D ** -0.5, act)[0]

    # bias
    out["bias"] = None
    out["bias_row_tokens"] = 0
    if shape.bias == "zipf":
        out["bias"] = _zipf_bias(sd.rng("bias"), E, shape.zipf_s, shape.zipf_std)[None, :]
    elif shape.bias == "segments":
        if shape.emulate_all_ranks:
            out["bias"] = np.stack([
                _segment_bias(sd.rng("bias", s), T, E, shape.segment_tokens,
                              shape.segment_hot, shape.segment_boost) for s in range(R)])
        else:
            out["bias"] = _segment_bias(sd.rng("bias"), T, E, shape.segment_tokens,
                                        shape.segment_hot, shape.segment_boost)
        out["bias_row_tokens"] = shape.segment_tokens

    # receiver (one-rank workloads)
    if shape.receiver == "hot_expert":
        b = out["bias"][0]
        hot = int(np.flatnonzero(b == b.max())[0])
        out["receiver"] = hot // X
    else:
        out["receiver"] = 0

    # tokens: rank s draws from stream ("x", s), so a one-rank workload's own
    # tokens are the receiver's tokens of the all-rank emulation
    if shape.emulate_all_ranks:
        if grid:
            if not grid_sum_bound_ok(shape):
                raise ValueError("exact-grid construction needs d_model * 8 * 255 < 2**24")
            out["x"] = _store(np.stack([_grid_x(sd.rng("x", s), (T, D)) for s in range(R)]), act)
        else:
            out["x"] = _normal_parts(sd, "x", R, (T, D), 1.0, act)
    else:
        if grid and not grid_sum_bound_ok(shape):
            raise ValueError("exact-grid construction needs d_model * 8 * 255 < 2**24")
        out["x"] = source_tokens(shape, seed, out["receiver"], grid)
        if shape.foreign == "routed":
            out["sources"] = lambda s, _sh=shape, _seed=seed, _g=grid: source_tokens(_sh, _seed, s, _g)

    if full or shape.emulate_all_ranks:
        n_exp = E if shape.emulate_all_ranks else X
        out["w13"] = _normal_parts(sd, "w13", n_exp, (2 * H, L), L ** -0.5, act)
        out["w2"] = _normal_parts(sd, "w2", n_exp, (L, H), H ** -0.5, act)
        out["w_up"] = _normal_parts(sd, "w_up", 1, (D, L), L ** -0.5, act)[0]
        out["ws13"] = _normal_parts(sd, "ws13", S, (2 * HS, D), D ** -0.5, act)
        out["ws2"] = _normal_parts(sd, "ws2", S, (D, HS), HS ** -0.5, act)

    if not shape.emulate_all_ranks and with_foreign:
        if send_cap is None:
            raise ValueError("send_cap is required for one-rank workloads")
        if shape.foreign == "drawn":
            fid, frows = foreign_pools(shape, sd, int(send_cap), out["receiver"], out["bias"])
            out["foreign_ids"], out["foreign_rows"] = fid, frows
        if full:
            out["foreign_ret"] = foreign_returns(shape, sd, int(send_cap), out["receiver"])
    return out


def foreign_pools(shape, sd, cap, receiver, bias):
    """Pools that ranks s != receiver send to the receiver.

    ids [R][cap] int32 (global expert ids of the receiver, -1 = empty slot),
    rows [R][cap][L] storage dtype.  Row s == receiver is left empty (-1): the
    measured rank's own pool comes from its own dispatch.  Model per source:
      * rank0 receiver, no segments: n ~ Binomial(T*k, 1/R) rows, ids uniform
        over the receiver's X experts;
      * hot_expert receiver: every pool full (n = cap), the hottest local
        expert with probability 0.85, the rest uniform;
      * segments: per segment of segment_tokens tokens, m of the receiver's
        experts are among the segment's hot experts (hypergeometric draw);
        each hot local expert gets Binomial(seg_tokens*k, 1/hot) rows, the
        other local experts Binomial(seg_tokens*k, 1/(4E)) rows each, in
        segment order; the sequence is cut at cap.
    """
    R, T, k, E, X, L = (shape.n_ranks, shape.tokens, shape.top_k, shape.n_experts,
                        shape.local_experts, shape.latent)
    ids = np.full((R, cap), -1, dtype=np.int32)
    base = receiver * X
    for s in range(R):
        if s == receiver:
            continue
        rng = sd.rng("foreign_pools", s)
        if shape.receiver == "hot_expert":
            b = bias[0, base:base + X]
            hot = int(np.argmax(b))
            others = [j for j in range(X) if j != hot]
            pick_hot = rng.random(cap) < 0.85
            seq = np.where(pick_hot, hot, rng.choice(others, size=cap)).astype(np.int32)
        elif shape.bias == "segments":
            parts = []
            nseg = -(-T // shape.segment_tokens)
            for g in range(nseg):
                ntok = min(shape.segment_tokens, T - g * shape.segment_tokens)
                m = rng.hypergeometric(X, E - X, shape.segment_hot)
                hot = rng.choice(X, size=m, replace=False) if m else np.zeros(0, int)
                seg = []
                for j in range(X):
                    p = 1.0 / shape.segment_hot if j in hot else 1.0 / (4 * E)
                    seg.append(np.full(rng.binomial(ntok * k, p), j, dtype=np.int32))
                seg = np.concatenate(seg)
                rng.shuffle(seg)
                parts.append(seg)
            seq = np.concatenate(parts)[:cap]
        else:
            n = min(int(rng.binomial(T * k, 1.0 / R)), cap)
            seq = rng.integers(0, X, size=n, dtype=np.int32)
        ids[s, :len(seq)] = seq + base
    rows = _normal_parts(sd, "foreign_rows", R, (cap, L), 1.0, shape.act)
    rows[receiver] = 0
    return ids, rows


def foreign_returns(shape, sd, cap, receiver):
    """Rows the other ranks return for the receiver's own tokens: [R][cap][L].

    Every slot holds a draw of N(0, 0.6^2) (about the spread of an expert
    output for N(0,1) latents); only slots the receiver actually filled are
    ever read.  Row d == receiver is zero: it is produced locally.
    """
    ret = _normal_parts(sd, "foreign_returns", shape.n_ranks, (cap, shape.latent), 0.6, shape.act)
    ret[receiver] = 0
    return ret
