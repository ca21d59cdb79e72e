"""Device buffers and the call sequence of the MoE layer on one GPU.

torch provides device memory, copies and streams; every step of the layer is
a libmoe call (see binding.py).  Two layouts of the expert-parallel domain
are provided:

* ``OneRankLayer``: one rank's share at its real shape.  The rank's own
  tokens go through route -> pack; its receive buffer holds its own pool for
  itself plus the pools the other ranks sent; its combine reads the rows it
  computed for itself plus the rows the other ranks returned (inputs).  When
  the workload gives the other ranks' tokens, their pools are made at set-up
  by running those ranks' route -> pack through the same library calls
  (untimed: it stands for what the other GPUs do); otherwise they are
  inputs.  The only copies in a step are the self-blocks of the exchanges.
* ``AllRanksLayer``: every rank of a small domain on one device.  All send
  pools sit in one [R_src][R_dst][send_cap][stride] block and all return rows
  in one [R_recv][R_src][send_cap][L] block, so each exchange is a strided
  view: zero copies.
"""

import numpy as np
import torch

from . import binding as B


def upload(arr, device):
    """Host array (uint16 bf16 bit patterns, float32, int32 or raw bytes) -> device tensor."""
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    if a.dtype in (np.int32, np.uint8):
        return torch.from_numpy(a).to(device)
    raise TypeError(f"unsupported host dtype {a.dtype}")


def rank_blocks(R, shape, dtype, device):
    """An [R][*shape] tensor whose per-rank blocks each start 256-byte aligned
    (the library takes 16-byte aligned activation pointers; a plain [R][T][n]
    tensor puts rank r at r*T*n elements, unaligned for odd widths)."""
    n = int(np.prod(shape))
    es = torch.empty((), dtype=dtype).element_size()
    stride = -(-n * es // 256) * 256 // es
    return torch.empty((R, stride), dtype=dtype, device=device)[:, :n].unflatten(1, tuple(shape))


def upload_rank_blocks(arr, device):
    """upload() of a host [R][...] array into 256-byte aligned per-rank blocks."""
    t = upload(arr, device)
    out = rank_blocks(t.shape[0], t.shape[1:], t.dtype, device)
    out.copy_(t)
    return out


def _act(shape):
    return torch.bfloat16 if shape.act == "bf16" else torch.float32


def pool_block_host(ids, rows, prow, act):
    """Host bytes of pools in the row layout of moe_pack_pools: [n][cap][prow]."""
    n, cap = ids.shape
    L = rows.shape[-1]
    esize = 2 if act == "bf16" else 4
    out = np.zeros((n, cap, prow), dtype=np.uint8)
    payload = np.ascontiguousarray(rows).view(np.uint8).reshape(n, cap, L * esize)
    out[:, :, :L * esize] = payload
    out[:, :, L * esize:L * esize + 4] = np.ascontiguousarray(ids, dtype=np.int32).view(np.uint8).reshape(n, cap, 4)
    return out


class OneRankLayer:
    """One EP rank's layer.  ``inp`` is a workload.gen.generate() dict."""

    def __init__(self, shape, inp, device="cuda", gather="fused", keep_source_logits=False, live_waves=0):
        self.shape, self.device = shape, device
        self.gather = gather
        # waves whose scratch (hidden rows, partial tiles) the workspace holds at once
        self.live_waves = live_waves if live_waves else shape.waves
        # keep_source_logits: the router logits each other rank computed at
        # set-up, as host float32 arrays (source_logits[s]), for inspection
        self.source_logits = {} if keep_source_logits else None
        r = int(inp["receiver"])
        self.rank = r
        self.dims = B.make_dims(shape, my_rank=r, live_waves=self.live_waves)
        self.scap, self.rcap, self.prow = B.capacity(self.dims)
        T, D, L, E, k, R = shape.tokens, shape.d_model, shape.latent, shape.n_experts, shape.top_k, shape.n_ranks
        X, W, H = shape.local_experts, shape.waves, shape.expert_hidden
        WX = X // W
        act = _act(shape)
        dev = device
        self.full = shape.layer == "full"
        # inputs
        self.x = upload(inp["x"], dev)
        self.w_router = upload(inp["w_router"], dev)
        self.w_down = upload(inp["w_down"], dev)
        self.bias = None if inp["bias"] is None else upload(np.ascontiguousarray(inp["bias"], np.float32), dev)
        self.bias_row_tokens = int(inp["bias_row_tokens"])
        # route / pack outputs
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        self.z = torch.empty((T, L), dtype=act, device=dev)
        self.idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.send_pools = torch.empty((R, self.scap, self.prow), dtype=torch.uint8, device=dev)
        self.slot_of = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.send_count = torch.empty((R,), dtype=torch.int32, device=dev)
        # receive side: slot s holds the pool source s sent; slot r is our own pool
        if "sources" in inp:
            self.recv_pools = torch.zeros((R, self.scap, self.prow), dtype=torch.uint8, device=dev)
        else:
            self.recv_pools = upload(pool_block_host(inp["foreign_ids"], inp["foreign_rows"], self.prow, shape.act),
                                     dev)
        self.row_src = torch.empty((W, WX, self.rcap), dtype=torch.int32, device=dev)
        self.wave_count = torch.empty((W, WX), dtype=torch.int32, device=dev)
        self.wave_buf = torch.empty((WX, self.rcap, L), dtype=act, device=dev) if gather == "buffer" else None
        self.ws = torch.empty((B.workspace_size(self.dims),), dtype=torch.uint8, device=dev)
        if self.full:
            self.w13 = upload(inp["w13"], dev)
            self.w2 = upload(inp["w2"], dev)
            self.w_up = upload(inp["w_up"], dev)
            self.ws13 = upload(inp["ws13"], dev)
            self.ws2 = upload(inp["ws2"], dev)
            self.ret_send = torch.zeros((R, self.scap, L), dtype=act, device=dev)
            self.ret_recv = upload(inp["foreign_ret"], dev)
            self.out = torch.empty((T, D), dtype=act, device=dev)
            self._ev_go, self._ev_shared, self._ev_ranked = torch.cuda.Event(), torch.cuda.Event(), torch.cuda.Event()
        self.source_demand = {}
        if "sources" in inp:
            self._route_other_ranks(inp["sources"])

    def _route_other_ranks(self, sources):
        """Each other rank s routes its own tokens and packs its pools; keep the
        pool it sends to this rank (uses this layer's dispatch buffers, which
        the rank's own dispatch overwrites later)."""
        from concurrent.futures import ThreadPoolExecutor
        others = [s for s in range(self.shape.n_ranks) if s != self.rank]
        with ThreadPoolExecutor(max_workers=8) as ex:  # host draws overlap the GPU work
            drawn = ex.map(sources, others)
            for s, host_x in zip(others, drawn):
                self._route_one(s, host_x)
        torch.cuda.synchronize()

    def _route_one(self, s, host_x):
        xs = upload(host_x, self.device)
        d = self.dims
        B.route(d, xs, self.w_router, self.w_down, self.bias, self.bias_row_tokens, self.logits, self.z,
                self.idx, self.w, self.ws)
        B.pack_pools(d, self.z, self.idx, self.send_pools, self.scap * self.prow, self.slot_of, self.send_count,
                     self.ws)
        self.recv_pools[s].copy_(self.send_pools[self.rank])
        if self.source_logits is not None:
            self.source_logits[s] = self.logits.cpu().numpy()
        # rows source s wants to send here, before its send cap (the count a
        # dropless exchange would send ahead of the rows)
        self.source_demand[s] = B.drop_stats(d, self.ws, raise_on_bad_ids=False).send_demand[self.rank]

    @property
    def esize(self):
        return 2 if self.shape.act == "bf16" else 4

    def dispatch(self, stream=None):
        d = self.dims
        B.route(d, self.x, self.w_router, self.w_down, self.bias, self.bias_row_tokens, self.logits, self.z,
                self.idx, self.w, self.ws, stream)
        B.pack_pools(d, self.z, self.idx, self.send_pools, self.scap * self.prow, self.slot_of,
                     self.send_count, self.ws, stream)
        # self-block of the dispatch exchange
        self.recv_pools[self.rank].copy_(self.send_pools[self.rank])

    def receive_rank(self, stream=None):
        B.recv_rank(self.dims, self.recv_pools, self.scap * self.prow, self.ws, stream)

    def receive_wave(self, w, stream=None):
        B.recv_waves(self.dims, self.recv_pools, self.scap * self.prow, w, self.wave_buf, self.row_src[w],
                     self.wave_count[w], self.ws, stream)

    def expert_wave(self, w, stream=None):
        B.expert_gemm(self.dims, w, self.wave_buf, self.recv_pools, self.scap * self.prow, self.row_src[w],
                      self.wave_count[w], self.w13, self.w2, self.ret_send, self.scap * self.shape.latent * self.esize,
                      self.ws, stream)

    def shared(self, stream=None):
        B.shared_experts(self.dims, self.x, self.ws13, self.ws, stream)

    def combine(self, stream=None):
        # self-block of the return exchange
        self.ret_recv[self.rank].copy_(self.ret_send[self.rank])
        B.combine(self.dims, self.ret_recv, self.scap * self.shape.latent * self.esize, self.slot_of, self.w,
                  self.w_up, self.ws2, self.out, self.ws, stream)

    def run(self, stream=None, side=None):
        """One batch on `stream` (torch's current stream if None).  With `side`,
        a second stream, the shared experts and the waves of odd scratch
        blocks (wave w is in block w mod live_waves) run there, beside the
        routed path and the other waves: the shared experts start once
        everything queued before on `stream` (the previous batch's combine,
        which reads their output) is done, the side waves once the receive
        ranking is, and the combine waits for both.  A block's waves always
        share a stream, so they run in order; with one live wave every wave
        runs on `stream`."""
        main = stream if stream is not None else torch.cuda.current_stream()
        waves = self.shape.waves
        with torch.cuda.stream(main):
            if self.full:
                if side is not None:
                    self._ev_go.record(main)
                    side.wait_event(self._ev_go)
                    self.shared(side)
                else:
                    self.shared(main)
            self.dispatch(main)
            self.receive_rank(main)
            # a shared wave buffer ("buffer" gather) keeps the waves in order
            two = side is not None and self.full and self.wave_buf is None and self.live_waves > 1
            if two:
                self._ev_ranked.record(main)
                side.wait_event(self._ev_ranked)
            for w in range(waves):
                st = side if two and (w % self.live_waves) % 2 else main
                self.receive_wave(w, st)
                if self.full:
                    self.expert_wave(w, st)
            if self.full:
                if side is not None:
                    self._ev_shared.record(side)
                    main.wait_event(self._ev_shared)
                self.combine(main)

    def drop_report(self, stream=None):
        return B.drop_stats(self.dims, self.ws, stream, raise_on_bad_ids=False).as_dict()

    def memory(self):
        """Device bytes of one step's buffers.  The SwiGLU hidden rows of a wave
        ([X/W][recv_cap][H] activations) are the part of the receive bank that
        the waves keep small; the workspace holds live_waves such blocks."""
        sh = self.shape
        rows = getattr(self, "wave_rows", 0) or (sh.local_experts // sh.waves) * self.rcap
        hidden_wave = rows * sh.expert_hidden * self.esize if self.full else 0
        exch = self.send_pools.numel() + self.recv_pools.numel()
        ret = (self.ret_send.numel() + self.ret_recv.numel()) * self.esize if self.full else 0
        return {"live_waves": self.live_waves, "hidden_rows_per_wave_bytes": hidden_wave,
                "hidden_rows_live_bytes": hidden_wave * self.live_waves, "workspace_bytes": self.ws.numel(),
                "wave_buffer_bytes": 0 if self.wave_buf is None else self.wave_buf.numel() * self.esize,
                "exchange_pool_bytes": exch, "return_row_bytes": ret}


class RaggedOneRankLayer(OneRankLayer):
    """One EP rank's layer with the dropless ragged exchange (the counterpart of
    RaggedAllRanksLayer at one rank's real shape).  The rank packs its rows
    back to back by destination (moe_pack_ragged, no send cap).  At set-up the
    other ranks route and pack their own tokens the same way (untimed: it
    stands for the other GPUs) and their counts toward this rank fix where
    every source's segment sits in the receive buffer; the inputs are the same
    every step, so the counts are too, and a step copies only the self
    segments of the two exchanges.  ``foreign_ret`` rows (the rows the other
    ranks return, [R][pool_rows][L]) are laid into this rank's ragged order
    once.  ``expert_rows`` is the receive cap of every expert.  With
    ``ragged_banks`` each wave's hidden rows are laid end to end in one bank
    sized to the largest number of rows any wave keeps (moe_dims.wave_rows),
    from per-expert arrival counts taken at set-up (the counts a dropless
    exchange would send ahead of the rows, split by expert); otherwise every
    expert has a bank of expert_rows rows."""

    def __init__(self, shape, inp, expert_rows, device="cuda", gather="fused", ragged_banks=True, live_waves=2):
        from workload.configs import exact_fit
        if "sources" not in inp:
            raise ValueError("the ragged layer needs a workload whose other ranks route their own tokens")
        self.shape, self.device, self.gather = shape, device, gather
        self.live_waves = min(live_waves, shape.waves) if live_waves else shape.waves
        self.source_logits = None
        r = int(inp["receiver"])
        self.rank = r
        T, D, L, E, k, R = shape.tokens, shape.d_model, shape.latent, shape.n_experts, shape.top_k, shape.n_ranks
        X, W = shape.local_experts, shape.waves
        WX = X // W
        act = _act(shape)
        dev = device
        self.full = shape.layer == "full"
        self._fit = lambda pool_rows: exact_fit(shape, pool_rows, int(expert_rows))
        # set-up dims: neither cap is used by route and pack, and cap 1 keeps
        # the receive parts of the set-up workspace small
        setup_dims = B.make_dims(exact_fit(shape, 1, 1), my_rank=r)
        self.rcap = int(expert_rows)
        self.prow = B.capacity(setup_dims)[2]
        self.x = upload(inp["x"], dev)
        self.w_router = upload(inp["w_router"], dev)
        self.w_down = upload(inp["w_down"], dev)
        self.bias = None if inp["bias"] is None else upload(np.ascontiguousarray(inp["bias"], np.float32), dev)
        self.bias_row_tokens = int(inp["bias_row_tokens"])
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        self.z = torch.empty((T, L), dtype=act, device=dev)
        self.idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.send_rows = torch.empty((T * k, self.prow), dtype=torch.uint8, device=dev)
        self.send_off = torch.empty((R + 1,), dtype=torch.int32, device=dev)
        self.slot_of = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.send_count = torch.empty((R,), dtype=torch.int32, device=dev)
        ws_setup = torch.zeros((B.workspace_size(setup_dims),), dtype=torch.uint8, device=dev)
        # the other ranks' segments toward this rank, and this rank's own count
        segs = {}
        for s in range(R):
            host_x = inp["x"] if s == r else inp["sources"](s)
            xs = upload(host_x, dev)
            B.route(setup_dims, xs, self.w_router, self.w_down, self.bias, self.bias_row_tokens, self.logits,
                    self.z, self.idx, self.w, ws_setup)
            B.pack_ragged(setup_dims, self.z, self.idx, self.send_rows, self.send_off, self.slot_of,
                          self.send_count, ws_setup)
            off = self.send_off.cpu().numpy()
            segs[s] = self.send_rows[int(off[r]):int(off[r + 1])].clone()
            if s == r:
                self.own_off = off.astype(np.int64)
        cnt = np.array([segs[s].shape[0] for s in range(R)], dtype=np.int64)
        self.seg_off = np.concatenate([[0], np.cumsum(cnt)])
        self.n_recv = int(self.seg_off[-1])
        self.view_rows = max(-(-self.n_recv // R), 1)
        self.scap = self.view_rows
        self.recv_pools = torch.empty((R * self.view_rows, self.prow), dtype=torch.uint8, device=dev)
        self.recv_pools.view(torch.int32)[self.n_recv:, (L * self.esize) // 4] = -1
        for s in range(R):   # the own segment too: a step copies the same rows again
            if cnt[s]:
                self.recv_pools[self.seg_off[s]:self.seg_off[s + 1]].copy_(segs[s])
        del segs, ws_setup
        self.wave_rows = 0
        if ragged_banks:
            arr = receive_arrivals(shape, exact_fit(shape, self.view_rows, 1), r, self.recv_pools,
                                   self.view_rows * self.prow, dev)
            self.wave_rows = max(int(sum(arr[w * WX:(w + 1) * WX])) for w in range(W))
        self.recv_dims = B.make_dims(self._fit(self.view_rows), my_rank=r, wave_rows=self.wave_rows,
                                     live_waves=self.live_waves)
        assert B.capacity(self.recv_dims)[:2] == (self.view_rows, self.rcap)
        # one workspace and one set of dims for the whole step (moe_pack_ragged
        # ignores the send cap, moe_combine reads the ragged return rows with
        # any cap)
        self.dims = self.recv_dims
        self.ws = self.ws_recv = torch.zeros((B.workspace_size(self.recv_dims),), dtype=torch.uint8, device=dev)
        self.row_src = torch.empty((W, WX, self.rcap), dtype=torch.int32, device=dev)
        self.wave_count = torch.empty((W, WX), dtype=torch.int32, device=dev)
        self.wave_buf = torch.empty((WX, self.rcap, L), dtype=act, device=dev) if gather == "buffer" else None
        self.source_demand = {s: int(cnt[s]) for s in range(R) if s != r}
        if self.full:
            self.w13 = upload(inp["w13"], dev)
            self.w2 = upload(inp["w2"], dev)
            self.w_up = upload(inp["w_up"], dev)
            self.ws13 = upload(inp["ws13"], dev)
            self.ws2 = upload(inp["ws2"], dev)
            self.ret_send = torch.zeros((R * self.view_rows, L), dtype=act, device=dev)
            self.ret_back = torch.zeros((T * k, L), dtype=act, device=dev)
            fr = upload(inp["foreign_ret"], dev)                 # [R][pool_rows][L]
            own_cnt = np.diff(self.own_off)
            for d in range(R):
                c = int(own_cnt[d])
                if d != r and c:
                    assert c <= fr.shape[1], "foreign_ret has fewer rows than this rank sends"
                    self.ret_back[self.own_off[d]:self.own_off[d] + c].copy_(fr[d, :c])
            del fr
            self.out = torch.empty((T, D), dtype=act, device=dev)
            self._ev_go, self._ev_shared, self._ev_ranked = torch.cuda.Event(), torch.cuda.Event(), torch.cuda.Event()
        torch.cuda.synchronize()

    def dispatch(self, stream=None):
        d, r = self.dims, self.rank
        B.route(d, self.x, self.w_router, self.w_down, self.bias, self.bias_row_tokens, self.logits, self.z,
                self.idx, self.w, self.ws, stream)
        B.pack_ragged(d, self.z, self.idx, self.send_rows, self.send_off, self.slot_of, self.send_count, self.ws,
                      stream)
        # self segment of the dispatch exchange (its place fixed by the count exchange)
        c = int(self.own_off[r + 1] - self.own_off[r])
        if c:
            self.recv_pools[self.seg_off[r]:self.seg_off[r] + c].copy_(
                self.send_rows[self.own_off[r]:self.own_off[r] + c])

    def receive_rank(self, stream=None):
        B.recv_rank(self.recv_dims, self.recv_pools, self.view_rows * self.prow, self.ws_recv, stream)

    def receive_wave(self, w, stream=None):
        B.recv_waves(self.recv_dims, self.recv_pools, self.view_rows * self.prow, w, self.wave_buf, self.row_src[w],
                     self.wave_count[w], self.ws_recv, stream)

    def expert_wave(self, w, stream=None):
        B.expert_gemm(self.recv_dims, w, self.wave_buf, self.recv_pools, self.view_rows * self.prow,
                      self.row_src[w], self.wave_count[w], self.w13, self.w2, self.ret_send,
                      self.view_rows * self.shape.latent * self.esize, self.ws_recv, stream)

    def combine(self, stream=None):
        r = self.rank
        c = int(self.own_off[r + 1] - self.own_off[r])
        if c:   # self segment of the return exchange
            self.ret_back[self.own_off[r]:self.own_off[r] + c].copy_(self.ret_send[self.seg_off[r]:self.seg_off[r] + c])
        scap = B.capacity(self.dims)[0]
        B.combine(self.dims, self.ret_back, scap * self.shape.latent * self.esize, self.slot_of, self.w, self.w_up,
                  self.ws2, self.out, self.ws, stream)

    def footprint(self):
        """Bytes of the exchange buffers and the workspace."""
        n = self.send_rows.numel() + self.recv_pools.numel() + self.ws.numel()
        if self.full:
            n += (self.ret_send.numel() + self.ret_back.numel()) * self.esize
        return n


def receive_arrivals(shape, fit_shape, rank, recv_pools, src_stride_bytes, device):
    """Rows arriving at each local expert of ``rank`` from the pools in
    ``recv_pools`` (a set-up pass of moe_recv_rank with a small workspace:
    the ranking does not depend on the expert widths or the receive cap)."""
    from dataclasses import replace
    probe = replace(fit_shape, expert_hidden=64, shared_experts=0, shared_hidden=64)
    d = B.make_dims(probe, my_rank=rank, live_waves=1, wave_rows=1)
    ws = torch.zeros((B.workspace_size(d),), dtype=torch.uint8, device=device)
    B.recv_rank(d, recv_pools, src_stride_bytes, ws)
    rep = B.drop_stats(d, ws, raise_on_bad_ids=False)
    return list(rep.expert_arrivals[:shape.local_experts])


class AllRanksLayer:
    """Every rank of a small EP domain on one device (zero-copy exchanges)."""

    def __init__(self, shape, inp, device="cuda", gather="fused"):
        self.shape, self.device, self.gather = shape, device, gather
        T, D, L, E, k, R = shape.tokens, shape.d_model, shape.latent, shape.n_experts, shape.top_k, shape.n_ranks
        X, W = shape.local_experts, shape.waves
        WX = X // W
        act = _act(shape)
        dev = device
        self.dims = [B.make_dims(shape, my_rank=r) for r in range(R)]
        self.scap, self.rcap, self.prow = B.capacity(self.dims[0])
        self.x = upload_rank_blocks(inp["x"], dev)                      # [R][T][D]
        self.w_router = upload(inp["w_router"], dev)
        self.w_down = upload(inp["w_down"], dev)
        bias = inp["bias"]
        if bias is not None and bias.ndim == 2:
            bias = np.broadcast_to(bias, (R,) + bias.shape)
        self.bias = None if bias is None else upload_rank_blocks(np.ascontiguousarray(bias, np.float32), dev)
        self.bias_row_tokens = int(inp["bias_row_tokens"])
        self.w13 = upload(inp["w13"], dev)                              # [E][2H][L]
        self.w2 = upload(inp["w2"], dev)                                # [E][L][H]
        self.w_up = upload(inp["w_up"], dev)
        self.ws13 = upload(inp["ws13"], dev)
        self.ws2 = upload(inp["ws2"], dev)
        self.logits = rank_blocks(R, (T, E), torch.float32, dev)
        self.z = torch.empty((R, T, L), dtype=act, device=dev)
        self.idx = torch.empty((R, T, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((R, T, k), dtype=torch.float32, device=dev)
        self.pools = torch.empty((R, R, self.scap, self.prow), dtype=torch.uint8, device=dev)   # [src][dst]
        self.slot_of = torch.empty((R, T, k), dtype=torch.int32, device=dev)
        self.send_count = torch.empty((R, R), dtype=torch.int32, device=dev)
        self.row_src = torch.empty((R, W, WX, self.rcap), dtype=torch.int32, device=dev)
        self.wave_count = torch.empty((R, W, WX), dtype=torch.int32, device=dev)
        # "buffer" gather: one wave buffer per (rank, wave), all kept for inspection
        self.wave_buf = (torch.empty((R, W, WX, self.rcap, L), dtype=act, device=dev) if gather == "buffer"
                         else None)
        self.ret = torch.zeros((R, R, self.scap, L), dtype=act, device=dev)                     # [recv][src]
        self.out = rank_blocks(R, (T, D), act, dev)
        self.ws = [torch.empty((B.workspace_size(self.dims[0]),), dtype=torch.uint8, device=dev)
                   for _ in range(R)]

    def run(self, stream=None):
        sh = self.shape
        R, L = sh.n_ranks, sh.latent
        esize = 2 if sh.act == "bf16" else 4
        pool_bytes = self.scap * self.prow
        for s in range(R):
            d = self.dims[s]
            bias = None if self.bias is None else self.bias[s]
            B.route(d, self.x[s], self.w_router, self.w_down, bias, self.bias_row_tokens, self.logits[s],
                    self.z[s], self.idx[s], self.w[s], self.ws[s], stream)
            B.pack_pools(d, self.z[s], self.idx[s], self.pools[s], pool_bytes, self.slot_of[s],
                         self.send_count[s], self.ws[s], stream)
        X = sh.local_experts
        for r in range(R):
            d = self.dims[r]
            recv_view = self.pools[0, r]                 # pool from source s at + s * R * pool_bytes
            B.recv_rank(d, recv_view, R * pool_bytes, self.ws[r], stream)
            for w in range(sh.waves):
                wb = None if self.wave_buf is None else self.wave_buf[r, w]
                B.recv_waves(d, recv_view, R * pool_bytes, w, wb, self.row_src[r, w],
                             self.wave_count[r, w], self.ws[r], stream)
                B.expert_gemm(d, w, wb, recv_view, R * pool_bytes, self.row_src[r, w],
                              self.wave_count[r, w], self.w13[r * X:(r + 1) * X], self.w2[r * X:(r + 1) * X],
                              self.ret[r], self.scap * L * esize, self.ws[r], stream)
        for s in range(R):
            d = self.dims[s]
            ret_view = self.ret[0, s]                    # rows from receiver d at + d * R * scap * L
            B.shared_experts(d, self.x[s], self.ws13, self.ws[s], stream)
            B.combine(d, ret_view, R * self.scap * L * esize, self.slot_of[s], self.w[s], self.w_up, self.ws2,
                      self.out[s], self.ws[s], stream)

    def drop_reports(self, stream=None):
        return [B.drop_stats(self.dims[r], self.ws[r], stream, raise_on_bad_ids=False).as_dict()
                for r in range(self.shape.n_ranks)]


def _ceil_div(a, b):
    return -(-a // b)


class RaggedAllRanksLayer:
    """Every rank of a small EP domain on one device with the dropless ragged
    exchange: each rank packs its rows back to back by destination
    (moe_pack_ragged) and nothing is capped on the send side.  The row counts
    are exchanged first (a host read of send_count here); each receiver's
    buffer then holds the segments sent to it laid end to end, source by
    source, viewed by the receive calls as R pools of ceil(n/R) rows with id
    -1 past the n received rows; the return rows go back into each sender's
    ragged order.  The two exchanges are device copies standing for the
    ragged all-to-all.  ``expert_rows`` sizes every expert's bank (the
    receive cap).  ``wave_rows``: 0 keeps a bank of expert_rows hidden rows
    per expert; None lays each wave's hidden rows end to end in one bank sized
    to the rows that receiver's fullest wave keeps (per-expert arrival counts
    at set-up, see RaggedOneRankLayer); a number forces that bank size."""

    def __init__(self, shape, inp, expert_rows, device="cuda", gather="fused", wave_rows=None):
        from workload.configs import exact_fit
        self.wave_rows_arg = wave_rows
        self.shape, self.device, self.gather = shape, device, gather
        T, D, L, E, k, R = shape.tokens, shape.d_model, shape.latent, shape.n_experts, shape.top_k, shape.n_ranks
        X, W = shape.local_experts, shape.waves
        WX = X // W
        act = _act(shape)
        dev = device
        self.expert_rows = int(expert_rows)
        self._fit = lambda pool_rows: exact_fit(shape, pool_rows, self.expert_rows)
        # send side (route, pack, shared experts, combine): neither cap is used,
        # and cap 1 keeps the receive parts of its workspace small
        self.send_dims = [B.make_dims(exact_fit(shape, 1, 1), my_rank=r) for r in range(R)]
        self.rcap = self.expert_rows
        self.prow = B.capacity(self.send_dims[0])[2]
        self.x = upload_rank_blocks(inp["x"], dev)
        self.w_router = upload(inp["w_router"], dev)
        self.w_down = upload(inp["w_down"], dev)
        bias = inp["bias"]
        if bias is not None and bias.ndim == 2:
            bias = np.broadcast_to(bias, (R,) + bias.shape)
        self.bias = None if bias is None else upload_rank_blocks(np.ascontiguousarray(bias, np.float32), dev)
        self.bias_row_tokens = int(inp["bias_row_tokens"])
        self.w13 = upload(inp["w13"], dev)
        self.w2 = upload(inp["w2"], dev)
        self.w_up = upload(inp["w_up"], dev)
        self.ws13 = upload(inp["ws13"], dev)
        self.ws2 = upload(inp["ws2"], dev)
        self.logits = rank_blocks(R, (T, E), torch.float32, dev)
        self.z = torch.empty((R, T, L), dtype=act, device=dev)
        self.idx = torch.empty((R, T, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((R, T, k), dtype=torch.float32, device=dev)
        self.send_rows = torch.empty((R, T * k, self.prow), dtype=torch.uint8, device=dev)
        self.send_off = torch.empty((R, R + 1), dtype=torch.int32, device=dev)
        self.slot_of = torch.empty((R, T, k), dtype=torch.int32, device=dev)
        self.send_count = torch.empty((R, R), dtype=torch.int32, device=dev)
        self.ret_back = torch.zeros((R, T * k, L), dtype=act, device=dev)   # returned rows, sender's order
        self.row_src = torch.empty((R, W, WX, self.rcap), dtype=torch.int32, device=dev)
        self.wave_count = torch.empty((R, W, WX), dtype=torch.int32, device=dev)
        self.wave_buf = torch.empty((WX, self.rcap, L), dtype=act, device=dev) if gather == "buffer" else None
        self.out = rank_blocks(R, (T, D), act, dev)
        self.ws_send = [torch.zeros((B.workspace_size(d),), dtype=torch.uint8, device=dev) for d in self.send_dims]
        self.recv_dims, self.recv, self.ret, self.ws_recv, self.seg_off = [], [], [], [], []

    def run(self, stream=None):
        sh = self.shape
        R, L, X = sh.n_ranks, sh.latent, sh.local_experts
        esize = 2 if sh.act == "bf16" else 4
        for s in range(R):
            d = self.send_dims[s]
            bias = None if self.bias is None else self.bias[s]
            B.route(d, self.x[s], self.w_router, self.w_down, bias, self.bias_row_tokens, self.logits[s],
                    self.z[s], self.idx[s], self.w[s], self.ws_send[s], stream)
            B.pack_ragged(d, self.z[s], self.idx[s], self.send_rows[s], self.send_off[s], self.slot_of[s],
                          self.send_count[s], self.ws_send[s], stream)
        # the count exchange
        torch.cuda.synchronize()
        cnt = self.send_count.cpu().numpy().astype(np.int64)      # [src][dst]
        off = self.send_off.cpu().numpy().astype(np.int64)        # [src][R+1]
        self.recv_dims, self.recv, self.ret, self.ws_recv, self.seg_off = [], [], [], [], []
        id_col = (L * esize) // 4
        for r in range(R):
            n = int(cnt[:, r].sum())
            view_rows = max(_ceil_div(n, R), 1)
            seg = np.concatenate([[0], np.cumsum(cnt[:, r])])
            buf = torch.empty((R * view_rows, self.prow), dtype=torch.uint8, device=self.device)
            buf.view(torch.int32)[n:, id_col] = -1
            for s in range(R):                                  # the dispatch exchange
                c = int(cnt[s, r])
                if c:
                    buf[seg[s]:seg[s] + c].copy_(self.send_rows[s, off[s, r]:off[s, r] + c])
            wave_rows = self.wave_rows_arg
            if wave_rows is None:
                arr = receive_arrivals(sh, self._fit(view_rows), r, buf, view_rows * self.prow, self.device)
                WX = X // sh.waves
                wave_rows = max(int(sum(arr[w * WX:(w + 1) * WX])) for w in range(sh.waves))
            d = B.make_dims(self._fit(view_rows), my_rank=r, wave_rows=wave_rows)
            assert B.capacity(d)[:2] == (view_rows, self.rcap)
            ws = torch.zeros((B.workspace_size(d),), dtype=torch.uint8, device=self.device)
            ret = torch.zeros((R * view_rows, L), dtype=self.out.dtype, device=self.device)
            pool_bytes = view_rows * self.prow
            B.recv_rank(d, buf, pool_bytes, ws, stream)
            for w in range(sh.waves):
                B.recv_waves(d, buf, pool_bytes, w, self.wave_buf, self.row_src[r, w], self.wave_count[r, w], ws,
                             stream)
                B.expert_gemm(d, w, self.wave_buf, buf, pool_bytes, self.row_src[r, w], self.wave_count[r, w],
                              self.w13[r * X:(r + 1) * X], self.w2[r * X:(r + 1) * X], ret, view_rows * L * esize,
                              ws, stream)
            for s in range(R):                                  # the return exchange
                c = int(cnt[s, r])
                if c:
                    self.ret_back[s, off[s, r]:off[s, r] + c].copy_(ret[seg[s]:seg[s] + c])
            self.recv_dims.append(d)
            self.recv.append(buf)
            self.ret.append(ret)
            self.ws_recv.append(ws)
            self.seg_off.append(seg)
        for s in range(R):
            d = self.send_dims[s]
            B.shared_experts(d, self.x[s], self.ws13, self.ws_send[s], stream)
            scap = B.capacity(d)[0]
            B.combine(d, self.ret_back[s], scap * L * esize, self.slot_of[s], self.w[s], self.w_up, self.ws2,
                      self.out[s], self.ws_send[s], stream)

    def drop_reports(self, stream=None):
        """Send fields from each rank's dispatch, receive fields from its receive."""
        out = []
        for r in range(self.shape.n_ranks):
            snd = B.drop_stats(self.send_dims[r], self.ws_send[r], stream, raise_on_bad_ids=False).as_dict()
            rcv = B.drop_stats(self.recv_dims[r], self.ws_recv[r], stream, raise_on_bad_ids=False).as_dict()
            for key in ("recv_arrivals", "recv_kept", "recv_dropped", "recv_bad_ids", "expert_arrivals",
                        "expert_kept"):
                snd[key] = rcv[key]
            out.append(snd)
        return out
