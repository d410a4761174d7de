"""GPU-vs-oracle harness: runs the HIP path through the C ABI and the CPU oracle on the same seeded inputs.

The oracle gets its own copy of the host rows, drawn from the workload generator, never from the GPU path.
Requests are independent, so at full sizes the oracle follows a sample of requests through every step.
"""
from __future__ import annotations

import sys
from typing import List, Optional, Sequence

import numpy as np
import torch

import hierarchical_memory_amd as hm
import oracle
import workload


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def ring_tail(rows: np.ndarray, tail0: int, T: int) -> np.ndarray:
    """Device tail of one request laid out as the boundary defines it: a ring of T rows holding the tokens
    [tail0, tail0 + T), token x in row x mod T (rows of tokens past the pool stay zero)."""
    H, rb = rows.shape
    tail = np.zeros((T, rb), np.uint8)
    for x in range(max(0, tail0), min(H, tail0 + T)):
        tail[x % T] = rows[x]
    return tail


def order_sorted_by_stamp(order: np.ndarray, stamp: np.ndarray) -> bool:
    """The library's LRU order list must list slots by ascending (stamp, slot)."""
    o = order.astype(np.int64)
    if sorted(o.tolist()) != list(range(len(o))):
        return False
    keys = stamp[o].astype(np.int64) * (1 << 20) + o
    return bool((np.diff(keys) > 0).all())


class Pair:
    def __init__(self, w: workload.Workload, sample: Optional[Sequence[int]] = None, gather: Optional[bool] = None,
                 n_steps: Optional[int] = None, ids: Optional[np.ndarray] = None, tail0: Optional[np.ndarray] = None,
                 policy: int = 0):
        self.w = w
        self.R, self.k, self.B, self.H = w.num_requests, w.top_k, w.buffer_slots, w.host_rows
        self.T, self.rb = w.tail_tokens, w.row_bytes
        self.gather = w.fused_gather if gather is None else gather
        self.sample = list(range(self.R)) if sample is None else list(sample)
        self.n_steps = (w.steps if ids is None else ids.shape[1]) if n_steps is None else n_steps
        log(f"[pair] {w.name}: R={self.R} k={self.k} B={self.B} H={self.H} T={self.T} steps={self.n_steps} "
            f"sample={self.sample[:8]}{'...' if len(self.sample) > 8 else ''}")
        cfg = hm.config(self.R, self.k, self.B, 0.0, self.rb, self.H, self.T, policy)
        self.sw = hm.SwapIn(cfg)
        workload.fill_rows_ptr(self.sw.host_pool_address(), 0, self.R * self.H, w.row_elems, w.row_seed)
        self.tail0_dev = None
        self.tail0 = None
        if self.T:
            pool = self.sw.host_pool()
            self.tail0 = np.full(self.R, w.tail0, np.int32) if tail0 is None else np.asarray(tail0, np.int32)
            self.tail0_dev = torch.from_numpy(self.tail0).cuda()
            # device tail rows = the host rows [tail0, tail0 + T) of each request (zeros past the pool's end)
            tail = np.stack([ring_tail(pool[r], int(self.tail0[r]), self.T) for r in range(self.R)])
            self.sw.tail.copy_(torch.from_numpy(tail))
        # the oracle's own rows, from the generator
        n = len(self.sample)
        host_o = np.empty((n, self.H, self.rb), np.uint8)
        for j, r in enumerate(self.sample):
            workload.fill_rows(host_o[j].view(np.uint16).reshape(self.H, w.row_elems), r * self.H, self.H,
                               w.row_elems, w.row_seed)
        tail_o = None
        if self.T:
            tail_o = np.stack([ring_tail(host_o[j], int(self.tail0[r]), self.T) for j, r in enumerate(self.sample)])
            if not len(self.sample):
                tail_o = np.zeros((0, self.T, self.rb), np.uint8)
        self.o = oracle.Oracle(n, self.B, self.k, self.H, self.rb, T=self.T, host=host_o, tail=tail_o, policy=policy)
        self.ids = workload.streams(w, n_steps=self.n_steps) if ids is None else np.ascontiguousarray(ids, np.int32)
        self.sample_t = torch.tensor(self.sample, dtype=torch.long, device="cuda")
        self.outs = self.sw.outputs(self.gather)
        self.t = 0

    def step(self, check_state: bool = False) -> None:
        ids = self.ids[:, self.t]
        topk = torch.from_numpy(np.ascontiguousarray(ids)).cuda()
        out, miss, status, g = self.sw.resolve(topk, self.tail0_dev, self.gather, outputs=self.outs)
        o_out, o_miss, o_status, o_g = self.o.step(ids[self.sample], None if self.tail0 is None else
                                                   self.tail0[self.sample], gather=self.gather)
        s = self.sample_t
        got_out = out[s].cpu().numpy()
        assert (got_out == o_out).all(), self._where("out", got_out, o_out)
        assert (miss[s].cpu().numpy() == o_miss).all(), self._where("miss", miss[s].cpu().numpy(), o_miss)
        assert (status[s].cpu().numpy() == o_status).all(), self._where("status", status[s].cpu().numpy(), o_status)
        if self.gather:
            got_g = g[s].cpu().numpy()
            assert (got_g == o_g).all(), self._where("gather", got_g, o_g)
        self.last_oracle_gather = o_g
        self.t += 1
        if check_state:
            self.check_state()

    def _where(self, what, got, exp) -> str:
        bad = np.argwhere(got != exp)
        return f"{self.w.name} step {self.t}: {what} differs at {bad[:5].tolist()} (of {len(bad)})"

    def check_state(self) -> None:
        s = self.sample_t
        sw, o = self.sw, self.o
        for name, got, exp in (("slot_tok", sw.slot_tok[s], o.slot_tok), ("stamp", sw.stamp[s], o.stamp),
                               ("page", sw.page[s], o.page), ("step", sw.step[s], o.t)):
            g = got.cpu().numpy()
            assert (g == exp).all(), self._where(name, g, exp)
        hot = sw.hot[s].cpu().numpy()
        assert (hot == o.hot).all(), self._where("hot", hot, o.hot)
        order = sw.lru_order[s].cpu().numpy().view(np.uint16)
        for j in range(len(self.sample)):
            assert order_sorted_by_stamp(order[j], o.stamp[j]), f"{self.w.name} step {self.t}: LRU order"

    def run(self, check_every: int = 1) -> None:
        for t in range(self.n_steps):
            last = t == self.n_steps - 1
            self.step(check_state=last or (check_every and (t % check_every == 0)))
            if t and t % 128 == 0:
                log(f"[pair] {self.w.name}: step {t} ok")
        log(f"[pair] {self.w.name}: {self.n_steps} steps bit-exact on requests {self.sample[:8]}")

    def check_all_requests(self, rows_per_request: int = 64, seed: int = 0) -> None:
        """Properties that hold at any size, on every request (not only the sampled ones)."""
        sw = self.sw
        st = sw.slot_tok.cpu().numpy()
        stamp = sw.stamp.cpu().numpy()
        page = sw.page.cpu().numpy()
        step = sw.step.cpu().numpy()
        order = sw.lru_order.cpu().numpy().view(np.uint16)
        pool = sw.host_pool()
        rng = np.random.default_rng(seed)
        for r in range(self.R):
            occ = np.nonzero(st[r] >= 0)[0]
            assert len(np.unique(st[r][occ])) == len(occ)
            assert (page[r][st[r][occ]] == occ).all() and int((page[r] >= 0).sum()) == len(occ)
            assert (stamp[r][st[r] < 0] == -1).all() and (stamp[r][occ] >= 0).all() and (stamp[r][occ] < step[r]).all()
            assert order_sorted_by_stamp(order[r], stamp[r])
            pick = rng.choice(occ, size=min(rows_per_request, len(occ)), replace=False) if len(occ) else occ
            if len(pick):
                hot_rows = sw.hot[r][torch.from_numpy(pick).cuda()].cpu().numpy()
                assert (hot_rows == pool[r][st[r][pick]]).all(), f"request {r}: slot bytes differ from host rows"
        log(f"[pair] {self.w.name}: invariants hold on all {self.R} requests")

    def close(self) -> None:
        self.sw.close()
