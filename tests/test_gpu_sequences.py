"""GPU parity over random sequences of calls: every entry point of the C ABI interleaved on one context.

Each sequence mixes fused resolves (with and without the gather), plan + copy (with and without the gather),
the static-plan step, accepted and rejected trials, trials made stale by an offload before their commit,
offloads, tail advances, partial resets and unfused gathers, in a seeded random order, on a small shape with a
device tail. After every call its outputs and the whole device state (tables, stamps, step counters, hot rows,
tail rows, tail starts, the host pool) must equal the oracle's, bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hierarchical_memory_amd  # noqa: F401  (raises if the HIP library is missing)
    yield
    torch.cuda.synchronize()


import oracle  # noqa: E402
import workload  # noqa: E402
from tests.parity import Pair, log  # noqa: E402

OPS = ("resolve", "resolve_gather", "plan_copy", "plan_copy_gather", "trial_accept", "trial_reject", "offload",
       "advance_tail", "reset_some", "gather", "trial_offload_commit", "static_step")


def _ids(rng, R, k, H):
    """Mostly valid distinct ids, with some padding, out-of-range and repeated ones."""
    ids = np.stack([rng.choice(H, size=k, replace=False) for _ in range(R)]).astype(np.int32)
    weird = rng.random(ids.shape) < 0.05
    ids[weird] = rng.integers(-2, H + 2, size=int(weird.sum()))
    return ids


def _clone(o: oracle.Oracle) -> oracle.Oracle:
    c = oracle.Oracle(o.n, o.B, o.k, o.H, o.rb, T=o.T, host=o.host.copy(),
                      tail=None if o.tail is None else o.tail.copy(), policy=o.policy)
    for name in ("slot_tok", "stamp", "page", "t", "hot"):
        getattr(c, name)[...] = getattr(o, name)
    return c


def _expected_gather(o: oracle.Oracle, out: np.ndarray) -> np.ndarray:
    """The rows the resolved indices name, read from the oracle's state: hot slot, tail row, or zeros."""
    g = np.zeros(out.shape + (o.rb,), np.uint8)
    for r in range(out.shape[0]):
        for i, v in enumerate(out[r]):
            if 0 <= v < o.B:
                g[r, i] = o.hot[r, v]
            elif o.B <= v < o.B + o.T:
                g[r, i] = o.tail[r, v - o.B]
    return g


def _eq(got, exp, what, op, n):
    got = got.cpu().numpy() if hasattr(got, "cpu") else got
    assert (got == exp).all(), f"call {n} ({op}): {what} differs at {np.argwhere(got != exp)[:5].tolist()}"


@pytest.mark.parametrize("seed", range(24))
def test_random_call_sequences(seed):
    import hierarchical_memory_amd as hm
    rng = np.random.default_rng(500 + seed)
    R, k, H, T, rb = 5, 40, 700, 48, 64
    B = int(rng.integers(k, 3 * k))
    policy = seed % 2
    w = workload.SINGLE_4K.with_(name=f"sequence_{seed}", num_requests=R, top_k=k, buffer_slots=B, host_rows=H, L0=H,
                                 tail_tokens=T, row_elems=rb // 2, steps=1, fused_gather=True)
    tail0 = rng.integers(H // 2, H - T - 150, size=R).astype(np.int32)
    p = Pair(w, ids=np.zeros((R, 1, k), np.int32), tail0=tail0, gather=True, policy=policy)
    sw, o, ctx = p.sw, p.o, p.sw.ctx
    out, miss, status, g = sw.outputs(gather=True)
    g2 = torch.empty_like(g)
    plan, trial = sw.plan_buffer(), sw.trial_buffer()
    st = torch.zeros(R, dtype=torch.int32, device="cuda")
    pool = sw.host_pool()
    resolved = False
    for n in range(60):
        op = OPS[int(rng.integers(len(OPS)))]
        if op == "gather" and not resolved:
            op = "resolve"
        ids = _ids(rng, R, k, H)
        topk = torch.from_numpy(ids).cuda()
        if op == "trial_offload_commit":
            # a trial, an offload in between, then the commit: stale for every request (the offload changed each
            # one), so the state is the offload's alone
            hm.hs_trial(ctx, topk, p.tail0_dev, out, miss, status, g, trial)
            o_out, o_miss, o_st, o_g = _clone(o).step(ids, p.tail0, gather=True)
            _eq(out, o_out, "trial out", op, n)
            _eq(g, o_g, "trial rows", op, n)
            m_rows = int(rng.integers(1, 6))
            pos = rng.integers(0, H - m_rows, size=R).astype(np.int32)
            rows = rng.integers(0, 256, size=(R, m_rows, rb), dtype=np.uint8)
            hm.hs_offload(ctx, torch.from_numpy(rows).cuda(), torch.from_numpy(pos).cuda())
            o.offload(rows, pos)
            st.zero_()
            hm.hs_commit(ctx, trial, g, None, st)
            _eq(st, np.full(R, hm.HS_STATUS_STALE, np.int32), "commit status", op, n)
            resolved = True
        elif op in ("resolve", "resolve_gather", "plan_copy", "plan_copy_gather", "trial_accept", "trial_reject",
                    "static_step"):
            gather = op in ("resolve_gather", "plan_copy_gather", "trial_accept", "trial_reject")
            if op == "static_step":
                gather = bool(rng.integers(0, 2))
                hm.hs_step_static(ctx, topk, p.tail0_dev, out, miss, status, g if gather else None)
            elif op in ("resolve", "resolve_gather"):
                hm.hs_resolve(ctx, topk, p.tail0_dev, out, miss, status, g if gather else None)
            elif op in ("plan_copy", "plan_copy_gather"):
                hm.hs_plan(ctx, topk, p.tail0_dev, out, miss, status, plan, row_sources=gather)
                hm.hs_copy(ctx, plan, miss, g if gather else None)
            else:
                hm.hs_trial(ctx, topk, p.tail0_dev, out, miss, status, g, trial)
                accept = torch.full((R,), 1 if op == "trial_accept" else 0, dtype=torch.int32, device="cuda")
                st.zero_()
                hm.hs_commit(ctx, trial, g, accept, st)
                _eq(st, np.zeros(R, np.int32), "commit status", op, n)
            ref = _clone(o) if op == "trial_reject" else o
            o_out, o_miss, o_st, o_g = ref.step(ids, p.tail0, gather=gather)
            _eq(out, o_out, "out", op, n)
            _eq(miss, o_miss, "miss", op, n)
            _eq(status, o_st, "status", op, n)
            if gather:
                _eq(g, o_g, "gathered rows", op, n)
            resolved = True
        elif op == "offload":
            m = int(rng.integers(1, 12))
            pos = rng.integers(-2, H - m + 3, size=R).astype(np.int32)  # some runs cross either end of the pool
            rows = rng.integers(0, 256, size=(R, m, rb), dtype=np.uint8)
            st.zero_()
            hm.hs_offload(ctx, torch.from_numpy(rows).cuda(), torch.from_numpy(pos).cuda(), st)
            _eq(st, o.offload(rows, pos), "offload status", op, n)
        elif op == "advance_tail":
            old = p.tail0.copy()
            step = np.minimum(rng.integers(0, T + 1, size=R), H - T - old).astype(np.int32)
            hm.hs_advance_tail(ctx, p.tail0_dev, torch.from_numpy(step).cuda(), st)
            _eq(st, o.advance_tail(p.tail0, step), "advance status", op, n)
            _eq(p.tail0_dev, p.tail0, "tail0", op, n)
            # the tokens entering the window: the caller writes their rows into the ring, on both sides
            for r in range(R):
                for x in range(int(old[r]) + T, int(p.tail0[r]) + T):
                    o.tail[r, x % T] = o.host[r, x]
                    sw.tail[r, x % T] = torch.from_numpy(pool[r, x].copy()).cuda()
        elif op == "reset_some":
            reqs = rng.choice(R, size=int(rng.integers(1, R + 1)), replace=False).astype(np.int32)
            sw.reset(torch.from_numpy(reqs).cuda())
            o.reset(reqs.tolist())
        else:  # gather of the last resolve's outputs, from the current rows
            hm.hs_gather(ctx, out, g2)
            _eq(g2, _expected_gather(o, out.cpu().numpy()), "unfused gather", op, n)
        torch.cuda.synchronize()
        p.check_state()
        _eq(sw.tail, o.tail, "tail rows", op, n)
        assert (pool == o.host).all(), f"call {n} ({op}): host pool differs"
    log(f"[sequence {seed}] B={B} policy={policy}: 60 calls bit-exact")
    p.close()
