"""GPU parity: the HIP path through the C ABI against the CPU oracle, bit for bit.

Every output (slots, miss counts, status), every table (slot table, stamps, page table, step counters), the
hot buffer's bytes and the gathered rows must equal the oracle's. Nothing here has a floating-point
tolerance: rows are copied, not computed.
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


import workload  # noqa: E402
from tests.parity import Pair, log  # noqa: E402


def _random_ids(rng, R, steps, k, H, extra_low=-3, extra_high=3, p_weird=0.1):
    """Random selections, mostly valid distinct ids, sometimes padding, out-of-range or repeated ids."""
    ids = np.empty((R, steps, k), np.int32)
    for r in range(R):
        for t in range(steps):
            row = rng.choice(H, size=k, replace=k > H).astype(np.int32) if H >= 1 else np.zeros(k, np.int32)
            weird = rng.random(k) < p_weird
            row[weird] = rng.integers(extra_low, H + extra_high, size=int(weird.sum()))
            ids[r, t] = row
    return ids


TINY = [  # (k, B, H, T, row_bytes)
    (1, 1, 3, 0, 16), (2, 3, 6, 0, 16), (3, 4, 6, 0, 48), (3, 3, 5, 2, 16), (7, 9, 30, 0, 32),
    (12, 20, 40, 6, 16), (33, 40, 100, 0, 1152), (64, 64, 200, 0, 64), (65, 130, 257, 17, 80),
    (2, 4, 6, 1, 1 << 20),  # the largest row: 1 MiB
]


@pytest.mark.parametrize("k,B,H,T,rb", TINY, ids=[f"k{k}_B{B}_H{H}_T{T}_rb{rb}" for k, B, H, T, rb in TINY])
def test_tiny_random(k, B, H, T, rb):
    rng = np.random.default_rng(k * 1000 + B)
    R, steps = 16, 12
    w = workload.SINGLE_4K.with_(name=f"tiny_k{k}_B{B}", num_requests=R, top_k=k, buffer_slots=B, host_rows=H,
                                 L0=H, tail_tokens=T, row_elems=rb // 2, steps=steps, fused_gather=True)
    ids = _random_ids(rng, R, steps, k, H)
    tail0 = rng.integers(0, H + 1, size=R).astype(np.int32) if T else None
    p = Pair(w, ids=ids, tail0=tail0, gather=True)
    p.run(check_every=1)
    p.close()


def _random_shape(seed):
    rng = np.random.default_rng(10_000 + seed)
    k = int(rng.integers(1, 700))
    B = int(rng.integers(k, 3 * k + 2))
    H = int(rng.integers(max(B // 2, 2), 4 * B + 8))
    T = int(rng.integers(1, 64)) if rng.random() < 0.4 else 0
    rb = int(rng.choice([16, 48, 80, 1152, 16 * int(rng.integers(1, 160))]))
    R = int(rng.integers(1, 24))
    policy = int(rng.integers(0, 2))
    gather = bool(rng.random() < 0.5)
    return rng, R, k, B, H, T, rb, policy, gather


@pytest.mark.parametrize("seed", range(64))
def test_random_shapes(seed):
    """Seeded random shapes (k, B, context, tail, row size, policy, fused gather), with padding, bad and repeated
    ids, k and B off the 16-byte vector path; every step and the final state against the oracle."""
    rng, R, k, B, H, T, rb, policy, gather = _random_shape(seed)
    steps = 6
    log(f"[random shape {seed}] R={R} k={k} B={B} H={H} T={T} rb={rb} policy={policy} gather={gather}")
    w = workload.SINGLE_4K.with_(name=f"random_{seed}", num_requests=R, top_k=k, buffer_slots=B, host_rows=H, L0=H,
                                 tail_tokens=T, row_elems=rb // 2, steps=steps, fused_gather=gather)
    ids = _random_ids(rng, R, steps, k, H, p_weird=0.05)
    tail0 = rng.integers(0, H + 1, size=R).astype(np.int32) if T else None
    p = Pair(w, ids=ids, tail0=tail0, gather=gather, policy=policy)
    p.run(check_every=2)
    p.close()


@pytest.mark.parametrize("seed", range(32))
def test_random_shapes_rank_layout(seed):
    """Small random k and B with a long context (H >= 82,000: no room for a token -> slot table), so every
    launch takes the rank layout; ids drawn from a window of about 3B tokens so that slots are hit, with
    padding, bad and repeated ids, a device tail on some seeds, FIFO on others, with and without the gather."""
    import hierarchical_memory_amd as hm
    rng = np.random.default_rng(20_000 + seed)
    k = int(rng.integers(1, 300))
    B = int(rng.integers(k, 3 * k + 2))
    H = int(rng.integers(82_000, 120_000))
    T = int(rng.integers(1, 64)) if seed % 3 == 0 else 0
    rb = int(rng.choice([16, 48, 1152]))
    R = int(rng.integers(1, 12))
    policy, gather, steps = seed % 2, bool(seed % 4 < 2), 6
    sizes = hm.hs_required_sizes(hm.config(R, k, B, 0.0, rb, H, T, policy))
    assert sizes.token_slot_table == 0
    lo = int(rng.integers(0, H - 3 * B - 8))
    ids = np.empty((R, steps, k), np.int32)
    for r in range(R):
        for t in range(steps):
            row = (lo + rng.choice(3 * B, size=k, replace=False)).astype(np.int32)
            weird = rng.random(k) < 0.05
            row[weird] = rng.integers(-3, H + 3, size=int(weird.sum()))
            ids[r, t] = row
    log(f"[rank shape {seed}] R={R} k={k} B={B} H={H} T={T} rb={rb} policy={policy} gather={gather}")
    w = workload.SINGLE_4K.with_(name=f"rank_{seed}", num_requests=R, top_k=k, buffer_slots=B, host_rows=H, L0=H,
                                 tail_tokens=T, row_elems=rb // 2, steps=steps, fused_gather=gather)
    tail0 = (lo + rng.integers(0, 3 * B, size=R)).astype(np.int32) if T else None
    p = Pair(w, ids=ids, tail0=tail0, gather=gather, policy=policy)
    p.run(check_every=1)
    p.close()


def test_context_of_262144_tokens():
    """A 262,144-token context at k = 2048, B = 4096 (the rank layout, about 150 KiB of LDS): fused resolve with a
    gather, then plan + copy, step by step against the oracle, with a repeated id on odd steps."""
    import hierarchical_memory_amd as hm
    H = 262144
    w = workload.SINGLE_4K.with_(name="context_262144", num_requests=3, top_k=2048, buffer_slots=4096, host_rows=H,
                                 L0=H, window=12000, row_elems=32, steps=8, fused_gather=True)
    sizes = hm.hs_required_sizes(hm.config(3, 2048, 4096, 0.0, 64, H))
    assert sizes.token_slot_table == 0 and sizes.lds_bytes <= 159 * 1024
    ids = workload.streams(w)
    ids[:, 1::2, 9] = ids[:, 1::2, 4]
    p = Pair(w, ids=ids, gather=True)
    p.run(check_every=1)
    p.close()
    p = Pair(w, ids=ids)
    plan = p.sw.plan_buffer()
    out, miss, status, _ = p.outs
    for t in range(w.steps):
        step_ids = p.ids[:, t]
        hm.hs_plan(p.sw.ctx, torch.from_numpy(np.ascontiguousarray(step_ids)).cuda(), None, out, miss, status, plan)
        hm.hs_copy(p.sw.ctx, plan, miss)
        o_out, o_miss, o_status, _ = p.o.step(step_ids[p.sample])
        assert (out.cpu().numpy() == o_out).all() and (miss.cpu().numpy() == o_miss).all()
        assert (status.cpu().numpy() == o_status).all()
        p.t += 1
        p.check_state()
    p.close()


@pytest.mark.parametrize("seed", range(20))
def test_random_shapes_sparse_layout(seed):
    """Contexts of 600,000 to 1,200,000 tokens with small k and B: past the flat bitmaps' LDS, so every launch
    takes the two-level rank layout. Most ids come from a window of about 3B tokens (slots are hit), the rest
    from the whole context (many 32-token words, most holding one id); padding, bad and repeated ids, a device
    tail on some seeds, FIFO on others, with and without the gather."""
    import hierarchical_memory_amd as hm
    rng = np.random.default_rng(30_000 + seed)
    k = int(rng.integers(1, 300))
    B = int(rng.integers(k, 3 * k + 2))
    H = int(rng.integers(600_000, 1_200_000))
    T = int(rng.integers(1, 64)) if seed % 3 == 0 else 0
    rb = int(rng.choice([16, 32]))
    R = int(rng.integers(1, 5))
    policy, gather, steps = seed % 2, bool(seed % 4 < 2), 6
    sizes = hm.hs_required_sizes(hm.config(R, k, B, 0.0, rb, H, T, policy))
    assert sizes.token_slot_table == 0 and sizes.sparse_rank == 1
    lo = int(rng.integers(0, H - 3 * B - 8))
    ids = np.empty((R, steps, k), np.int32)
    for r in range(R):
        for t in range(steps):
            near = (lo + rng.choice(3 * B, size=k, replace=False)).astype(np.int32)
            far = rng.integers(0, H, size=k).astype(np.int32)
            row = np.where(rng.random(k) < 0.7, near, far)
            weird = rng.random(k) < 0.05
            row[weird] = rng.integers(-3, H + 3, size=int(weird.sum()))
            ids[r, t] = row
    log(f"[sparse shape {seed}] R={R} k={k} B={B} H={H} T={T} rb={rb} policy={policy} gather={gather}")
    w = workload.SINGLE_4K.with_(name=f"sparse_{seed}", num_requests=R, top_k=k, buffer_slots=B, host_rows=H, L0=H,
                                 tail_tokens=T, row_elems=rb // 2, steps=steps, fused_gather=gather)
    tail0 = (lo + rng.integers(0, 3 * B, size=R)).astype(np.int32) if T else None
    p = Pair(w, ids=ids, tail0=tail0, gather=gather, policy=policy)
    p.run(check_every=1)
    p.close()


@pytest.mark.parametrize("tail", [0, 8192])
def test_context_of_one_million_tokens(tail):
    """A 1,048,576-token context at k = 2048, B = 4096 (the two-level rank layout), with and without a device
    tail of 8192 tokens at its end: fused resolve with a gather, then plan + copy, step by step against the
    oracle, with a repeated id on odd steps."""
    import hierarchical_memory_amd as hm
    H = 1 << 20
    w = workload.SINGLE_4K.with_(name=f"context_1M_T{tail}", num_requests=2, top_k=2048, buffer_slots=4096,
                                 host_rows=H, L0=H, window=12000, row_elems=32, steps=8, fused_gather=True,
                                 tail_tokens=tail)
    sizes = hm.hs_required_sizes(hm.config(2, 2048, 4096, 0.0, 64, H, tail))
    assert sizes.token_slot_table == 0 and sizes.sparse_rank == 1 and sizes.lds_bytes <= 159 * 1024
    ids = workload.streams(w)
    ids[:, 1::2, 9] = ids[:, 1::2, 4]
    tail0 = np.full(2, H - tail, np.int32) if tail else None
    log(f"[1M context] tail {tail}: fused with gather")
    p = Pair(w, ids=ids, tail0=tail0, gather=True)
    p.run(check_every=1)
    p.close()
    log(f"[1M context] tail {tail}: plan + copy")
    p = Pair(w, ids=ids, tail0=tail0)
    plan = p.sw.plan_buffer()
    out, miss, status, _ = p.outs
    for t in range(w.steps):
        step_ids = p.ids[:, t]
        hm.hs_plan(p.sw.ctx, torch.from_numpy(np.ascontiguousarray(step_ids)).cuda(), p.tail0_dev, out, miss,
                   status, plan)
        hm.hs_copy(p.sw.ctx, plan, miss)
        o_out, o_miss, o_status, _ = p.o.step(step_ids[p.sample], None if tail0 is None else tail0[p.sample])
        assert (out.cpu().numpy() == o_out).all() and (miss.cpu().numpy() == o_miss).all()
        assert (status.cpu().numpy() == o_status).all()
        p.t += 1
        p.check_state()
    p.close()
    log(f"[1M context] tail {tail}: trial + commit")
    p = Pair(w, ids=ids, tail0=tail0, gather=True)
    trial = p.sw.trial_buffer()
    out, miss, status, g = p.outs
    for t in range(4):
        step_ids = p.ids[:, t]
        hm.hs_trial(p.sw.ctx, torch.from_numpy(np.ascontiguousarray(step_ids)).cuda(), p.tail0_dev, out, miss,
                    status, g, trial)
        o_out, o_miss, o_status, o_g = p.o.step(step_ids[p.sample], None if tail0 is None else tail0[p.sample],
                                                gather=True)
        assert (out.cpu().numpy() == o_out).all() and (miss.cpu().numpy() == o_miss).all()
        assert (g.cpu().numpy() == o_g).all()
        hm.hs_commit(p.sw.ctx, trial, g)
        p.t += 1
        p.check_state()
    p.close()


def test_direct_layout_eight_slots_per_thread():
    """B = 8192 with a short context: the direct layout with 8 ids and 8 slots per thread, every thread holding
    two 4-slot chunks; fused resolve with a gather, then plan + copy, step by step against the oracle."""
    import hierarchical_memory_amd as hm
    H = 12000
    w = workload.SINGLE_4K.with_(name="B8192", num_requests=2, top_k=2048, buffer_slots=8192, host_rows=H, L0=H,
                                 window=6000, row_elems=32, steps=10, fused_gather=True)
    sizes = hm.hs_required_sizes(hm.config(2, 2048, 8192, 0.0, 64, H))
    assert sizes.token_slot_table == 3
    ids = workload.streams(w)
    ids[:, 1::3, 7] = ids[:, 1::3, 3]  # a repeated id now and then
    p = Pair(w, ids=ids, gather=True)
    p.run(check_every=1)
    p.close()
    p = Pair(w, ids=ids)
    plan = p.sw.plan_buffer()
    out, miss, status, _ = p.outs
    for t in range(w.steps):
        step_ids = p.ids[:, t]
        hm.hs_plan(p.sw.ctx, torch.from_numpy(np.ascontiguousarray(step_ids)).cuda(), None, out, miss, status, plan)
        hm.hs_copy(p.sw.ctx, plan, miss)
        o_out, o_miss, o_status, _ = p.o.step(step_ids[p.sample])
        assert (out.cpu().numpy() == o_out).all() and (miss.cpu().numpy() == o_miss).all()
        assert (status.cpu().numpy() == o_status).all()
        p.t += 1
        p.check_state()
    p.close()


@pytest.mark.parametrize("H", [8192, 120_000], ids=["direct", "rank"])
@pytest.mark.parametrize("path", ["fused", "plan_copy", "plan_copy_gather", "trial_commit", "static"])
def test_degenerate_steps_every_path(path, H):
    """Degenerate steps through every path of a step, against the oracle: a step of padding only, a step that
    hits every id (no miss: empty plan lists, nothing to copy), a step of ids past the context (every one bad),
    between ordinary steps; k 512, B 1024, with the token -> slot table (8192 rows) and without (120,000)."""
    import hierarchical_memory_amd as hm
    R, k, B = 3, 512, 1024
    w = workload.SINGLE_4K.with_(name=f"degenerate_{path}_{H}", num_requests=R, top_k=k, buffer_slots=B,
                                 host_rows=H, L0=H, window=2000, row_elems=32, steps=8, fused_gather=True)
    sizes = hm.hs_required_sizes(hm.config(R, k, B, 0.0, 64, H))
    assert sizes.token_slot_table == (3 if H == 8192 else 0)
    ids = workload.streams(w)
    ids[:, 2] = -1                      # padding only
    ids[:, 3] = ids[:, 1]               # every id resident: no miss
    ids[:, 4] = H + np.arange(k)        # every id past the context
    ids[0, 5, :] = -1                   # one request padded, the others ordinary
    gather = path in ("fused", "plan_copy_gather", "trial_commit", "static")
    p = Pair(w, ids=ids, gather=gather)
    out, miss, status, g = p.outs
    plan = p.sw.plan_buffer() if path.startswith("plan") else None
    trial = p.sw.trial_buffer() if path == "trial_commit" else None
    for t in range(w.steps):
        step_ids = np.ascontiguousarray(p.ids[:, t])
        topk = torch.from_numpy(step_ids).cuda()
        log(f"[degenerate {path} H={H}] step {t}")
        if path == "fused":
            hm.hs_resolve(p.sw.ctx, topk, None, out, miss, status, g)
        elif path == "plan_copy":
            hm.hs_plan(p.sw.ctx, topk, None, out, miss, status, plan)
            hm.hs_copy(p.sw.ctx, plan, miss)
        elif path == "plan_copy_gather":
            hm.hs_plan(p.sw.ctx, topk, None, out, miss, status, plan, row_sources=True)
            hm.hs_copy(p.sw.ctx, plan, miss, g)
        elif path == "trial_commit":
            hm.hs_trial(p.sw.ctx, topk, None, out, miss, status, g, trial)
            hm.hs_commit(p.sw.ctx, trial, g)
        else:
            hm.hs_step_static(p.sw.ctx, topk, None, out, miss, status, g)
        o_out, o_miss, o_status, o_g = p.o.step(step_ids[p.sample], gather=gather)
        assert (out.cpu().numpy() == o_out).all(), f"step {t}: slots"
        assert (miss.cpu().numpy() == o_miss).all() and (status.cpu().numpy() == o_status).all(), f"step {t}"
        if gather:
            assert (g.cpu().numpy() == o_g).all(), f"step {t}: gathered rows"
        if t in (2, 3, 4):
            assert (o_miss == 0).all()
        if t == 4:
            assert (o_status == hm.HS_STATUS_BAD_ID).all()
        p.t += 1
        p.check_state()
    p.close()


@pytest.mark.parametrize("policy", [0, 1], ids=["lru", "fifo"])
@pytest.mark.parametrize("path", ["fused", "fused_gather", "plan_copy", "trial_commit", "static"])
def test_rank_layout_four_slots_per_thread(path, policy):
    """The rank layout at B = 4096 (four slots per thread: stamps and slot-table entries written back as whole
    16-byte rows) through every path of a step, LRU and FIFO, against the oracle: k 2048, a 150,000-token
    context (no room for a token -> slot table) with a 2048-token device tail; repeated ids, padding and bad
    ids on some steps, and a step that hits every id."""
    import hierarchical_memory_amd as hm
    R, k, B, H, T = 2, 2048, 4096, 150_000, 2048
    w = workload.SINGLE_4K.with_(name=f"rank_rows_{path}_{policy}", num_requests=R, top_k=k, buffer_slots=B,
                                 host_rows=H, L0=H, window=6000, partB_permille=200, row_elems=32, steps=8,
                                 fused_gather=True, tail_tokens=T)
    sizes = hm.hs_required_sizes(hm.config(R, k, B, 0.0, 64, H, T, policy))
    assert sizes.token_slot_table == 0 and sizes.sparse_rank == 0
    ids = workload.streams(w)
    ids[:, 2, 7] = ids[:, 2, 3]          # a repeated id
    ids[:, 3, :100] = -1                 # padding
    ids[:, 3, 100:105] = H + 5           # bad ids
    ids[:, 5] = ids[:, 4]                # every id hit
    gather = path != "fused" and path != "plan_copy"
    p = Pair(w, ids=ids, gather=gather, policy=policy)
    out, miss, status, g = p.outs
    plan = p.sw.plan_buffer() if path == "plan_copy" else None
    trial = p.sw.trial_buffer() if path == "trial_commit" else None
    for t in range(w.steps):
        step_ids = np.ascontiguousarray(p.ids[:, t])
        topk = torch.from_numpy(step_ids).cuda()
        log(f"[rank rows {path} policy={policy}] step {t}")
        if path == "fused":
            hm.hs_resolve(p.sw.ctx, topk, p.tail0_dev, out, miss, status)
        elif path == "fused_gather":
            hm.hs_resolve(p.sw.ctx, topk, p.tail0_dev, out, miss, status, g)
        elif path == "plan_copy":
            hm.hs_plan(p.sw.ctx, topk, p.tail0_dev, out, miss, status, plan)
            hm.hs_copy(p.sw.ctx, plan, miss)
        elif path == "trial_commit":
            hm.hs_trial(p.sw.ctx, topk, p.tail0_dev, out, miss, status, g, trial)
            hm.hs_commit(p.sw.ctx, trial, g)
        else:
            hm.hs_step_static(p.sw.ctx, topk, p.tail0_dev, out, miss, status, g)
        o_out, o_miss, o_status, o_g = p.o.step(step_ids[p.sample], p.tail0[p.sample], gather=gather)
        assert (out.cpu().numpy() == o_out).all(), f"step {t}: slots"
        assert (miss.cpu().numpy() == o_miss).all() and (status.cpu().numpy() == o_status).all(), f"step {t}"
        if gather:
            assert (g.cpu().numpy() == o_g).all(), f"step {t}: gathered rows"
        if t == 5:
            assert (o_miss == 0).all()
        p.t += 1
        p.check_state()
    p.close()


def test_single_request_full():
    p = Pair(workload.SINGLE_4K, gather=True)
    p.run(check_every=1)
    p.close()


def test_grow_32_requests_full():
    p = Pair(workload.GROW_32)
    p.run(check_every=16)
    p.check_all_requests()
    p.close()


@pytest.mark.parametrize("w", workload.sweep_workloads(), ids=lambda w: w.name)
def test_buffer_sweep(w):
    p = Pair(w, sample=[0, 21, 42, 63])
    p.run(check_every=64)
    p.check_all_requests(rows_per_request=16)
    p.close()


def test_concurrency_256_requests_full():
    p = Pair(workload.CONC_256, sample=[0, 85, 170, 255])
    p.run(check_every=64)
    p.check_all_requests(rows_per_request=16)
    p.close()


def test_hybrid_tail_fused_gather_full():
    p = Pair(workload.HYBRID_64, sample=[0, 31, 63])
    p.run(check_every=32)
    p.check_all_requests(rows_per_request=16)
    p.close()


def test_unfused_gather_matches_fused():
    import hierarchical_memory_amd as hm
    w = workload.HYBRID_64.with_(num_requests=8, steps=6)
    p = Pair(w, sample=[0, 7], gather=True)
    for _ in range(w.steps):
        p.step()
        out, _, _, g = p.outs
        g2 = torch.empty_like(g)
        hm.hs_gather(p.sw.ctx, out, g2)
        assert torch.equal(g, g2)
    p.close()


GATHER_CASES = [  # (k, B, H, T, row_bytes); a workgroup of the gather covers max(1, 768 // (row_bytes / 16)) rows
    (33, 40, 100, 0, 1152),  # 10 rows per workgroup: the last of 4 workgroups holds 3
    (65, 130, 257, 17, 80),  # 153 rows per workgroup: one partial workgroup; tail rows
    (5, 8, 20, 3, 16384),  # 1024 chunks per row: one row per workgroup in two passes, the second ragged
    (2, 4, 6, 1, 1 << 20),  # the largest row: 65536 chunks, one row per workgroup in 86 passes
    (2048, 4096, 8192, 0, 1152),
]


@pytest.mark.parametrize("k,B,H,T,rb", GATHER_CASES, ids=[f"k{k}_B{B}_T{T}_rb{rb}" for k, B, H, T, rb in GATHER_CASES])
def test_unfused_gather_against_oracle(k, B, H, T, rb):
    """hs_gather after each step equals the oracle's gathered rows (padding, bad and repeated ids included)."""
    import hierarchical_memory_amd as hm
    rng = np.random.default_rng(k + rb)
    R, steps = 4, 5
    w = workload.SINGLE_4K.with_(name=f"gather_k{k}_rb{rb}", num_requests=R, top_k=k, buffer_slots=B, host_rows=H,
                                 L0=H, tail_tokens=T, row_elems=rb // 2, steps=steps, fused_gather=True)
    ids = _random_ids(rng, R, steps, k, H)
    tail0 = rng.integers(0, H + 1, size=R).astype(np.int32) if T else None
    p = Pair(w, ids=ids, tail0=tail0, gather=True)
    g2 = torch.full((R, k, rb), 0xAB, dtype=torch.uint8, device="cuda")
    for _ in range(steps):
        p.step()
        out = p.outs[0]
        hm.hs_gather(p.sw.ctx, out, g2)
        got = g2.cpu().numpy()
        assert (got == p.last_oracle_gather).all(), p._where("unfused gather", got, p.last_oracle_gather)
    p.close()


def test_maximum_request_count():
    """65535 requests (the largest count, and the largest grid dimension the kernels use for it): fused resolve
    with the gather, plan + copy with the gather, unfused gather and offload, every request against the oracle."""
    import hierarchical_memory_amd as hm
    rng = np.random.default_rng(65535)
    R, k, B, H, rb, steps = 65535, 4, 8, 24, 16, 4
    w = workload.SINGLE_4K.with_(name="max_requests", num_requests=R, top_k=k, buffer_slots=B, host_rows=H, L0=H,
                                 row_elems=rb // 2, steps=steps, fused_gather=True)
    ids = np.stack([np.stack([rng.choice(H, size=k, replace=False) for _ in range(steps)]) for _ in range(R)])
    p = Pair(w, ids=ids.astype(np.int32), gather=True)
    p.step(check_state=True)
    out, miss, status, g = p.outs
    plan = p.sw.plan_buffer()
    topk = torch.from_numpy(np.ascontiguousarray(p.ids[:, 1])).cuda()
    hm.hs_plan(p.sw.ctx, topk, None, out, miss, status, plan, row_sources=True)
    hm.hs_copy(p.sw.ctx, plan, miss, g)
    o_out, o_miss, _, o_g = p.o.step(p.ids[:, 1], gather=True)
    assert (out.cpu().numpy() == o_out).all() and (miss.cpu().numpy() == o_miss).all()
    assert (g.cpu().numpy() == o_g).all()
    p.t += 1
    p.check_state()
    g2 = torch.empty_like(g)
    hm.hs_gather(p.sw.ctx, out, g2)
    assert torch.equal(g2, g)
    rows = rng.integers(0, 256, size=(R, 2, rb), dtype=np.uint8)
    pos = rng.integers(0, H - 1, size=R).astype(np.int32)
    st = torch.zeros(R, dtype=torch.int32, device="cuda")
    hm.hs_offload(p.sw.ctx, torch.from_numpy(rows).cuda(), torch.from_numpy(pos).cuda(), st)
    assert (st.cpu().numpy() == p.o.offload(rows, pos)).all()
    torch.cuda.synchronize()
    assert (p.sw.host_pool() == p.o.host).all()
    # a step through plan + copy without a gather (workgroups bound to requests)
    topk = torch.from_numpy(np.ascontiguousarray(p.ids[:, 2])).cuda()
    hm.hs_plan(p.sw.ctx, topk, None, out, miss, status, plan)
    hm.hs_copy(p.sw.ctx, plan, miss)
    o_out, o_miss, _, _ = p.o.step(p.ids[:, 2])
    assert (out.cpu().numpy() == o_out).all() and (miss.cpu().numpy() == o_miss).all()
    p.t += 1
    p.check_state()
    for _ in range(3, steps):
        p.step(check_state=True)
    p.close()


@pytest.mark.parametrize("R", [1, 2, 33, 127, 128, 129, 300])
def test_plan_then_copy_request_counts(R):
    """hs_plan + hs_copy without a gather on either side of the copy's two grids (with fewer requests than its
    128 workgroups every workgroup takes an equal share of the step's missed rows; with more, workgroups are
    bound to requests): one request padded and one hitting every id at one step, so some requests have no
    miss; every request's outputs, tables and rows against the oracle."""
    import hierarchical_memory_amd as hm
    rng = np.random.default_rng(4000 + R)
    k, B, H, rb, steps = 24, 48, 160, 48, 4
    w = workload.SINGLE_4K.with_(name=f"copy_R{R}", num_requests=R, top_k=k, buffer_slots=B, host_rows=H, L0=H,
                                 row_elems=rb // 2, steps=steps, fused_gather=False)
    ids = np.stack([np.stack([rng.choice(H, size=k, replace=False) for _ in range(steps)]) for _ in range(R)])
    ids = ids.astype(np.int32)
    ids[0, 2] = -1                      # request 0: padding only at step 2
    if R > 1:
        ids[R - 1, 2] = ids[R - 1, 1]   # the last request: every id hit at step 2
    p = Pair(w, ids=ids, gather=False)  # every request against the oracle
    out, miss, status, _ = p.outs
    plan = p.sw.plan_buffer()
    for t in range(steps):
        step_ids = np.ascontiguousarray(p.ids[:, t])
        hm.hs_plan(p.sw.ctx, torch.from_numpy(step_ids).cuda(), None, out, miss, status, plan)
        hm.hs_copy(p.sw.ctx, plan, miss)
        o_out, o_miss, o_status, _ = p.o.step(step_ids)
        assert (out.cpu().numpy() == o_out).all() and (miss.cpu().numpy() == o_miss).all()
        assert (status.cpu().numpy() == o_status).all()
        if t == 2:
            assert o_miss[0] == 0 and o_miss[R - 1] == 0
        p.t += 1
        p.check_state()
    p.close()


def test_buffer_equals_topk_and_whole_context():
    """B = k (every free slot shares the previous step's stamp) and B >= context (compulsory misses only)."""
    for B in (256, 4096):
        p = Pair(workload.SINGLE_4K.with_(buffer_slots=B))
        p.run(check_every=8)
        p.close()


def test_run_twice_identical():
    outs = []
    for _ in range(2):
        p = Pair(workload.GROW_32.with_(num_requests=8, steps=24), sample=[3])
        res = []
        for _ in range(p.n_steps):
            p.step()
            res.append(p.outs[0].cpu().numpy().copy())
        res.append(p.sw.stamp.cpu().numpy())
        res.append(p.sw.hot.cpu().numpy())
        outs.append(res)
        p.close()
    for a, b in zip(*outs):
        assert (a == b).all()


def test_partial_reset_mid_run():
    import hierarchical_memory_amd as hm
    w = workload.GROW_32.with_(num_requests=6, steps=20)
    p = Pair(w)
    for t in range(w.steps):
        if t == 9:
            ids = torch.tensor([1, 4, 99, -1], dtype=torch.int32, device="cuda")  # 99 and -1 are skipped
            hm.hs_reset(p.sw.ctx, ids)
            p.o.reset([1, 4])
            p.check_state()
        p.step(check_state=True)
    p.close()


def test_padding_bad_and_repeated_ids():
    w = workload.SINGLE_4K.with_(num_requests=4, top_k=16, buffer_slots=20, host_rows=50, L0=50, steps=6)
    ids = np.array([[[3, 3, -1, 60, -5, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17]] * 6] * 4, np.int32)
    ids[1] = -1
    ids[2, :, 0] = 49
    p = Pair(w, ids=ids)
    p.run(check_every=1)
    st = p.outs[2].cpu().numpy()
    assert st.tolist() == [3, 0, 1, 3]
    p.close()


@pytest.mark.parametrize("path", ["fused", "plan_copy", "trial_commit"])
def test_corrupt_state_is_reported_not_used(path):
    """A request whose slot table holds an impossible token is refused by every path of a step (status
    HS_STATUS_BAD_STATE, no miss, outputs -1, its state untouched: no row copied, no record committed) while
    the other requests step as the oracle does."""
    import hierarchical_memory_amd as hm
    w = workload.SINGLE_4K.with_(num_requests=3, steps=4)
    p = Pair(w, sample=[0, 2], gather=path == "trial_commit")
    p.step()
    # corrupt request 1's slot table from the host: the kernel must refuse it and leave its state alone
    p.sw.slot_tok[1, 5] = w.host_rows + 7
    before = [t.clone() for t in (p.sw.slot_tok, p.sw.stamp, p.sw.page, p.sw.step, p.sw.hot, p.sw.lru_order)]
    out, miss, status, g = p.outs
    if path == "fused":
        p.step()
    else:
        step_ids = np.ascontiguousarray(p.ids[:, p.t])
        topk = torch.from_numpy(step_ids).cuda()
        if path == "plan_copy":
            plan = p.sw.plan_buffer()
            hm.hs_plan(p.sw.ctx, topk, None, out, miss, status, plan)
            hm.hs_copy(p.sw.ctx, plan, miss)
        else:
            trial = p.sw.trial_buffer()
            cstat = torch.zeros(3, dtype=torch.int32, device="cuda")
            hm.hs_trial(p.sw.ctx, topk, None, out, miss, status, g, trial)
            hm.hs_commit(p.sw.ctx, trial, g, None, cstat)
            assert cstat[1].item() == hm.HS_STATUS_STALE and cstat[0].item() == 0 and cstat[2].item() == 0
        o_out, o_miss, o_status, _ = p.o.step(step_ids[p.sample])
        assert (out.cpu().numpy()[p.sample] == o_out).all() and (miss.cpu().numpy()[p.sample] == o_miss).all()
        assert (status.cpu().numpy()[p.sample] == o_status).all()
        p.t += 1
    assert status[1].item() == hm.HS_STATUS_BAD_STATE and miss[1].item() == 0 and (out[1] == -1).all()
    for b, a in zip(before, (p.sw.slot_tok, p.sw.stamp, p.sw.page, p.sw.step, p.sw.hot, p.sw.lru_order)):
        assert torch.equal(b[1], a[1])
    p.check_state()
    p.close()


def test_graph_replay_equals_eager():
    """The resolve never waits on the host and keeps its step counter on the device, so a captured graph
    replays it; every replay must equal an eager run on the same inputs."""
    w = workload.GROW_32.with_(num_requests=4, steps=10)
    eager = Pair(w, sample=[])
    graph = Pair(w, sample=[0, 1, 2, 3])
    topk = torch.empty((w.num_requests, w.top_k), dtype=torch.int32, device="cuda")
    g_out = graph.sw.outputs(False)
    # warm up on a side stream, then capture one resolve
    topk.copy_(torch.from_numpy(np.ascontiguousarray(graph.ids[:, 0])))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    cg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cg, stream=s):
        graph.sw.resolve(topk, None, False, outputs=g_out)
    torch.cuda.synchronize()
    for t in range(w.steps):
        topk.copy_(torch.from_numpy(np.ascontiguousarray(graph.ids[:, t])))
        cg.replay()
        torch.cuda.synchronize()
        eager.step()
        e_out = eager.outs[0]
        assert torch.equal(g_out[0], e_out) and torch.equal(g_out[1], eager.outs[1])
        # and the oracle agrees with the replay
        o_out, o_miss, _, _ = graph.o.step(graph.ids[:, t])
        assert (g_out[0].cpu().numpy() == o_out).all()
        graph.t += 1
    graph.check_state()
    for name in ("slot_tok", "stamp", "page", "step", "hot"):
        assert torch.equal(getattr(graph.sw, name), getattr(eager.sw, name)), name
    eager.close()
    graph.close()


def test_two_contexts_of_different_shapes():
    """A context keeps working after another one of a smaller shape (less LDS) is created on the device."""
    big = Pair(workload.GROW_32.with_(num_requests=4, steps=6))
    small = Pair(workload.SINGLE_4K.with_(steps=6, top_k=16, buffer_slots=32, host_rows=64, L0=64, window=64))
    for _ in range(6):
        big.step()
        small.step()
    big.check_state()
    small.check_state()
    big.close()
    small.close()


def test_bind_rejects_host_memory():
    """Binding checks that every buffer is device memory of the context's device."""
    import hierarchical_memory_amd as hm
    cfg = hm.config(2, 8, 16, 0.0, 64, 32)
    ctx = hm.hs_create(cfg)
    try:
        dev = dict(hot=torch.zeros((2, 16, 64), dtype=torch.uint8, device="cuda"), tail=None,
                   slot_tok=torch.empty((2, 16), dtype=torch.int32, device="cuda"),
                   stamp=torch.empty((2, 16), dtype=torch.int32, device="cuda"),
                   lru_order=torch.empty((2, 16), dtype=torch.int16, device="cuda"),
                   page=torch.empty((2, 32), dtype=torch.int32, device="cuda"),
                   step=torch.empty((2,), dtype=torch.int32, device="cuda"),
                   epoch=torch.empty((2,), dtype=torch.int32, device="cuda"))
        for host in (torch.empty((2, 32), dtype=torch.int32),
                     torch.empty((2, 32), dtype=torch.int32, pin_memory=True)):
            with pytest.raises(hm.HiSparseError) as err:
                hm.hs_bind_device(ctx, **dict(dev, page=host))
            assert err.value.code == hm.HS_E_INVALID and "page" in str(err.value)
        hm.hs_bind_device(ctx, **dev)  # all device memory: accepted
    finally:
        hm.hs_destroy(ctx)


def test_largest_shape_that_fits_lds():
    """Near the LDS limit of one workgroup: a wide buffer and a long context."""
    import hierarchical_memory_amd as hm
    cfg = hm.config(2, 2048, 8192, 0.0, 1152, 120000)
    s = hm.hs_required_sizes(cfg)
    assert s.lds_bytes > 128 * 1024
    w = workload.SINGLE_4K.with_(name="wide", num_requests=2, top_k=2048, buffer_slots=8192, host_rows=120000,
                                 L0=120000, window=20000, steps=10)
    p = Pair(w)
    p.run(check_every=3)
    p.close()


def test_shared_missed_token_array_near_the_lds_limit():
    """At k = 2048, B = 8192, H = 180000 a separate missed-token array would pass 159 KiB of LDS, so the missed
    tokens share the rank-to-slot table and the kernel keeps its settling pass: steps without and with repeated
    ids, fused and through plan + copy."""
    import hierarchical_memory_amd as hm
    s = hm.hs_required_sizes(hm.config(2, 2048, 8192, 0.0, 1152, 180000))
    assert s.token_slot_table == 0 and s.lds_bytes_rank + 4 * 2048 > 159 * 1024
    w = workload.SINGLE_4K.with_(name="wide_shared", num_requests=2, top_k=2048, buffer_slots=8192,
                                 host_rows=180000, L0=180000, window=20000, steps=8)
    ids = workload.streams(w)
    ids[:, 1::2, 7] = ids[:, 1::2, 3]  # odd steps repeat an id
    p = Pair(w, ids=ids)
    p.run(check_every=1)
    p.close()
    p = Pair(w, ids=ids)
    plan = p.sw.plan_buffer()
    out, miss, status, _ = p.outs
    for t in range(w.steps):
        step_ids = p.ids[:, t]
        hm.hs_plan(p.sw.ctx, torch.from_numpy(np.ascontiguousarray(step_ids)).cuda(), None, out, miss, status, plan)
        hm.hs_copy(p.sw.ctx, plan, miss)
        o_out, o_miss, o_status, _ = p.o.step(step_ids[p.sample])
        s = p.sample_t
        assert (out[s].cpu().numpy() == o_out).all() and (miss[s].cpu().numpy() == o_miss).all()
        assert (status[s].cpu().numpy() == o_status).all()
        p.t += 1
        p.check_state()
    p.close()


@pytest.mark.parametrize("base", [workload.CONC_256, workload.GROW_32], ids=["256req_shape", "32req_shape"])
def test_direct_layout_with_repeated_ids(base):
    """At the 256- and 32-request shapes every launch takes the direct layout (a token -> slot entry per host
    row): each selected id is tested against the slot table from its own side. A request whose selection repeats
    an id ranks its ids in the table's region instead, so the lowest position keeps the id. Requests 1 and 3
    repeat an id on odd steps; fused without and with a gather, and plan + copy, step by step against the
    oracle."""
    import hierarchical_memory_amd as hm
    bits = 3
    w = base.with_(name=base.name + "_4req", num_requests=4, steps=8)
    sizes = hm.hs_required_sizes(hm.config(w.num_requests, w.top_k, w.buffer_slots, 0.0, w.row_bytes, w.host_rows))
    assert sizes.token_slot_table == bits
    ids = workload.streams(w)
    ids[1, 1::2, 7] = ids[1, 1::2, 3]
    ids[3, 1::2, 100] = ids[3, 1::2, 2000]
    for gather in (False, True):
        p = Pair(w, ids=ids, gather=gather)
        p.run(check_every=1)
        assert (p.outs[2].cpu().numpy()[[1, 3]] != 0).any(), "the repeated ids were not reported"
        p.close()
    p = Pair(w, ids=ids)
    plan = p.sw.plan_buffer()
    out, miss, status, _ = p.outs
    for t in range(w.steps):
        step_ids = p.ids[:, t]
        hm.hs_plan(p.sw.ctx, torch.from_numpy(np.ascontiguousarray(step_ids)).cuda(), None, out, miss, status, plan)
        hm.hs_copy(p.sw.ctx, plan, miss)
        o_out, o_miss, o_status, _ = p.o.step(step_ids[p.sample])
        s = p.sample_t
        assert (out[s].cpu().numpy() == o_out).all() and (miss[s].cpu().numpy() == o_miss).all()
        assert (status[s].cpu().numpy() == o_status).all()
        p.t += 1
        p.check_state()
    p.close()


def _check_plan(plan_r, out_r, ids_r, m):
    """The plan lists the step's missed ids in ascending order with the slots they were given."""
    toks = plan_r[0][:m]
    assert (np.diff(toks) > 0).all() if m > 1 else True
    pos = {int(x): i for i, x in enumerate(ids_r)}
    assert [int(out_r[pos[int(x)]]) for x in toks] == plan_r[1][:m].tolist()


def test_plan_then_copy_matches_oracle():
    import hierarchical_memory_amd as hm
    w = workload.GROW_32.with_(num_requests=8, steps=40)
    p = Pair(w, sample=[0, 5, 7])
    plan = p.sw.plan_buffer()
    out, miss, status, _ = p.outs
    for t in range(w.steps):
        ids = p.ids[:, t]
        topk = torch.from_numpy(np.ascontiguousarray(ids)).cuda()
        hm.hs_plan(p.sw.ctx, topk, None, out, miss, status, plan)
        hm.hs_copy(p.sw.ctx, plan, miss)
        o_out, o_miss, o_status, _ = p.o.step(ids[p.sample])
        s = p.sample_t
        assert (out[s].cpu().numpy() == o_out).all() and (miss[s].cpu().numpy() == o_miss).all()
        assert (status[s].cpu().numpy() == o_status).all()
        pl, oc, mc = plan.cpu().numpy(), out.cpu().numpy(), miss.cpu().numpy()
        for r in range(w.num_requests):
            _check_plan(pl[r], oc[r], ids[r], int(mc[r]))
        p.t += 1
        if t % 8 == 0 or t == w.steps - 1:
            p.check_state()
    p.close()


COPY_GATHER_CASES = [  # (k, B, H, T, row_bytes, policy)
    (200, 330, 1500, 0, 80, 0),
    (200, 330, 1500, 40, 80, 0),  # device tail
    (34, 40, 300, 7, 1152, 1),  # 3 rows per workgroup, the last of 12 holds 1; FIFO
    (5, 8, 60, 3, 16384, 0),  # 1024 chunks per row: one row per workgroup in four passes
    (2, 4, 6, 1, 1 << 20, 1),  # the largest row (1 MiB); FIFO
]


def test_gathering_copy_of_a_plan_without_row_sources():
    """hs_copy with a gather output takes each position's row source from the plan, and writes a missed row to
    its slot from the position that gathers it; a plan made without HS_PLAN_ROW_SOURCES leaves that part as it
    was (here: arbitrary values, in and out of every range). The gathered rows and the new slots' rows are then
    undefined, but every access stays in bounds, the page table is published from the miss list, and the
    outputs and every table match the oracle."""
    import hierarchical_memory_amd as hm
    rng = np.random.default_rng(77)
    R, k, B, H, T, rb = 3, 64, 128, 1000, 16, 48
    w = workload.SINGLE_4K.with_(name="copy_without_sources", num_requests=R, top_k=k, buffer_slots=B,
                                 host_rows=H, L0=H, tail_tokens=T, row_elems=rb // 2, window=400, steps=5,
                                 partB_permille=200, fused_gather=True)
    p = Pair(w, gather=True)
    out, miss, status, g = p.outs
    plan = p.sw.plan_buffer()
    edges = np.array([-2 - k - 5, -2 - k, -3 - k, -2, -1, 0, B - 1, B, B + T - 1, B + T, B + T + 7, 1 << 30,
                      -(1 << 30)], np.int32)
    for t in range(w.steps):
        src = rng.integers(-5000, 5000, size=(R, k)).astype(np.int32)
        src[:, :len(edges)] = edges
        plan[:, 3].copy_(torch.from_numpy(src))
        step_ids = np.ascontiguousarray(p.ids[:, t])
        hm.hs_plan(p.sw.ctx, torch.from_numpy(step_ids).cuda(), p.tail0_dev, out, miss, status, plan)
        hm.hs_copy(p.sw.ctx, plan, miss, g)
        o_out, o_miss, o_status, _ = p.o.step(step_ids, p.tail0)
        assert (out.cpu().numpy() == o_out).all() and (miss.cpu().numpy() == o_miss).all()
        assert (status.cpu().numpy() == o_status).all()
        p.t += 1
        for name, got, exp in (("slot_tok", p.sw.slot_tok, p.o.slot_tok), ("stamp", p.sw.stamp, p.o.stamp),
                               ("page", p.sw.page, p.o.page), ("step", p.sw.step, p.o.t)):
            assert (got.cpu().numpy() == exp).all(), f"step {t}: {name}"
    p.close()


@pytest.mark.parametrize("k,B,H,T,rb,policy", COPY_GATHER_CASES,
                         ids=[f"k{c[0]}_T{c[3]}_rb{c[4]}_p{c[5]}" for c in COPY_GATHER_CASES])
def test_plan_then_copy_with_gather(k, B, H, T, rb, policy):
    """hs_plan, then hs_copy with a gather output: the gathered rows, the hot rows and every table equal the
    oracle's fused step (padding, bad and repeated ids included; with and without a device tail; ragged and
    large rows; both policies)."""
    import hierarchical_memory_amd as hm
    rng = np.random.default_rng(31 + k + T)
    R, steps = 6, 8
    w = workload.SINGLE_4K.with_(name=f"copy_gather_k{k}_T{T}", num_requests=R, top_k=k, buffer_slots=B,
                                 host_rows=H, L0=H, tail_tokens=T, row_elems=rb // 2, steps=steps, fused_gather=True)
    ids = _random_ids(rng, R, steps, k, H, p_weird=0.05)
    tail0 = rng.integers(H // 2, H - T, size=R).astype(np.int32) if T else None
    p = Pair(w, ids=ids, tail0=tail0, gather=True, policy=policy)
    out, miss, status, g = p.outs
    plan = p.sw.plan_buffer()
    for t in range(steps):
        topk = torch.from_numpy(np.ascontiguousarray(ids[:, t])).cuda()
        g.fill_(0xCD)
        hm.hs_plan(p.sw.ctx, topk, p.tail0_dev, out, miss, status, plan, row_sources=True)
        hm.hs_copy(p.sw.ctx, plan, miss, g)
        o_out, o_miss, o_st, o_g = p.o.step(ids[:, t], p.tail0, gather=True)
        assert (out.cpu().numpy() == o_out).all() and (miss.cpu().numpy() == o_miss).all()
        assert (status.cpu().numpy() == o_st).all()
        assert (g.cpu().numpy() == o_g).all(), f"step {t}: gathered rows differ"
        p.t += 1
        p.check_state()
    p.close()


def test_copy_overlapped_on_second_stream():
    """Plans on the main stream, copies on a second stream, two steps in flight with double-buffered plans;
    after the last copy every table and every hot row equals the oracle's."""
    import hierarchical_memory_amd as hm
    w = workload.GROW_32.with_(num_requests=8, steps=30)
    p = Pair(w, sample=list(range(8)))
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    plans = [p.sw.plan_buffer() for _ in range(2)]
    misses = [torch.empty((w.num_requests,), dtype=torch.int32, device="cuda") for _ in range(2)]
    out, _, status, _ = p.outs
    copied = [None, None]
    topk_all = torch.from_numpy(np.ascontiguousarray(p.ids.transpose(1, 0, 2))).cuda()
    torch.cuda.synchronize()
    for t in range(w.steps):
        b = t % 2
        if copied[b] is not None:
            main.wait_event(copied[b])  # the copy that read this plan buffer is done
        hm.hs_plan(p.sw.ctx, topk_all[t], None, out, misses[b], status, plans[b], main)
        planned = torch.cuda.Event()
        planned.record(main)
        side.wait_event(planned)
        hm.hs_copy(p.sw.ctx, plans[b], misses[b], stream=side)
        copied[b] = torch.cuda.Event()
        copied[b].record(side)
        o_out, o_miss, _, _ = p.o.step(p.ids[:, t])
        assert (out.cpu().numpy() == o_out).all() and (misses[b].cpu().numpy() == o_miss).all()
        p.t += 1
    torch.cuda.synchronize()
    p.check_state()
    p.close()


def test_copy_with_gather_overlapped_on_second_stream():
    """The pipelined step: plans on the main stream, copy-and-gather on a second stream, two steps in flight
    (plans and gather outputs double-buffered); every gathered row and, at the end, every table and hot row
    equal the oracle's."""
    import hierarchical_memory_amd as hm
    w = workload.HYBRID_64.with_(num_requests=6, steps=24)
    p = Pair(w, sample=list(range(6)), gather=True)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    R, k, rb = w.num_requests, w.top_k, w.row_bytes
    plans = [p.sw.plan_buffer() for _ in range(2)]
    misses = [torch.empty((R,), dtype=torch.int32, device="cuda") for _ in range(2)]
    gathers = [torch.empty((R, k, rb), dtype=torch.uint8, device="cuda") for _ in range(2)]
    out, _, status, _ = p.outs
    copied = [None, None]
    expected = [None, None]
    topk_all = torch.from_numpy(np.ascontiguousarray(p.ids.transpose(1, 0, 2))).cuda()
    torch.cuda.synchronize()
    for t in range(w.steps):
        b = t % 2
        if copied[b] is not None:
            copied[b].synchronize()  # the copy of step t - 2 is done: check its rows, then reuse its buffers
            assert (gathers[b].cpu().numpy() == expected[b]).all(), f"step {t - 2}: gathered rows differ"
        hm.hs_plan(p.sw.ctx, topk_all[t], p.tail0_dev, out, misses[b], status, plans[b], main, row_sources=True)
        planned = torch.cuda.Event()
        planned.record(main)
        side.wait_event(planned)
        hm.hs_copy(p.sw.ctx, plans[b], misses[b], gathers[b], stream=side)
        copied[b] = torch.cuda.Event()
        copied[b].record(side)
        o_out, o_miss, _, o_g = p.o.step(p.ids[:, t], p.tail0, gather=True)
        expected[b] = o_g
        assert (out.cpu().numpy() == o_out).all() and (misses[b].cpu().numpy() == o_miss).all()
        p.t += 1
    torch.cuda.synchronize()
    for b in range(2):
        assert (gathers[b].cpu().numpy() == expected[b]).all()
    p.check_state()
    p.close()


def test_snapshot_restore_resume():
    """A snapshot of the seven device buffers, restored, resumes exactly like the uninterrupted run."""
    w = workload.GROW_32.with_(num_requests=4, steps=24)
    p = Pair(w)
    for _ in range(10):
        p.step()
    names = ("hot", "slot_tok", "stamp", "lru_order", "page", "step")
    snap = {n: getattr(p.sw, n).clone() for n in names}
    o_snap = {n: getattr(p.o, n).copy() for n in ("hot", "slot_tok", "stamp", "page", "t")}
    first = []
    for _ in range(10, 20):
        p.step()
        first.append(p.outs[0].cpu().numpy().copy())
    for n in names:
        getattr(p.sw, n).copy_(snap[n])
    for n, v in o_snap.items():
        getattr(p.o, n)[...] = v
    p.t = 10
    for i in range(10, 20):
        p.step()
        assert (p.outs[0].cpu().numpy() == first[i - 10]).all()
    p.check_state()
    p.close()


def test_export_import_state_replays_exactly():
    """hs_export_state / hs_import_state: a snapshot of tables and rows taken after 10 steps, imported after 10
    more, replays those 10 steps with the same outputs and ends in the same state; a tables-only import leaves
    the hot rows as they are; the oracle agrees with the replay."""
    import hierarchical_memory_amd as hm
    w = workload.GROW_32.with_(num_requests=4, steps=24)
    p = Pair(w, gather=True)
    for _ in range(10):
        p.step()
    snap = p.sw.state_buffer(hm.HS_STATE_TABLES | hm.HS_STATE_ROWS)
    hm.hs_export_state(p.sw.ctx, snap)
    o_snap = {n: getattr(p.o, n).copy() for n in ("hot", "slot_tok", "stamp", "page", "t")}
    first = []
    for _ in range(10, 20):
        p.step()
        first.append((p.outs[0].cpu().numpy().copy(), p.outs[3].cpu().numpy().copy()))
    end = p.sw.state_buffer()
    hm.hs_export_state(p.sw.ctx, end)
    hm.hs_import_state(p.sw.ctx, snap)
    for n, v in o_snap.items():
        getattr(p.o, n)[...] = v
    p.t = 10
    p.check_state()
    for i in range(10, 20):
        p.step()
        assert (p.outs[0].cpu().numpy() == first[i - 10][0]).all() and (p.outs[3].cpu().numpy() == first[i - 10][1]).all()
    again = p.sw.state_buffer()
    hm.hs_export_state(p.sw.ctx, again)
    assert torch.equal(end, again)
    # tables only: the rows stay as they are
    tables = p.sw.state_buffer(hm.HS_STATE_TABLES)
    hm.hs_export_state(p.sw.ctx, tables, hm.HS_STATE_TABLES)
    hot = p.sw.hot.clone()
    p.sw.hot.fill_(3)
    hm.hs_import_state(p.sw.ctx, tables, hm.HS_STATE_TABLES)
    assert (p.sw.hot == 3).all()
    p.sw.hot.copy_(hot)
    p.check_state()
    # a buffer too small, or a what of nothing, is refused before any copy
    with pytest.raises(hm.HiSparseError) as err:
        hm.hs_export_state(p.sw.ctx, tables, hm.HS_STATE_TABLES | hm.HS_STATE_ROWS)
    assert err.value.code == hm.HS_E_INVALID
    with pytest.raises(hm.HiSparseError):
        hm.hs_import_state(p.sw.ctx, tables, 0)
    p.close()


def test_commit_after_an_offload_or_reset_is_stale():
    """A trial, then an offload of the rows it fetched (the host pool now holds other rows), then the commit:
    the commit is refused (HS_STATUS_STALE) and leaves the state as the offload left it, so no slot ends up with
    a row the host pool no longer holds; a new trial and commit then serve the offloaded rows. Likewise a trial
    made before a reset cannot be committed after the same number of steps has brought the step counter back."""
    import hierarchical_memory_amd as hm
    w = workload.GROW_32.with_(num_requests=4, steps=12)
    p = Pair(w, gather=True)
    R, rb = w.num_requests, w.row_bytes
    trial = p.sw.trial_buffer()
    out, miss, status, g = p.outs
    cstat = torch.zeros((R,), dtype=torch.int32, device="cuda")
    for _ in range(4):
        p.step()
    ids = np.ascontiguousarray(p.ids[:, 4])
    topk = torch.from_numpy(ids).cuda()
    hm.hs_trial(p.sw.ctx, topk, None, out, miss, status, g, trial)
    torch.cuda.synchronize()
    # offload 8 rows per request over the first missed tokens of the trial: the host pool changes under them
    rec = trial.view(R, -1).cpu().numpy()
    pos = rec[:, 4].astype(np.int32).copy()  # each request's smallest missed token
    rows = np.random.default_rng(3).integers(0, 256, size=(R, 8, rb), dtype=np.uint8)
    hm.hs_offload(p.sw.ctx, torch.from_numpy(rows).cuda(), torch.from_numpy(pos).cuda())
    p.o.offload(rows, pos)
    hm.hs_commit(p.sw.ctx, trial, g, None, cstat)
    assert (cstat.cpu().numpy() == hm.HS_STATUS_STALE).all()
    p.check_state()  # the oracle had the offload, not the trial
    p.step(check_state=True)  # the same selection again: the missed rows come from the new host rows
    # reset, the same number of steps again, then an old trial: stale
    hm.hs_trial(p.sw.ctx, torch.from_numpy(np.ascontiguousarray(p.ids[:, 5])).cuda(), None, out, miss, status, g, trial)
    step_before = int(p.sw.step[0].item())
    p.sw.reset()
    p.o.reset()
    for t in range(step_before):
        p.o.step(p.ids[:, t])
        hm.hs_resolve(p.sw.ctx, torch.from_numpy(np.ascontiguousarray(p.ids[:, t])).cuda(), None, out, miss, status, g)
    assert int(p.sw.step[0].item()) == step_before
    hm.hs_commit(p.sw.ctx, trial, g, None, cstat)
    assert (cstat.cpu().numpy() == hm.HS_STATUS_STALE).all()
    p.check_state()
    p.close()


def test_commit_after_a_tail_advance_or_an_import_is_stale():
    """A trial made before a tail advance that moves the windows, or before a state import (even of the very
    state the trial was made from), is refused at commit (HS_STATUS_STALE) and leaves the state as the advance
    or the import left it; the run then continues in parity."""
    import hierarchical_memory_amd as hm
    w = workload.HYBRID_64.with_(num_requests=4, steps=12)
    p = Pair(w, gather=True)
    R = w.num_requests
    trial = p.sw.trial_buffer()
    out, miss, status, g = p.outs
    cstat = torch.full((R,), -1, dtype=torch.int32, device="cuda")
    for _ in range(4):
        p.step()
    hm.hs_trial(p.sw.ctx, torch.from_numpy(np.ascontiguousarray(p.ids[:, 4])).cuda(), p.tail0_dev, out, miss,
                status, g, trial)
    n = np.full(R, 16, np.int32)
    hm.hs_advance_tail(p.sw.ctx, p.tail0_dev, torch.from_numpy(n).cuda())
    t0_o = np.ascontiguousarray(p.tail0[p.sample])
    p.o.advance_tail(t0_o, n[p.sample])
    hm.hs_commit(p.sw.ctx, trial, g, None, cstat)
    assert (cstat.cpu().numpy() == hm.HS_STATUS_STALE).all()
    p.tail0 = p.tail0_dev.cpu().numpy().astype(np.int32)
    assert (p.tail0[p.sample] == t0_o).all()
    p.check_state()  # the advance's state: no trial applied
    p.step(check_state=True)
    # an import of the current state itself: a trial made before it is still stale
    snap = p.sw.state_buffer(hm.HS_STATE_TABLES)
    hm.hs_trial(p.sw.ctx, torch.from_numpy(np.ascontiguousarray(p.ids[:, p.t])).cuda(), p.tail0_dev, out, miss,
                status, g, trial)
    hm.hs_export_state(p.sw.ctx, snap, hm.HS_STATE_TABLES)
    hm.hs_import_state(p.sw.ctx, snap, hm.HS_STATE_TABLES)
    cstat.fill_(-1)
    hm.hs_commit(p.sw.ctx, trial, g, None, cstat)
    assert (cstat.cpu().numpy() == hm.HS_STATUS_STALE).all()
    p.check_state()
    for _ in range(2):
        p.step(check_state=True)
    p.close()


def test_import_tables_and_rebuild_order():
    """Tables computed elsewhere (here by the oracle, on the CPU) are imported without an order list;
    hs_rebuild_order derives it from the stamps and the run continues in parity."""
    import hierarchical_memory_amd as hm
    w = workload.GROW_32.with_(num_requests=3, steps=20)
    p = Pair(w)
    ids = p.ids
    for t in range(8):  # the oracle alone
        p.o.step(ids[:, t])
    for n_gpu, n_o in (("slot_tok", "slot_tok"), ("stamp", "stamp"), ("page", "page"), ("step", "t"), ("hot", "hot")):
        getattr(p.sw, n_gpu).copy_(torch.from_numpy(np.ascontiguousarray(getattr(p.o, n_o))))
    p.sw.lru_order.zero_()
    hm.hs_rebuild_order(p.sw.ctx)
    p.t = 8
    p.check_state()
    for _ in range(8, w.steps):
        p.step(check_state=True)
    p.close()


def _oracle_copy(o):
    import copy
    c = copy.copy(o)
    for n in ("slot_tok", "stamp", "page", "t", "hot"):
        setattr(c, n, getattr(o, n).copy())
    return c


def test_trial_commit_retry_matches_oracle():
    """hs_trial changes nothing; its outputs and gathered rows equal the oracle's on a copy of the state.
    hs_commit applies the accepted requests only; a record committed twice is stale the second time."""
    import hierarchical_memory_amd as hm
    w = workload.GROW_32.with_(num_requests=6, steps=14)
    p = Pair(w, gather=True)
    R = w.num_requests
    trial = p.sw.trial_buffer()
    out, miss, status, g = p.outs
    cstat = torch.zeros((R,), dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(11)
    names = ("slot_tok", "stamp", "lru_order", "page", "step", "hot")
    for t in range(w.steps):
        ids = p.ids[:, t]
        # a first try with another selection (the next request's ids), rejected
        alt = np.ascontiguousarray(np.roll(ids, 1, axis=0))
        before = {n: getattr(p.sw, n).clone() for n in names}
        hm.hs_trial(p.sw.ctx, torch.from_numpy(alt).cuda(), None, out, miss, status, g, trial)
        oc = _oracle_copy(p.o)
        o_out, o_miss, o_st, o_g = oc.step(alt, gather=True)
        assert (out.cpu().numpy() == o_out).all() and (miss.cpu().numpy() == o_miss).all()
        assert (status.cpu().numpy() == o_st).all() and (g.cpu().numpy() == o_g).all()
        for n in names:
            assert torch.equal(before[n], getattr(p.sw, n)), f"trial changed {n}"
        hm.hs_commit(p.sw.ctx, trial, g, torch.zeros((R,), dtype=torch.int32, device="cuda"), cstat)
        for n in names:
            assert torch.equal(before[n], getattr(p.sw, n)), f"rejected commit changed {n}"
        # the real selection, accepted for a random subset of the requests
        hm.hs_trial(p.sw.ctx, torch.from_numpy(np.ascontiguousarray(ids)).cuda(), None, out, miss, status, g, trial)
        oc = _oracle_copy(p.o)
        o_out, o_miss, o_st, o_g = oc.step(ids, gather=True)
        assert (out.cpu().numpy() == o_out).all() and (g.cpu().numpy() == o_g).all()
        accept = rng.integers(0, 2, size=R).astype(np.int32)
        accept[t % R] = 1
        hm.hs_commit(p.sw.ctx, trial, g, torch.from_numpy(accept).cuda(), cstat)
        assert (cstat.cpu().numpy() == 0).all()
        for r in np.nonzero(accept)[0]:
            for n in ("slot_tok", "stamp", "page", "t", "hot"):
                getattr(p.o, n)[r] = getattr(oc, n)[r]
        p.t += 1
        p.check_state()
        # committing the same records again: every accepted request is now stale
        hm.hs_commit(p.sw.ctx, trial, g, torch.from_numpy(accept).cuda(), cstat)
        assert (cstat.cpu().numpy() == accept * hm.HS_STATUS_STALE).all()
        p.check_state()
    p.close()


def test_trial_commit_hybrid_tail():
    """Trial and commit with a device tail: resident ids resolve in place and take no slot."""
    import hierarchical_memory_amd as hm
    w = workload.HYBRID_64.with_(num_requests=4, steps=10)
    p = Pair(w, gather=True)
    trial = p.sw.trial_buffer()
    out, miss, status, g = p.outs
    for t in range(w.steps):
        ids = p.ids[:, t]
        hm.hs_trial(p.sw.ctx, torch.from_numpy(np.ascontiguousarray(ids)).cuda(), p.tail0_dev, out, miss, status,
                    g, trial)
        o_out, o_miss, o_st, o_g = p.o.step(ids, p.tail0, gather=True)
        assert (out.cpu().numpy() == o_out).all() and (g.cpu().numpy() == o_g).all()
        hm.hs_commit(p.sw.ctx, trial, g)
        p.t += 1
        p.check_state()
    p.close()


FIFO_CASES = [workload.SINGLE_4K, workload.GROW_32.with_(num_requests=8, steps=64),
              workload.HYBRID_64.with_(num_requests=4, steps=24),
              workload.SWEEP_BASE.with_(num_requests=4, steps=48, buffer_slots=2048)]


@pytest.mark.parametrize("w", FIFO_CASES, ids=lambda w: w.name)
def test_fifo_policy(w):
    """FIFO replacement (hits do not refresh stamps) against the oracle run with the same policy."""
    import hierarchical_memory_amd as hm
    p = Pair(w, policy=hm.HS_EVICT_FIFO)
    p.run(check_every=4)
    p.close()


def test_fifo_plan_trial_commit():
    import hierarchical_memory_amd as hm
    w = workload.GROW_32.with_(num_requests=4, steps=16)
    p = Pair(w, policy=hm.HS_EVICT_FIFO, gather=True)
    plan, trial = p.sw.plan_buffer(), p.sw.trial_buffer()
    out, miss, status, g = p.outs
    for t in range(w.steps):
        ids = np.ascontiguousarray(p.ids[:, t])
        topk = torch.from_numpy(ids).cuda()
        if t % 2:
            hm.hs_plan(p.sw.ctx, topk, None, out, miss, status, plan)
            hm.hs_copy(p.sw.ctx, plan, miss)
        else:
            hm.hs_trial(p.sw.ctx, topk, None, out, miss, status, g, trial)
            hm.hs_commit(p.sw.ctx, trial, g)
        o_out, o_miss, _, _ = p.o.step(ids)
        assert (out.cpu().numpy() == o_out).all() and (miss.cpu().numpy() == o_miss).all()
        p.t += 1
        p.check_state()
    p.close()


def test_offload_rows_then_resolve():
    """hs_offload writes device rows into the host pool (and into the hot slot of a token that has one);
    later resolves fetch the new rows. Pool, slots and every later output equal the oracle's."""
    import hierarchical_memory_amd as hm
    w = workload.GROW_32.with_(num_requests=6, steps=20)
    p = Pair(w)
    R, rb = w.num_requests, w.row_bytes
    for _ in range(8):
        p.step()
    n = 700
    rows = np.empty((R, n, rb), np.uint8)
    workload.fill_rows(rows.view(np.uint16).reshape(R * n, rb // 2), 0, R * n, rb // 2, 4242)
    pos = np.array([0, 5000, 30000, w.host_rows - 300, 32000, 12345], np.int32)
    status = torch.zeros((R,), dtype=torch.int32, device="cuda")
    hm.hs_offload(p.sw.ctx, torch.from_numpy(rows).cuda(), torch.from_numpy(pos).cuda(), status)
    o_st = p.o.offload(rows, pos)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == o_st).all() and o_st[3] == hm.HS_STATUS_BAD_ID
    pool = p.sw.host_pool()
    for r in range(R):
        a = int(pos[r])
        b = min(w.host_rows, a + n)
        assert (pool[r][a:b] == p.o.host[r][a:b]).all() and (pool[r][a:b] == rows[r][:b - a]).all()
    p.check_state()
    for _ in range(8, w.steps):
        p.step(check_state=True)
    p.close()


def test_large_topk_equal_buffer():
    """k = B = 4096 (the largest top-k whose workgroup fits the LDS with this context): every free slot is a
    victim each step."""
    w = workload.SINGLE_4K.with_(name="k4096", num_requests=3, top_k=4096, buffer_slots=4096, host_rows=16384,
                                 L0=16384, window=8192, steps=10)
    p = Pair(w)
    p.run(check_every=2)
    p.close()


@pytest.mark.parametrize("path", ["fused", "fused_gather", "plan_copy"])
def test_largest_topk_and_buffer(path):
    """k = 4096 with B = 8192 and a 40,000-token context, near the LDS cap of one workgroup (the direct layout
    with eight ids and eight slots per thread without a gather, the rank layout with one), a repeated id on
    some steps; every step and the state against the oracle."""
    import hierarchical_memory_amd as hm
    R, k, B, H = 2, 4096, 8192, 40_000
    sizes = hm.hs_required_sizes(hm.config(R, k, B, 0.0, 64, H))
    assert sizes.lds_bytes > 150 * 1024 and sizes.token_slot_table == 1
    w = workload.SINGLE_4K.with_(name=f"k4096_B8192_{path}", num_requests=R, top_k=k, buffer_slots=B,
                                 host_rows=H, L0=H, window=12000, row_elems=32, steps=8,
                                 fused_gather=path == "fused_gather")
    ids = workload.streams(w)
    ids[:, 1::3, 11] = ids[:, 1::3, 2]
    if path != "plan_copy":
        p = Pair(w, ids=ids, gather=path == "fused_gather")
        p.run(check_every=1)
        p.close()
        return
    p = Pair(w, ids=ids)
    plan = p.sw.plan_buffer()
    out, miss, status, _ = p.outs
    for t in range(w.steps):
        step_ids = np.ascontiguousarray(p.ids[:, t])
        hm.hs_plan(p.sw.ctx, torch.from_numpy(step_ids).cuda(), None, out, miss, status, plan)
        hm.hs_copy(p.sw.ctx, plan, miss)
        o_out, o_miss, o_status, _ = p.o.step(step_ids[p.sample])
        assert (out.cpu().numpy() == o_out).all() and (miss.cpu().numpy() == o_miss).all()
        assert (status.cpu().numpy() == o_status).all()
        p.t += 1
        p.check_state()
    p.close()


def test_many_small_requests():
    """1500 requests (1500 workgroups, more than the 256 CUs), tiny k and B."""
    rng = np.random.default_rng(8)
    w = workload.SINGLE_4K.with_(name="many", num_requests=1500, top_k=8, buffer_slots=8, host_rows=64, L0=64,
                                 steps=6, row_elems=8)
    ids = _random_ids(rng, 1500, 6, 8, 64, p_weird=0.05)
    p = Pair(w, ids=ids, sample=[0, 1, 777, 1499])
    p.run(check_every=1)
    p.check_all_requests(rows_per_request=4)
    p.close()


def test_whole_set_kept():
    """keep = 100 %: k misses at step 0, none after; slots and rows never move."""
    p = Pair(workload.SINGLE_4K.with_(keep_permille=1000))
    p.run(check_every=4)
    assert int(p.outs[1][0].item()) == 0
    p.close()


def test_graph_replay_plan_copy_and_trial_commit():
    """The split step (plan + copy) and the retryable step (trial + commit) captured in HIP graphs: every
    replay, with eager work and synchronisation between replays, equals the oracle."""
    import hierarchical_memory_amd as hm
    w = workload.GROW_32.with_(num_requests=4, steps=12)
    for kind in ("split", "trial"):
        p = Pair(w, gather=True)
        topk = torch.empty((w.num_requests, w.top_k), dtype=torch.int32, device="cuda")
        out, miss, status, g = p.outs
        plan, trial = p.sw.plan_buffer(), p.sw.trial_buffer()
        cstat = torch.zeros((w.num_requests,), dtype=torch.int32, device="cuda")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg, stream=s):
            if kind == "split":
                hm.hs_plan(p.sw.ctx, topk, None, out, miss, status, plan)
                hm.hs_copy(p.sw.ctx, plan, miss)
            else:
                hm.hs_trial(p.sw.ctx, topk, None, out, miss, status, g, trial)
                hm.hs_commit(p.sw.ctx, trial, g, None, cstat)
        torch.cuda.synchronize()
        for t in range(w.steps):
            ids = np.ascontiguousarray(p.ids[:, t])
            topk.copy_(torch.from_numpy(ids))
            cg.replay()
            torch.cuda.synchronize()
            o_out, o_miss, _, o_g = p.o.step(ids, gather=True)
            assert (out.cpu().numpy() == o_out).all() and (miss.cpu().numpy() == o_miss).all(), (kind, t)
            if kind == "trial":
                assert (g.cpu().numpy() == o_g).all() and (cstat.cpu().numpy() == 0).all()
            p.t += 1
            p.check_state()
        p.close()


def test_advance_tail_then_resolve():
    """The tail window moves forward: the leaving tokens' ring rows (overwritten first with fresh rows, as a
    model would produce them) go to the host pool, tail0 advances on the device, and those tokens then
    resolve through the hot buffer — all equal to the oracle."""
    import hierarchical_memory_amd as hm
    w = workload.HYBRID_64.with_(num_requests=4, steps=18)
    p = Pair(w, gather=True)
    R, T, rb = w.num_requests, w.tail_tokens, w.row_bytes
    for _ in range(6):
        p.step()
    n = np.array([64, 1000, 0, 20000], np.int32)  # the last is clamped to T
    fresh = np.empty((R, T, rb), np.uint8)
    workload.fill_rows(fresh.view(np.uint16).reshape(R * T, rb // 2), 0, R * T, rb // 2, 555)
    p.sw.tail.copy_(torch.from_numpy(fresh))
    p.o.tail[...] = fresh[p.sample]
    status = torch.full((R,), -1, dtype=torch.int32, device="cuda")
    hm.hs_advance_tail(p.sw.ctx, p.tail0_dev, torch.from_numpy(n).cuda(), status)
    t0_o = np.ascontiguousarray(p.tail0[p.sample])
    old = t0_o.copy()
    o_st = p.o.advance_tail(t0_o, n[p.sample])
    torch.cuda.synchronize()
    new_t0 = p.tail0_dev.cpu().numpy()
    assert (new_t0 == old + np.minimum(n, T)).all() and (new_t0[p.sample] == t0_o).all()
    assert (status.cpu().numpy() == 0).all() and (o_st == 0).all()
    pool = p.sw.host_pool()
    for j, r in enumerate(p.sample):
        for x in range(int(old[j]), int(new_t0[r]), 97):
            assert (pool[r][x] == fresh[r][x % T]).all() and (p.o.host[j][x] == pool[r][x]).all()
    p.tail0 = new_t0.astype(np.int32)
    p.check_state()
    for _ in range(6, w.steps):
        p.step(check_state=True)
    p.close()
