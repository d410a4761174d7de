"""Pins of the CPU oracle against facts fixed outside it.

The oracle is the reference every GPU result is compared with, so it is itself
checked against things it does not compute: a hand-worked trace, a second
formulation of LRU (a list, not a sort over stamps), closed forms of special
cases, and invariants that hold after every step. A mutation test then plants
plausible mistakes in a copy of the oracle's source and checks that these pins
catch each one.
"""
from __future__ import annotations

import itertools
import os
import random

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
import workload
from tests.brute_lru import ListLRU

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def make_host(n, H, row_bytes, seed=7):
    """Distinct seeded rows, so a wrong row shows up in a byte comparison."""
    host = np.empty((n, H, row_bytes), np.uint8)
    workload.fill_rows(host.view(np.uint16).reshape(n * H, row_bytes // 2), 0, n * H, row_bytes // 2, seed)
    return host


def check_invariants(o: oracle.Oracle, r: int, ids, out, miss, status, tail0=None, gathered=None):
    """Invariants that hold after every step (any sizes)."""
    B, H = o.B, o.H
    st_, stamp, page = o.slot_tok[r], o.stamp[r], o.page[r]
    occupied = np.nonzero(st_ >= 0)[0]
    # slot table injective on occupied slots; page table is its inverse
    assert len(set(st_[occupied].tolist())) == len(occupied)
    assert (page[st_[occupied]] == occupied).all()
    assert int((page >= 0).sum()) == len(occupied)
    # empty slots carry stamp -1, occupied ones a past step
    assert (stamp[st_ < 0] == -1).all()
    assert (stamp[occupied] >= 0).all() and (stamp[occupied] < o.t[r]).all()
    # every occupied slot holds its token's host row
    if len(occupied):
        assert (o.hot[r][occupied] == o.host[r][st_[occupied]]).all()
    # hits + misses + resident = valid ids
    valid = [x for x in ids if x != -1]
    res = sum(1 for v in out if v >= B)
    ok = sum(1 for v in out if v >= 0)
    if status == 0:
        assert ok == len(valid)
    n_hit = ok - res - miss
    assert n_hit >= 0
    # every resolved id maps to its own row
    for i, x in enumerate(ids):
        v = out[i]
        if 0 <= v < B:
            assert st_[v] == x and page[x] == v
            if o.policy == oracle.LRU:
                assert stamp[v] == o.t[r] - 1
            else:
                assert stamp[v] <= o.t[r] - 1
        elif v >= B:
            assert tail0 is not None and v == B + x % o.T
        if gathered is not None:
            if v >= 0:
                assert (gathered[i] == o.host[r][x]).all()
            else:
                assert (gathered[i] == 0).all()


# --------------------------------------------------------------------------- worked example

def _read_golden(name):
    lines = [l.strip() for l in open(os.path.join(GOLDEN, name)) if l.strip() and not l.startswith("#")]
    kv, steps = {}, []
    for l in lines:
        if l.startswith("step "):
            a, b, c = l[5:].split("|")
            steps.append(([int(v) for v in a.split()], [int(v) for v in b.split()[1:]], int(c.split()[1])))
        else:
            key, *vals = l.split()
            kv[key] = [int(v) for v in vals]
    return kv, steps


def test_worked_example():
    kv, steps = _read_golden("worked_example_B3_k2.txt")
    B, k, H = kv["B"][0], kv["k"][0], kv["H"][0]
    o = oracle.Oracle(1, B, k, H, 16, host=make_host(1, H, 16))
    for ids, out_exp, miss_exp in steps:
        out, miss, status, _ = o.step(np.array([ids], np.int32))
        assert out[0].tolist() == out_exp and miss[0] == miss_exp and status[0] == 0
    assert o.slot_tok[0].tolist() == kv["final_slot_tok"]
    assert o.stamp[0].tolist() == kv["final_stamp"]
    assert o.page[0].tolist() == kv["final_page"]
    assert o.t[0] == kv["final_t"][0]


# --------------------------------------------------------------------------- list LRU, exhaustive

def _compare_with_list(o, lru, r, ids, tail0=None):
    out, miss, status, _ = o.step(np.array([ids], np.int32), None if tail0 is None else np.array([tail0], np.int32))
    out_l, miss_l, status_l = lru.step(ids, tail0)
    assert out[0].tolist() == out_l
    assert miss[0] == miss_l and status[0] == status_l
    assert o.slot_tok[r].tolist() == lru.slot_tok()
    assert o.stamp[r].tolist() == lru.stamps()
    assert o.page[r].tolist() == lru.page()
    assert o.t[r] == lru.t
    check_invariants(o, r, ids, out[0].tolist(), miss[0], status[0], tail0)


@pytest.mark.parametrize("policy", [oracle.LRU, oracle.FIFO], ids=["lru", "fifo"])
def test_list_lru_exhaustive_tiny(policy):
    """Every sequence of 3 steps of k-subsets of 6 tokens (k <= 3), every B in [k, 4], with the ids of each
    step in two orders: the oracle and the list model agree on every output and every table."""
    H = 6
    rb = 16
    host = make_host(1, H, rb)
    n_cases = 0
    for k in (1, 2, 3):
        subsets = [list(c) for c in itertools.combinations(range(H), k)]
        for B in range(k, 5):
            for seq in itertools.product(subsets, repeat=3):
                for flip in (False, True):
                    o = oracle.Oracle(1, B, k, H, rb, host=host, policy=policy)
                    lru = ListLRU(B, H, fifo=policy == oracle.FIFO)
                    for ids in seq:
                        ids = ids[::-1] if flip else ids
                        _compare_with_list(o, lru, 0, ids)
                    n_cases += 1
    assert n_cases > 10000


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(st.data())
def test_list_lru_random(data):
    """Random sizes, padding, out-of-range and repeated ids, and a device tail."""
    k = data.draw(st.integers(1, 12))
    B = data.draw(st.integers(k, 20))
    H = data.draw(st.integers(1, 40))
    T = data.draw(st.integers(0, 6))
    use_tail = data.draw(st.booleans()) and T > 0
    tail0 = data.draw(st.integers(0, H)) if use_tail else None
    steps = data.draw(st.integers(1, 8))
    policy = data.draw(st.sampled_from([oracle.LRU, oracle.FIFO]))
    o = oracle.Oracle(1, B, k, H, 16, T=T, host=make_host(1, H, 16), policy=policy)
    lru = ListLRU(B, H, T, fifo=policy == oracle.FIFO)
    for _ in range(steps):
        ids = data.draw(st.lists(st.integers(-3, H + 2), min_size=k, max_size=k))
        _compare_with_list(o, lru, 0, ids, tail0)


# --------------------------------------------------------------------------- closed forms

def test_cold_start():
    """From an empty buffer, the j-th smallest selected id takes slot j (empty slots go in index order),
    with stamp 0; the other slots stay empty."""
    rng = np.random.default_rng(3)
    for B, k, H in [(8, 8, 50), (512, 256, 4096), (4096, 2048, 40960), (6144, 2048, 65536)]:
        ids = rng.choice(H, size=k, replace=False).astype(np.int32)
        o = oracle.Oracle(1, B, k, H, 16, host=make_host(1, H, 16))
        out, miss, status, _ = o.step(ids[None])
        order = np.argsort(ids)
        assert miss[0] == k and status[0] == 0
        assert (out[0][order] == np.arange(k)).all()
        assert (o.slot_tok[0][:k] == np.sort(ids)).all() and (o.slot_tok[0][k:] == -1).all()
        assert (o.stamp[0][:k] == 0).all() and (o.stamp[0][k:] == -1).all()


def test_buffer_holds_whole_context():
    """B >= number of tokens: only compulsory misses. A token seen for the first time at step t takes slot
    (distinct tokens seen before t) + (its rank among step t's new tokens); its slot's stamp is the last step
    that selected it."""
    w = workload.SINGLE_4K.with_(buffer_slots=4096, steps=64)
    ids = workload.streams(w)[0]
    o = oracle.Oracle(1, 4096, w.top_k, w.host_rows, 16, host=make_host(1, w.host_rows, 16))
    seen_order = {}
    last = {}
    for t in range(w.steps):
        out, miss, status, _ = o.step(ids[t][None])
        new = sorted(x for x in ids[t].tolist() if x not in seen_order)
        base = len(seen_order)
        for j, x in enumerate(new):
            seen_order[x] = base + j
        for x in ids[t].tolist():
            last[x] = t
        assert miss[0] == len(new)
        assert [seen_order[x] for x in ids[t].tolist()] == out[0].tolist()
    for x, s in seen_order.items():
        assert o.slot_tok[0][s] == x and o.stamp[0][s] == last[x]


def test_buffer_equals_topk():
    """B = k: after every step the buffer holds exactly the selected set; misses are the ids not selected in
    the previous step, and (all free slots then sharing stamp t-1) the j-th smallest new id goes to the j-th
    smallest free slot."""
    w = workload.SINGLE_4K.with_(buffer_slots=256)
    ids = workload.streams(w)[0]
    k = w.top_k
    o = oracle.Oracle(1, k, k, w.host_rows, 16, host=make_host(1, w.host_rows, 16))
    prev_slots = {}
    for t in range(w.steps):
        out, miss, status, _ = o.step(ids[t][None])
        cur = ids[t].tolist()
        new = sorted(set(cur) - set(prev_slots))
        assert miss[0] == len(new)
        assert set(o.slot_tok[0].tolist()) == set(cur)
        if t > 0:
            kept_slots = {prev_slots[x] for x in cur if x in prev_slots}
            free = sorted(set(range(k)) - kept_slots)
            for j, x in enumerate(new):
                assert out[0][cur.index(x)] == free[j]
        prev_slots = {x: int(out[0][i]) for i, x in enumerate(cur)}


def test_fifo_closed_forms():
    """FIFO: a hit never refreshes a stamp. Keeping the whole set, stamps stay at the step the slots were
    filled (0); with a buffer holding the whole context, a token's slot is the same as under LRU (only
    compulsory misses) but its stamp is the first step that selected it."""
    w = workload.SINGLE_4K.with_(keep_permille=1000)
    ids = workload.streams(w)[0]
    o = oracle.Oracle(1, w.buffer_slots, w.top_k, w.host_rows, 16, host=make_host(1, w.host_rows, 16),
                      policy=oracle.FIFO)
    for t in range(w.steps):
        out, miss, status, _ = o.step(ids[t][None])
        assert miss[0] == (w.top_k if t == 0 else 0)
        occ = o.slot_tok[0] >= 0
        assert (o.stamp[0][occ] == 0).all() and (o.stamp[0][~occ] == -1).all()
    w = workload.SINGLE_4K.with_(buffer_slots=4096)
    ids = workload.streams(w)[0]
    lru = oracle.Oracle(1, 4096, w.top_k, w.host_rows, 16, host=make_host(1, w.host_rows, 16))
    fifo = oracle.Oracle(1, 4096, w.top_k, w.host_rows, 16, host=make_host(1, w.host_rows, 16), policy=oracle.FIFO)
    first = {}
    for t in range(w.steps):
        a = lru.step(ids[t][None])[0]
        b = fifo.step(ids[t][None])[0]
        assert (a == b).all()
        for x in ids[t].tolist():
            first.setdefault(x, t)
    for s in np.nonzero(fifo.slot_tok[0] >= 0)[0]:
        assert fifo.stamp[0][s] == first[int(fifo.slot_tok[0][s])]


def test_same_set_every_step():
    """Keeping the whole set (p = 1): k misses at step 0, none after; slots never move; stamps track the step."""
    w = workload.SINGLE_4K.with_(keep_permille=1000)
    ids = workload.streams(w)[0]
    o = oracle.Oracle(1, w.buffer_slots, w.top_k, w.host_rows, 16, host=make_host(1, w.host_rows, 16))
    first = None
    for t in range(w.steps):
        out, miss, status, _ = o.step(ids[t][None])
        assert set(ids[t].tolist()) == set(ids[0].tolist())
        assert miss[0] == (w.top_k if t == 0 else 0)
        m = dict(zip(ids[t].tolist(), out[0].tolist()))
        first = first or m
        assert m == first
        occ = o.slot_tok[0] >= 0
        assert (o.stamp[0][occ] == t).all() and (o.stamp[0][~occ] == -1).all()


# --------------------------------------------------------------------------- invariants on real streams

@pytest.mark.parametrize("w", [workload.SINGLE_4K,
                               workload.GROW_32.with_(num_requests=2, steps=24),
                               workload.HYBRID_64.with_(num_requests=2, steps=12, L0=20000, host_rows=20000,
                                                        tail_tokens=2000, top_k=512, buffer_slots=1024)],
                         ids=lambda w: w.name)
def test_invariants_on_workload_streams(w):
    n = w.num_requests
    ids = workload.streams(w)
    rb = 16
    host = make_host(n, w.host_rows, rb)
    tail = None
    tail0 = None
    if w.tail_tokens:
        tail0 = np.full(n, w.tail0, np.int32)
        tail = np.zeros((n, w.tail_tokens, rb), np.uint8)
        for x in range(w.tail0, w.tail0 + w.tail_tokens):  # ring row x mod T
            tail[:, x % w.tail_tokens] = host[:, x]
    o = oracle.Oracle(n, w.buffer_slots, w.top_k, w.host_rows, rb, T=w.tail_tokens, host=host, tail=tail)
    last = [dict() for _ in range(n)]
    for t in range(w.steps):
        out, miss, status, g = o.step(ids[:, t], tail0, gather=True)
        for r in range(n):
            check_invariants(o, r, ids[r, t].tolist(), out[r].tolist(), miss[r], status[r],
                             None if tail0 is None else int(tail0[r]), g[r])
            for x in ids[r, t].tolist():
                last[r][x] = t
            # stamp of a buffered token's slot = the last step that selected it
            occ = np.nonzero(o.slot_tok[r] >= 0)[0]
            for s in occ:
                assert o.stamp[r][s] == last[r][int(o.slot_tok[r][s])]
            assert min(w.buffer_slots, sum(1 for x in last[r] if tail0 is None or x < tail0[r])) == len(occ)


def test_error_paths():
    """Padding leaves state alone; out-of-range, outside-the-tail and repeated ids give -1 and a status bit,
    the first of repeated ids being the one resolved."""
    H, B, k = 20, 8, 6
    o = oracle.Oracle(1, B, k, H, 16, T=4, host=make_host(1, H, 16))
    out, miss, status, _ = o.step(np.array([[-1, -1, -1, -1, -1, -1]], np.int32))
    assert (out == -1).all() and miss[0] == 0 and status[0] == 0 and (o.slot_tok == -1).all() and o.t[0] == 1
    out, miss, status, _ = o.step(np.array([[3, 25, 3, -7, 5, -1]], np.int32))
    assert out[0].tolist() == [0, -1, -1, -1, 1, -1] and miss[0] == 2
    assert status[0] == oracle.BAD_ID | oracle.DUP_ID
    out, miss, status, _ = o.step(np.array([[14, 18, 19, 15, 3, 14]], np.int32), np.array([15], np.int32))
    # 14 < tail0: a miss; 15..18 resident (T=4, ring row x mod 4); 19 outside the tail window; last 14 repeated
    assert out[0].tolist() == [2, 8 + 18 % 4, -1, 8 + 15 % 4, 0, -1] and status[0] == oracle.BAD_ID | oracle.DUP_ID
    o.reset()
    assert (o.slot_tok == -1).all() and (o.stamp == -1).all() and (o.page == -1).all() and o.t[0] == 0


# --------------------------------------------------------------------------- mutation test

MUTANTS = {
    "equal stamps: highest slot first": ("if (p->val != q->val) return p->val < q->val ? -1 : 1;",
                                         "if (p->val != q->val) return p->val > q->val ? -1 : 1;"),
    "misses paired in selection order": ("qsort(misses, (size_t)m, sizeof(pair_t), by_key_then_val);", ""),
    "hit stamps not refreshed": ("if (hit[s]) stamp[s] = t;", "if (hit[s]) stamp[s] = stamp[s];"),
    "new slot stamped t-1": ("stamp[v] = t;", "stamp[v] = t - 1;"),
    "evicted token left in page table": ("if (y != -1) page[y] = -1;", "if (y != -1) page[y] = page[y];"),
    "wrong host row": ("host + (int64_t)x * rb", "host + (int64_t)(x ^ 1) * rb"),
    "victims from the newest end": ("const int32_t v = cand[j].val;", "const int32_t v = cand[c - 1 - j].val;"),
    "duplicate not rejected": ("if (seen[x]) { status |= ORACLE_DUP_ID; continue; }", ""),
    "tail window not checked": ("if (resident && (int64_t)x - (int64_t)tail0 >= (int64_t)T)", "if (0)"),
    "tail index off by one": ("out[i] = B + x % T;", "out[i] = B + (x + 1) % T;"),
    "tail indexed from tail0": ("out[i] = B + x % T;", "out[i] = B + (x - tail0);"),
    "step counter not advanced": ("*t_io = t + 1;", "*t_io = t;"),
    "FIFO refreshes hit stamps": ("if (d->policy == ORACLE_LRU)\n    for", "if (1)\n    for"),
    "LRU leaves hit stamps alone": ("if (d->policy == ORACLE_LRU)\n    for", "if (d->policy == ORACLE_FIFO)\n    for"),
    "offload leaves the hot slot stale": (
        "if (page[x] != -1) memcpy(hot + (int64_t)page[x] * rb, rows + (int64_t)j * rb, (size_t)rb);", ""),
    "offloaded rows in reverse order": ("memcpy(host + x * rb, rows + (int64_t)j * rb, (size_t)rb);",
                                        "memcpy(host + x * rb, rows + (int64_t)(n - 1 - j) * rb, (size_t)rb);"),
    "leaving tail rows not written to the host": ("memcpy(host + x * rb, tail + (x % d->T) * rb, (size_t)rb);", ""),
    "tail window not advanced": ("*tail0 += n;", "*tail0 += 0;"),
    "tail advance not clamped to the ring": ("if (n > d->T) n = d->T;", ""),
}


def _run_pins_against(lib_path: str) -> bool:
    """True when every pin passes for the oracle library at lib_path."""
    import tests.test_oracle_pins as me
    real = oracle.load

    def fake(path=None):
        return real(lib_path)

    oracle.load = fake
    try:
        me.test_worked_example()
        host = make_host(1, 6, 16)
        for k in (1, 2, 3):
            for B in range(k, 5):
                for seq in itertools.product(list(itertools.combinations(range(6), k)), repeat=2):
                    o = oracle.Oracle(1, B, k, 6, 16, host=host)
                    lru = ListLRU(B, 6)
                    for ids in seq:
                        _compare_with_list(o, lru, 0, list(ids)[::-1])
        for k in (1, 2, 3):
            for B in range(k, 5):
                for seq in itertools.product(list(itertools.combinations(range(6), k)), repeat=2):
                    o = oracle.Oracle(1, B, k, 6, 16, host=host, policy=oracle.FIFO)
                    lst = ListLRU(B, 6, fifo=True)
                    for ids in seq:
                        _compare_with_list(o, lst, 0, list(ids)[::-1])
        me.test_cold_start()
        me.test_offload_keeps_slots_consistent()
        me.test_advance_tail_moves_rows_to_host()
        me.test_buffer_equals_topk()
        me.test_error_paths()
        me.test_fifo_closed_forms()
        rng = random.Random(5)
        for _ in range(200):
            k = rng.randint(1, 8); B = rng.randint(k, 12); H = rng.randint(2, 24); T = rng.randint(0, 4)
            tail0 = rng.randint(0, H) if T else None
            o = oracle.Oracle(1, B, k, H, 16, T=T, host=make_host(1, H, 16))
            lru = ListLRU(B, H, T)
            for _ in range(rng.randint(1, 6)):
                _compare_with_list(o, lru, 0, [rng.randint(-2, H + 1) for _ in range(k)], tail0)
        return True
    except AssertionError:
        return False
    finally:
        oracle.load = real


def test_pins_pass_on_real_oracle():
    assert _run_pins_against(oracle.build(force=False))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, name
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    lib = oracle.build(force=True, src=str(mut), dst=str(tmp_path / "libmutant.so"))
    assert not _run_pins_against(lib), f"no pin caught: {name}"


def test_offload_keeps_slots_consistent():
    """Offloaded rows replace host rows, and the hot row of a token that sits in a slot; rows outside the pool
    are skipped with the bad-id bit. Afterwards every slot still holds its token's host row and a gather
    returns the new rows."""
    w = workload.SINGLE_4K.with_(num_requests=2, steps=12)
    ids = workload.streams(w)
    host = make_host(2, w.host_rows, 32)
    o = oracle.Oracle(2, w.buffer_slots, w.top_k, w.host_rows, 32, host=host)
    for t in range(6):
        o.step(ids[:, t])
    n = 300
    rows = np.empty((2, n, 32), np.uint8)
    workload.fill_rows(rows.view(np.uint16).reshape(2 * n, 16), 0, 2 * n, 16, 99)
    pos = np.array([w.host_rows - 200, 1000], np.int32)  # request 0 runs past the end of its pool
    in_slots = [int((o.page[1][1000:1300] >= 0).sum())]
    assert in_slots[0] > 0
    st = o.offload(rows, pos)
    assert st.tolist() == [oracle.BAD_ID, 0]
    assert (o.host[0][w.host_rows - 200:] == rows[0][:200]).all()
    assert (o.host[1][1000:1300] == rows[1]).all()
    for r in range(2):
        occ = np.nonzero(o.slot_tok[r] >= 0)[0]
        assert (o.hot[r][occ] == o.host[r][o.slot_tok[r][occ]]).all()
    for t in range(6, 12):
        out, miss, status, g = o.step(ids[:, t], gather=True)
        for r in range(2):
            check_invariants(o, r, ids[r, t].tolist(), out[r].tolist(), miss[r], status[r], None, g[r])


def test_advance_tail_moves_rows_to_host():
    """Advancing the tail window: the leaving tokens' ring rows become their host rows, tail0 moves, and those
    tokens then resolve through the hot buffer (a miss fetches the former tail row)."""
    w = workload.HYBRID_64.with_(num_requests=2, steps=10, L0=3000, host_rows=3000, tail_tokens=400, top_k=64,
                                 buffer_slots=128)
    ids = workload.streams(w)
    rb = 32
    host = make_host(2, w.host_rows, rb)
    tail0 = np.full(2, w.tail0, np.int32)
    tail = np.zeros((2, w.tail_tokens, rb), np.uint8)
    workload.fill_rows(tail.view(np.uint16).reshape(2 * w.tail_tokens, rb // 2), 0, 2 * w.tail_tokens, rb // 2, 77)
    o = oracle.Oracle(2, w.buffer_slots, w.top_k, w.host_rows, rb, T=w.tail_tokens, host=host, tail=tail)
    for t in range(4):
        o.step(ids[:, t], tail0)
    old_tail0 = tail0.copy()
    before = o.tail.copy()
    st = o.advance_tail(tail0, np.array([50, 500], np.int32))  # the second clamps to T = 400
    assert st.tolist() == [0, 0]
    assert tail0.tolist() == [old_tail0[0] + 50, old_tail0[1] + 400]
    for r, n in ((0, 50), (1, 400)):
        for x in range(old_tail0[r], old_tail0[r] + n):
            assert (o.host[r][x] == before[r][x % w.tail_tokens]).all()
    # a token that just left the tail is now a miss whose row comes from the host (the former tail row)
    x = int(old_tail0[0])
    sel = np.array([[x] + list(range(1, w.top_k)), list(range(w.top_k))], np.int32)
    out, miss, status, g = o.step(sel, tail0, gather=True)
    assert 0 <= out[0][0] < w.buffer_slots and (g[0][0] == before[0][x % w.tail_tokens]).all()
    for r in range(2):
        check_invariants(o, r, sel[r].tolist(), out[r].tolist(), miss[r], status[r], int(tail0[r]), g[r])
