"""hs_step_static (the split step with its plan in the library's static device array, for callers that cannot
allocate) against the split step it stands for, hs_plan + hs_copy with a plan buffer: outputs, gathered rows and
the whole state bit for bit, on two shapes called one after the other (the second smaller, so its plan only
partly overwrites what the first left in the shared array), and a context whose plan is too large is refused."""
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


def _twin(hm, w):
    cfg = hm.config(w.num_requests, w.top_k, w.buffer_slots, 0.0, w.row_bytes, w.host_rows, w.tail_tokens)
    sw = hm.SwapIn(cfg)
    workload.fill_rows_ptr(sw.host_pool_address(), 0, w.num_requests * w.host_rows, w.row_elems, w.row_seed)
    if w.tail_tokens:
        pool = sw.host_pool()
        ring = np.arange(w.tail0, w.tail0 + w.tail_tokens) % w.tail_tokens
        rows = np.empty((w.num_requests, w.tail_tokens, w.row_bytes), np.uint8)
        rows[:, ring] = pool[:, w.tail0:w.tail0 + w.tail_tokens]
        sw.tail.copy_(torch.from_numpy(rows))
    return sw


def _state(sw):
    return [sw.slot_tok, sw.stamp, sw.lru_order, sw.page, sw.step, sw.hot]


@pytest.mark.parametrize("order", ["large_then_small"])
def test_static_step_matches_plan_and_copy(order):
    import hierarchical_memory_amd as hm
    large = workload.GROW_32.with_(name="static_large", num_requests=6, steps=10)
    small = workload.HYBRID_64.with_(name="static_small", num_requests=3, top_k=512, buffer_slots=1024,
                                     host_rows=8192, L0=8192, tail_tokens=1024, steps=10)
    for w, gather in ((large, False), (small, True)):
        ref, dut = _twin(hm, w), _twin(hm, w)
        assert w.num_requests * 4 * w.top_k * 4 <= hm.HS_STATIC_PLAN_BYTES
        ids = workload.streams(w)
        tail0 = torch.full((w.num_requests,), w.tail0, dtype=torch.int32, device="cuda") if w.tail_tokens else None
        ro, do_ = ref.outputs(gather), dut.outputs(gather)
        plan = ref.plan_buffer()
        for t in range(w.steps):
            topk = torch.from_numpy(np.ascontiguousarray(ids[:, t])).cuda()
            hm.hs_plan(ref.ctx, topk, tail0, ro[0], ro[1], ro[2], plan, row_sources=gather)
            hm.hs_copy(ref.ctx, plan, ro[1], ro[3])
            hm.hs_step_static(dut.ctx, topk, tail0, do_[0], do_[1], do_[2], do_[3])
            torch.cuda.synchronize()
            for a, b in zip(ro, do_):
                if a is not None:
                    assert torch.equal(a, b), f"{w.name} step {t}: outputs differ"
            for a, b in zip(_state(ref), _state(dut)):
                assert torch.equal(a, b), f"{w.name} step {t}: state differs"
        assert int(do_[1].sum().item()) > 0, "no misses: the copy was not exercised"
        ref.close()
        dut.close()


def test_static_step_refuses_a_plan_past_the_array():
    import hierarchical_memory_amd as hm
    R, k = 300, 2048  # plan 300 x 4 x 2048 x 4 bytes, past 8 MiB
    assert R * 4 * k * 4 > hm.HS_STATIC_PLAN_BYTES
    sw = hm.SwapIn(hm.config(R, k, k, 0.0, 16, 4096))
    out, miss, status, _ = sw.outputs()
    topk = torch.zeros((R, k), dtype=torch.int32, device="cuda")
    with pytest.raises(hm.HiSparseError) as err:
        hm.hs_step_static(sw.ctx, topk, None, out, miss, status)
    assert err.value.code == hm.HS_E_INVALID and "static plan" in str(err.value)
    sw.close()
