"""The seeded input generator: the C generator equals its pure-Python twin, and its streams have the shape
the workloads describe (k distinct ids per step, the kept share of the previous step, the forced current
token, the refill ranges)."""
import numpy as np
import pytest

import workload


SMALL = [workload.SINGLE_4K,
         workload.GROW_32.with_(L0=3000, top_k=200, window=300, host_rows=3100),
         workload.SWEEP_BASE.with_(L0=5000, host_rows=5000, top_k=300, keep_permille=950),
         workload.HYBRID_64.with_(L0=20000, host_rows=20000, tail_tokens=1000, top_k=300)]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_c_matches_python_twin(w):
    assert (workload.streams(w, n_steps=8, requests=3) == workload.streams_py(w, 8, 3)).all()


@pytest.mark.parametrize("w", workload.ALL, ids=lambda w: w.name)
def test_stream_shape(w):
    n_steps = min(w.steps, 40)
    s = workload.streams(w, n_steps=n_steps, requests=min(w.num_requests, 4))
    k = w.top_k
    keep = w.keep_permille * k // 1000
    for r in range(s.shape[0]):
        for t in range(n_steps):
            ids = s[r, t]
            L = w.L0 + (t if w.grow else 0)
            assert len(set(ids.tolist())) == k and ids.min() >= 0 and ids.max() < L <= w.host_rows
            if w.grow:
                assert L - 1 in ids
            if t:
                prev = set(s[r, t - 1].tolist())
                new = [x for x in ids.tolist() if x not in prev]
                # a refill draw may land on an id the previous step had but did not keep
                assert k - len(new) >= keep
                n_new = k - keep - (1 if w.grow else 0)
                nB = w.partB_permille * n_new // 1000
                if w.tail_tokens:
                    assert sum(1 for x in new if x >= w.tail0) <= nB
                    assert sum(1 for x in new if x < w.tail0) <= n_new - nB


def test_rows_deterministic_and_normal():
    a = np.empty((300, 576), np.uint16)
    workload.fill_rows(a, 0, 300, 576, 11)
    b = np.empty((100, 576), np.uint16)
    workload.fill_rows(b, 200, 100, 576, 11)
    assert (a[200:] == b).all()
    f = (a.astype(np.uint32) << 16).view(np.float32)
    assert abs(f.mean()) < 0.02 and abs(f.std() - 1) < 0.02
    assert len({r.tobytes() for r in a}) == 300
