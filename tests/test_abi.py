"""The C ABI without a GPU: the library loads, exports what include/hisparse.h declares, and rejects bad
configurations with an error code and a message before touching the device."""
import ctypes
import json
import os
import re

import pytest

import hierarchical_memory_amd as hm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def declared_functions():
    src = open(os.path.join(ROOT, "include", "hisparse.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|void|const char\*)\s+(hs_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 9
    lib = ctypes.CDLL(hm.library_path())
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(hm.EXPORTED)


@pytest.mark.parametrize("kw,msg", [
    (dict(num_requests=0), "num_requests"),
    (dict(top_k=0), "top_k"),
    (dict(top_k=9000, device_buffer_size=9000), "top_k"),
    (dict(device_buffer_size=100), "device_buffer_size"),
    (dict(device_buffer_size=70000), "device_buffer_size"),
    (dict(row_bytes=1000), "row_bytes"),
    (dict(row_bytes=0), "row_bytes"),
    (dict(host_to_device_ratio=0.0), "host_to_device_ratio"),
    (dict(host_to_device_ratio=-1.0), "host_to_device_ratio"),
    (dict(tail_tokens=-1), "tail_tokens"),
    (dict(max_context=-5), "max_context"),
    (dict(device_buffer_size=40000, max_context=1 << 20), "LDS"),
    (dict(eviction_policy=2), "eviction_policy"),
    # R x H x row_bytes ~ 2^67 would wrap a 64-bit size
    (dict(num_requests=65535, top_k=8, device_buffer_size=8, max_context=2**31 - 1, row_bytes=1 << 20), "host pool"),
    (dict(num_requests=65535, top_k=8, device_buffer_size=8, max_context=1 << 24, row_bytes=1 << 20), "host pool"),
])
def test_bad_config_rejected(kw, msg):
    base = dict(num_requests=4, top_k=256, device_buffer_size=512, host_to_device_ratio=8.0, row_bytes=1152,
                max_context=0, tail_tokens=0, eviction_policy=0)
    base.update(kw)
    cfg = hm.HsConfig(**base)
    with pytest.raises(hm.HiSparseError) as e:
        hm.hs_required_sizes(cfg)
    assert e.value.code == hm.HS_E_INVALID and msg in str(e.value)
    with pytest.raises(hm.HiSparseError):
        hm.hs_create(cfg)  # fails in the same host-side check, before any HIP call


def test_null_arguments():
    lib = hm.lib()
    assert lib.hs_required_sizes(None, None) == hm.HS_E_INVALID
    assert lib.hs_create(None, None) == hm.HS_E_INVALID
    assert lib.hs_resolve(None, None, None, None, None, None, None, None) == hm.HS_E_INVALID
    assert lib.hs_reset(None, None, -1, None) == hm.HS_E_INVALID
    assert lib.hs_gather(None, None, None, None) == hm.HS_E_INVALID
    assert lib.hs_bind_device(None, None) == hm.HS_E_INVALID
    assert "NULL" in hm.hs_last_error()
    lib.hs_destroy(None)


def test_launch_configs_from_the_pages():
    lines = [l for l in open(os.path.join(GOLDEN, "hisparse_launch_configs.txt")) if l.startswith("{")]
    got = []
    for l in lines:
        cfg = hm.config_from_hisparse_json(l.strip(), num_requests=32)
        s = hm.hs_required_sizes(cfg)
        got.append((cfg.top_k, cfg.device_buffer_size, s.host_rows))
    # host rows = ratio x buffer slots
    assert got == [(2048, 6144, 61440), (2048, 4096, 32768)]
    with pytest.raises(ValueError):
        hm.config_from_hisparse_json('{"top_k": 1, "device_buffer": 2}', 1)


def test_sizes_of_the_workloads():
    import workload
    for w in workload.ALL:
        s = hm.hs_required_sizes(hm.config(w.num_requests, w.top_k, w.buffer_slots, 0.0, w.row_bytes, w.host_rows,
                                           w.tail_tokens))
        assert s.host_rows == w.host_rows
        assert s.host_pool_bytes == w.num_requests * w.host_rows * w.row_bytes
        assert s.lds_bytes <= 159 * 1024
        assert s.hot_bytes == w.num_requests * w.buffer_slots * w.row_bytes


MISC = 4 * (8 * 16 + 8)  # the scan and flag words every layout carries


def _words(H):
    return (H + 31) // 32


def test_lds_layout_takes_the_missed_token_array_where_it_fits():
    """The rank layout needs about 21k + 7B + 10 ceil(H/32) bytes of LDS; the missed tokens get 4k bytes of their
    own only while the total stays within 159 KiB (near the limit they share the rank-to-slot table)."""
    def base(k, B, H):
        return 21 * k + 7 * B + 10 * _words(H) + MISC

    def lds(k, B, H):
        return hm.hs_required_sizes(hm.config(2, k, B, 0.0, 1152, H)).lds_bytes_rank

    for k, B, H in ((2048, 4096, 40960), (2048, 4096, 131072), (256, 512, 4096), (2048, 8192, 131072),
                    (2048, 4096, 262144)):
        extra = lds(k, B, H) - base(k, B, H)
        assert 4 * k <= extra <= 4 * k + 256, (k, B, H, extra)
        assert lds(k, B, H) <= 159 * 1024
    for k, B, H in ((2048, 8192, 180000), (4096, 4096, 150000)):
        extra = lds(k, B, H) - base(k, B, H)
        assert 0 <= extra <= 256, (k, B, H, extra)
        assert lds(k, B, H) + 4 * k > 159 * 1024


def test_context_length_limits_of_the_rank_layouts():
    """At k = 2048 and B = 4096 the flat rank layout holds about 290,000 host rows per request (262,144 take
    it). Past that the two-level layout takes over: its bitmaps run over at most k compact words, plus a coarse
    bitmap of one bit per 32 host rows and its uint16 prefix counts, up to about 10.5 million host rows; past
    159 KiB the shape is refused."""
    def req(H):
        return hm.hs_required_sizes(hm.config(2, 2048, 4096, 0.0, 64, H))
    ok = req(262144)
    assert ok.lds_bytes <= 159 * 1024 and ok.token_slot_table == 0 and ok.sparse_rank == 0
    limit = 159 * 1024 - (21 * 2048 + 7 * 4096 + MISC)
    h_max = (limit // 10) * 32
    assert 280000 < h_max < 300000
    assert req(h_max - 4096).sparse_rank == 0
    for H in (h_max + 32 * 64, 1 << 20, 3_000_000):
        s = req(H)
        wc = -(-H // 1024)  # coarse words
        base = 39 * 2048 + 7 * 4096 + 6 * wc + MISC
        assert s.sparse_rank == 1 and s.token_slot_table == 0
        assert 0 <= s.lds_bytes - base <= 256 and s.lds_bytes <= 159 * 1024, (H, s.lds_bytes, base)
    # near the limit the missed tokens share the rank -> slot table (4k bytes fewer)
    wc_max = (159 * 1024 - (35 * 2048 + 7 * 4096 + MISC)) // 6
    assert 10_000_000 < wc_max * 1024 < 11_000_000
    assert req(wc_max * 1024 - 64 * 1024).sparse_rank == 1
    with pytest.raises(hm.HiSparseError) as err:
        req(wc_max * 1024 + 64 * 1024)
    assert err.value.code == hm.HS_E_INVALID and "LDS" in str(err.value)


def test_binding_refuses_host_tensors():
    """Per-call buffers must be GPU tensors: a CPU tensor is refused before anything reaches the library."""
    import torch
    cpu = torch.zeros(8, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        hm.hs_resolve(None, cpu, None, cpu, cpu, cpu)
    with pytest.raises(ValueError, match="GPU tensor"):
        hm.hs_gather(None, cpu, cpu)


def test_build_script_loads_without_the_built_library():
    """build() must work on a fresh checkout: loading the build script may not import the package, whose import
    needs the library that the script is about to build."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys, os, __graft_entry__ as g; "
            "m = g._load_by_path('_hs_build', os.path.join(g.ROOT, 'hierarchical_memory_amd', 'build.py')); "
            "assert callable(m.build); "
            "assert 'hierarchical_memory_amd' not in sys.modules, 'the package was imported'")
    res = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_token_slot_table_where_it_fits():
    """Launches take the direct layout (a uint16 token -> slot entry per host row) where it fits in 159 KiB and
    B <= 8192: about 8k + 5B + T/8 + 6 ceil(H/32) + max(2H, 6 ceil(H/32) + 4k, 4k + 2B) bytes, 4k more with a
    gather output; elsewhere the rank layout."""
    cap = 159 * 1024
    # (k, B, H, T, expected bits): 256-request, 32-request and single-request shapes both ways, hybrid and sweep
    # shapes neither, a buffer past the direct kernel's 8192 slots neither
    cases = ((2048, 4096, 40960, 0, 3), (2048, 4096, 33024, 0, 3), (256, 512, 4096, 0, 3), (2048, 4096, 131072, 8192, 0),
             (2048, 2048, 65536, 0, 0), (2048, 6144, 65536, 0, 0), (64, 9000, 4096, 0, 0), (2048, 8192, 8192, 100, 3))
    for k, B, H, T, bits in cases:
        s = hm.hs_required_sizes(hm.config(2, k, B, 0.0, 1152, H, T))
        assert s.token_slot_table == bits, (k, B, H, s.token_slot_table)
        W = _words(H)
        for bit, got, extra in ((1, s.lds_bytes_launch, 0), (2, s.lds_bytes_launch_gather, 4 * k)):
            if bits & bit:
                region = max(2 * H, 6 * W + 4 * k, 4 * k + 2 * B)  # table, repeat arrays, staged lists
                est = 8 * k + 4 * B + 4 * ((B + 3) // 4) + 6 * W + 4 * ((T + 31) // 32) + MISC + region + extra
                assert est <= got <= est + 256 and got <= cap, (k, B, H, bit, got, est)
            else:
                assert got == s.lds_bytes_rank, (k, B, H, bit, got, s.lds_bytes_rank)
        assert s.lds_bytes == max(s.lds_bytes_launch, s.lds_bytes_launch_gather)


@pytest.fixture()
def fake_ctx():
    """A context key registered with the sizes of a real configuration (host-only), so the binding's argument
    checks run; no call below gets past them to the library."""
    cfg = hm.config(3, 8, 16, 0.0, 64, 100, 4)
    key = 0x5EED0000
    hm.hisparse._register(key, cfg, hm.hs_required_sizes(cfg))
    yield ctypes.c_void_p(key)
    hm.hisparse._CTX_SIZES.pop(key, None)


def _i32(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.int32)


def test_binding_checks_dtype_and_size(fake_ctx):
    """Every per-call tensor is checked for dtype and size against the context before its pointer is taken: an
    int64 id list, a short output, a gather output of too few bytes, a 2-D offload row block are refused with a
    message that names the argument; a well-formed CPU tensor gets as far as the device check."""
    import torch
    ctx = fake_ctx
    R, k, rb = 3, 8, 64
    good = dict(topk=_i32(R, k), tail0=_i32(R), out=_i32(R, k), miss=_i32(R), status=_i32(R))
    cases = [
        (hm.hs_resolve, dict(good, topk=torch.zeros((R, k), dtype=torch.int64)), "topk must be a torch.int32"),
        (hm.hs_resolve, dict(good, out=_i32(R, k - 1)), "out has 21 elements"),
        (hm.hs_resolve, dict(good, miss=_i32(R - 1)), "miss has 2 elements"),
        (hm.hs_resolve, dict(good, tail0=torch.zeros(R, dtype=torch.int64)), "tail0 must be a torch.int32"),
        (hm.hs_resolve, dict(good, gather=torch.zeros((R, k, rb - 1), dtype=torch.uint8)), "gather has"),
        (hm.hs_plan, dict(good, plan=_i32(R, 3, k)), "plan has 72 elements"),
        (hm.hs_trial, dict(good, gather=torch.zeros((R, k, rb), dtype=torch.uint8), trial=_i32(4)), "trial has"),
        (hm.hs_trial, dict(good, gather=None, trial=_i32(1 << 16)), "gather must not be None"),
        (hm.hs_step_static, dict(good, status=torch.zeros(R, dtype=torch.float32)), "status must be a torch.int32"),
    ]
    for fn, kw, msg in cases:
        with pytest.raises(ValueError, match=msg):
            fn(ctx, **kw)
    with pytest.raises(ValueError, match="plan has"):
        hm.hs_copy(ctx, _i32(R, 2, k), _i32(R))
    with pytest.raises(ValueError, match="gather has"):
        hm.hs_gather(ctx, _i32(R, k), torch.zeros(10, dtype=torch.uint8))
    with pytest.raises(ValueError, match="accept has"):
        hm.hs_commit(ctx, _i32(1 << 16), torch.zeros((R, k, rb), dtype=torch.uint8), accept=_i32(1))
    with pytest.raises(ValueError, match="3 dimensions"):
        hm.hs_offload(ctx, torch.zeros((R, 2 * rb), dtype=torch.uint8), _i32(R))
    with pytest.raises(ValueError, match="rows must be"):
        hm.hs_offload(ctx, torch.zeros((R, 2, rb // 2), dtype=torch.uint8), _i32(R))
    with pytest.raises(ValueError, match="n must be a torch.int32"):
        hm.hs_advance_tail(ctx, _i32(R), torch.zeros(R, dtype=torch.int64))
    with pytest.raises(ValueError, match="request_ids must be a torch.int32"):
        hm.hs_reset(ctx, torch.zeros(2, dtype=torch.int64))
    # well-formed arguments on the CPU: refused only because they are not GPU tensors
    with pytest.raises(ValueError, match="GPU tensor"):
        hm.hs_resolve(ctx, **good)
    with pytest.raises(ValueError, match="GPU tensor"):
        hm.hs_offload(ctx, torch.zeros((R, 2, rb), dtype=torch.uint8), _i32(R))


def test_state_snapshot_sizes():
    """hs_export_state / hs_import_state lay the selected buffers out at 256-byte aligned offsets: tables (slot
    table, stamps, order list, page table, step counters) and rows (hot, tail)."""
    cfg = hm.config(3, 8, 16, 0.0, 64, 100, 4)
    s = hm.hs_required_sizes(cfg)
    a256 = lambda b: (b + 255) // 256 * 256  # noqa: E731
    assert s.state_tables_bytes == sum(a256(b) for b in (3 * 16 * 4, 3 * 16 * 4, 3 * 16 * 2, 3 * 100 * 4, 3 * 4))
    assert s.state_rows_bytes == a256(3 * 16 * 64) + a256(3 * 4 * 64)
    assert s.epoch_bytes == 3 * 4
    lib = hm.lib()
    assert lib.hs_export_state(None, None, 0, 1, None) == hm.HS_E_INVALID
    assert lib.hs_import_state(None, None, 0, 1, None) == hm.HS_E_INVALID
