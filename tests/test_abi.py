"""The C-ABI library loads on any host and exports every entry point that
include/csahca.h declares (no device work)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csahca.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ca_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("ca_compress_prefill", "ca_compress_decode", "ca_index_topk_prefill", "ca_index_topk_decode",
                 "ca_csa_attend_prefill", "ca_csa_attend_decode", "ca_hca_attend_prefill", "ca_hca_attend_decode",
                 "ca_window_append", "ca_store_entries"):
        assert want in names


def test_library_exports_every_declared_symbol():
    from long_context_attention_17_amd import binding
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(binding.EXPORTED)


def test_host_helpers_match_the_record_layout():
    import oracle
    from long_context_attention_17_amd import binding as ca
    for fmt in (ca.F32, ca.BF16, ca.FP8MIX, ca.E4M3, ca.FP4):
        for D, R in ((512, 64), (64, 8), (64, 0), (32, 0), (128, 0)):
            if fmt == ca.FP8MIX and (D - R) % 64:
                continue
            if fmt in (ca.E4M3, ca.FP4) and R:
                continue
            assert ca.record_stride(fmt, D, R) == oracle.record_stride(fmt, D, R)
            assert ca.page_bytes(fmt, D, R, 64) == oracle.page_bytes(fmt, D, R, 64)
    assert ca.record_stride(ca.FP8MIX, 512, 64) == 640
    assert ca.page_bytes(ca.E4M3, 64, 0, 64) == 4352
    assert ca.page_bytes(ca.FP4, 64, 0, 64) == 64 * (32 + 2) and ca.page_bytes(ca.FP4, 48, 0, 64) == -1
    assert ca.record_stride(9, 512, 64) == -1


def test_argument_errors_are_reported_without_launching():
    """Validation happens on the host before any launch, so these need no GPU."""
    from long_context_attention_17_amd import binding as ca
    lib = ca.lib()
    p = ca.CompressParams(0, 1, ca.BF16, 1, 1, 1e-6, 1e4)
    rc = lib.ca_compress_prefill(ctypes.byref(p), None, None, None, None, None, None, None, 16, 0, 0, None, None)
    assert rc == -1 and b"cache descriptor is NULL" in lib.ca_last_error()
    cache = ca._Cache(ca.FP8MIX, 500, 64, 64, None, 0, None, 0, 0)
    rc = lib.ca_store_entries(ctypes.byref(cache), 0, 0, 0, None, None, 1e-6, 1, 1e4, 1, None)
    assert rc == -3 and b"fp8-mixed" in lib.ca_last_error()
    cache = ca._Cache(ca.BF16, 512, 64, 48, None, 0, None, 0, 0)
    rc = lib.ca_store_entries(ctypes.byref(cache), 0, 0, 0, None, None, 1e-6, 1, 1e4, 1, None)
    assert rc == -1 and b"power of two" in lib.ca_last_error()
    ip = ca.IndexParams(8, 64, 4, 0, ca.BF16)
    cache = ca._Cache(ca.E4M3, 64, 0, 64, None, 0, None, 0, 0)
    rc = lib.ca_index_topk_decode(ctypes.byref(ip), None, None, None, 0, 0, ctypes.byref(cache), None, None, None,
                                  None, 0, None, 0, None)
    assert rc == -1                      # k must be positive
    ip = ca.IndexParams(8, 64, 4, 16, ca.BF16, ca.FP4)
    rc = lib.ca_index_topk_decode(ctypes.byref(ip), None, None, None, 0, 0, ctypes.byref(cache), None, None, None,
                                  None, 0, None, 0, None)
    assert rc == -1 and b"q_quant" in lib.ca_last_error()   # FP4 queries need an FP4 pool
    wp = ca.WindowParams(512, 64, ca.BF16, ca.BF16, 1e-6, 1e4)
    rc = lib.ca_decode_append(ctypes.byref(wp), None, None, None, 0, None, 128, 1, None, 0, None)
    assert rc == -1 and b"n_jobs" in lib.ca_last_error()
    job = ca.DecodeEntryJob(ca.CompressParams(4, 1, ca.BF16, 1, 1, 1e-6, 1e4), None, None, None, None, None,
                            ctypes.pointer(ca._Cache(ca.FP8MIX, 512, 64, 64, None, 0, None, 8, 0)))
    rc = lib.ca_decode_append(ctypes.byref(wp), None, None, None, 8, None, 128, 8, ctypes.byref(job), 1, None)
    assert rc == -1 and b"NULL" in lib.ca_last_error()      # missing rows / ring
    assert lib.ca_decode_append(ctypes.byref(wp), None, None, None, 0, None, 128, 1, ctypes.byref(job), 1, None) == 0
    # one-call decode steps: the checks of the calls they combine, before any launch
    jobs = (ca.DecodeEntryJob * 2)(job, job)
    ip = ca.IndexParams(8, 64, 8, 16, ca.BF16, 0)                          # ratio 8 vs the jobs' 4
    ap = ca.AttendParams(64, 512, 64, 128, ca.BF16, ca.BF16, ca.BF16, 0.04, 1e-6, 1e4)
    rc = lib.ca_csa_decode_step(ctypes.byref(wp), None, None, None, 128, 8, jobs, ctypes.byref(ip), None, None, None,
                                None, None, 0, ctypes.byref(ap), None, None, None, 0, 0, None, None, None, None, 0, None)
    assert rc == -1 and b"ratios differ" in lib.ca_last_error()
    rc = lib.ca_hca_decode_step(ctypes.byref(wp), None, None, None, 128, 8, jobs, None, None, None, None, 0, 0,
                                None, None, None, None, 0, None)
    assert rc == -1 and b"params NULL" in lib.ca_last_error()
    assert lib.ca_hca_decode_step(ctypes.byref(wp), None, None, None, 128, 8, jobs, ctypes.byref(ap), None, None,
                                  None, 0, 0, None, None, None, None, 0, None) == 0          # B = 0: nothing to do
    ap = ca.AttendParams(64, 512, 64, 128, ca.BF16, ca.BF16, ca.BF16, 0.04, 1e-6, 1e4)
    cache = ca._Cache(ca.E4M3, 512, 0, 64, None, 0, None, 0, 0)
    rc = lib.ca_hca_attend_decode(ctypes.byref(ap), None, None, ctypes.byref(cache), 128, None, 1, 0, None, 1, None,
                                  None, None, None, 0, None)
    assert rc == -2                      # indexer pools cannot be attended
    # empty inputs are valid no-ops
    cache = ca._Cache(ca.BF16, 512, 64, 64, None, 0, None, 1, 0)
    p = ca.CompressParams(4, 1, ca.BF16, 1, 1, 1e-6, 1e4)
    assert lib.ca_compress_prefill(ctypes.byref(p), None, None, None, None, None, None, None, 3, 0, 0,
                                   ctypes.byref(cache), None) == 0
    # a continuation whose rows complete no new entry is a valid no-op too
    assert lib.ca_compress_prefill(ctypes.byref(p), None, None, None, None, None, None, None, 3, 5, 0,
                                   ctypes.byref(cache), None) == 0
    assert lib.ca_compress_prefill(ctypes.byref(p), None, None, None, None, None, None, None, 3, -1, 0,
                                   ctypes.byref(cache), None) == -1


def test_timer_argument_errors_need_no_device():
    """The launch timer rejects bad arguments before it creates any HIP event."""
    from long_context_attention_17_amd import binding as ca
    lib = ca.lib()
    assert lib.ca_timer_start(1 << 4, 16) == -1           # unknown kernel bit
    assert lib.ca_timer_start(1, 0) == -1                 # no launches to time
    assert lib.ca_timer_start(1, (1 << 20) + 1) == -1     # above the launch cap
    ms, n = ctypes.c_double(-1.0), ctypes.c_int64(-1)
    assert lib.ca_timer_read(-1, ctypes.byref(ms), ctypes.byref(n)) == -1
    assert lib.ca_timer_read(ca.TIMED_PROJ_GEMM + 1, ctypes.byref(ms), ctypes.byref(n)) == -1
    assert lib.ca_timer_read(ca.TIMED_HCA_ATTEND, None, ctypes.byref(n)) == -1
    # nothing was timed: reading reports zero launches without touching the device
    assert lib.ca_timer_read(ca.TIMED_HCA_ATTEND, ctypes.byref(ms), ctypes.byref(n)) == 0
    assert (ms.value, n.value) == (0.0, 0)
    assert lib.ca_timer_stop() == 0


def test_fp4_queries_need_fp4_keys():
    from long_context_attention_17_amd.configs import CONFIGS
    import dataclasses
    cfg = dataclasses.replace(CONFIGS[5], idx="fp4", idx_q="fp4")
    assert cfg.idx_q == "fp4"
    with pytest.raises(ValueError):
        dataclasses.replace(CONFIGS[5], idx_q="fp4")          # e4m3 keys
    with pytest.raises(ValueError):
        dataclasses.replace(CONFIGS[5], idx="fp4", idx_q="bf16")


def test_decode_split_plan_depends_on_the_row_alone():
    """The decode attention's split plan: chunks never exceed one workgroup's item table
    (2,176 items), are whole 64-item tiles, cover the row exactly, and never outnumber what
    the workspace holds for a row of at most max_items items -- for every row length,
    including rows longer than 16 x 2,176 items (the plan takes only the row's length)."""
    from long_context_attention_17_amd import binding as ca
    ap = ca.AttendParams(128, 512, 64, 128, ca.BF16, ca.BF16, ca.BF16, 0.04, 1e-6, 1e4)
    totals = list(range(0, 5000)) + list(range(5000, 300000, 97)) + [34816, 34817, 34816 * 2 + 1, 262144 + 128]
    for max_items in (129, 2176, 8320, 34816, 40000, 262272):
        _, _, ms = ca.attend_decode_plan(ap, max_items)
        for total in totals:
            if total > max_items:
                continue
            ln, n, _ = ca.attend_decode_plan(ap, total)
            assert ln <= 2176 and ln % 64 == 0 and ln >= 256, (total, ln)
            assert n >= 1 and n * ln >= total and (n - 1) * ln < max(total, 1), (total, ln, n)
            assert n <= ms, (total, max_items, n, ms)
    # rows up to 16 chunks of the 256-item minimum stay at 16 chunks; longer rows get more
    assert ca.attend_decode_plan(ap, 8320)[:2] == (576, 15)
    assert ca.attend_decode_plan(ap, 2176)[:2] == (256, 9)
    assert ca.attend_decode_plan(ap, 40000)[1] == 19
    with pytest.raises(ca.CAError):
        ca.attend_decode_plan(ap, -1)


def test_decode_window_ring_must_hold_the_window():
    """A decode ring of fewer than n_win slots would alias window positions."""
    from long_context_attention_17_amd import binding as ca
    lib = ca.lib()
    ap = ca.AttendParams(64, 512, 64, 128, ca.BF16, ca.BF16, ca.BF16, 0.04, 1e-6, 1e4)
    cache = ca._Cache(ca.FP8MIX, 512, 64, 64, ctypes.c_void_p(16), 1, ctypes.c_void_p(16), 4, 4)
    dummy = ctypes.c_void_p(16)
    rc = lib.ca_hca_attend_decode(ctypes.byref(ap), dummy, dummy, ctypes.byref(cache), 128, dummy, 1, 1000, dummy,
                                  64, dummy, dummy, None, dummy, 1 << 30, None)
    assert rc == -1 and b"n_win" in lib.ca_last_error()
    wp = ca.WindowParams(512, 64, ca.BF16, ca.BF16, 1e-6, 1e4)
    job = ca.DecodeEntryJob(ca.CompressParams(128, 0, ca.BF16, 1, 1, 1e-6, 1e4), dummy, dummy, dummy, None, dummy,
                            ctypes.pointer(cache))
    rc = lib.ca_hca_decode_step(ctypes.byref(wp), dummy, dummy, dummy, 64, 1, ctypes.byref(job), ctypes.byref(ap),
                                dummy, dummy, dummy, 1, 1000, dummy, dummy, None, dummy, 1 << 30, None)
    assert rc == -1 and b"n_win" in lib.ca_last_error()


def test_no_alloc_step_rejects_a_step_beyond_its_scratch():
    """The allocation-free HCA step refuses, before any device work, a step whose attention
    workspace would exceed the library's static scratch."""
    from long_context_attention_17_amd import binding as ca
    lib = ca.lib()
    cap = lib.ca_static_scratch_bytes()
    assert cap == 64 << 20
    ap = ca.AttendParams(128, 512, 64, 128, ca.BF16, ca.BF16, ca.BF16, 0.04, 1e-6, 1e4)
    assert ca.attend_workspace(ap, 64, 1 << 22, 0, 128) > cap
    wp = ca.WindowParams(512, 64, ca.BF16, ca.BF16, 1e-6, 1e4)
    cache = ca._Cache(ca.FP8MIX, 512, 64, 64, ctypes.c_void_p(16), 1, ctypes.c_void_p(16), 64, 1 << 16)
    d = ctypes.c_void_p(16)
    job = ca.DecodeEntryJob(ca.CompressParams(128, 0, ca.BF16, 1, 1, 1e-6, 1e4), d, d, d, None, d,
                            ctypes.pointer(cache))
    rc = lib.ca_hca_decode_step_noalloc(ctypes.byref(wp), d, d, d, 128, 64, ctypes.byref(job), ctypes.byref(ap), d, d,
                                        d, 64, 1 << 22, d, d, None, None)
    assert rc == -4 and b"static scratch" in lib.ca_last_error()


def test_decode_state_sizes_and_errors():
    """ca_state_bytes: the window row, each tail ring and the whole pages holding pos/ratio
    entries of each cache, every part 256-byte aligned; bad arguments are refused on the host."""
    from long_context_attention_17_amd import binding as ca
    lib = ca.lib()
    d = 256                                                # an aligned non-null stand-in address
    st = ca.DecodeState()
    st.window, st.W, st.S, st.win_dim, st.win_format, st.n_jobs = d, 128, 4, 512, ca.BF16, 2
    c0 = ca._Cache(ca.FP8MIX, 512, 64, 64, ctypes.c_void_p(d), 100, ctypes.c_void_p(d), 4, 50)
    c1 = ca._Cache(ca.E4M3, 64, 0, 64, ctypes.c_void_p(d), 100, ctypes.c_void_p(d), 4, 50)
    st.tail[0], st.tail[1] = d, d
    st.tail_floats[0], st.tail_floats[1] = 8 * 4 * 512, 8 * 4 * 64
    st.cache[0], st.cache[1] = ctypes.pointer(c0), ctypes.pointer(c1)
    st.ratio[0], st.ratio[1] = 4, 4
    pos = 1001                                             # 250 entries: 4 pages of 64
    want = 128 * 512 * 2 + 8 * 4 * 512 * 4 + 8 * 4 * 64 * 4 + 4 * 64 * 640 + 4 * (64 * 64 + 64 * 4)
    assert ca.state_bytes(st, pos) == want
    assert ca.state_bytes(st, 0) == 128 * 512 * 2 + 8 * 4 * 512 * 4 + 8 * 4 * 64 * 4
    assert lib.ca_state_bytes(ctypes.byref(st), 64 * 50 * 4 + 4) == -1     # more pages than the table holds
    assert b"beyond the page table" in lib.ca_last_error()
    rc = lib.ca_state_save(ctypes.byref(st), 4, pos, ctypes.c_void_p(d), want, None)
    assert rc == -1 and b"seq 4" in lib.ca_last_error()
    rc = lib.ca_state_save(ctypes.byref(st), 0, pos, ctypes.c_void_p(d), want - 1, None)
    assert rc == -4
    st.window = 264                                        # misaligned
    assert lib.ca_state_bytes(ctypes.byref(st), pos) == -1 and b"aligned" in lib.ca_last_error()


def test_sublayer_projection_arguments_need_no_device():
    """The projection entry points check their arguments and size their workspaces on the
    host: bad widths and misaligned weights are rejected before any launch, T = 0 is a no-op,
    and only decode-sized T (too few output tiles to fill the chip) needs K-split partials."""
    from long_context_attention_17_amd import binding as ca
    lib = ca.lib()
    fake = 1 << 20                                   # aligned stand-in addresses (never dereferenced)
    qp = ca.QueryProjParams(7168, 1536, 128 * 512, 64 * 128, 64, fake, fake, fake, fake)
    op = ca.OutProjParams(128, 512, 1024, 7168, fake, fake)
    assert lib.ca_query_proj(None, None, 0, None, None, None, None, None, 0, None) == -1
    assert lib.ca_query_proj(ctypes.byref(qp), None, 0, None, None, None, None, None, 0, None) == 0
    assert lib.ca_out_proj(ctypes.byref(op), None, 0, None, None, None, 0, None) == 0
    assert lib.ca_query_proj(ctypes.byref(qp), None, 4, None, None, None, None, None, 0, None) == -1   # NULL buffers
    assert lib.ca_query_proj(ctypes.byref(qp), None, -1, None, None, None, None, None, 0, None) == -1
    bad = ca.QueryProjParams(7168 + 32, 1536, 128 * 512, 64 * 128, 64, fake, fake, fake, fake)
    assert lib.ca_query_proj(ctypes.byref(bad), None, 0, None, None, None, None, None, 0, None) == -3
    bad = ca.QueryProjParams(7168, 1536, 128 * 512, 64 * 128, 0, fake, fake, fake, fake)        # n_qi without n_i
    assert lib.ca_query_proj(ctypes.byref(bad), None, 0, None, None, None, None, None, 0, None) == -1
    bad = ca.QueryProjParams(7168, 1536, 128 * 512, 64 * 128, 64, fake + 2, fake, fake, fake)
    assert lib.ca_query_proj(ctypes.byref(bad), None, 0, None, None, None, None, None, 0, None) == -1
    assert "aligned" in lib.ca_last_error().decode()
    bad = ca.OutProjParams(60, 512, 1024, 7168, fake, fake)                                    # 8 heads a group
    assert lib.ca_out_proj(ctypes.byref(bad), None, 0, None, None, None, 0, None) == -3
    assert lib.ca_query_proj_workspace(ctypes.byref(qp), 32768) == 0
    assert lib.ca_out_proj_workspace(ctypes.byref(op), 32768) == 0
    assert lib.ca_query_proj_workspace(ctypes.byref(qp), 8) > 0       # h W^DQ: 13 output tiles at T = 8
    assert lib.ca_out_proj_workspace(ctypes.byref(op), 8) > 0
    assert lib.ca_query_proj_workspace(None, 8) == 0


def test_attention_rejects_pools_and_windows_beyond_31_bit_item_indices():
    """Attention items are addressed by pool record index or window row in 31 bits: a pool of
    2^31 - 1 or more records, or a decode window of 2^31 - 1 or more rows, is refused on the
    host before any launch (fake, never dereferenced addresses)."""
    from long_context_attention_17_amd import binding as ca
    lib = ca.lib()
    fake = 1 << 20
    p = ca.AttendParams(64, 512, 64, 128, ca.BF16, ca.BF16, ca.BF16, 512 ** -0.5, 1e-6, 1e4, None)

    def hca_decode(n_pages, W, B=1):
        c = ca._Cache(ca.FP8MIX, 512, 64, 64, fake, n_pages, fake, B, 16)
        return lib.ca_hca_attend_decode(ctypes.byref(p), fake, fake, ctypes.byref(c), 128, fake, B, 1024, fake, W,
                                        fake, fake, None, fake, 1 << 30, None)

    big = (1 << 31) // 64                           # pages of 64 records: 2^31 records
    assert hca_decode(big, 128) == -3 and "records" in lib.ca_last_error().decode()
    assert hca_decode(big - 1, (1 << 31) // 8, B=8) == -3 and "window" in lib.ca_last_error().decode()


def test_attention_rejects_rows_beyond_the_32_bit_split_plan():
    """The kernels take a row's split plan in 32-bit arithmetic: a call whose rows may hold
    2^31 - 4,096 or more items (here CSA with k near 2^31) is refused on the host before
    any launch (fake, never dereferenced addresses); k + n_win below the limit passes
    that check and fails later on the workspace instead."""
    from long_context_attention_17_amd import binding as ca
    lib = ca.lib()
    fake = 1 << 20
    p = ca.AttendParams(64, 512, 64, 128, ca.BF16, ca.BF16, ca.BF16, 512 ** -0.5, 1e-6, 1e4, None)
    c = ca._Cache(ca.FP8MIX, 512, 64, 64, fake, 16, fake, 1, 16)

    def csa_decode(k):
        return lib.ca_csa_attend_decode(ctypes.byref(p), fake, fake, ctypes.byref(c), fake, fake, k, 4, fake, 1, 1024,
                                        fake, 128, fake, fake, None, None, 0, None)

    assert csa_decode((1 << 31) - 1024) == -3 and "2^31 - 4096 or more items" in lib.ca_last_error().decode()
    rc = csa_decode((1 << 31) - 4096 - 256)
    assert rc != 0 and "2^31 - 4096" not in lib.ca_last_error().decode()
