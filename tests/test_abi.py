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
    assert lib.ca_timer_start(1 << 3, 16) == -1           # unknown kernel bit
    assert lib.ca_timer_start(1, 0) == -1                 # no launches to time
    assert lib.ca_timer_start(1, (1 << 20) + 1) == -1     # above the launch cap
    ms, n = ctypes.c_double(-1.0), ctypes.c_int64(-1)
    assert lib.ca_timer_read(-1, ctypes.byref(ms), ctypes.byref(n)) == -1
    assert lib.ca_timer_read(ca.TIMED_INDEX_SCORES + 1, ctypes.byref(ms), ctypes.byref(n)) == -1
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
