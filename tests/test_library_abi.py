"""The C-ABI library builds, loads and exports every symbol its header declares.

CPU only: nothing here launches a kernel.  Calls that return before any HIP
work (argument validation, workspace sizing, status strings) are exercised.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


@pytest.fixture(scope="module")
def lib():
    from speculative_decoding_sampling_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    return ctypes.CDLL(build.LIB)


def declared_functions():
    names = []
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            with open(os.path.join(INCLUDE, h)) as f:
                names += re.findall(r"SPECV_API\s+[\w\s\*]+?\b(specv_\w+)\s*\(", f.read())
    return names


def test_header_declares_the_api():
    names = declared_functions()
    assert set(names) == {"specv_workspace_bytes", "specv_verify", "specv_verify_debug",
                          "specv_verify_timed", "specv_num_stages", "specv_stage_name",
                          "specv_path_kind", "specv_set_small_batch_limit",
                          "specv_verify_noalloc",
                          "specv_status_string", "specv_version", "specv_selftest_exp64",
                          "specv_selftest_set_small_poll_limit",
                          "specv_bench_row_stats", "specv_sample",
                          "specv_acceptance_rates", "specv_round_stats",
                          "specv_monitor_state_bytes", "specv_monitor_reset",
                          "specv_monitor_update", "specv_lm_head_workspace_bytes",
                          "specv_verify_lm_head", "specv_bench_lm_head",
                          "specv_lm_head_packed_weight_bytes",
                          "specv_lm_head_pack_weight"}, names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_only_the_c_api_is_exported(lib):
    import subprocess
    from speculative_decoding_sampling_amd import build
    out = subprocess.run(["nm", "-D", "--defined-only", build.LIB], capture_output=True,
                         text=True).stdout
    funcs = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert funcs == set(declared_functions()), funcs


def test_workspace_sizes(lib):
    f = lib.specv_workspace_bytes
    f.argtypes = [ctypes.c_int] * 5 + [ctypes.c_float]
    f.restype = ctypes.c_size_t
    n3 = f(64, 4, 128256, 1, 0, 1.0)
    assert n3 > 0 and n3 % 256 == 0
    assert f(64, 4, 128256, 1, 0, 1.0) == n3                      # pure function of sizes
    assert f(128, 4, 128256, 1, 0, 1.0) > n3
    assert f(0, 4, 100, 0, 0, 1.0) == 0                           # B < 1
    assert f(1, 65, 100, 0, 0, 1.0) == 0                          # K > SPECV_MAX_K
    assert f(1, 64, 100, 0, 0, 1.0) > 0                           # K = SPECV_MAX_K
    assert f(1, 4, 0, 0, 0, 1.0) == 0                             # V < 1
    assert f(1, 4, 100, 7, 0, 1.0) == 0                           # unknown dtype
    assert f(1, 4, 100, 0, 0, 0.0) == 0                           # top_p out of range
    assert f(256, 8, 152064, 0, 50, 0.9) > 0                      # the top-k/top-p workload
    assert f(1, 4, 300000, 0, 50, 0.9) > 0                        # large V: the radix select
    assert f(4, 4, 1000, 0, 0, 0.9) > 0 and f(4, 4, 1000, 0, 999, 1.0) > 0


def test_validation_returns_before_any_gpu_work(lib):
    v = lib.specv_verify
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    v.argtypes = [vp, vp, ci, vp, vp, vp, vp, ci, ci, ci, cf, ci, cf, ci, vp, vp, vp,
                  ctypes.c_size_t, vp]
    v.restype = ci
    dummy = ctypes.c_void_p(4096)
    base = [dummy, dummy, 1, dummy, dummy, dummy, dummy, 4, 4, 1000, 1.0, 0, 1.0, -1,
            dummy, dummy, dummy, 1 << 20, None]

    def call(**kw):
        args = list(base)
        idx = {"B": 7, "K": 8, "V": 9, "T": 10, "top_k": 11, "top_p": 12, "eos": 13,
               "target": 0, "ws_bytes": 17}
        for k, val in kw.items():
            args[idx[k]] = val
        return v(*args)

    assert call(B=0) == 1
    assert call(K=65) == 1
    assert call(V=0) == 1
    assert call(T=0.0) == 1
    assert call(T=float("nan")) == 1
    assert call(top_p=0.0) == 1
    assert call(eos=1000) == 1
    assert call(target=None) == 1
    assert call(top_k=10, ws_bytes=16) == 2    # filtered path: workspace too small
    assert call(top_k=129, ws_bytes=16) == 2   # radix-select path: workspace too small
    assert call(top_k=0, top_p=0.9, ws_bytes=16) == 2
    assert call(ws_bytes=16) == 2              # workspace too small


def test_noalloc_rejects_sizes_beyond_its_scratch_without_device_work(lib):
    v = lib.specv_verify_noalloc
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    v.argtypes = [vp, vp, ci, vp, vp, vp, vp, ci, ci, ci, cf, ci, cf, ci, vp, vp, vp]
    v.restype = ci
    d = ctypes.c_void_p(4096)
    # B=256, K=8, V=152064 with top-k 50 needs ~98 MB: beyond the 16 MiB scratch
    assert v(d, d, 0, d, d, d, d, 256, 8, 152064, 1.0, 50, 0.9, -1, d, d, None) == 5
    assert v(d, d, 0, d, d, d, d, 0, 8, 152064, 1.0, 50, 0.9, -1, d, d, None) == 1   # B < 1
    s = lib.specv_status_string
    s.argtypes = [ctypes.c_int]
    s.restype = ctypes.c_char_p
    assert s(5).startswith(b"sizes need more scratch")


def test_stage_names(lib):
    lib.specv_stage_name.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.specv_stage_name.restype = ctypes.c_char_p
    lib.specv_num_stages.argtypes = [ctypes.c_int]
    for kind, first in ((0, b"row_stats"), (1, b"filter_cand"), (2, b"filter_rows"),
                        (3, b"verify_small")):
        n = lib.specv_num_stages(kind)
        names = [lib.specv_stage_name(kind, i) for i in range(n)]
        assert n >= 1 and names[0] == first and all(names)
        assert lib.specv_stage_name(kind, n) is None
        assert lib.specv_stage_name(kind, -1) is None
    assert lib.specv_num_stages(4) == 0 and lib.specv_stage_name(4, 0) is None
    assert lib.specv_num_stages(3) == 1          # the small-batch path is one kernel
    pk = lib.specv_path_kind
    pk.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float]
    pk.restype = ctypes.c_int
    assert pk(64, 4, 128256, 0, 1.0) == 0 and pk(64, 4, 128256, 128256, 1.0) == 0   # filters off
    assert pk(256, 8, 152064, 50, 0.9) == 1 and pk(1, 0, 152064, 100, 1.0) == 1      # candidates
    assert pk(1, 1, 152064, 128, 1.0) == 2   # 128 at 19 chunks: slots beyond the on-chip list
    assert pk(64, 4, 152064, 0, 0.9) == 2 and pk(1, 4, 152064, 1000, 1.0) == 2      # radix
    assert pk(1, 4, 300000, 50, 0.9) == 2                                           # chunks
    # small sizes without filters: B (K+1) ceil(V/2048) within the limit (384 by default)
    assert pk(8, 4, 4096, 0, 1.0) == 3 and pk(1, 5, 32000, 0, 1.0) == 3
    assert pk(1, 5, 32000, 0, 0.9) == 2                   # filters keep their own paths
    assert pk(24, 3, 2048 * 4, 0, 1.0) == 3 and pk(24, 3, 2048 * 4 + 1, 0, 1.0) == 0
    lim = lib.specv_set_small_batch_limit
    lim.argtypes = [ctypes.c_longlong]
    lim.restype = ctypes.c_longlong
    old = lim(0)
    try:
        assert old == 384 and pk(8, 4, 4096, 0, 1.0) == 0
        ws = lib.specv_workspace_bytes
        ws.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                       ctypes.c_float]
        ws.restype = ctypes.c_size_t
        big = ws(8, 4, 4096, 0, 0, 1.0)
        assert lim(1 << 40) == 0 and pk(64, 4, 128256, 0, 1.0) == 3
        assert ws(8, 4, 4096, 0, 0, 1.0) > big            # the pass runs for every row pair
        assert lim(-5) == 1 << 40 and pk(8, 4, 4096, 0, 1.0) == 0   # negative: off
    finally:
        lim(old)


def test_status_strings(lib):
    s = lib.specv_status_string
    s.argtypes = [ctypes.c_int]
    s.restype = ctypes.c_char_p
    assert s(0) == b"ok" and s(1) == b"invalid argument"
    assert lib.specv_version() == 103


def test_bench_hook_rejects_bad_arguments(lib):
    f = lib.specv_bench_row_stats
    vp, i, fl, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    f.argtypes = [vp, vp, vp, vp, i, i, i, i, i, fl, vp, sz, i, vp, vp, vp]
    f.restype = i
    one = (vp * 1)(16)
    ok = dict(targets=one, drafts=one, toks=one, lens=one, nsets=1, dtype=1, B=2, K=3, V=4096,
              T=1.0, ws=16, wsb=1 << 20, reps=4, start=16, stop=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["targets"], a["drafts"], a["toks"], a["lens"], a["nsets"], a["dtype"], a["B"],
                 a["K"], a["V"], a["T"], a["ws"], a["wsb"], a["reps"], None, a["start"],
                 a["stop"])

    assert call(nsets=0) == 1
    assert call(reps=0) == 1
    assert call(start=None) == 1
    assert call(T=0.0) == 1
    assert call(targets=(vp * 1)(0)) == 1
    assert call(wsb=16) == 2


def test_sample_rejects_bad_arguments(lib):
    f = lib.specv_sample
    vp, i, fl, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    f.argtypes = [vp, i, vp, i, i, fl, i, fl, vp, vp, sz, vp]
    f.restype = i
    ok = dict(logits=16, dtype=1, u=16, R=4, V=1000, T=1.0, k=0, p=1.0, out=16, ws=16,
              wsb=1 << 20)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["logits"], a["dtype"], a["u"], a["R"], a["V"], a["T"], a["k"], a["p"],
                 a["out"], a["ws"], a["wsb"], None)

    assert call(R=0) == 1
    assert call(logits=None) == 1
    assert call(u=None) == 1
    assert call(out=None) == 1
    assert call(T=-1.0) == 1
    assert call(p=0.0) == 1
    assert call(k=10, p=0.5, wsb=16) == 2            # filtered workspace too small
    assert call(wsb=16) == 2


def test_acceptance_rates_reject_bad_arguments(lib):
    f = lib.specv_acceptance_rates
    vp, i, fl, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    f.argtypes = [vp, vp, i, vp, i, i, i, fl, i, fl, vp, vp, sz, vp]
    f.restype = i
    ok = dict(t=16, d=16, dtype=1, dl=16, B=2, K=3, V=1000, T=1.0, k=0, p=1.0, beta=16, ws=16,
              wsb=1 << 20)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["t"], a["d"], a["dtype"], a["dl"], a["B"], a["K"], a["V"], a["T"], a["k"],
                 a["p"], a["beta"], a["ws"], a["wsb"], None)

    assert call(B=0) == 1
    assert call(dl=None) == 1
    assert call(beta=None) == 1
    assert call(d=None) == 1
    assert call(T=0.0) == 1
    assert call(k=0, p=0.5, wsb=16) == 2             # top-p alone: radix-select workspace
    assert call(p=1.5) == 1 and call(k=-1) == 1
    assert call(wsb=16) == 2
    assert call(K=0, d=None, wsb=1 << 20) == 0       # nothing to compute, nothing launched


def test_round_stats_reject_bad_arguments(lib):
    f = lib.specv_round_stats
    vp, i = ctypes.c_void_p, ctypes.c_int
    f.argtypes = [vp, vp, vp, vp, vp, i, i, vp, vp, vp, vp]
    f.restype = i
    ok = dict(dt=16, dl=16, out=16, n=16, beta=None, B=4, K=3, acc=16, exp=None, tot=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["dt"], a["dl"], a["out"], a["n"], a["beta"], a["B"], a["K"], a["acc"],
                 a["exp"], a["tot"], None)

    assert call(B=0) == 1
    assert call(K=65) == 1 and call(K=-1) == 1
    assert call(dt=None) == 1
    assert call(out=None) == 1 and call(n=None) == 1 and call(dl=None) == 1
    assert call(exp=16) == 1                         # expected tokens need beta
    assert call(dl=18) == 1                          # misaligned
    assert call(tot=20) == 1                         # int64 totals must be 8-aligned


def test_monitor_sizes_and_bad_arguments(lib):
    sb = lib.specv_monitor_state_bytes
    sb.argtypes = [ctypes.c_int, ctypes.c_int]
    sb.restype = ctypes.c_size_t
    assert sb(1, 1) == 32 and sb(3, 4) == 3 * 32 and sb(2, 5) == 2 * 48
    assert sb(0, 4) == 0 and sb(4, 0) == 0 and sb(4, 4097) == 0 and sb(1, 4096) == 4100 * 4
    rs = lib.specv_monitor_reset
    rs.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    rs.restype = ctypes.c_int
    assert rs(None, 4, 8, None) == 1 and rs(16, 0, 8, None) == 1 and rs(16, 4, 0, None) == 1
    assert rs(24, 4, 8, None) == 1                   # state must be 16-aligned
    f = lib.specv_monitor_update
    vp, i = ctypes.c_void_p, ctypes.c_int
    f.argtypes = [vp, vp, vp, vp, i, i, i, i, vp, vp, vp, vp]
    f.restype = i
    ok = dict(dt=16, dl=16, out=16, n=16, B=4, K=3, mk=6, W=8, st=16, nxt=16, rate=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["dt"], a["dl"], a["out"], a["n"], a["B"], a["K"], a["mk"], a["W"], a["st"],
                 a["nxt"], a["rate"], None)

    assert call(B=0) == 1 and call(K=65) == 1
    assert call(mk=0) == 1 and call(mk=65) == 1
    assert call(W=0) == 1 and call(W=4097) == 1
    assert call(st=None) == 1 and call(nxt=None) == 1 and call(dt=None) == 1
    assert call(st=20) == 1 and call(rate=20) == 1


def test_lm_head_workspace_sizes(lib):
    f = lib.specv_lm_head_workspace_bytes
    f.argtypes = [ctypes.c_int] * 5 + [ctypes.c_float]
    f.restype = ctypes.c_size_t
    g = lib.specv_workspace_bytes
    g.argtypes = [ctypes.c_int] * 5 + [ctypes.c_float]
    g.restype = ctypes.c_size_t
    n = f(64, 4, 128256, 4096, 0, 1.0)
    # the unfiltered bf16 layout plus the LM head's tile statistics
    assert n >= g(64, 4, 128256, 1, 0, 1.0) + 64 * 5 * ((128256 + 255) // 256) * 8
    assert n % 256 == 0
    assert f(64, 4, 128256, 4096, 0, 1.0) == f(64, 4, 128256, 64, 0, 1.0)   # D only validated
    assert f(64, 4, 128256, 100, 0, 1.0) == 0                     # D not a multiple of 64
    assert f(64, 4, 128256, 0, 0, 1.0) == 0
    assert f(64, 4, 128256, 65536 + 64, 0, 1.0) == 0              # above SPECV_MAX_D
    assert f(0, 4, 100, 64, 0, 1.0) == 0 and f(1, 65, 100, 64, 0, 1.0) == 0
    assert f(1, 4, 0, 64, 0, 1.0) == 0
    # with top-k / top-p: the filtered layout plus the tile statistics
    nf = f(64, 4, 128256, 4096, 50, 0.9)
    assert nf >= g(64, 4, 128256, 1, 50, 0.9) + 64 * 5 * ((128256 + 255) // 256) * 8
    assert f(64, 4, 128256, 4096, 0, 0.9) > 0 and f(64, 4, 128256, 4096, -1, 0.9) == 0


def test_lm_head_packed_weight_sizes_and_validation(lib):
    f = lib.specv_lm_head_packed_weight_bytes
    f.argtypes = [ctypes.c_int] * 2
    f.restype = ctypes.c_size_t
    # whole 128-id tiles of D bf16 values each
    assert f(128256, 4096) == 1002 * 128 * 4096 * 2
    assert f(128, 64) == 128 * 64 * 2
    assert f(129, 64) == 256 * 64 * 2
    assert f(1, 64) == 128 * 64 * 2
    assert f(0, 64) == 0 and f(100, 0) == 0 and f(100, 96) == 0 and f(100, 65536 + 64) == 0
    p = lib.specv_lm_head_pack_weight
    vp = ctypes.c_void_p
    p.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, vp]
    p.restype = ctypes.c_int
    src, dst = vp(1 << 20), vp(1 << 30)
    assert p(None, dst, 100, 64, None) == 1
    assert p(src, None, 100, 64, None) == 1
    assert p(vp((1 << 20) + 8), dst, 100, 64, None) == 1         # not 16-byte aligned
    assert p(src, vp((1 << 30) + 4), 100, 64, None) == 1
    assert p(src, dst, 100, 96, None) == 1                       # D not a multiple of 64
    assert p(src, dst, 0, 64, None) == 1
    assert p(src, vp((1 << 20) + 4096), 100, 64, None) == 1      # overlaps the source
    assert p(vp((1 << 20) + 4096), src, 100, 64, None) == 1


def test_lm_head_validation_returns_before_any_gpu_work(lib):
    v = lib.specv_verify_lm_head
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    v.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, ci, cf, ci, vp, vp, vp, vp,
                  ctypes.c_size_t, vp, vp, vp, vp, vp]
    v.restype = ci
    d = ctypes.c_void_p(4096)
    base = [d, d, d, d, d, d, d, 4, 4, 1000, 64, 1.0, 0, 1.0, -1, d, d, d, d, 1 << 30, None,
            None, None, None, None]
    idx = {"hidden": 0, "weight": 1, "B": 7, "K": 8, "V": 9, "D": 10, "T": 11, "top_k": 12,
           "top_p": 13, "eos": 14, "out": 15, "ws": 18, "ws_bytes": 19}

    def call(**kw):
        args = list(base)
        for k, val in kw.items():
            args[idx[k]] = val
        return v(*args)

    assert call(D=100) == 1
    assert call(D=0) == 1
    assert call(B=0) == 1
    assert call(K=65) == 1
    assert call(T=0.0) == 1
    assert call(eos=1000) == 1
    assert call(hidden=None) == 1
    assert call(hidden=ctypes.c_void_p(4104)) == 1               # not 16-byte aligned
    assert call(weight=ctypes.c_void_p(4098)) == 1
    assert call(out=None) == 1
    assert call(ws_bytes=16) == 2
    assert call(ws=None) == 2
    assert call(D=65536 + 64) == 4                                # SPECV_EUNSUPPORTED
    assert call(top_k=-1) == 1 and call(top_p=0.0) == 1
    assert call(top_k=50, top_p=0.9, ws_bytes=16) == 2            # filtered: workspace
