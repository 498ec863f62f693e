"""ctypes binding for libspecverify (argument marshalling only).

Every step of the verification runs in the HIP library; this module checks
tensor shapes and dtypes, allocates outputs and a workspace with torch, and
passes raw device pointers plus the current HIP stream through the C ABI
declared in ``include/specverify.h``.  If the library is not built the
binding raises: there is no fallback.
"""

import ctypes
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspecverify.so")

SPECV_F32, SPECV_BF16 = 0, 1
SPECV_OK, SPECV_EINVAL, SPECV_EWORKSPACE, SPECV_EHIP, SPECV_EUNSUPPORTED = 0, 1, 2, 3, 4
SPECV_ESCRATCH = 5
NOALLOC_SCRATCH_BYTES = 16 << 20
MAX_K = 64
MAX_WINDOW = 4096
TOTAL_FIELDS = ("requests", "errors", "drafted", "accepted", "emitted", "eos_stops",
                "full_accepts", "rejections")

PATH_ERROR, PATH_REJECT, PATH_BONUS, PATH_EOS = -1, 0, 1, 2

_lib = None
_lock = threading.Lock()
_workspaces = {}


class SpecVerifyError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"specv_verify failed with status {status}: {msg}")
        self.status = status


def library_path():
    return _LIB_PATH


def load_library():
    """Load libspecverify.so and declare its C signatures (once)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is not built; run `python -m speculative_decoding_sampling_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        c_int, c_float, c_vp, c_size = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
        lib.specv_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int, c_float]
        lib.specv_workspace_bytes.restype = c_size
        common = [c_vp, c_vp, c_int, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_float, c_int,
                  c_float, c_int, c_vp, c_vp, c_vp, c_size, c_vp]
        lib.specv_verify.argtypes = common
        lib.specv_verify.restype = c_int
        lib.specv_verify_debug.argtypes = common + [c_vp, c_vp, c_vp, c_vp]
        lib.specv_verify_debug.restype = c_int
        lib.specv_verify_timed.argtypes = common + [c_vp]
        lib.specv_verify_timed.restype = c_int
        lib.specv_verify_noalloc.argtypes = common[:16] + [c_vp]
        lib.specv_verify_noalloc.restype = c_int
        lib.specv_sample.argtypes = [c_vp, c_int, c_vp, c_int, c_int, c_float, c_int, c_float, c_vp,
                                     c_vp, c_size, c_vp]
        lib.specv_sample.restype = c_int
        lib.specv_acceptance_rates.argtypes = [c_vp, c_vp, c_int, c_vp, c_int, c_int, c_int,
                                               c_float, c_int, c_float, c_vp, c_vp, c_size, c_vp]
        lib.specv_acceptance_rates.restype = c_int
        lib.specv_round_stats.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_vp, c_vp,
                                          c_vp, c_vp]
        lib.specv_round_stats.restype = c_int
        lib.specv_monitor_state_bytes.argtypes = [c_int, c_int]
        lib.specv_monitor_state_bytes.restype = c_size
        lib.specv_monitor_reset.argtypes = [c_vp, c_int, c_int, c_vp]
        lib.specv_monitor_reset.restype = c_int
        lib.specv_monitor_update.argtypes = [c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int,
                                             c_vp, c_vp, c_vp, c_vp]
        lib.specv_monitor_update.restype = c_int
        lib.specv_path_kind.argtypes = [c_int, c_int, c_int, c_int, ctypes.c_float]
        lib.specv_path_kind.restype = c_int
        lib.specv_set_small_batch_limit.argtypes = [ctypes.c_longlong]
        lib.specv_set_small_batch_limit.restype = ctypes.c_longlong
        lib.specv_num_stages.argtypes = [c_int]
        lib.specv_num_stages.restype = c_int
        lib.specv_stage_name.argtypes = [c_int, c_int]
        lib.specv_stage_name.restype = ctypes.c_char_p
        lib.specv_status_string.argtypes = [c_int]
        lib.specv_status_string.restype = ctypes.c_char_p
        lib.specv_selftest_exp64.argtypes = [c_vp, c_vp, c_int, c_vp]
        lib.specv_selftest_exp64.restype = c_int
        lib.specv_bench_row_stats.argtypes = [c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int,
                                              c_int, c_float, c_vp, c_size, c_int, c_vp, c_vp,
                                              c_vp]
        lib.specv_bench_row_stats.restype = c_int
        lib.specv_lm_head_packed_weight_bytes.argtypes = [c_int, c_int]
        lib.specv_lm_head_packed_weight_bytes.restype = c_size
        lib.specv_lm_head_pack_weight.argtypes = [c_vp, c_vp, c_int, c_int, c_vp]
        lib.specv_lm_head_pack_weight.restype = c_int
        lib.specv_lm_head_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int, c_float]
        lib.specv_lm_head_workspace_bytes.restype = c_size
        lib.specv_verify_lm_head.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int,
                                             c_int, c_int, c_float, c_int, c_float, c_int, c_vp,
                                             c_vp, c_vp, c_vp, c_size, c_vp, c_vp, c_vp, c_vp,
                                             c_vp]
        lib.specv_verify_lm_head.restype = c_int
        lib.specv_bench_lm_head.argtypes = [c_vp, c_vp, c_int, c_int, c_int, c_float, c_vp, c_vp,
                                            c_size, c_int, c_vp, c_vp, c_vp]
        lib.specv_bench_lm_head.restype = c_int
        lib.specv_version.argtypes = []
        lib.specv_version.restype = c_int
        _lib = lib
        return lib


def status_string(status):
    return load_library().specv_status_string(int(status)).decode()


def path_kind(B, K, V, top_k=0, top_p=1.0):
    """0: no filters; 1: top-k / top-p by the candidate select; 2: by the radix
    select; 3: no filters, small sizes (one kernel after the row statistics)."""
    return int(load_library().specv_path_kind(int(B), int(K), int(V), int(top_k), float(top_p)))


def set_small_batch_limit(limit):
    """Largest B * (K+1) * ceil(V / 2048) of an unfiltered call that takes
    path 3 (default 384; 0: never, a huge value: always).  Process-wide;
    returns the previous limit."""
    return int(load_library().specv_set_small_batch_limit(int(limit)))


def stage_names(kind=0):
    """Names of the kernel stages a call on path ``kind`` (see path_kind) launches, in order."""
    lib = load_library()
    return [lib.specv_stage_name(int(kind), i).decode() for i in range(lib.specv_num_stages(int(kind)))]


def selftest_exp64(x):
    """The sampler's device float64 exp applied to a float64 GPU tensor (test hook)."""
    lib = load_library()
    if x.dtype != torch.float64 or x.device.type != "cuda" or not x.is_contiguous():
        raise ValueError("x must be a contiguous float64 GPU tensor")
    y = torch.empty_like(x)
    st = lib.specv_selftest_exp64(_ptr(x), _ptr(y), x.numel(),
                                  ctypes.c_void_p(torch.cuda.current_stream(x.device).cuda_stream))
    if st != SPECV_OK:
        raise SpecVerifyError(st, status_string(st))
    return y


def sample(logits, u, temperature=1.0, top_k=0, top_p=1.0, *, out_tokens=None, workspace=None,
           stream=None):
    """Draw one token per row of ``logits`` [R, V] (bf16 or fp32) from its
    processed distribution (temperature, top-k, top-p) at the uniforms ``u``
    [R] (fp32), by inverse CDF over ascending token ids.  Returns
    ``out_tokens`` [R] int32 (-1 for a row with no finite logit or a uniform
    outside [0, 1)).  Asynchronous on ``stream``."""
    lib = load_library()
    dev = logits.device
    if dev.type != "cuda" or logits.dim() != 2:
        raise ValueError("logits must be a [R, V] GPU tensor")
    R, V = logits.shape
    code = _dtype_code(logits)
    _check(logits, "logits", None, (R, V), dev)
    _check(u, "u", torch.float32, (R,), dev)
    if out_tokens is None:
        out_tokens = torch.empty((R,), dtype=torch.int32, device=dev)
    _check(out_tokens, "out_tokens", torch.int32, (R,), dev)
    nbytes = int(lib.specv_workspace_bytes(R, 0, V, code, int(top_k), float(top_p)))
    if workspace is None:
        workspace = _workspace(dev, nbytes)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    st = lib.specv_sample(_ptr(logits), code, _ptr(u), R, V, float(temperature), int(top_k),
                          float(top_p), _ptr(out_tokens), _ptr(workspace),
                          workspace.numel() * workspace.element_size(),
                          ctypes.c_void_p(stream.cuda_stream))
    if st != SPECV_OK:
        raise SpecVerifyError(st, status_string(st))
    return out_tokens


def acceptance_rates(target_logits, draft_logits, draft_len, temperature=1.0, top_k=0, top_p=1.0,
                     *, beta=None, workspace=None, stream=None):
    """Per-position acceptance rates sum_x min(p_k(x), q_k(x)) of a batch
    (target [B, K+1, V], draft [B, K, V], draft_len [B] int32), as a [B, K]
    float32 tensor; -1 where a position was not drafted or a row has no
    finite logit.  Asynchronous on ``stream``."""
    lib = load_library()
    dev = target_logits.device
    if dev.type != "cuda" or target_logits.dim() != 3:
        raise ValueError("target_logits must be a [B, K+1, V] GPU tensor")
    B, K1, V = target_logits.shape
    K = K1 - 1
    code = _dtype_code(target_logits)
    _check(target_logits, "target_logits", None, (B, K + 1, V), dev)
    _check(draft_logits, "draft_logits", target_logits.dtype, (B, K, V), dev)
    _check(draft_len, "draft_len", torch.int32, (B,), dev)
    if beta is None:
        beta = torch.empty((B, K), dtype=torch.float32, device=dev)
    _check(beta, "beta", torch.float32, (B, K), dev)
    nbytes = int(lib.specv_workspace_bytes(B, K, V, code, int(top_k), float(top_p)))
    if workspace is None:
        workspace = _workspace(dev, nbytes)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    st = lib.specv_acceptance_rates(_ptr(target_logits), _ptr(draft_logits), code,
                                    _ptr(draft_len), B, K, V, float(temperature), int(top_k),
                                    float(top_p), _ptr(beta), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    ctypes.c_void_p(stream.cuda_stream))
    if st != SPECV_OK:
        raise SpecVerifyError(st, status_string(st))
    return beta


def _round_args(draft_tokens, draft_len, out_tokens, n_emitted):
    dev = out_tokens.device
    if dev.type != "cuda" or out_tokens.dim() != 2:
        raise ValueError("out_tokens must be a [B, K+1] GPU tensor")
    B, K1 = out_tokens.shape
    K = K1 - 1
    _check(out_tokens, "out_tokens", torch.int32, (B, K + 1), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _check(draft_len, "draft_len", torch.int32, (B,), dev)
    _check(n_emitted, "n_emitted", torch.int32, (B,), dev)
    return dev, B, K


def round_stats(draft_tokens, draft_len, out_tokens, n_emitted, beta=None, *, accepted=None,
                expected=None, totals=None, stream=None):
    """Statistics of one verified round from a ``verify`` call's inputs and
    outputs.  Returns (accepted [B] int32, expected [B] float32 or None,
    totals [8] int64 in ``TOTAL_FIELDS`` order); ``expected`` (E[N] from the
    per-position rates) needs ``beta`` from ``acceptance_rates``.
    Asynchronous on ``stream``."""
    lib = load_library()
    dev, B, K = _round_args(draft_tokens, draft_len, out_tokens, n_emitted)
    if accepted is None:
        accepted = torch.empty(B, dtype=torch.int32, device=dev)
    _check(accepted, "accepted", torch.int32, (B,), dev)
    if beta is not None:
        _check(beta, "beta", torch.float32, (B, K), dev)
        if expected is None:
            expected = torch.empty(B, dtype=torch.float32, device=dev)
    if expected is not None:
        _check(expected, "expected", torch.float32, (B,), dev)
    if totals is None:
        totals = torch.empty(len(TOTAL_FIELDS), dtype=torch.int64, device=dev)
    _check(totals, "totals", torch.int64, (len(TOTAL_FIELDS),), dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    st = lib.specv_round_stats(_ptr(draft_tokens), _ptr(draft_len), _ptr(out_tokens),
                               _ptr(n_emitted), _ptr(beta), B, K, _ptr(accepted), _ptr(expected),
                               _ptr(totals), ctypes.c_void_p(stream.cuda_stream))
    if st != SPECV_OK:
        raise SpecVerifyError(st, status_string(st))
    return accepted, expected, totals


class DraftLengthMonitor:
    """Per-request acceptance-rate windows and the adaptive draft length, held
    in device memory (``specv_monitor_*``).  ``update`` takes one verified
    round and returns the next round's draft lengths, without a host sync."""

    def __init__(self, batch, window, max_k, device, stream=None):
        self.lib = load_library()
        self.B, self.window, self.max_k = int(batch), int(window), int(max_k)
        self.device = torch.device(device)
        nbytes = int(self.lib.specv_monitor_state_bytes(self.B, self.window))
        if nbytes == 0 or not 1 <= self.max_k <= MAX_K:
            raise ValueError(f"bad monitor sizes: batch={batch} window={window} max_k={max_k}")
        self.state = torch.empty((nbytes + 15) // 16 * 16, dtype=torch.uint8, device=self.device)
        self.reset(stream)

    def _stream(self, stream):
        return torch.cuda.current_stream(self.device) if stream is None else stream

    def reset(self, stream=None):
        st = self.lib.specv_monitor_reset(_ptr(self.state), self.B, self.window,
                                          ctypes.c_void_p(self._stream(stream).cuda_stream))
        if st != SPECV_OK:
            raise SpecVerifyError(st, status_string(st))

    def update(self, draft_tokens, draft_len, out_tokens, n_emitted, *, next_draft_len=None,
               rate=None, stream=None):
        """Returns (next_draft_len [B] int32, rate [B] float64); pass
        ``next_draft_len=draft_len`` to update the draft lengths in place."""
        dev, B, K = _round_args(draft_tokens, draft_len, out_tokens, n_emitted)
        if B != self.B or dev != self.device:
            raise ValueError(f"monitor holds {self.B} requests on {self.device}")
        if next_draft_len is None:
            next_draft_len = torch.empty(B, dtype=torch.int32, device=dev)
        _check(next_draft_len, "next_draft_len", torch.int32, (B,), dev)
        if rate is None:
            rate = torch.empty(B, dtype=torch.float64, device=dev)
        _check(rate, "rate", torch.float64, (B,), dev)
        st = self.lib.specv_monitor_update(_ptr(draft_tokens), _ptr(draft_len), _ptr(out_tokens),
                                           _ptr(n_emitted), B, K, self.max_k, self.window,
                                           _ptr(self.state), _ptr(next_draft_len), _ptr(rate),
                                           ctypes.c_void_p(self._stream(stream).cuda_stream))
        if st != SPECV_OK:
            raise SpecVerifyError(st, status_string(st))
        return next_draft_len, rate


def bench_row_stats(sets, workspace, reps, temperature=1.0, stream=None, start=None, stop=None):
    """Benchmark hook: the row-statistics kernel alone, ``reps`` launches
    cycling through ``sets`` (dicts as ``verify`` takes, same sizes), between
    the HIP events ``start`` and ``stop`` (raw handles) recorded on ``stream``."""
    lib = load_library()
    t0 = sets[0]["target_logits"]
    B, K1, V = t0.shape
    n = len(sets)
    arr = lambda key: (ctypes.c_void_p * n)(*[s[key].data_ptr() if s[key].numel() else 0
                                               for s in sets])
    for s in sets:
        if s["target_logits"].shape != t0.shape or s["target_logits"].dtype != t0.dtype:
            raise ValueError("all sets must share shape and dtype")
    if stream is None:
        stream = torch.cuda.current_stream(t0.device)
    st = lib.specv_bench_row_stats(arr("target_logits"), arr("draft_logits"), arr("draft_tokens"),
                                   arr("draft_len"), n, _dtype_code(t0), B, K1 - 1, V,
                                   float(temperature), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), int(reps),
                                   ctypes.c_void_p(stream.cuda_stream), start, stop)
    if st != SPECV_OK:
        raise SpecVerifyError(st, status_string(st))


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return SPECV_BF16
    if t.dtype == torch.float32:
        return SPECV_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def workspace_bytes(B, K, V, dtype, top_k=0, top_p=1.0):
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    return int(load_library().specv_workspace_bytes(int(B), int(K), int(V), code, int(top_k),
                                                   float(top_p)))


def _workspace(device, nbytes):
    key = (device.index if device.index is not None else torch.cuda.current_device())
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _check(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def verify(target_logits, draft_logits, draft_tokens, draft_len, u, u_final, temperature=1.0,
           top_k=0, top_p=1.0, eos_id=-1, *, out_tokens=None, n_emitted=None, workspace=None,
           debug=False, stream=None, events=None):
    """Run one batched verification step on the GPU.

    Shapes: target_logits [B, K+1, V] (bf16 or fp32), draft_logits [B, K, V]
    (same dtype), draft_tokens [B, K] int32, draft_len [B] int32, u [B, K]
    fp32, u_final [B] fp32.  Returns a dict with ``out_tokens`` [B, K+1] and
    ``n_emitted`` [B] (int32), plus ``accept_prob``, ``residual_mass``,
    ``stop_pos`` and ``path`` when ``debug`` is true.  The call is
    asynchronous on ``stream`` (default: the current stream).  ``events``, a
    ctypes array of ``len(stage_names()) + 1`` HIP event handles, selects the
    timing entry point, which records them around every kernel stage.
    """
    lib = load_library()
    dev = target_logits.device
    if dev.type != "cuda":
        raise ValueError("target_logits must be a GPU tensor")
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, K+1, V]")
    B, K1, V = target_logits.shape
    K = K1 - 1
    code = _dtype_code(target_logits)
    _check(target_logits, "target_logits", None, (B, K + 1, V), dev)
    _check(draft_logits, "draft_logits", target_logits.dtype, (B, K, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _check(draft_len, "draft_len", torch.int32, (B,), dev)
    _check(u, "u", torch.float32, (B, K), dev)
    _check(u_final, "u_final", torch.float32, (B,), dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    if n_emitted is None:
        n_emitted = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(out_tokens, "out_tokens", torch.int32, (B, K + 1), dev)
    _check(n_emitted, "n_emitted", torch.int32, (B,), dev)
    nbytes = int(lib.specv_workspace_bytes(B, K, V, code, int(top_k), float(top_p)))
    if workspace is None:
        workspace = _workspace(dev, nbytes)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    args = [_ptr(target_logits), _ptr(draft_logits), code, _ptr(draft_tokens), _ptr(draft_len),
            _ptr(u), _ptr(u_final), B, K, V, float(temperature), int(top_k), float(top_p),
            int(eos_id), _ptr(out_tokens), _ptr(n_emitted), _ptr(workspace),
            workspace.numel() * workspace.element_size(), sptr]
    res = {"out_tokens": out_tokens, "n_emitted": n_emitted}
    if events is not None:
        if debug:
            raise ValueError("events and debug are exclusive")
        status = lib.specv_verify_timed(*args, ctypes.cast(events, ctypes.c_void_p))
    elif debug:
        res["accept_prob"] = torch.empty((B, K), dtype=torch.float32, device=dev)
        res["residual_mass"] = torch.empty((B,), dtype=torch.float64, device=dev)
        res["stop_pos"] = torch.empty((B,), dtype=torch.int32, device=dev)
        res["path"] = torch.empty((B,), dtype=torch.int32, device=dev)
        status = lib.specv_verify_debug(*args, _ptr(res["accept_prob"]), _ptr(res["residual_mass"]),
                                        _ptr(res["stop_pos"]), _ptr(res["path"]))
    else:
        status = lib.specv_verify(*args)
    if status != SPECV_OK:
        raise SpecVerifyError(status, status_string(status))
    return res


def verify_noalloc(target_logits, draft_logits, draft_tokens, draft_len, u, u_final,
                   temperature=1.0, top_k=0, top_p=1.0, eos_id=-1, *, out_tokens, n_emitted,
                   stream=None):
    """``specv_verify_noalloc``: the verification step with the library's fixed
    device scratch instead of a workspace.  The outputs must be passed in;
    nothing is allocated.  Same shapes and dtypes as ``verify``."""
    lib = load_library()
    dev = target_logits.device
    if dev.type != "cuda" or target_logits.dim() != 3:
        raise ValueError("target_logits must be a [B, K+1, V] GPU tensor")
    B, K1, V = target_logits.shape
    K = K1 - 1
    code = _dtype_code(target_logits)
    _check(target_logits, "target_logits", None, (B, K + 1, V), dev)
    _check(draft_logits, "draft_logits", target_logits.dtype, (B, K, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _check(draft_len, "draft_len", torch.int32, (B,), dev)
    _check(u, "u", torch.float32, (B, K), dev)
    _check(u_final, "u_final", torch.float32, (B,), dev)
    _check(out_tokens, "out_tokens", torch.int32, (B, K + 1), dev)
    _check(n_emitted, "n_emitted", torch.int32, (B,), dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    status = lib.specv_verify_noalloc(
        _ptr(target_logits), _ptr(draft_logits), code, _ptr(draft_tokens), _ptr(draft_len),
        _ptr(u), _ptr(u_final), B, K, V, float(temperature), int(top_k), float(top_p),
        int(eos_id), _ptr(out_tokens), _ptr(n_emitted), ctypes.c_void_p(stream.cuda_stream))
    if status != SPECV_OK:
        raise SpecVerifyError(status, status_string(status))
    return {"out_tokens": out_tokens, "n_emitted": n_emitted}


class PackedLmHeadWeight:
    """An LM-head weight [V, D] bf16 in the layout the fused call reads
    (``specv_lm_head_pack_weight``): ``data`` is the packed device buffer."""

    def __init__(self, data, V, D):
        self.data, self.V, self.D = data, int(V), int(D)


def lm_head_packed_weight_bytes(V, D):
    return int(load_library().specv_lm_head_packed_weight_bytes(int(V), int(D)))


def pack_lm_head_weight(weight, stream=None):
    """Repack an LM-head weight [V, D] bf16 (GPU) once for ``verify_lm_head``;
    asynchronous on ``stream``."""
    lib = load_library()
    if weight.device.type != "cuda" or weight.dim() != 2:
        raise ValueError("weight must be a [V, D] GPU tensor")
    V, D = weight.shape
    _check(weight, "weight", torch.bfloat16, (V, D), weight.device)
    nbytes = lm_head_packed_weight_bytes(V, D)
    if nbytes == 0:
        raise SpecVerifyError(SPECV_EINVAL, f"unsupported LM-head shape V={V} D={D}")
    data = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=weight.device)
    if stream is None:
        stream = torch.cuda.current_stream(weight.device)
    st = lib.specv_lm_head_pack_weight(_ptr(weight), _ptr(data), V, D,
                                       ctypes.c_void_p(stream.cuda_stream))
    if st != SPECV_OK:
        raise SpecVerifyError(st, status_string(st))
    return PackedLmHeadWeight(data, V, D)


def lm_head_workspace_bytes(B, K, V, D, top_k=0, top_p=1.0):
    return int(load_library().specv_lm_head_workspace_bytes(int(B), int(K), int(V), int(D),
                                                            int(top_k), float(top_p)))


def verify_lm_head(hidden, packed_weight, draft_logits, draft_tokens, draft_len, u, u_final,
                   temperature=1.0, eos_id=-1, *, top_k=0, top_p=1.0, target_logits=None,
                   out_tokens=None, n_emitted=None, workspace=None, debug=False, stream=None):
    """The verification step fused with the target model's LM head.

    Shapes: hidden [B, K+1, D] bf16 (the target model's final hidden states),
    packed_weight a ``PackedLmHeadWeight`` (``pack_lm_head_weight`` of the
    [V, D] bf16 weight), draft_logits [B, K, V] bf16, draft_tokens
    [B, K] int32, draft_len [B] int32, u [B, K] fp32, u_final [B] fp32; D a
    multiple of 64.  Returns a dict with ``target_logits`` [B, K+1, V] bf16
    (the LM head's output), ``out_tokens`` and ``n_emitted``, plus the
    ``verify`` diagnostics when ``debug`` is true.  Asynchronous on
    ``stream``."""
    lib = load_library()
    dev = hidden.device
    if dev.type != "cuda" or hidden.dim() != 3 or not isinstance(packed_weight, PackedLmHeadWeight):
        raise ValueError("hidden must be a [B, K+1, D] GPU tensor and packed_weight a "
                         "PackedLmHeadWeight")
    B, K1, D = hidden.shape
    K = K1 - 1
    V = packed_weight.V
    if packed_weight.D != D:
        raise ValueError(f"packed weight has D={packed_weight.D}, hidden D={D}")
    bf = torch.bfloat16
    _check(hidden, "hidden", bf, (B, K + 1, D), dev)
    _check(packed_weight.data, "packed_weight", bf, (lm_head_packed_weight_bytes(V, D) // 2,), dev)
    _check(draft_logits, "draft_logits", bf, (B, K, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _check(draft_len, "draft_len", torch.int32, (B,), dev)
    _check(u, "u", torch.float32, (B, K), dev)
    _check(u_final, "u_final", torch.float32, (B,), dev)
    if target_logits is None:
        target_logits = torch.empty((B, K + 1, V), dtype=bf, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    if n_emitted is None:
        n_emitted = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(target_logits, "target_logits", bf, (B, K + 1, V), dev)
    _check(out_tokens, "out_tokens", torch.int32, (B, K + 1), dev)
    _check(n_emitted, "n_emitted", torch.int32, (B,), dev)
    nbytes = lm_head_workspace_bytes(B, K, V, D, top_k, top_p)
    if workspace is None:
        workspace = _workspace(dev, nbytes)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    res = {"target_logits": target_logits, "out_tokens": out_tokens, "n_emitted": n_emitted}
    diag = [None, None, None, None]
    if debug:
        res["accept_prob"] = torch.empty((B, K), dtype=torch.float32, device=dev)
        res["residual_mass"] = torch.empty((B,), dtype=torch.float64, device=dev)
        res["stop_pos"] = torch.empty((B,), dtype=torch.int32, device=dev)
        res["path"] = torch.empty((B,), dtype=torch.int32, device=dev)
        diag = [res["accept_prob"], res["residual_mass"], res["stop_pos"], res["path"]]
    st = lib.specv_verify_lm_head(_ptr(hidden), _ptr(packed_weight.data), _ptr(draft_logits),
                                  _ptr(draft_tokens), _ptr(draft_len), _ptr(u), _ptr(u_final), B,
                                  K, V, D, float(temperature), int(top_k), float(top_p),
                                  int(eos_id), _ptr(target_logits),
                                  _ptr(out_tokens), _ptr(n_emitted), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(),
                                  ctypes.c_void_p(stream.cuda_stream), *[_ptr(t) for t in diag])
    if st != SPECV_OK:
        raise SpecVerifyError(st, status_string(st))
    return res


def bench_lm_head(hidden, packed_weight, logits, workspace, reps, temperature=1.0, stream=None,
                  start=None, stop=None):
    """Benchmark hook: the LM-head kernel alone (hidden [M, D] and logits
    [M, V] bf16, a ``PackedLmHeadWeight``), ``reps`` launches between the HIP
    events ``start`` and ``stop`` (raw handles) recorded on ``stream``."""
    lib = load_library()
    M, D = hidden.shape
    V = packed_weight.V
    if packed_weight.D != D:
        raise ValueError(f"packed weight has D={packed_weight.D}, hidden D={D}")
    if stream is None:
        stream = torch.cuda.current_stream(hidden.device)
    st = lib.specv_bench_lm_head(_ptr(hidden), _ptr(packed_weight.data), M, D, V, float(temperature),
                                 _ptr(logits), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), int(reps),
                                 ctypes.c_void_p(stream.cuda_stream), start, stop)
    if st != SPECV_OK:
        raise SpecVerifyError(st, status_string(st))
