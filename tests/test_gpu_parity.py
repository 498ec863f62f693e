"""Parity of the HIP path with the fp64 oracle, through the C ABI (GPU only).

Bars: tokens and counts bit-exact except where the oracle flags a decision
as within rounding reach; accept probabilities and residual masses within
1e-5 absolute.  Sizes keep the oracle to seconds yet span many chunks and a
ragged tail (V is never a multiple of the chunk sizes used here).
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
from speculative_decoding_sampling_amd import binding  # noqa: E402
from speculative_decoding_sampling_amd.workloads import f32, make_workload, upload  # noqa: E402
from tests.parity import compare, flag_ceiling, to_numpy  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(params=["four_kernel", "one_kernel_tail"])
def unfiltered_path(request):
    """Runs a test on each unfiltered path: the four-kernel path (the
    small-batch limit at 0) and the small-batch tail (the limit so large
    that every unfiltered call takes it)."""
    old = binding.set_small_batch_limit(0 if request.param == "four_kernel" else 1 << 40)
    yield request.param
    binding.set_small_batch_limit(old)


def oracle_sampler(z, T, k, p, uni):
    P, _ = O.processed_distribution(z, f32(T), k, f32(p))
    return O.icdf(P, uni)[0]


def run_gpu(w, **kw):
    args = upload(w, DEV)
    args.update(kw)
    res = binding.verify(**args, debug=True)
    torch.cuda.synchronize()
    return to_numpy(res)


def run_oracle(w, requests=None, **kw):
    p = dict(temperature=w.T, top_k=w.top_k, top_p=w.top_p, eos_id=w.eos_id)
    p.update(kw)
    # The call receives temperature and top_p as float32; the oracle gets the same values.
    return O.verify(w.target, w.draft, w.draft_tokens, w.draft_len, w.u, w.u_final,
                    f32(p["temperature"]), p["top_k"], f32(p["top_p"]), p["eos_id"], w.dtype,
                    requests=requests)


def assert_parity(w, requests=None, label="", check_flags=True):
    """GPU against oracle on one workload; unless the case forces near-ties on
    purpose (check_flags=False), the oracle may flag at most
    flag_ceiling(positions) requests (checked by compare)."""
    print(f"[parity] cfg={w.cfg} seed={w.seed} B={w.B} K={w.K} V={w.V} {w.dtype} {label}",
          flush=True)
    g = run_gpu(w)
    o = run_oracle(w, requests)
    rep = compare(g, o, w.K, check_flags=check_flags)
    print(f"  requests={rep['requests']} positions={rep['positions']} flagged={rep['flagged']} "
          f"kinds={rep['flag_kinds']} max_alpha_err={rep['max_alpha_err']:.2e} "
          f"max_mass_err={rep['max_mass_err']:.2e}", flush=True)
    assert not rep["mismatches"], rep["mismatches"][:5]
    return rep, g, o


@pytest.mark.parametrize("cfg,B", [(1, None), (2, None), (3, 8), (5, 16)])
def test_parity_reduced_batch(cfg, B, unfiltered_path):
    assert_parity(make_workload(cfg, B=B))


@pytest.mark.parametrize("cfg", [1, 2])
def test_parity_seed_sweep(cfg):
    flagged = positions = 0
    for i in range(12):
        rep, _, _ = assert_parity(make_workload(cfg, seed=1000 + cfg + 100 * i))
        flagged += rep["flagged"]
        positions += rep["positions"]
    print(f"  sweep cfg={cfg}: flagged {flagged} of {positions} positions")


@pytest.mark.parametrize("cfg", [3, 5])
def test_parity_full_size(cfg):
    w = make_workload(cfg)
    rep, g, o = assert_parity(w, label="full size")
    # every request took one of the four paths and emitted a sane count
    n = g["n_emitted"]
    assert np.all((n == -1) | ((n >= 1) & (n <= w.draft_len + 1)))


@pytest.mark.parametrize("cfg,B", [(1, None), (2, None), (3, 8), (5, 16)])
def test_small_batch_tail_equals_four_kernel_path(cfg, B):
    # The same inputs through both unfiltered paths: the small-batch tail runs
    # the same accept scan, chunk pass and draw code on the same row
    # statistics, so every output agrees (the residual mass up to the order
    # of float64 sums, which is the same too).  Workload 5 brings ragged
    # lengths, p == q requests and EOS; the default limit puts workloads 1
    # and 2 on the tail.
    w = make_workload(cfg, B=B)
    print(f"[tail] cfg={cfg} B={w.B} K={w.K} V={w.V} kind="
          f"{binding.path_kind(w.B, w.K, w.V)}", flush=True)
    if cfg in (1, 2):
        assert binding.path_kind(w.B, w.K, w.V) == 3
    old = binding.set_small_batch_limit(0)
    try:
        four = run_gpu(w)
        binding.set_small_batch_limit(1 << 40)
        tail = run_gpu(w)
    finally:
        binding.set_small_batch_limit(old)
    for k in ("out_tokens", "n_emitted", "stop_pos", "path", "accept_prob"):
        assert np.array_equal(four[k], tail[k], equal_nan=True), k
    rel = np.abs(four["residual_mass"] - tail["residual_mass"]) / np.maximum(
        np.abs(four["residual_mass"]), 1e-300)
    assert np.all(rel <= 1e-12), float(rel.max())
    rep = compare(tail, run_oracle(w), w.K)
    assert not rep["mismatches"], rep["mismatches"][:3]


def test_small_path_shares_one_workspace_across_sizes():
    # The one-kernel small-batch path publishes row statistics and chunk-pass
    # records through tagged words that no call clears.  One zeroed workspace
    # (every request's call counter starting equal) serves, in turn,
    # verifications of two sizes whose draft lengths change from call to call
    # and draft-side sampling calls of a third size; every call must match the
    # oracle, so no word left by another call -- of these sizes or of others
    # -- passes for one of the current call's.
    w1, w2 = make_workload(1), make_workload(2)
    for w in (w1, w2):
        assert binding.path_kind(w.B, w.K, w.V) == 3
    R = w1.B * w1.K
    assert binding.path_kind(R, 0, w1.V) == 3
    nbytes = max(binding.workspace_bytes(w1.B, w1.K, w1.V, torch.float32),
                 binding.workspace_bytes(w2.B, w2.K, w2.V, torch.bfloat16),
                 binding.workspace_bytes(R, 0, w1.V, torch.float32))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(77)
    drows = upload(w1, DEV)["draft_logits"].reshape(R, w1.V)
    for step in range(6):
        for w in (w1, w2):
            # every drafted token was drawn from q, so any length up to K is valid
            w.draft_len = rng.integers(0, w.K + 1, size=w.B).astype(np.int32)
            print(f"[share] step={step} cfg={w.cfg} draft_len={w.draft_len.tolist()}", flush=True)
            g = to_numpy(binding.verify(**upload(w, DEV), workspace=ws, debug=True))
            torch.cuda.synchronize()
            rep = compare(g, run_oracle(w), w.K)
            assert not rep["mismatches"], (step, w.cfg, rep["mismatches"][:3])
        un = ((rng.integers(0, 1 << 24, size=R)) * 2.0 ** -24).astype(np.float32)
        tok = binding.sample(drows, torch.from_numpy(un).to(DEV), w1.T, workspace=ws)
        torch.cuda.synchronize()
        ref, fk = oracle_sample(w1.draft.reshape(R, w1.V), un, w1.T, 0, 1.0, w1.dtype)
        sure = fk == O.FLAG_NONE
        assert np.array_equal(tok.cpu().numpy()[sure], ref[sure]), step


def test_small_path_waits_that_run_out_are_request_errors():
    # The one-kernel path bounds every wait between its workgroups; a wait that
    # runs out makes its request an error instead of hanging.  A test hook caps
    # the polls at one, so most waits run out (every kernel still ends
    # normally): each request is then an error (every output -1) or the
    # oracle's.  The draws of such a call advance their call counters while
    # workgroups of the request may not yet have read them, so those tag their
    # words with the advanced counter; the next eager call on the same
    # workspace, polling normally, must still match the oracle everywhere.
    import ctypes
    lib = binding.load_library()
    lib.specv_selftest_set_small_poll_limit.restype = ctypes.c_int
    lib.specv_selftest_set_small_poll_limit.argtypes = [ctypes.c_int]
    w = make_workload(1)
    assert binding.path_kind(w.B, w.K, w.V) == 3
    ws = torch.zeros(binding.workspace_bytes(w.B, w.K, w.V, torch.float32), dtype=torch.uint8,
                     device=DEV)
    ora = run_oracle(w)
    old = lib.specv_selftest_set_small_poll_limit(1)
    try:
        print("[timeout] one poll per wait", flush=True)
        g = to_numpy(binding.verify(**upload(w, DEV), workspace=ws, debug=True))
        torch.cuda.synchronize()
    finally:
        lib.specv_selftest_set_small_poll_limit(old)
    err = g["n_emitted"] == -1
    print(f"[timeout] {int(err.sum())} of {w.B} requests timed out", flush=True)
    for b in np.nonzero(err)[0]:
        assert np.all(g["out_tokens"][b] == -1) and g["path"][b] == -1, b
    rep = compare(g, ora, w.K)
    assert all(m[0] in set(np.nonzero(err)[0].tolist()) for m in rep["mismatches"]), \
        rep["mismatches"][:3]
    for step in range(3):
        print(f"[timeout] normal call {step}", flush=True)
        g = to_numpy(binding.verify(**upload(w, DEV), workspace=ws, debug=True))
        torch.cuda.synchronize()
        rep = compare(g, ora, w.K)
        assert not rep["mismatches"], (step, rep["mismatches"][:3])


def test_p_equals_q_is_always_bonus_with_alpha_exactly_one(unfiltered_path):
    # EOS off: with p == q an accepted draft may itself be the EOS token.
    w = make_workload(5, B=16)
    w.draft[:] = w.target[:, :w.K]
    g = run_gpu(w, eos_id=-1)
    assert np.array_equal(g["path"], np.full(w.B, binding.PATH_BONUS))
    assert np.array_equal(g["n_emitted"], w.draft_len + 1)
    for b in range(w.B):
        assert np.all(g["accept_prob"][b, :w.draft_len[b]] == 1.0)
    rep = compare(g, run_oracle(w, eos_id=-1), w.K)
    assert not rep["mismatches"], rep["mismatches"][:3]


def test_deterministic_bitwise(unfiltered_path):
    w = make_workload(3, B=8)
    a, b = run_gpu(w), run_gpu(w)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k


def test_per_request_errors_are_isolated(unfiltered_path):
    w = make_workload(1)
    w.draft_len[0] = 5                       # draft_len > K
    w.draft_len[1] = -1                      # negative draft_len
    w.draft_tokens[2, 3] = w.V               # token out of range
    w.u[3, 1] = 1.0                          # uniform outside [0, 1)
    w.u_final[4] = np.nan                    # final uniform not a number
    w.draft[5, 2, w.draft_tokens[5, 2]] = -np.inf   # q(x) == 0
    g = run_gpu(w)
    for b in range(6):
        assert g["n_emitted"][b] == -1 and np.all(g["out_tokens"][b] == -1)
        assert g["path"][b] == binding.PATH_ERROR
    rep = compare(g, run_oracle(w), w.K)
    assert not rep["mismatches"], rep["mismatches"][:3]


def test_draft_len_zero_and_k_zero(unfiltered_path):
    w = make_workload(1)
    w.draft_len[:] = 0
    assert_parity(w, label="draft_len=0")
    # K = 0: only the bonus row exists
    t = torch.from_numpy(w.target[:, :1].copy()).to(DEV)
    d = torch.empty((w.B, 0, w.V), dtype=torch.float32, device=DEV)
    res = binding.verify(t, d, torch.empty((w.B, 0), dtype=torch.int32, device=DEV),
                         torch.zeros(w.B, dtype=torch.int32, device=DEV),
                         torch.empty((w.B, 0), dtype=torch.float32, device=DEV),
                         torch.from_numpy(w.u_final).to(DEV), 1.0, debug=True)
    torch.cuda.synchronize()
    o = O.verify(w.target[:, :1], w.draft[:, :0], w.draft_tokens[:, :0], np.zeros(w.B, np.int32),
                 w.u[:, :0], w.u_final, 1.0)
    assert np.array_equal(res["out_tokens"].cpu().numpy(), o["out_tokens"])
    assert np.array_equal(res["n_emitted"].cpu().numpy(), o["n_emitted"])


@pytest.mark.parametrize("V", [1, 3, 4097, 10007])
def test_unaligned_and_tiny_vocabularies(V, unfiltered_path):
    rng = np.random.default_rng(V)
    B, K = 6, 3
    t = rng.normal(0, 2, size=(B, K + 1, V)).astype(np.float32)
    d = (t[:, :K] + rng.normal(0, 0.6, size=(B, K, V))).astype(np.float32)
    toks = np.array([[int(np.argmax(d[b, k] + rng.gumbel(size=V))) for k in range(K)]
                     for b in range(B)], dtype=np.int32)
    from speculative_decoding_sampling_amd.workloads import Workload, to_bf16_bits, uniforms
    for dtype in ("f32", "bf16"):
        tt = to_bf16_bits(t) if dtype == "bf16" else t
        dd = to_bf16_bits(d) if dtype == "bf16" else d
        w = Workload(cfg=0, seed=V, B=B, K=K, V=V, dtype=dtype, T=f32(0.9), top_k=0, top_p=1.0,
                     eos_id=-1, target=np.ascontiguousarray(tt), draft=np.ascontiguousarray(dd),
                     draft_tokens=toks, draft_len=np.array([3, 2, 1, 0, 3, 3], np.int32),
                     u=uniforms(rng, (B, K)), u_final=uniforms(rng, (B,)))
        assert_parity(w, label=f"V={V}")


def _custom_workload(t, d, draft_len, rng, dtype="f32", T=1.0, seed=0):
    from speculative_decoding_sampling_amd.workloads import Workload, to_bf16_bits, uniforms
    B, K1, V = t.shape
    K = K1 - 1
    # draft tokens drawn from the draft rows (Gumbel-max on z / T)
    toks = np.array([[int(np.argmax(d[b, k] / np.float32(T) + rng.gumbel(size=V)))
                      for k in range(K)] for b in range(B)], dtype=np.int32).reshape(B, K)
    tt = to_bf16_bits(t) if dtype == "bf16" else t
    dd = to_bf16_bits(d) if dtype == "bf16" else d
    return Workload(cfg=0, seed=seed, B=B, K=K, V=V, dtype=dtype, T=f32(T), top_k=0, top_p=1.0,
                    eos_id=-1, target=np.ascontiguousarray(tt), draft=np.ascontiguousarray(dd),
                    draft_tokens=toks, draft_len=np.asarray(draft_len, np.int32),
                    u=uniforms(rng, (B, K)), u_final=uniforms(rng, (B,)))


def test_maximum_draft_length(unfiltered_path):
    # K = 64, the largest draft length the call takes (SPECV_MAX_K): drafts
    # close to the target so the first-rejection scan runs deep, one request
    # whose draft rows equal its target rows (every draft accepted, then the
    # bonus draw from target row 64, which has no scan lane of its own), and
    # ragged lengths from 0 to 64
    rng = np.random.default_rng(64)
    B, K, V = 6, 64, 1500
    t = rng.normal(0, 2, size=(B, K + 1, V)).astype(np.float32)
    d = (t[:, :K] + rng.normal(0, 0.03, size=(B, K, V))).astype(np.float32)
    d[1] = t[1, :K]
    w = _custom_workload(t, d, [64, 64, 40, 0, 63, 17], rng, seed=64)
    rep, g, o = assert_parity(w, label="K=64")
    assert o["path"][1] == O.PATH_BONUS and o["n_emitted"][1] == 65
    # a rejection in the upper half of the 64-lane scan
    assert any(o["path"][b] == O.PATH_REJECT and o["stop_pos"][b] >= 32 for b in range(B))


def test_maximum_draft_length_filtered():
    # K = 64 on the top-k / top-p path: the scan reads the bonus row's
    # filtered statistics apart from the 64 lanes' rows.
    rng = np.random.default_rng(65)
    B, K, V = 4, 64, 3000
    t = rng.normal(0, 2, size=(B, K + 1, V)).astype(np.float32)
    d = (t[:, :K] + rng.normal(0, 0.02, size=(B, K, V))).astype(np.float32)
    d[0] = t[0, :K]
    w = _custom_workload(t, d, [64, 64, 31, 64], rng, seed=65)
    w.top_k, w.top_p = 30, f32(0.9)
    redraw_tokens(w, 65)
    rep, g, o = assert_parity(w, label="K=64 filtered")
    assert o["path"][0] == O.PATH_BONUS and o["n_emitted"][0] == 65


def test_maximum_vocabulary():
    # V = 4194304, the largest vocabulary the call takes (SPECV_MAX_V): the
    # sampler's 2048-token chunks reach their table limit of 2048 per row
    rng = np.random.default_rng(22)
    B, K, V = 2, 2, 1 << 22
    t = rng.normal(0, 2, size=(B, K + 1, V)).astype(np.float32)
    d = (t[:, :K] + rng.normal(0, 0.7, size=(B, K, V)).astype(np.float32)).astype(np.float32)
    w = _custom_workload(t, d, [2, 1], rng, dtype="bf16", seed=22)
    assert_parity(w, label="V=2^22")


@pytest.mark.parametrize("V", [4097, 10007, 20011])
def test_unaligned_vocabularies_filtered(V):
    # Rows that are not 16-byte aligned and a ragged last chunk on the top-k /
    # top-p path (the candidate pass's element loads), drafts drawn from the
    # filtered draft distribution.
    rng = np.random.default_rng(V + 1)
    B, K, top_k, top_p = 5, 3, 20, 0.9
    t = rng.normal(0, 2, size=(B, K + 1, V)).astype(np.float32)
    d = (t[:, :K] + rng.normal(0, 0.6, size=(B, K, V))).astype(np.float32)
    from speculative_decoding_sampling_amd.workloads import Workload, to_bf16_bits, uniforms
    for dtype in ("f32", "bf16"):
        tt = to_bf16_bits(t) if dtype == "bf16" else t
        dd = to_bf16_bits(d) if dtype == "bf16" else d
        uni = uniforms(rng, (B, K))
        toks = np.array([[oracle_sampler(O.widen_row(dd[b, k], dtype), f32(0.9), top_k,
                                         f32(top_p), float(uni[b, k])) for k in range(K)]
                         for b in range(B)], dtype=np.int32)
        w = Workload(cfg=0, seed=V, B=B, K=K, V=V, dtype=dtype, T=f32(0.9), top_k=top_k,
                     top_p=f32(top_p), eos_id=-1, target=np.ascontiguousarray(tt),
                     draft=np.ascontiguousarray(dd), draft_tokens=toks,
                     draft_len=np.array([3, 2, 1, 0, 3], np.int32),
                     u=uniforms(rng, (B, K)), u_final=uniforms(rng, (B,)))
        assert_parity(w, label=f"V={V} filtered {dtype}")


def test_exhaustive_cells_match_oracle():
    # Thousands of random V=3, K=2 requests over the worked example's
    # distributions: tokens must match the oracle request for request.
    p_rows = [np.array([0.5, 0.3, 0.2]), np.array([0.1, 0.6, 0.3]), np.array([0.25, 0.25, 0.5])]
    q_rows = [np.array([0.6, 0.1, 0.3]), np.array([0.3, 0.3, 0.4])]
    K, V = 2, 3
    rng = np.random.default_rng(0)
    B = 4000
    toks = rng.integers(0, V, size=(B, K)).astype(np.int32)
    u = rng.random((B, K)).astype(np.float32)
    uf = rng.random(B).astype(np.float32)
    t = np.broadcast_to(np.log(np.array(p_rows, dtype=np.float32)), (B, K + 1, V)).copy()
    d = np.broadcast_to(np.log(np.array(q_rows, dtype=np.float32)), (B, K, V)).copy()
    from speculative_decoding_sampling_amd.workloads import Workload
    w = Workload(cfg=0, seed=0, B=B, K=K, V=V, dtype="f32", T=1.0, top_k=0, top_p=1.0,
                 eos_id=-1, target=t, draft=d, draft_tokens=toks,
                 draft_len=np.full(B, K, np.int32), u=u, u_final=uf)
    assert_parity(w, label="tiny-V exhaustive")


def test_host_argument_errors():
    w = make_workload(1)
    a = upload(w, DEV)
    bad = [
        dict(temperature=0.0), dict(temperature=-1.0), dict(temperature=float("inf")),
        dict(top_p=0.0), dict(top_p=1.5), dict(top_k=-1), dict(eos_id=w.V), dict(eos_id=-2),
    ]
    for kw in bad:
        args = dict(a)
        args.update(kw)
        with pytest.raises(binding.SpecVerifyError) as e:
            binding.verify(**args)
        assert e.value.status == binding.SPECV_EINVAL, kw
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(binding.SpecVerifyError) as e:
        binding.verify(**a, workspace=small)
    assert e.value.status == binding.SPECV_EWORKSPACE


def test_exp64_against_numpy():
    # The sampler's float64 exp (table-driven, Tang 1989; N = 512, cubic, one
    # FMA argument reduction) against numpy's exp: relative error below
    # 1e-14 + |x| * 1.2e-16 (its stated bound, plus 2 ulp for numpy's own
    # rounding), and 0 at and below -745.2.
    rng = np.random.default_rng(5)
    x = np.concatenate([-rng.random(400000) * 745.0, -rng.random(200000) * 40.0,
                        -rng.random(50000) * 1e-3, rng.random(50000) * 700.0,
                        [0.0, -0.0, -1e-300, -708.39, -709.0, -744.0, -745.0]])
    y = binding.selftest_exp64(torch.from_numpy(x).to(DEV)).cpu().numpy()
    ref = np.exp(x)
    normal = ref > 2.3e-308
    rel = np.abs(y[normal] - ref[normal]) / ref[normal]
    bound = 1e-14 + np.abs(x[normal]) * 1.2e-16 + 4.5e-16
    near = x[normal] >= -40.0
    print(f"  exp64: max rel {rel.max():.3g}; over x >= -40: {rel[near].max():.3g}; "
          f"max rel/bound {(rel / bound).max():.3f} over {normal.sum()} values")
    assert np.all(rel <= bound)
    sub = ~normal
    sub_bound = (1e-14 + np.abs(x[sub]) * 1.2e-16) * ref[sub] + 2 * 5e-324   # subnormal grid
    assert np.all(np.abs(y[sub] - ref[sub]) <= sub_bound)
    z = binding.selftest_exp64(torch.tensor([-np.inf, -746.0, -1e6], dtype=torch.float64,
                                            device=DEV)).cpu().numpy()
    assert np.all(z == 0.0)


def test_sampler_exact_path_with_many_near_ties(unfiltered_path):
    # Draft = target + N(0, 1e-4^2): nearly every token is a near tie, so the
    # chunks overflow their tie slots and the sampler takes its exact path.
    # u close to 1 forces rejections whenever p(x) < q(x).
    w = make_workload(3, B=8)
    from speculative_decoding_sampling_amd.workloads import from_bf16_bits
    rng = np.random.default_rng(9)
    t = from_bf16_bits(w.target).astype(np.float32)
    w.dtype = "f32"
    w.target = np.ascontiguousarray(t)
    w.draft = np.ascontiguousarray(t[:, :w.K] + rng.normal(0, 1e-4, size=t[:, :w.K].shape)
                                   .astype(np.float32))
    w.u[:] = np.float32(1.0 - 2.0 ** -24)
    rep, g, o = assert_parity(w, label="near-identical rows", check_flags=False)
    assert (o["path"] == O.PATH_REJECT).sum() >= 4


# ---------------------------------------------------------------------------
# top-k / top-p path
# ---------------------------------------------------------------------------

def redraw_tokens(w, seed):
    """Draft tokens from the processed draft distribution (the oracle's)."""
    from speculative_decoding_sampling_amd.workloads import uniforms
    rng = np.random.default_rng(seed)
    uni = uniforms(rng, (w.B, w.K))
    for b in range(w.B):
        for k in range(w.K):
            z = O.widen_row(w.draft[b, k], w.dtype)
            w.draft_tokens[b, k] = oracle_sampler(z, w.T, w.top_k, w.top_p, float(uni[b, k]))


def test_parity_topk_topp_reduced():
    w = make_workload(4, B=12, draft_sampler=oracle_sampler)
    rep, g, o = assert_parity(w)
    assert rep["positions"] > 0


def test_parity_topk_topp_with_eos():
    # EOS on the filtered path. The EOS id is the token the oracle accepts
    # furthest into some request's draft, so that request must stop there
    # on the EOS path rather than run on to a rejection or the bonus token.
    w = make_workload(4, B=16, draft_sampler=oracle_sampler)
    o0 = run_oracle(w, eos_id=-1)
    # without an EOS id every request ends on a rejection or the bonus token,
    # and its last accepted draft position is one before its stop position
    j, b = max((int(o0["stop_pos"][b]) - 1, b) for b in range(w.B))
    assert j >= 0, "no request accepts any draft token"
    w.eos_id = int(o0["out_tokens"][b, j])
    rep, g, o = assert_parity(w, label=f"filtered, eos={w.eos_id} at b={b} pos={j}")
    assert o["path"][b] == O.PATH_EOS and o["stop_pos"][b] <= j


def test_parity_topk_topp_full_size_sampled():
    w = make_workload(4, draft_sampler=oracle_sampler)          # B=256, K=8, V=152064 fp32
    rep, g, o = assert_parity(w, requests=list(range(0, w.B, 5)), label="full size, sampled")
    assert rep["requests"] == len(range(0, w.B, 5))


@pytest.mark.parametrize("top_k,top_p", [(40, 1.0), (7, 0.8), (128, 0.95), (1, 1.0)])
def test_parity_topk_bf16_with_ties(top_k, top_p):
    # bf16 logits repeat values, so the k-th logit is often tied: all ties stay.
    w = make_workload(3, B=6)
    w.top_k, w.top_p, w.T = top_k, f32(top_p), f32(0.9)
    redraw_tokens(w, top_k)
    assert_parity(w, label=f"bf16 top_k={top_k} top_p={top_p}")


def test_parity_filtered_ragged_bf16_with_eos():
    # the mixed-batch workload (ragged draft lengths, drafts equal to or far
    # from the target, bf16) through the top-k/top-p path, with an EOS id the
    # oracle accepts mid-draft
    w = make_workload(5, B=16)
    w.top_k, w.top_p, w.T = 40, f32(0.92), f32(0.8)
    redraw_tokens(w, 5)
    o0 = run_oracle(w, eos_id=-1)
    j, b = max((int(o0["stop_pos"][b]) - 1, b) for b in range(w.B))
    assert j >= 1, "no request accepts two draft tokens"
    w.eos_id = int(o0["out_tokens"][b, j])
    rep, g, o = assert_parity(w, label=f"filtered, eos={w.eos_id} at b={b} pos={j}")
    assert o["path"][b] == O.PATH_EOS and o["stop_pos"][b] <= j
    assert len(set(w.draft_len.tolist())) > 1


def test_filter_capacity_overflow_matches_oracle():
    # A row whose logits are all equal keeps every token under top-k (ties
    # kept): its 8192-token chunks hold far more candidates than their slots,
    # so the candidate merge hands the row to the radix select, and the kept
    # set (all 152064 tokens) is far beyond the kept list, so the draw is
    # streamed over the row.  Every request must still match the oracle.
    w = make_workload(4, B=4, draft_sampler=oracle_sampler)
    w.target[2, 0, :] = 0.0
    w.draft_tokens[2, 0] = int(np.argmax(w.draft[2, 0]))    # a draft token q keeps
    rep, g, o = assert_parity(w, label="all-equal target row")
    assert o["n_emitted"][2] > 0 and g["n_emitted"][2] == o["n_emitted"][2]


# ---------------------------------------------------------------------------
# top-k / top-p through the radix select: top-p alone, large top-k, kept sets
# beyond the 512-token list (streamed draws)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,B,top_k,top_p", [
    (3, 8, 0, 0.9),          # top-p alone, bf16 V=128256 (thousands of tokens kept)
    (4, 6, 0, 0.9),          # top-p alone, fp32 V=152064
    (3, 6, 1000, 1.0),       # top-k 1000 alone: 1000 kept, beyond the list
    (4, 6, 1000, 0.95),      # top-k 1000 then top-p
    (1, None, 300, 0.8),     # fp32 V=4096
    (2, 1, 0, 0.5),          # B=1, bf16 V=32000
])
def test_parity_radix_select(cfg, B, top_k, top_p):
    from speculative_decoding_sampling_amd import binding as bd
    w = make_workload(cfg, B=B, draft_sampler=oracle_sampler)
    w.top_k, w.top_p = top_k, f32(top_p)
    assert bd.path_kind(w.B, w.K, w.V, w.top_k, w.top_p) == 2
    redraw_tokens(w, 100 + cfg)
    rep, g, o = assert_parity(w, label=f"radix select top_k={top_k} top_p={top_p}")
    assert rep["positions"] > 0


def test_parity_radix_select_kept_sets_of_every_size():
    # top-p over rows whose spread differs request by request, so kept sets
    # run from one token to most of the vocabulary, on both sides of the list
    # size; ties from bf16 rounding and -inf masks in some rows.
    rng = np.random.default_rng(77)
    B, K, V = 8, 3, 20011
    scale = np.array([0.05, 0.5, 1.0, 2.0, 4.0, 8.0, 16.0, 0.2], dtype=np.float32)
    t = (rng.normal(0, 1, size=(B, K + 1, V)).astype(np.float32) * scale[:, None, None])
    d = (t[:, :K] + rng.normal(0, 0.3, size=(B, K, V)).astype(np.float32) * scale[:, None, None])
    t[1, :, rng.random(V) < 0.5] = -np.inf
    d[1, :, :] = np.where(np.isinf(t[1, :K]), -np.inf, d[1])
    w = _custom_workload(t, d.astype(np.float32), [3, 3, 2, 3, 1, 3, 0, 3], rng, dtype="bf16",
                         T=0.9, seed=77)
    w.top_k, w.top_p = 0, f32(0.95)
    redraw_tokens(w, 77)
    rep, g, o = assert_parity(w, label="kept sets of every size")
    P, _ = O.processed_distribution(O.widen_row(w.target[0, 0], "bf16"), f32(0.9), 0, f32(0.95))
    Q, _ = O.processed_distribution(O.widen_row(w.target[6, 0], "bf16"), f32(0.9), 0, f32(0.95))
    assert (P > 0).sum() > 512 and (Q > 0).sum() < 512


def test_radix_select_deterministic_bitwise():
    w = make_workload(4, B=4, draft_sampler=oracle_sampler)
    w.top_k, w.top_p = 0, f32(0.9)
    redraw_tokens(w, 9)
    a, b = run_gpu(w), run_gpu(w)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k


def test_many_draws_large_vocabulary_non_unit_temperature():
    # ~1000 inverse-CDF draws over V = 32000 at T = 0.8: a draw moves if the
    # two sides' CDFs differ by more than about 1e-10, e.g. through a
    # temperature that is not the same float on both sides.
    w = make_workload(2, B=1024)
    rep, g, o = assert_parity(w, label="1024 draws")
    assert rep["requests"] == 1024


@pytest.mark.parametrize("cfg,B,top_k,top_p", [(3, 8, None, None), (4, 6, None, None),
                                              (3, 6, 0, 0.9), (4, 3, 0, 0.9),
                                              (1, None, None, None), (2, None, None, None)])
def test_graph_replay_matches_eager(cfg, B, top_k, top_p):
    # One call captured in a HIP graph and replayed several times, with eager
    # calls on other inputs and synchronisations in between: every replay
    # gives the eager result on its inputs (the call records no memset, so
    # replays after the first are as good as the first).  Cases 3 and 4 take
    # the radix path (top-p alone): the bf16 histogram select with the
    # streamed draw's chunk pass, and the float32 multi-pass select; the last
    # two the small-batch tail, whose arrival counters the row-statistics
    # kernel clears in every call.
    filt = cfg == 4 or top_p is not None
    kw = dict(top_k=top_k, top_p=top_p, draft_sampler=oracle_sampler) if filt else {}
    w = make_workload(cfg, B=B, **kw)
    other = make_workload(cfg, B=B, seed=77, **kw)
    if top_p is not None:
        assert binding.path_kind(w.B, w.K, w.V, w.top_k, w.top_p) == 2
    if cfg in (1, 2):
        assert binding.path_kind(w.B, w.K, w.V, w.top_k, w.top_p) == 3
    a = upload(w, DEV)
    b = upload(other, DEV)
    ws = torch.empty(binding.workspace_bytes(w.B, w.K, w.V,
                                             torch.bfloat16 if w.dtype == "bf16" else torch.float32,
                                             w.top_k, f32(w.top_p)), dtype=torch.uint8, device=DEV)
    ref = {k: v.clone() for k, v in binding.verify(**a, workspace=ws).items()}
    ref_b = {k: v.clone() for k, v in binding.verify(**b, workspace=ws).items()}
    torch.cuda.synchronize()
    out_t = torch.full_like(ref["out_tokens"], -7)
    out_n = torch.full_like(ref["n_emitted"], -7)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.verify(**a, workspace=ws, out_tokens=out_t, n_emitted=out_n)
    for rep in range(4):
        out_t.fill_(-7)
        out_n.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_t, ref["out_tokens"]), rep
        assert torch.equal(out_n, ref["n_emitted"]), rep
        # eager work on other inputs, sharing the workspace, between replays
        r = binding.verify(**b, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(r["out_tokens"], ref_b["out_tokens"])


def test_bench_row_stats_hook_runs():
    # The benchmark hook launches the row-statistics kernel alone; afterwards a
    # full call on the same workspace still matches the oracle.
    import ctypes
    w = make_workload(3, B=4)
    a = upload(w, DEV)
    ws = torch.empty(binding.workspace_bytes(w.B, w.K, w.V, torch.bfloat16), dtype=torch.uint8,
                     device=DEV)
    lib = ctypes.CDLL("libamdhip64.so")
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert lib.hipEventCreate(ctypes.byref(e)) == 0
    binding.bench_row_stats([a, a], ws, 5, w.T, None, ev[0].value, ev[1].value)
    torch.cuda.synchronize()
    ms = ctypes.c_float()
    assert lib.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0 and ms.value > 0
    for e in ev:
        lib.hipEventDestroy(e)
    g = to_numpy(binding.verify(**a, workspace=ws, debug=True))
    torch.cuda.synchronize()
    rep = compare(g, run_oracle(w), w.K)
    assert not rep["mismatches"], rep["mismatches"][:5]


# ---------------------------------------------------------------------------
# Processed-distribution sampler (draft-side draws): specv_sample.

def oracle_sample(logits, u, T, top_k, top_p, dtype):
    """The oracle's draws: a verification with no drafts draws each row's bonus
    token from F(row) at u (same inverse CDF, same flags)."""
    R, V = logits.shape
    t = logits[:, None, :]
    o = O.verify(t, t[:, :0, :], np.zeros((R, 0), np.int32),
                 np.zeros(R, np.int32), np.zeros((R, 0), np.float32), u, f32(T), top_k,
                 f32(top_p), -1, dtype)
    return o["out_tokens"][:, 0], o["flag_kind"]


def upload_logits(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def assert_sample_parity(logits, u, T, top_k, top_p, dtype, label=""):
    y = binding.sample(upload_logits(logits, dtype), torch.from_numpy(u).to(DEV), T, top_k, top_p)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    yo, flags = oracle_sample(logits, u, T, top_k, top_p, dtype)
    certain = flags == O.FLAG_NONE
    bad = np.flatnonzero(certain & (y != yo))
    print(f"[sample] {label} R={len(u)} V={logits.shape[1]} {dtype} T={T} k={top_k} p={top_p}: "
          f"flagged {int((~certain).sum())}, mismatches {len(bad)}", flush=True)
    assert len(bad) == 0, [(int(r), int(y[r]), int(yo[r])) for r in bad[:5]]
    assert int((~certain).sum()) <= flag_ceiling(len(u))
    return y, yo


@pytest.mark.parametrize("cfg,R", [(1, 32), (2, None), (3, 48), (5, 32)])
def test_sample_matches_oracle_unfiltered(cfg, R, unfiltered_path):
    w = make_workload(cfg, B=R if cfg != 2 else None)
    rows = w.draft.reshape(-1, w.V)
    rng = np.random.default_rng(700 + cfg)
    from speculative_decoding_sampling_amd.workloads import uniforms
    u = uniforms(rng, rows.shape[0])
    assert_sample_parity(rows, u, w.T, 0, 1.0, w.dtype, label=f"cfg{cfg}")


@pytest.mark.parametrize("top_k,top_p", [(50, 0.9), (1, 1.0), (100, 0.95), (100, 1.0)])
def test_sample_matches_oracle_filtered(top_k, top_p):
    # top-k 100 without top-p keeps more than one wave's worth of tokens: the
    # merge's LDS sorts, not the one-wave register sorts
    w = make_workload(4, B=4, draft_sampler=oracle_sampler)
    rows = w.draft.reshape(-1, w.V)[:24]
    from speculative_decoding_sampling_amd.workloads import uniforms
    u = uniforms(np.random.default_rng(800 + top_k), rows.shape[0])
    assert_sample_parity(rows, u, w.T, top_k, top_p, w.dtype, label="cfg4 rows")


@pytest.mark.parametrize("top_k,top_p", [(0, 0.9), (1000, 1.0), (2000, 0.99)])
def test_sample_matches_oracle_radix_select(top_k, top_p):
    # the draft-side draw through the radix select, kept sets beyond the list
    # (the draw streamed over the row)
    w = make_workload(4, B=3, draft_sampler=oracle_sampler)
    rows = w.draft.reshape(-1, w.V)[:16]
    from speculative_decoding_sampling_amd.workloads import uniforms
    u = uniforms(np.random.default_rng(900 + top_k), rows.shape[0])
    assert_sample_parity(rows, u, w.T, top_k, top_p, w.dtype, label="cfg4 rows, radix select")


def test_sample_filtered_sparse_and_tied_rows():
    # The filter's radix select at its edges: fewer finite logits than top_k
    # (every one kept), exactly top_k, top_k + 1 with a tie at the k-th value
    # (both kept), finite logits only in the last chunk, many duplicates, and
    # an ordinary row; every row drawn at several uniforms.
    rng = np.random.default_rng(17)
    V, top_k = 20000, 50
    base = np.full((6, V), -np.inf, dtype=np.float32)
    base[0, rng.choice(V, 3, replace=False)] = rng.normal(0, 2, 3)
    base[1, rng.choice(V, top_k, replace=False)] = rng.normal(0, 2, top_k)
    ids = rng.choice(V, top_k + 1, replace=False)
    vals = np.sort(rng.normal(0, 2, top_k + 1))[::-1].copy()
    vals[top_k] = vals[top_k - 1]                    # a tie at the k-th largest
    base[2, ids] = vals
    base[3, V - 300:] = rng.normal(0, 2, 300)        # only the tail chunk is finite
    base[4] = np.round(rng.normal(0, 2, V) * 4) / 4  # many equal values
    base[5] = rng.normal(0, 2, V)
    rows = np.repeat(base, 4, axis=0)
    from speculative_decoding_sampling_amd.workloads import uniforms
    u = uniforms(np.random.default_rng(18), rows.shape[0])
    assert_sample_parity(rows, u, 0.7, top_k, 0.9, "f32", label="sparse/tied rows")
    assert_sample_parity(rows, u, 1.0, top_k, 1.0, "f32", label="sparse/tied rows, top-k only")


def test_sample_edge_cases(unfiltered_path):
    # u = 0 and the largest uniform below 1; a row with one finite logit; rows
    # with no finite logit or a uniform outside [0, 1) give -1, alone.
    rng = np.random.default_rng(11)
    V = 5000
    z = rng.normal(0, 2, size=(6, V)).astype(np.float32)
    z[2, :] = -np.inf
    z[2, 1234] = 0.5
    z[3, :] = -np.inf
    u = np.array([0.0, 1.0 - 2.0 ** -24, 0.5, 0.5, 1.0, -0.25], dtype=np.float32)
    y = binding.sample(upload_logits(z, "f32"), torch.from_numpy(u).to(DEV), 1.0).cpu().numpy()
    yo, _ = oracle_sample(z[:3], u[:3], 1.0, 0, 1.0, "f32")
    assert np.array_equal(y[:3], yo) and y[2] == 1234
    assert np.all(y[3:] == -1)


def test_full_round_with_gpu_drawn_drafts():
    # One whole synthetic round on the GPU: the draft tokens are drawn from the
    # draft logits by specv_sample with their own uniforms, then verified.  The
    # oracle draws the same tokens (except where it flags the draw) and the
    # verification matches it.
    w = make_workload(3, B=16)
    from speculative_decoding_sampling_amd.workloads import uniforms
    ud = uniforms(np.random.default_rng(913), (w.B, w.K))
    rows = w.draft.reshape(-1, w.V)
    y, yo = assert_sample_parity(rows, ud.reshape(-1), w.T, 0, 1.0, w.dtype, label="round drafts")
    w.draft_tokens = y.reshape(w.B, w.K).astype(np.int32)
    assert_parity(w, label="verify GPU-drawn drafts")


# ---------------------------------------------------------------------------
# Per-position acceptance rates: specv_acceptance_rates.

def assert_beta_parity(w, tol, label=""):
    a = upload(w, DEV)
    beta = binding.acceptance_rates(a["target_logits"], a["draft_logits"], a["draft_len"], w.T,
                                    w.top_k, w.top_p)
    torch.cuda.synchronize()
    g = beta.cpu().numpy().astype(np.float64)
    o = O.acceptance_rates(w.target, w.draft, w.draft_len, f32(w.T), w.top_k, f32(w.top_p),
                           w.dtype)
    drafted = o >= 0
    assert np.array_equal(g < 0, ~drafted), "undrafted / error positions differ"
    err = np.abs(g[drafted] - o[drafted])
    bad = []
    for b, k in zip(*np.nonzero(drafted & (np.abs(g - o) > tol))):
        # with top-p, a cut within 1e-10 of top_p may keep a different set
        marg = [O.processed_distribution(O.widen_row(r, w.dtype), f32(w.T), w.top_k,
                                         f32(w.top_p))[1]["topp_margin"]
                for r in (w.target[b, k], w.draft[b, k])]
        if min(marg) > O.TOPP_FLAG_ABS:
            bad.append((int(b), int(k), float(g[b, k]), float(o[b, k])))
    print(f"[beta] {label} cfg={w.cfg} B={w.B} K={w.K} V={w.V} {w.dtype}: "
          f"{int(drafted.sum())} positions, max err {err.max() if err.size else 0:.2e}, "
          f"mean beta {o[drafted].mean() if drafted.any() else 0:.4f}", flush=True)
    assert not bad, bad[:5]


@pytest.mark.parametrize("cfg,B", [(1, None), (2, None), (3, 8), (5, 16)])
def test_acceptance_rates_unfiltered(cfg, B):
    assert_beta_parity(make_workload(cfg, B=B), 1e-5)


def test_acceptance_rates_filtered():
    # float64 inside; the float32 result is within half an ulp (6e-8 at <= 1).
    assert_beta_parity(make_workload(4, B=6, draft_sampler=oracle_sampler), 1e-7)


@pytest.mark.parametrize("cfg,B,top_k,top_p", [(3, 4, 0, 0.9), (4, 3, 1000, 0.95)])
def test_acceptance_rates_radix_select(cfg, B, top_k, top_p):
    # beta through the radix select; kept sets beyond the list are streamed
    w = make_workload(cfg, B=B, draft_sampler=oracle_sampler)
    w.top_k, w.top_p = top_k, f32(top_p)
    assert_beta_parity(w, 1e-7, label=f"radix select top_k={top_k} top_p={top_p}")


def test_acceptance_rates_identical_rows_and_ragged():
    # draft == target gives beta = 1; positions past draft_len give -1.
    w = make_workload(5, B=16)
    w.draft = np.ascontiguousarray(w.target[:, :w.K])
    assert_beta_parity(w, 1e-5, label="draft == target")
    a = upload(w, DEV)
    g = binding.acceptance_rates(a["target_logits"], a["draft_logits"], a["draft_len"],
                                 w.T).cpu().numpy()
    for b in range(w.B):
        nb = int(w.draft_len[b])
        assert np.all(np.abs(g[b, :nb] - 1.0) < 1e-5) and np.all(g[b, nb:] == -1.0)
