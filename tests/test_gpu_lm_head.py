"""The verification fused with the target LM head, against the oracle (GPU only).

On small-integer inputs every float32 sum of the LM head is exact, so the
target logits must equal the oracle's bfloat16-rounded exact product bit for
bit, and the verification on them must match the oracle's as in the unfused
parity tests (tokens bit-exact except flagged decisions, accept
probabilities and residual masses within 1e-5).  On general inputs the
logits are checked against the float64 product within the float32
accumulation bound 2 D 2^-24 sum |h w|: between the roundings of the
product minus and plus the bound, equal to the rounded product where those
agree, and equal to it for all but a small fraction overall.  Shapes cover a partial row tile, several row blocks, a
ragged vocabulary tail and V not a multiple of 4.
"""

import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
from oracle import lm_head as OL  # noqa: E402
from speculative_decoding_sampling_amd import binding  # noqa: E402
from speculative_decoding_sampling_amd.workloads import (  # noqa: E402
    make_lm_head_workload, upload_lm_head)
from tests.parity import compare, to_numpy  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run_fused(w, **kw):
    args = upload_lm_head(w, DEV)
    args.update(kw)
    res = binding.verify_lm_head(**args, debug=True)
    torch.cuda.synchronize()
    out = to_numpy({k: v for k, v in res.items() if k != "target_logits"})
    out["target_bits"] = res["target_logits"].view(torch.int16).cpu().numpy().view(np.uint16)
    return out


@pytest.mark.parametrize("B,K,V,D,ragged,seed", [
    (4, 3, 5000, 256, False, 1),       # M = 16: one partial row tile; V tail
    (8, 4, 20000, 512, True, 2),       # M = 40: a full and a partial row tile; ragged drafts
    (70, 4, 3000, 128, False, 3),      # M = 350: two row blocks
    (2, 0, 4100, 64, False, 4),        # no drafts: bonus draws only
    (1, 5, 32000, 1024, False, 5),     # single request, low-latency shape
    (3, 2, 4097, 192, True, 6),        # V odd: element stores; D = 3 k blocks
    (2, 2, 200, 64, False, 7),         # V < 256: half a workgroup's waves past V
])
def test_fused_exact_parity(B, K, V, D, ragged, seed):
    print(f"[lm_head] B={B} K={K} V={V} D={D} ragged={ragged} seed={seed}", flush=True)
    w = make_lm_head_workload(B, K, V, D, seed=seed, ragged=ragged)
    g = run_fused(w)
    t_bits = OL.lm_head_target_bits(w.hidden, w.weight)
    assert np.array_equal(g["target_bits"], t_bits), int(np.sum(g["target_bits"] != t_bits))
    o = O.verify(t_bits, w.draft, w.draft_tokens, w.draft_len, w.u, w.u_final, w.T, 0, 1.0,
                 w.eos_id, "bf16")
    rep = compare(g, o, w.K)
    print(f"  requests={rep['requests']} positions={rep['positions']} flagged={rep['flagged']} "
          f"max_alpha_err={rep['max_alpha_err']:.2e} max_mass_err={rep['max_mass_err']:.2e}",
          flush=True)
    assert not rep["mismatches"], rep["mismatches"][:5]


@pytest.mark.parametrize("T,eos_id,seed", [(0.7, -1, 61), (1.3, 17, 62)])
def test_fused_exact_parity_temperature_and_eos(T, eos_id, seed):
    B, K, V, D = 16, 4, 6000, 256
    print(f"[lm_head] T={T} eos={eos_id} B={B} K={K} V={V} D={D} seed={seed}", flush=True)
    w = make_lm_head_workload(B, K, V, D, seed=seed, T=T, ragged=True, eos_id=eos_id)
    if eos_id >= 0:
        # make EOS occur: some drafted tokens are the EOS id (their acceptance
        # still follows p and q at that id)
        w.draft_tokens[::3, 0] = eos_id
    g = run_fused(w)
    t_bits = OL.lm_head_target_bits(w.hidden, w.weight)
    assert np.array_equal(g["target_bits"], t_bits)
    o = O.verify(t_bits, w.draft, w.draft_tokens, w.draft_len, w.u, w.u_final, w.T, 0, 1.0,
                 w.eos_id, "bf16")
    rep = compare(g, o, w.K)
    print(f"  requests={rep['requests']} positions={rep['positions']} flagged={rep['flagged']} "
          f"paths={np.bincount(o['path'] + 1, minlength=4).tolist()}", flush=True)
    assert not rep["mismatches"], rep["mismatches"][:5]


@pytest.mark.parametrize("B,K,V,D,top_k,top_p,seed", [
    (8, 4, 20000, 512, 50, 0.9, 71),     # the candidate select
    (6, 3, 6000, 256, 0, 0.9, 72),       # top-p alone: the radix select
    (3, 2, 4097, 192, 1000, 0.95, 73),   # top-k 1000 then top-p; V odd
])
def test_fused_exact_parity_filtered(B, K, V, D, top_k, top_p, seed):
    # top-k / top-p on the fused call: the filtered path runs on the LM
    # head's logits; drafts are drawn from the filtered draft rows
    print(f"[lm_head] filtered top_k={top_k} top_p={top_p} B={B} K={K} V={V} D={D}", flush=True)
    w = make_lm_head_workload(B, K, V, D, seed=seed, ragged=True, T=0.8)
    tp = float(np.float32(top_p))
    rng = np.random.default_rng(seed)
    for b in range(B):
        for k in range(K):
            P, _ = O.processed_distribution(O.widen_row(w.draft[b, k], "bf16"), w.T, top_k, tp)
            w.draft_tokens[b, k] = O.icdf(P, float(rng.random()))[0]
    g = run_fused(w, top_k=top_k, top_p=tp)
    t_bits = OL.lm_head_target_bits(w.hidden, w.weight)
    assert np.array_equal(g["target_bits"], t_bits)
    o = O.verify(t_bits, w.draft, w.draft_tokens, w.draft_len, w.u, w.u_final, w.T, top_k, tp,
                 w.eos_id, "bf16")
    rep = compare(g, o, w.K)
    print(f"  requests={rep['requests']} positions={rep['positions']} flagged={rep['flagged']} "
          f"max_alpha_err={rep['max_alpha_err']:.2e}", flush=True)
    assert not rep["mismatches"], rep["mismatches"][:5]
    assert rep["positions"] > 0


def test_fused_general_inputs_logits_within_accumulation_bound():
    B, K, V, D = 3, 3, 3001, 1024
    w = make_lm_head_workload(B, K, V, D, seed=21, exact=False)
    print(f"[lm_head] general inputs B={B} K={K} V={V} D={D}", flush=True)
    g = run_fused(w)
    exact = OL.lm_head_logits(w.hidden, w.weight)
    absprod = np.abs(OL.widen_bf16(w.hidden)).reshape(-1, D) @ np.abs(OL.widen_bf16(w.weight)).T
    bound = 2 * D * 2.0 ** -24 * absprod.reshape(exact.shape)   # any fp32 order, truncation too
    want = OL.round_bf16(exact)
    got = OL.widen_bf16(g["target_bits"])
    # rounding is monotone: a float32 sum within the bound of the exact value
    # rounds to a bfloat16 between these two, and to want where they agree
    lo, hi = OL.round_bf16(exact - bound), OL.round_bf16(exact + bound)
    assert np.all((lo <= got) & (got <= hi))
    certain = lo == hi
    assert np.array_equal(got[certain], want[certain])
    # typical float32 rounding is far inside the worst-case bound: nearly
    # every logit is the nearest bfloat16 of the exact product
    agree = float(np.mean(got == want))
    print(f"  certain {certain.mean():.4f}, equal to the rounded exact product {agree:.5f}",
          flush=True)
    assert agree > 0.99


@pytest.mark.parametrize("offset", [4, 1])
def test_fused_output_alignment_store_paths_agree(offset):
    # The logits written 16-byte aligned (whole rows through LDS) and at an
    # element offset of 8 bytes (8-byte stores per lane) or 2 bytes (element
    # stores): the same logits, statistics and draws.
    w = make_lm_head_workload(4, 3, 5000, 256, seed=41)
    print(f"[lm_head] output offset {2 * offset} bytes", flush=True)
    a = run_fused(w)
    n = w.B * (w.K + 1) * w.V
    buf = torch.zeros(n + 8, dtype=torch.bfloat16, device=DEV)
    b = run_fused(w, target_logits=buf[offset:offset + n].view(w.B, w.K + 1, w.V))
    for k in a:
        x, y = np.asarray(a[k]), np.asarray(b[k])
        same = np.array_equal(x, y, equal_nan=True) if x.dtype.kind == "f" else np.array_equal(x, y)
        assert same, k


def test_fused_deterministic():
    w = make_lm_head_workload(6, 4, 9000, 256, seed=31)
    a, b = run_fused(w), run_fused(w)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_fused_host_argument_errors():
    lib = binding.load_library()
    w = make_lm_head_workload(2, 2, 1000, 128, seed=41)
    args = upload_lm_head(w, DEV)
    B, K, V, D = w.B, w.K, w.V, w.D
    tl = torch.empty((B, K + 1, V), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((B, K + 1), dtype=torch.int32, device=DEV)
    n = torch.empty((B,), dtype=torch.int32, device=DEV)
    ws = torch.empty(binding.lm_head_workspace_bytes(B, K, V, D), dtype=torch.uint8, device=DEV)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = binding._ptr

    def call(D_=D, ws_bytes=None, hidden=None, T=1.0):
        h = args["hidden"] if hidden is None else hidden
        return lib.specv_verify_lm_head(
            p(h), p(args["packed_weight"].data), p(args["draft_logits"]), p(args["draft_tokens"]),
            p(args["draft_len"]), p(args["u"]), p(args["u_final"]), B, K, V, D_, T, 0, 1.0, -1,
            p(tl),
            p(out), p(n), p(ws), ws.numel() if ws_bytes is None else ws_bytes, s, None, None,
            None, None)

    assert call() == 0
    assert call(D_=100) == 1                     # not a multiple of 64
    assert call(D_=0) == 1
    assert call(T=0.0) == 1
    assert call(ws_bytes=16) == 2
    assert binding.lm_head_workspace_bytes(B, K, V, 100) == 0
    mis = torch.empty(B * (K + 1) * D + 8, dtype=torch.bfloat16, device=DEV)[1:]
    assert call(hidden=mis) == 1                 # hidden not 16-byte aligned
    torch.cuda.synchronize()


def test_bench_lm_head_hook_runs():
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    w = make_lm_head_workload(2, 1, 2000, 128, seed=51)
    a = upload_lm_head(w, DEV)
    M = w.B * (w.K + 1)
    hid = a["hidden"].reshape(M, w.D)
    logits = torch.empty((M, w.V), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(M * ((w.V + 255) // 256) * 8, dtype=torch.uint8, device=DEV)
    binding.bench_lm_head(hid, a["packed_weight"], logits, ws, 3, start=ev[0], stop=ev[1])
    torch.cuda.synchronize()
    t_bits = OL.lm_head_target_bits(w.hidden, w.weight).reshape(M, w.V)
    got = logits.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, t_bits)


@pytest.mark.parametrize("V,D", [(300, 128), (128, 64), (1, 192)])
def test_packed_weight_layout(V, D):
    # the documented layout: piece (t, kb, w, s, l) of 8 values holds
    # weight[128 t + 32 w + l % 32][64 kb + 32 (l / 32) + 8 s + i], zeros past V
    print(f"[lm_head] pack V={V} D={D}", flush=True)
    rng = np.random.default_rng(V + D)
    wbits = rng.integers(0, 0x7F7F, size=(V, D), dtype=np.uint16)
    wt = torch.from_numpy(wbits.view(np.int16)).to(DEV).view(torch.bfloat16)
    pk = binding.pack_lm_head_weight(wt)
    torch.cuda.synchronize()
    got = pk.data.view(torch.int16).cpu().numpy().view(np.uint16)
    ntile, nkb = (V + 127) // 128, D // 64
    assert got.size == ntile * 128 * D
    want = np.zeros(got.size, dtype=np.uint16)
    for t in range(ntile):
        for kb in range(nkb):
            for w in range(4):
                for s in range(4):
                    for l in range(64):
                        v = 128 * t + 32 * w + l % 32
                        piece = (((t * nkb + kb) * 4 + w) * 4 + s) * 64 + l
                        if v < V:
                            k = 64 * kb + 32 * (l // 32) + 8 * s
                            want[8 * piece:8 * piece + 8] = wbits[v, k:k + 8]
    assert np.array_equal(got, want)


def test_pack_argument_errors():
    lib = binding.load_library()
    wt = torch.zeros((256, 128), dtype=torch.bfloat16, device=DEV)
    n = binding.lm_head_packed_weight_bytes(256, 128)
    buf = torch.empty(n // 2 + 16, dtype=torch.bfloat16, device=DEV)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = binding._ptr
    assert lib.specv_lm_head_pack_weight(p(wt), p(buf), 256, 128, s) == 0
    assert lib.specv_lm_head_pack_weight(p(wt), p(buf[1:]), 256, 128, s) == 1   # misaligned
    assert lib.specv_lm_head_pack_weight(p(wt), p(wt), 256, 128, s) == 1        # in place
    assert lib.specv_lm_head_pack_weight(p(wt), p(buf), 256, 100, s) == 1
    with pytest.raises(TypeError):
        binding.pack_lm_head_weight(wt.float())
    torch.cuda.synchronize()


def test_fused_full_size_sampled():
    # the benchmarked launch: B=64, K=4, V=128256, D=4096; the oracle checks a
    # sample of requests (their 5 target rows bit for bit, then their
    # verification); every request's counts and padding are checked
    B, K, V, D = 64, 4, 128256, 4096
    print(f"[lm_head] full size B={B} K={K} V={V} D={D}", flush=True)
    w = make_lm_head_workload(B, K, V, D, seed=3003)
    g = run_fused(w)
    n, out = g["n_emitted"], g["out_tokens"]
    assert np.all((n >= 1) & (n <= w.draft_len + 1))
    for b in range(B):
        assert np.all(out[b, :n[b]] >= 0) and np.all(out[b, :n[b]] < V)
        assert np.all(out[b, n[b]:] == -1)
    sample = np.array([0, 7, 19, 26, 33, 41, 50, 63])
    t_bits = OL.lm_head_target_bits(w.hidden[sample], w.weight)
    got = g["target_bits"].reshape(B, K + 1, V)[sample]
    assert np.array_equal(got, t_bits), int(np.sum(got != t_bits))
    o = O.verify(t_bits, w.draft[sample], w.draft_tokens[sample], w.draft_len[sample],
                 w.u[sample], w.u_final[sample], w.T, 0, 1.0, w.eos_id, "bf16")
    gs = {k: v[sample] for k, v in g.items() if k != "target_bits"}
    rep = compare(gs, o, K)
    print(f"  sampled requests={rep['requests']} positions={rep['positions']} "
          f"flagged={rep['flagged']} paths={np.bincount(o['path'] + 1, minlength=4).tolist()}",
          flush=True)
    assert not rep["mismatches"], rep["mismatches"][:5]
