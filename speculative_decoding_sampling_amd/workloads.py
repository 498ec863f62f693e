"""Seeded synthetic inputs for the verification call.

This module only draws random inputs.  It holds none of the verification
arithmetic (no normalisers, acceptance tests or inverse-CDF draws), so the
HIP library and the fp64 oracle can both consume its output without sharing
any of the method's code.

The five workloads stand in for the decode workloads of the nickwang.xyz notes
"推测解码：草稿、验证与实际加速" (section "链、树与自推测是不同维度": batch 1–64,
verification budget 5–8), which ran on public datasets that are not used here.

Random-number contract (per workload, seed ``s``):
``SeedSequence(s).spawn(8)`` gives eight PCG64 streams, used in this order:
target logits, draft noise, target spike, draft-token draws, u, u_final,
draft lengths, request classes / EOS placement.  Logits are drawn in float32;
bf16 workloads round to nearest-even and form the draft from the *stored*
target.  Uniforms are ``(uint32 >> 8) * 2**-24`` so they are exact in float32.
"""

from dataclasses import dataclass, field

import numpy as np

# Fixed workloads: shape, dtype, value distribution, sampling parameters.
WORKLOADS = {
    1: dict(name="B8_K4_V4096_f32", B=8, K=4, V=4096, dtype="f32", T=1.0,
            top_k=0, top_p=1.0, eos_id=-1),
    2: dict(name="B1_K5_V32000_bf16", B=1, K=5, V=32000, dtype="bf16", T=0.8,
            top_k=0, top_p=1.0, eos_id=-1),
    3: dict(name="B64_K4_V128256_bf16", B=64, K=4, V=128256, dtype="bf16", T=1.0,
            top_k=0, top_p=1.0, eos_id=-1),
    4: dict(name="B256_K8_V152064_f32_topk50_topp0.9", B=256, K=8, V=152064, dtype="f32",
            T=0.7, top_k=50, top_p=0.9, eos_id=-1),
    5: dict(name="B64_Kragged8_V129280_bf16_eos", B=64, K=8, V=129280, dtype="bf16", T=1.0,
            top_k=0, top_p=1.0, eos_id=1),
}

CLASS_DEFAULT, CLASS_EQUAL, CLASS_FAR = 0, 1, 2


@dataclass
class Workload:
    cfg: int
    seed: int
    B: int
    K: int
    V: int
    dtype: str                  # "f32" or "bf16" (bf16 stored as uint16 bit patterns)
    T: float
    top_k: int
    top_p: float
    eos_id: int
    target: np.ndarray          # [B, K+1, V]
    draft: np.ndarray           # [B, K, V]
    draft_tokens: np.ndarray    # [B, K] int32
    draft_len: np.ndarray       # [B] int32
    u: np.ndarray               # [B, K] float32
    u_final: np.ndarray         # [B] float32
    classes: np.ndarray = field(default=None)   # [B] request class (workload 5)

    @property
    def elem_bytes(self):
        return 2 if self.dtype == "bf16" else 4

    @property
    def positions(self):
        """Verified draft positions in one call: sum of draft lengths."""
        return int(np.clip(self.draft_len, 0, self.K).sum())

    @property
    def algorithmic_bytes(self):
        """One read of every row the call needs: sum_b (2*n_b + 1) * V * elem."""
        n = np.clip(self.draft_len, 0, self.K).astype(np.int64)
        return int(((2 * n + 1) * self.V * self.elem_bytes).sum())


def f32(x):
    """x rounded to the nearest float32, as a Python float."""
    return float(np.float32(x))


def to_bf16_bits(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + rounding) >> np.uint32(16)).astype(np.uint16)


def from_bf16_bits(h):
    """bf16 bit patterns (uint16) -> float32, exact."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def uniforms(rng, shape):
    """Uniforms on the 2**-24 grid in [0, 1), exact in float32."""
    bits = rng.integers(0, 2 ** 32, size=shape, dtype=np.uint64).astype(np.uint32)
    return ((bits >> np.uint32(8)).astype(np.float64) * 2.0 ** -24).astype(np.float32)


def gumbel_max_token(z, T, rng):
    """Draw one token from softmax(z / T) with the Gumbel-max trick.

    This is the draft model's own sampler (upstream of verification); it
    needs no normaliser and no CDF.
    """
    g = -np.log(-np.log(rng.random(z.shape[0])))
    return int(np.argmax(z / T + g))


def make_workload(cfg, seed=None, B=None, draft_sampler=None, top_k=None, top_p=None):
    """Build workload ``cfg`` (1..5) with ``seed`` (default 1000 + cfg).

    ``B`` overrides the batch size (per-request shapes stay the same);
    ``top_k`` / ``top_p`` override the workload's filter settings (the logits
    are the same).
    Filtered workloads (top-k / top-p) need ``draft_sampler(z, T, top_k, top_p,
    uniform) -> token`` so that draft tokens come from the processed draft
    distribution; unfiltered workloads use Gumbel-max on z / T.
    """
    spec = WORKLOADS[cfg]
    seed = 1000 + cfg if seed is None else int(seed)
    B = spec["B"] if B is None else int(B)
    K, V, dtype = spec["K"], spec["V"], spec["dtype"]
    # The call takes temperature and top_p as float32: keep the values both
    # sides see identical.
    top_k = spec["top_k"] if top_k is None else int(top_k)
    top_p = spec["top_p"] if top_p is None else top_p
    T, top_p = f32(spec["T"]), f32(top_p)
    filtered = (0 < top_k < V) or top_p < 1.0
    if filtered and draft_sampler is None:
        raise ValueError("filtered workloads need a draft_sampler for the processed draft distribution")

    streams = [np.random.Generator(np.random.PCG64(s))
               for s in np.random.SeedSequence(seed).spawn(8)]
    r_t, r_dn, r_spike, r_tok, r_u, r_uf, r_len, r_cls = streams

    sigma_t = {1: 2.0, 2: 3.0, 3: 3.0, 4: 2.5, 5: 3.0}[cfg]
    t = r_t.standard_normal((B, K + 1, V), dtype=np.float32)
    t *= np.float32(sigma_t)
    if cfg == 3:                                 # +6 on one random token per target row
        spike = r_spike.integers(0, V, size=(B, K + 1))
        bi, ki = np.meshgrid(np.arange(B), np.arange(K + 1), indexing="ij")
        t[bi, ki, spike] += np.float32(6.0)
    if dtype == "bf16":
        t_bits = to_bf16_bits(t)
        t = from_bf16_bits(t_bits)

    classes = np.full(B, CLASS_DEFAULT, dtype=np.int32)
    noise = r_dn.standard_normal((B, K, V), dtype=np.float32)
    tk = t[:, :K, :]
    if cfg == 1:
        d = tk + np.float32(0.5) * noise
    elif cfg == 2:
        d = np.float32(0.9) * tk + noise
    elif cfg == 3:
        d = tk + np.float32(0.7) * noise
    elif cfg == 4:
        d = np.float32(0.8) * tk + np.float32(1.2) * noise
    else:
        n_eq = max(B // 8, 1) if B >= 2 else 0
        n_far = max(B // 8, 1) if B >= 3 else 0
        labels = np.array([CLASS_EQUAL] * n_eq + [CLASS_FAR] * n_far
                          + [CLASS_DEFAULT] * (B - n_eq - n_far), dtype=np.int32)
        classes = labels[r_cls.permutation(B)]
        sig = np.where(classes == CLASS_FAR, 4.0, 0.7).astype(np.float32)
        d = tk + sig[:, None, None] * noise
        d[classes == CLASS_EQUAL] = tk[classes == CLASS_EQUAL]
    del noise
    d = np.ascontiguousarray(d, dtype=np.float32)

    if cfg == 5:
        draft_len = r_len.integers(0, K + 1, size=B).astype(np.int32)
    else:
        draft_len = np.full(B, K, dtype=np.int32)

    if dtype == "bf16":
        d_bits = to_bf16_bits(d)
        d = from_bf16_bits(d_bits)

    eos_id = spec["eos_id"]
    if cfg == 5:
        # In a quarter of the default-class requests, one used row gets the EOS
        # logit raised to row max + 2 in both target and draft, so EOS happens.
        for b in np.flatnonzero(classes == CLASS_DEFAULT):
            if r_cls.random() < 0.25:
                k = int(r_cls.integers(0, max(int(draft_len[b]), 1)))
                t[b, k, eos_id] = t[b, k].max() + np.float32(2.0)
                d[b, k, eos_id] = d[b, k].max() + np.float32(2.0)
        t_bits = to_bf16_bits(t)
        t = from_bf16_bits(t_bits)
        d_bits = to_bf16_bits(d)
        d = from_bf16_bits(d_bits)

    tokens = np.zeros((B, K), dtype=np.int32)
    for b in range(B):
        for k in range(K):
            if filtered:
                uni = float(r_tok.random())
                tokens[b, k] = draft_sampler(d[b, k].astype(np.float64), T, top_k, top_p, uni)
            else:
                tokens[b, k] = gumbel_max_token(d[b, k].astype(np.float64), T, r_tok)

    u = uniforms(r_u, (B, K))
    u_final = uniforms(r_uf, (B,))

    if dtype == "bf16":
        target_arr, draft_arr = t_bits, d_bits
    else:
        target_arr, draft_arr = t, d
    return Workload(cfg=cfg, seed=seed, B=B, K=K, V=V, dtype=dtype, T=T, top_k=top_k,
                    top_p=top_p, eos_id=eos_id, target=np.ascontiguousarray(target_arr),
                    draft=np.ascontiguousarray(draft_arr), draft_tokens=tokens,
                    draft_len=draft_len, u=u, u_final=u_final, classes=classes)


@dataclass
class LmHeadWorkload:
    """Inputs of the verification fused with the target LM head."""
    seed: int
    B: int
    K: int
    V: int
    D: int
    T: float
    eos_id: int
    exact: bool                 # small-integer values: every float32 sum is exact
    hidden: np.ndarray          # [B, K+1, D] bf16 bit patterns (uint16)
    weight: np.ndarray          # [V, D] bf16 bit patterns (uint16)
    draft: np.ndarray           # [B, K, V] bf16 bit patterns (uint16)
    draft_tokens: np.ndarray    # [B, K] int32
    draft_len: np.ndarray       # [B] int32
    u: np.ndarray               # [B, K] float32
    u_final: np.ndarray         # [B] float32

    @property
    def positions(self):
        return int(np.clip(self.draft_len, 0, self.K).sum())

    @property
    def dtype(self):
        return "bf16"


# Exact LM-head inputs: hidden = i / 16, weight = j / 32 with i, j uniform on
# -8..8, so a logit is an integer multiple of 2**-9 whose partial sums stay
# below 2**24 in magnitude for D <= 4096 (exact in float32 in any order), with
# standard deviation sqrt(D) * 24 / 512 (3.0 at D = 4096).
_HID_SCALE, _W_SCALE = 16.0, 32.0


def _small_int_bf16(rng, shape, scale):
    i = rng.integers(-8, 9, size=shape, dtype=np.int8)
    return i, to_bf16_bits(i.astype(np.float32) / np.float32(scale))


def make_lm_head_workload(B, K, V, D, seed=2000, exact=True, T=1.0, draft_sigma=0.7,
                          ragged=False, eos_id=-1):
    """Seeded inputs of the fused call at batch B, K drafts, vocabulary V and
    hidden size D.

    ``exact`` draws small-integer hidden states and weights (see above);
    otherwise hidden ~ N(0, 1) and weight ~ N(0, (3 / sqrt(D))**2) in bf16
    (logits ~ N(0, 3**2), float32 sums rounded).  The draft logits are the
    target logits plus N(0, draft_sigma**2) noise, rounded to bf16 -- the
    target logits here are an exact float32 product of the integer draws
    (inputs to the draft only; the verification consumes its own); with
    ``exact`` false they come from the float32 product of the bf16 values.
    Draft tokens are drawn from the draft rows by Gumbel-max on z / T; draft
    lengths are K, or uniform on 0..K with ``ragged``.  Stream order of
    SeedSequence(seed).spawn(7): hidden, weight, draft noise, draft tokens,
    u, u_final, draft lengths.
    """
    if exact and D > 4096:
        raise ValueError("exact LM-head inputs need D <= 4096")
    rs = [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(7)]
    r_h, r_w, r_dn, r_tok, r_u, r_uf, r_len = rs
    M = B * (K + 1)
    if exact:
        hi, h_bits = _small_int_bf16(r_h, (M, D), _HID_SCALE)
        wi, w_bits = _small_int_bf16(r_w, (V, D), _W_SCALE)
        t = (hi.astype(np.float32) @ wi.astype(np.float32).T) / np.float32(_HID_SCALE * _W_SCALE)
        del wi
    else:
        h_bits = to_bf16_bits(r_h.standard_normal((M, D), dtype=np.float32))
        w_bits = to_bf16_bits(r_w.standard_normal((V, D), dtype=np.float32)
                              * np.float32(3.0 / np.sqrt(D)))
        t = from_bf16_bits(h_bits) @ from_bf16_bits(w_bits).T
    t = t.reshape(B, K + 1, V)
    T = f32(T)
    d = t[:, :K, :] + np.float32(draft_sigma) * r_dn.standard_normal((B, K, V), dtype=np.float32)
    d_bits = to_bf16_bits(d)
    d = from_bf16_bits(d_bits)
    del t
    tokens = np.zeros((B, K), dtype=np.int32)
    for b in range(B):
        for k in range(K):
            tokens[b, k] = gumbel_max_token(d[b, k].astype(np.float64), T, r_tok)
    u = uniforms(r_u, (B, K))
    u_final = uniforms(r_uf, (B,))
    if ragged:
        draft_len = r_len.integers(0, K + 1, size=B).astype(np.int32)
    else:
        draft_len = np.full(B, K, dtype=np.int32)
    return LmHeadWorkload(seed=seed, B=B, K=K, V=V, D=D, T=T, eos_id=eos_id, exact=exact,
                          hidden=np.ascontiguousarray(h_bits.reshape(B, K + 1, D)),
                          weight=np.ascontiguousarray(w_bits),
                          draft=np.ascontiguousarray(d_bits), draft_tokens=tokens,
                          draft_len=draft_len, u=u, u_final=u_final)


def upload_lm_head(w, device="cuda"):
    """Copy an LM-head workload to the GPU as ``binding.verify_lm_head`` takes it
    (the weight repacked once by the library, as at model load)."""
    import torch

    from speculative_decoding_sampling_amd import binding

    def bf(a):
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)

    return dict(
        hidden=bf(w.hidden),
        packed_weight=binding.pack_lm_head_weight(bf(w.weight)),
        draft_logits=bf(w.draft),
        draft_tokens=torch.from_numpy(w.draft_tokens).to(device),
        draft_len=torch.from_numpy(w.draft_len).to(device),
        u=torch.from_numpy(w.u).to(device),
        u_final=torch.from_numpy(w.u_final).to(device),
        temperature=w.T,
        eos_id=w.eos_id,
    )


def upload(w, device="cuda"):
    """Copy a workload's arrays to the GPU as the tensors ``binding.verify`` takes."""
    import torch

    def logits(a):
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(a).to(device)

    return dict(
        target_logits=logits(w.target),
        draft_logits=logits(w.draft),
        draft_tokens=torch.from_numpy(w.draft_tokens).to(device),
        draft_len=torch.from_numpy(w.draft_len).to(device),
        u=torch.from_numpy(w.u).to(device),
        u_final=torch.from_numpy(w.u_final).to(device),
        temperature=w.T,
        top_k=w.top_k,
        top_p=w.top_p,
        eos_id=w.eos_id,
    )


def make_round_outcomes(B, K, seed, draft_len=None, fail_frac=0.05, eos_frac=0.1, V=1000):
    """Random outcomes of one verified round, shaped as a verification call's
    inputs and outputs: (draft_tokens [B][K], draft_len [B], out_tokens
    [B][K+1], n_emitted [B]), all int32.

    Only random draws: draft_len (if not given) uniform in [0, K]; n_emitted
    uniform in [1, draft_len + 1]; the emitted tokens before the last repeat
    the drafts; the last one repeats the draft at its position for an
    ``eos_frac`` share of the rounds that stop inside the drafts and differs
    from it otherwise; a ``fail_frac`` share of rounds are failed ones
    (n_emitted = -1, out_tokens all -1).  Stream order of SeedSequence(seed)
    .spawn(4): draft tokens, draft lengths, stop positions, round kinds.
    """
    rs = [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(4)]
    toks = rs[0].integers(0, V, size=(B, K), dtype=np.int64).astype(np.int32)
    if draft_len is None:
        draft_len = rs[1].integers(0, K + 1, size=B)
    dl = np.asarray(draft_len, dtype=np.int32).copy()
    out = np.full((B, K + 1), -1, dtype=np.int32)
    n = np.full(B, -1, dtype=np.int32)
    stop = rs[2].random(B)
    kind = rs[3].random(B)
    for b in range(B):
        nb = int(dl[b])
        if kind[b] < fail_frac or nb < 0 or nb > K:
            continue
        last = min(int(stop[b] * (nb + 1)), nb)
        out[b, :last] = toks[b, :last]
        if last < nb and kind[b] < fail_frac + eos_frac:
            out[b, last] = toks[b, last]
        else:
            out[b, last] = (toks[b, last] + 1) % V if last < nb else V - 1 - b % V
        n[b] = last + 1
    return toks, dl, out, n
