"""GPU parity on the special cases of the gated delta rule (explainer page "論文解説:
Qwen3.8-Next の設計", ta-paperlens.web.app, section "GDNの中身", Eq. (1), with alpha and beta
in their closed ranges) through the three chunk-parallel plans (single pass, split, segmented)
and the decode kernel, against the fp64 oracle and, where Eq. (1) fixes the answer in closed form, against that answer too.

Cases: beta = 1 with basis keys (the written value is read back exactly, for any alpha and
state); beta = 0 with g = 0 (the state is kept bit for bit); g = -60 (memoryless); one key
repeated over whole chunks and keys at cosine 0.999 (an ill-conditioned I + A); split/resume
through the final state; superposition in (S0, v); exact scale invariance under powers of two;
|v| and S0 of order 1e5 and 1e-6 (the power-of-two operand scaling keeps the fp16 matrix-core
operands in range); the epsilon clamp of the L2-normalisation prologue on zero and sub-epsilon
rows.

Bars (tests/parity.py): bf16 inputs eps <= 2e-3 M, eps = max|X - R|, M = max|R|.
"""
import numpy as np
import pytest

import oracle
from gdn_inputs import GdnInputs, make_inputs, round_to
from parity import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"
# "segmented_formed": the segmented plan with GDN_SEG_NO_TM, both passes forming every chunk's
# (I + A)^-1 instead of the output pass reading the transition pass's records
PLANS = ["fused", "split", "segmented", "segmented_formed"]
ALL = 1 | 2 | 4  # GDN_QK_L2NORM | GDN_BETA_LOGIT | GDN_G_LOGIT


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_token_gdn_amd as gdn
    gdn.load_library()


def use_plan(monkeypatch, plan):
    """Pin the prefill plan; the segmented one with one chunk per segment, so that every chunk
    boundary is a segment boundary (transition, combine and entry state all exercised)."""
    monkeypatch.setenv("GDN_FORCE_VARIANT", plan.replace("_formed", ""))
    if plan.startswith("segmented"):
        monkeypatch.setenv("GDN_SEG_CHUNKS", "1")
    if plan == "segmented_formed":
        monkeypatch.setenv("GDN_SEG_NO_TM", "1")


def gdn_mod():
    import linear_attention_token_gdn_amd as gdn
    return gdn


def prefill(inp, chunk=64, s0="inp", scale=1.0):
    """o, final state of one gdn_chunk_fwd call (float64 numpy)."""
    gdn = gdn_mod()
    t = inp.to_torch(DEV)
    init = t["s0"] if isinstance(s0, str) else (None if s0 is None else torch.from_numpy(
        np.ascontiguousarray(s0, dtype=np.float32)).to(DEV))
    o, sT = gdn.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["g"], initial_state=init,
                          chunk=chunk, scale=scale)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), sT.double().cpu().numpy()


def decode(inp, scale=1.0):
    """T chained gdn_decode_step calls, then one gdn_decode_tokens call over the same tokens:
    (o, state) of each."""
    gdn = gdn_mod()
    t = inp.to_torch(DEV)
    B, T = inp.q.shape[:2]
    state = t["s0"].clone()
    outs = []
    for s in range(T):
        outs.append(gdn.decode_step(*[t[n][:, s].contiguous() for n in ("q", "k", "v", "beta", "g")],
                                    state, scale=scale))
    state2 = t["s0"].clone()
    o2, _ = gdn.decode_tokens(t["q"], t["k"], t["v"], t["beta"], t["g"], state2, scale=scale)
    torch.cuda.synchronize()
    return ((torch.stack(outs, 1).double().cpu().numpy(), state.double().cpu().numpy()),
            (o2.double().cpu().numpy(), state2.double().cpu().numpy()))


def ref(inp, s0="inp", scale=1.0):
    init = inp.s0 if isinstance(s0, str) else s0
    return oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, s0=init, scale=scale)


def inputs(q, k, v, beta, g, s0):
    """GdnInputs from float arrays (rounded to bf16; the state stays fp32)."""
    return GdnInputs(q=round_to(q, "bf16"), k=round_to(k, "bf16"), v=round_to(v, "bf16"),
                     beta=round_to(beta, "bf16"), g=round_to(g, "bf16"),
                     s0=None if s0 is None else np.asarray(s0, np.float32), dtype="bf16")


def basis_keys(rng, B, T, H, d):
    """k_t = e_pi(t): basis vectors in a random order, each reused after d tokens."""
    k = np.zeros((B, T, H, d), np.float32)
    for b in range(B):
        for h in range(H):
            perm = rng.permutation(d)
            k[b, np.arange(T), h, perm[np.arange(T) % d]] = 1.0
    return k


def check_all(what, pairs):
    for name, x, r in pairs:
        e = check(x, r, "bf16", "%s %s" % (what, name))
        print("%s %s: err %.2e (max %.2e)" % (what, name, e[0], e[1]))


# ------------------------------------------------------------------ beta = 1, basis keys
@pytest.mark.parametrize("plan", PLANS)
@pytest.mark.parametrize("decay", [False, True])
def test_beta_one_reads_back_the_written_value(plan, decay, monkeypatch):
    """beta = 1 and a unit key overwrite what the state holds under that key: with q_t = k_t
    the output is v_t exactly, for any alpha and any initial state (basis keys are exact in
    bf16; repeated keys are rewritten with their latest value)."""
    use_plan(monkeypatch, plan)
    rng = np.random.default_rng(900 + decay)
    B, T, H, d = 1, 200, 2, 128
    k = basis_keys(rng, B, T, H, d)
    v = rng.standard_normal((B, T, H, d)).astype(np.float32)
    g = -rng.uniform(0.0, 0.2, (B, T, H)) if decay else np.zeros((B, T, H))
    s0 = rng.standard_normal((B, H, d, d)).astype(np.float32) * 0.5
    inp = inputs(k, k, v, np.ones((B, T, H)), g, s0)
    o, sT = prefill(inp)
    ro, rS = ref(inp)
    check_all("beta=1 %s decay=%d" % (plan, decay), [("o", o, ro), ("S", sT, rS)])
    check(o, inp.v, "bf16", "beta=1 %s: o_t = v_t" % plan)


def test_beta_one_decode_reads_back_exactly():
    rng = np.random.default_rng(902)
    B, T, H, d = 4, 12, 2, 128
    k = basis_keys(rng, B, T, H, d)
    v = rng.standard_normal((B, T, H, d)).astype(np.float32)
    s0 = rng.standard_normal((B, H, d, d)).astype(np.float32)
    inp = inputs(k, k, v, np.ones((B, T, H)), -rng.uniform(0, 0.2, (B, T, H)), s0)
    (o1, S1), (o2, S2) = decode(inp)
    ro, rS = ref(inp)
    check_all("decode beta=1", [("o", o1, ro), ("S", S1, rS), ("o tokens", o2, ro),
                                ("S tokens", S2, rS)])
    check(o1, inp.v, "bf16", "decode beta=1: o_t = v_t")


# ------------------------------------------------------------------ beta = 0, g = 0
@pytest.mark.parametrize("plan", PLANS + ["decode"])
def test_beta_zero_without_decay_keeps_the_state(plan, monkeypatch):
    """beta = 0 and alpha = 1 leave the state untouched: S_T = S0 bit for bit (Delta = 0, and
    every power-of-two scaling is undone exactly) and o_t = S0^T q_t."""
    rng = np.random.default_rng(910)
    B, T, H, d = 2, 150, 2, 128
    inp = make_inputs(B, T, H, H, d, d, dtype="bf16", s0_std=1.0, seed=910)
    inp.beta[:] = 0.0
    inp.g[:] = 0.0
    ro, rS = ref(inp)
    if plan == "decode":
        (o, sT), (o2, S2) = decode(inp)
        np.testing.assert_array_equal(S2, inp.s0)
        check(o2, ro, "bf16", "beta=0 decode_tokens o")
    else:
        use_plan(monkeypatch, plan)
        o, sT = prefill(inp)
    np.testing.assert_array_equal(sT, inp.s0)
    check(o, ro, "bf16", "beta=0 %s o" % plan)


# ------------------------------------------------------------------ g = -60
@pytest.mark.parametrize("plan", PLANS + ["decode"])
def test_memoryless_gates(plan, monkeypatch):
    """alpha = e^-60: every token forgets the past, S_t ~ beta_t k_t v_t^T."""
    inp = make_inputs(2, 150 if plan != "decode" else 10, 2, 4, 128, 128, dtype="bf16",
                      s0_std=0.5, seed=920)
    inp.g[:] = -60.0
    ro, rS = ref(inp)
    if plan == "decode":
        (o, sT), (o2, S2) = decode(inp)
        check_all("g=-60 decode_tokens", [("o", o2, ro), ("S", S2, rS)])
    else:
        use_plan(monkeypatch, plan)
        o, sT = prefill(inp)
    check_all("g=-60 %s" % plan, [("o", o, ro), ("S", sT, rS)])
    # the closed-form limit, from the stored inputs (the state left by the last token)
    b, t = 0, inp.q.shape[1] - 1
    for h in range(inp.v.shape[2]):
        kk = inp.k[b, t, h // 2].astype(np.float64)
        lim = inp.beta[b, t, h] * np.outer(kk, inp.v[b, t, h])
        assert np.abs(rS[b, h] - lim).max() <= 1e-12 * max(1.0, np.abs(lim).max())


# ------------------------------------------------------------------ ill-conditioned chunks
@pytest.mark.parametrize("plan", PLANS)
@pytest.mark.parametrize("kind", ["repeated", "cos0.999"])
def test_repeated_and_near_parallel_keys(plan, kind, monkeypatch):
    """One key for a whole chunk (A is a full strictly lower triangle of beta_r e^(..)), or
    keys at cosine ~0.999 to a common direction, with random beta and a strong initial state."""
    use_plan(monkeypatch, plan)
    rng = np.random.default_rng(930)
    B, T, H, d = 1, 190, 2, 128
    base = make_inputs(B, T, H, H, d, d, dtype="bf16", s0_std=0.3, seed=930)
    k = np.empty((B, T, H, d))
    for c0 in range(0, T, 64):
        k0 = rng.standard_normal((B, 1, H, d))
        k0 /= np.linalg.norm(k0, axis=-1, keepdims=True)
        n = min(64, T - c0)
        if kind == "repeated":
            k[:, c0:c0 + n] = k0
        else:
            x = k0 + 0.0045 * rng.standard_normal((B, n, H, d))
            k[:, c0:c0 + n] = x / np.linalg.norm(x, axis=-1, keepdims=True)
    inp = inputs(base.q, k, base.v, base.beta, base.g, base.s0)
    o, sT = prefill(inp)
    ro, rS = ref(inp)
    check_all("%s keys %s" % (kind, plan), [("o", o, ro), ("S", sT, rS)])


# ------------------------------------------------------------------ split / resume
@pytest.mark.parametrize("plan", PLANS)
def test_split_and_resume_through_the_final_state(plan, monkeypatch):
    """run(T1) then run(T2 | initial = final(T1)) = run(T1 + T2)."""
    use_plan(monkeypatch, plan)
    inp = make_inputs(1, 250, 2, 4, 128, 128, dtype="bf16", s0_std=0.02, seed=940)
    T1 = 100  # not a multiple of the chunk: the first call ends in a partial chunk

    def part(a, b, s0):
        return GdnInputs(q=inp.q[:, a:b], k=inp.k[:, a:b], v=inp.v[:, a:b], beta=inp.beta[:, a:b],
                         g=inp.g[:, a:b], s0=s0, dtype="bf16")
    o1, S1 = prefill(part(0, T1, inp.s0))
    o2, S2 = prefill(part(T1, 250, None), s0=S1.astype(np.float32))
    o, sT = prefill(inp)
    ro, rS = ref(inp)
    os = np.concatenate([o1, o2], axis=1)
    check_all("split/resume %s" % plan, [("o joined", os, ro), ("S joined", S2, rS),
                                          ("o one call", o, ro), ("S one call", sT, rS)])
    check(os, o, "bf16", "split/resume %s: joined vs one call" % plan)


# ------------------------------------------------------------------ linearity in (S0, v)
@pytest.mark.parametrize("plan", PLANS + ["decode"])
def test_superposition_in_state_and_values(plan, monkeypatch):
    """(S0, V) -> (O, S_T) is linear for fixed q, k, beta, g: run(S0, V) = run(S0, 0) +
    run(0, V)."""
    inp = make_inputs(1, 130 if plan != "decode" else 9, 2, 4, 128, 128, dtype="bf16",
                      s0_std=0.05, seed=950)
    only_s = GdnInputs(q=inp.q, k=inp.k, v=np.zeros_like(inp.v), beta=inp.beta, g=inp.g,
                       s0=inp.s0, dtype="bf16")
    only_v = GdnInputs(q=inp.q, k=inp.k, v=inp.v, beta=inp.beta, g=inp.g,
                       s0=np.zeros_like(inp.s0), dtype="bf16")
    if plan == "decode":
        run = lambda x: decode(x)[0]
    else:
        use_plan(monkeypatch, plan)
        run = prefill
    o, sT = run(inp)
    oa, Sa = run(only_s)
    ob, Sb = run(only_v)
    ro, rS = ref(inp)
    check_all("superposition %s" % plan, [("o", o, ro), ("S", sT, rS), ("o sum", oa + ob, ro),
                                           ("S sum", Sa + Sb, rS)])


# ------------------------------------------------------------------ magnitudes
@pytest.mark.parametrize("plan", PLANS + ["decode"])
@pytest.mark.parametrize("k2", [-24, 16])
def test_power_of_two_scale_invariance(plan, k2, monkeypatch):
    """Scaling v and S0 by 2^k scales o and S_T by exactly 2^k (bit for bit): the fp16 operand
    copies carry a power-of-two scale of their own, so they are the same bits at any
    magnitude."""
    inp = make_inputs(1, 150 if plan != "decode" else 7, 2, 4, 128, 128, dtype="bf16",
                      s0_std=0.05, seed=960)
    f = np.float32(2.0 ** k2)
    big = GdnInputs(q=inp.q, k=inp.k, v=inp.v * f, beta=inp.beta, g=inp.g, s0=inp.s0 * f,
                    dtype="bf16")
    if plan == "decode":
        run = lambda x: decode(x)[0]
    else:
        use_plan(monkeypatch, plan)
        run = prefill
    o, sT = run(inp)
    ob, Sb = run(big)
    np.testing.assert_array_equal(ob, o * float(f))
    np.testing.assert_array_equal(Sb, sT * float(f))


@pytest.mark.parametrize("plan", PLANS + ["decode"])
@pytest.mark.parametrize("mag", [1e5, 1e-6])
def test_large_and_small_values_and_state(plan, mag, monkeypatch):
    """|v| and S0 far outside fp16's comfortable range (1e5 overflows fp16 by itself once
    accumulated; 1e-6 sits in its subnormals): parity with the oracle at the usual bar."""
    inp = make_inputs(2, 150 if plan != "decode" else 9, 2, 4, 128, 128, dtype="bf16",
                      s0_std=1.0, seed=970)
    inp = GdnInputs(q=inp.q, k=inp.k, v=round_to(inp.v * mag, "bf16"), beta=inp.beta, g=inp.g,
                    s0=(inp.s0 * mag).astype(np.float32), dtype="bf16")
    ro, rS = ref(inp)
    if plan == "decode":
        (o, sT), (o2, S2) = decode(inp)
        check_all("|v|~%g decode_tokens" % mag, [("o", o2, ro), ("S", S2, rS)])
    else:
        use_plan(monkeypatch, plan)
        o, sT = prefill(inp)
    check_all("|v|~%g %s" % (mag, plan), [("o", o, ro), ("S", sT, rS)])


# ------------------------------------------------------------------ the prologue's epsilon
@pytest.mark.parametrize("plan", PLANS + ["decode"])
def test_l2norm_epsilon_clamp(plan, monkeypatch):
    """GDN_QK_L2NORM divides by max(||x||, 1e-6): a zero row stays zero (the token writes and
    erases nothing, and reads out 0), a row of norm 1e-8 is scaled by 1e6 (to norm 0.01)."""
    rng = np.random.default_rng(980)
    T, Hk, Hv, d = 140 if plan != "decode" else 8, 2, 4, 128
    q = rng.standard_normal((T, Hk, d))
    k = rng.standard_normal((T, Hk, d))
    for x in (q, k):
        x[3] = 0.0                                            # zero rows
        x[5] *= 1e-8 / np.linalg.norm(x[5], axis=-1, keepdims=True)  # below the epsilon
    q[7, 1] = 0.0
    k[2:6:2, 0] = 0.0
    v = rng.standard_normal((T, Hv, d))
    beta = rng.standard_normal((T, Hv))       # logits
    g = rng.uniform(2.0, 6.0, (T, Hv))        # logits of alpha
    x = {n: round_to(a, "bf16") for n, a in (("q", q), ("k", k), ("v", v), ("beta", beta),
                                            ("g", g))}
    s0 = (rng.standard_normal((1, Hv, d, d)) * 0.1).astype(np.float32)
    cu = np.array([0, T], np.int64)
    ro, rS = oracle.run_packed(x["q"], x["k"], x["v"], x["beta"], x["g"], cu, s0=s0, flags=ALL)
    gdn = gdn_mod()
    t = {n: torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(torch.bfloat16)
         for n, a in x.items()}
    s0_t = torch.from_numpy(s0).to(DEV)
    if plan == "decode":
        o, sT = gdn.decode_tokens(*[t[n][None] for n in ("q", "k", "v", "beta", "g")], s0_t,
                                  flags=ALL)
        o = o[0]
    else:
        use_plan(monkeypatch, plan)
        o, sT = gdn.chunk_fwd_varlen(t["q"][None], t["k"][None], t["v"][None], t["beta"][None],
                                     t["g"][None], initial_state=s0_t, flags=ALL)
        o = o[0]
    torch.cuda.synchronize()
    check_all("eps clamp %s" % plan, [("o", o.double().cpu().numpy(), ro),
                                       ("S", sT.double().cpu().numpy(), rS)])
