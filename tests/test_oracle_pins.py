"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

The rule is Eq. (1) of the explainer page "論文解説: Qwen3.8-Next の設計"
(ta-paperlens.web.app), section "GDNの中身: 足すのではなく、消してから書く":
S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, read out as
o_t = S_t^T q_t after the update.  None of these tests re-types the oracle's
loop: each one checks a closed form, an invariant, a hand-worked example, an
exact rational brute force, or an independently derived (chunked or dense
transition-matrix) form of the same operator.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from gdn_inputs import make_inputs, round_to_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _unit_keys(rng, shape, dk):
    """Keys with entries +-1/sqrt(dk) for dk a power of four -> exact unit norm in binary."""
    s = math.isqrt(dk)
    assert s * s == dk and (s & (s - 1)) == 0
    signs = rng.choice([-1.0, 1.0], size=shape + (dk,))
    return (signs / s).astype(np.float32)


# ---------------------------------------------------------------- worked example
def test_worked_example_golden():
    rows, S_rows = [], []
    with open(os.path.join(GOLDEN, "worked_example_d2_t4.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0] == "S":
                S_rows.append([float(x) for x in parts[1:]])
            else:
                rows.append([float(x) for x in parts])
    rows = np.array(rows)
    T = rows.shape[0]
    k = rows[:, 1:3].reshape(1, T, 1, 2)
    v = rows[:, 3:5].reshape(1, T, 1, 2)
    beta = rows[:, 5].reshape(1, T, 1)
    g = rows[:, 6].reshape(1, T, 1)
    q = rows[:, 7:9].reshape(1, T, 1, 2)
    o_expect = rows[:, 9:11]
    o, sT = oracle.run(q, k, v, beta, g)
    o = o[0, :, 0, :]
    np.testing.assert_array_equal(o[:3], o_expect[:3])
    np.testing.assert_allclose(o[3], o_expect[3], rtol=1e-8, atol=0)
    np.testing.assert_allclose(sT[0, 0], np.array(S_rows), rtol=1e-8, atol=1e-9)


# ---------------------------------------------------------------- P1: beta = 1 writes exactly
@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 32), (4, 8)])
def test_beta_one_overwrites_exactly(dk, dv):
    """beta=1, ||k||=1, any alpha, any state: S_t^T k_t = v_t, so querying k_t returns v_t."""
    rng = _rng(11)
    B, T, H = 2, 9, 3
    k = _unit_keys(rng, (B, T, H), dk)
    q = k.copy()
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    beta = np.ones((B, T, H), np.float32)
    g = -rng.uniform(0.0, 3.0, (B, T, H)).astype(np.float32)
    s0 = rng.standard_normal((B, H, dk, dv))
    o, _ = oracle.run(q, k, v, beta, g, s0=s0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P2: beta = 0 only decays
@pytest.mark.parametrize("dk,dv", [(8, 8), (16, 4)])
def test_beta_zero_is_pure_decay(dk, dv):
    rng = _rng(12)
    B, T, H = 1, 13, 2
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    beta = np.zeros((B, T, H), np.float32)
    g = -rng.uniform(0.001, 0.5, (B, T, H)).astype(np.float32)
    s0 = rng.standard_normal((B, H, dk, dv))
    o, sT = oracle.run(q, k, v, beta, g, s0=s0)
    gam = np.cumsum(g.astype(np.float64), axis=1)                      # [B,T,H], inclusive
    expect_o = np.exp(gam)[..., None] * np.einsum("bthi,bhij->bthj", q.astype(np.float64), s0)
    np.testing.assert_allclose(o, expect_o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sT, np.exp(gam[:, -1])[..., None, None] * s0, rtol=1e-12)
    # with g = 0 the state is kept exactly
    o0, sT0 = oracle.run(q, k, v, beta, np.zeros_like(g), s0=s0)
    np.testing.assert_array_equal(sT0, s0)


# ---------------------------------------------------------------- P3: delta rule retrieval
def test_orthonormal_keys_store_and_overwrite():
    """alpha=1, beta=1, S0=0, basis keys: reading an earlier key returns its latest value exactly."""
    rng = _rng(13)
    dk, dv = 16, 8
    perm = rng.permutation(dk)
    writes = list(perm[:10]) + [perm[2], perm[5]]          # two rewrites of earlier keys
    T = len(writes) + dk
    k = np.zeros((1, T, 1, dk), np.float32)
    q = np.zeros_like(k)
    v = np.zeros((1, T, 1, dv), np.float32)
    beta = np.zeros((1, T, 1), np.float32)
    g = np.zeros((1, T, 1), np.float32)
    latest = {}
    for t, key in enumerate(writes):
        k[0, t, 0, key] = 1.0
        q[0, t, 0, key] = 1.0
        v[0, t, 0] = rng.standard_normal(dv).astype(np.float32)
        beta[0, t, 0] = 1.0
        latest[key] = v[0, t, 0].copy()
    for j in range(dk):                                    # read phase: beta = 0, alpha = 1
        t = len(writes) + j
        q[0, t, 0, j] = 1.0
        k[0, t, 0, (j + 1) % dk] = 1.0
    o, _ = oracle.run(q, k, v, beta, g)
    for j in range(dk):
        want = latest.get(j, np.zeros(dv, np.float32))
        np.testing.assert_array_equal(o[0, len(writes) + j, 0], want)
    # plain accumulation (no erase) would have returned v_old + v_new for rewritten keys
    assert not np.allclose(o[0, len(writes) + perm[2], 0], v[0, 2, 0] + v[0, 10, 0])


# ---------------------------------------------------------------- P4: memoryless limit
def test_strong_decay_is_memoryless():
    rng = _rng(14)
    B, T, H, dk, dv = 1, 7, 2, 8, 8
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    beta = rng.uniform(0.1, 0.9, (B, T, H)).astype(np.float32)
    g = np.full((B, T, H), -60.0, np.float32)
    s0 = rng.standard_normal((B, H, dk, dv))
    o, sT = oracle.run(q, k, v, beta, g, s0=s0)
    kq = np.einsum("bthi,bthi->bth", k.astype(np.float64), q.astype(np.float64))
    expect = (beta * kq)[..., None] * v
    np.testing.assert_allclose(o, expect, rtol=1e-13, atol=1e-15)
    expect_s = beta[:, -1, :, None, None] * np.einsum("bhi,bhj->bhij", k[:, -1].astype(np.float64),
                                                      v[:, -1].astype(np.float64))
    np.testing.assert_allclose(sT, expect_s, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- P5: linearity in (S0, V)
def test_linear_in_state_and_values():
    rng = _rng(15)
    B, T, H, dk, dv = 1, 11, 2, 8, 6
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    beta = rng.uniform(0, 1, (B, T, H)).astype(np.float32)
    g = -rng.uniform(0.001, 0.3, (B, T, H)).astype(np.float32)
    # values on a 2^-8 grid so that va + 3 vb is exact in float32
    va = (rng.integers(-512, 512, (B, T, H, dv)) / 256.0).astype(np.float32)
    vb = (rng.integers(-512, 512, (B, T, H, dv)) / 256.0).astype(np.float32)
    sa = rng.standard_normal((B, H, dk, dv))
    sb = rng.standard_normal((B, H, dk, dv))
    oa, Sa = oracle.run(q, k, va, beta, g, s0=sa)
    ob, Sb = oracle.run(q, k, vb, beta, g, s0=sb)
    oc, Sc = oracle.run(q, k, va + 3 * vb, beta, g, s0=sa + 3 * sb)
    np.testing.assert_allclose(oc, oa + 3 * ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Sc, Sa + 3 * Sb, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- P6: dv columns independent
def test_value_columns_are_independent():
    inp = make_inputs(1, 17, 2, 2, 8, 12, dtype="f32", s0_std=0.5, seed=16)
    perm = _rng(16).permutation(12)
    o, S = oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, s0=inp.s0)
    op, Sp = oracle.run(inp.q, inp.k, inp.v[..., perm], inp.beta, inp.g, s0=inp.s0[..., perm])
    np.testing.assert_array_equal(op, o[..., perm])
    np.testing.assert_array_equal(Sp, S[..., perm])
    # the first 5 columns alone give the same numbers
    o5, S5 = oracle.run(inp.q, inp.k, inp.v[..., :5], inp.beta, inp.g, s0=inp.s0[..., :5])
    np.testing.assert_array_equal(o5, o[..., :5])


# ---------------------------------------------------------------- P7: split / resume
def test_split_and_resume():
    inp = make_inputs(2, 40, 2, 4, 8, 8, dtype="bf16", s0_std=0.1, seed=17)
    o, S = oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, s0=inp.s0)
    t1 = 23
    sl = lambda a, a0, a1: np.ascontiguousarray(a[:, a0:a1])
    o1, S1 = oracle.run(*(sl(x, 0, t1) for x in (inp.q, inp.k, inp.v, inp.beta, inp.g)), s0=inp.s0)
    o2, S2 = oracle.run(*(sl(x, t1, 40) for x in (inp.q, inp.k, inp.v, inp.beta, inp.g)), s0=S1)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), o)
    np.testing.assert_array_equal(S2, S)


# ---------------------------------------------------------------- P8: chunked form
def chunked_form(q, k, v, beta, g, s0, C, scale=1.0):
    """Chunk-parallel rewriting of Eq. (1), derived independently of the oracle.

    Within a chunk of C' <= C tokens with start state S: gamma = cumsum(g),
    D_rs = exp(gamma_r - gamma_s) (s <= r), A = strictly_lower(diag(beta)(K K^T * D)),
    Tm = (I + A)^-1, U = Tm diag(beta) V, W = Tm diag(beta exp(gamma)) K,
    Delta = U - W S, O = scale (diag(exp(gamma)) Q S + (lower(Q K^T) * D) Delta),
    S <- exp(gamma_last) S + Ktilde^T Delta with Ktilde_s = exp(gamma_last - gamma_s) k_s.
    """
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    G = Hv // Hk
    o = np.zeros((B, T, Hv, dv))
    S_out = np.zeros((B, Hv, dk, dv))
    for b in range(B):
        for hv in range(Hv):
            hq = hv // G
            S = np.zeros((dk, dv)) if s0 is None else np.array(s0[b, hv], dtype=np.float64)
            for t0 in range(0, T, C):
                t1 = min(T, t0 + C)
                Q = q[b, t0:t1, hq].astype(np.float64)
                K = k[b, t0:t1, hq].astype(np.float64)
                V = v[b, t0:t1, hv].astype(np.float64)
                bt = beta[b, t0:t1, hv].astype(np.float64)
                gam = np.cumsum(g[b, t0:t1, hv].astype(np.float64))
                Dm = np.exp(np.tril(gam[:, None] - gam[None, :]))
                Dm = np.tril(Dm)
                A = np.tril(bt[:, None] * (K @ K.T) * Dm, -1)
                Tm = np.linalg.inv(np.eye(t1 - t0) + A)
                U = Tm @ (bt[:, None] * V)
                W = Tm @ ((bt * np.exp(gam))[:, None] * K)
                Delta = U - W @ S
                P = np.tril(Q @ K.T) * Dm
                o[b, t0:t1, hv] = scale * (np.exp(gam)[:, None] * (Q @ S) + P @ Delta)
                Kt = np.exp(gam[-1] - gam)[:, None] * K
                S = np.exp(gam[-1]) * S + Kt.T @ Delta
            S_out[b, hv] = S
    return o, S_out


@pytest.mark.parametrize("C", [1, 2, 4, 7, 16, 64])
def test_chunked_form_matches(C):
    inp = make_inputs(1, 61, 2, 4, 8, 5, dtype="bf16", s0_std=0.3, seed=18)
    o, S = oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, s0=inp.s0, scale=0.75)
    oc, Sc = chunked_form(inp.q, inp.k, inp.v, inp.beta, inp.g, inp.s0, C, scale=0.75)
    np.testing.assert_allclose(oc, o, rtol=1e-11, atol=1e-12 * np.abs(o).max())
    np.testing.assert_allclose(Sc, S, rtol=1e-11, atol=1e-12 * np.abs(S).max())


# ---------------------------------------------------------------- P9: brute force
def test_dense_transition_products():
    """S_T = (A_T...A_1) S0 + sum_t (A_T...A_{t+1}) beta_t k_t v_t^T, A_t = alpha_t (I - beta_t k_t k_t^T)."""
    inp = make_inputs(1, 8, 1, 1, 6, 4, dtype="f32", s0_std=1.0, seed=19)
    o, S = oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, s0=inp.s0)
    dk = 6
    kk = inp.k[0, :, 0].astype(np.float64)
    vv = inp.v[0, :, 0].astype(np.float64)
    qq = inp.q[0, :, 0].astype(np.float64)
    bb = inp.beta[0, :, 0].astype(np.float64)
    aa = np.exp(inp.g[0, :, 0].astype(np.float64))
    A = [aa[t] * (np.eye(dk) - bb[t] * np.outer(kk[t], kk[t])) for t in range(8)]
    for T in range(1, 9):
        prod = np.eye(dk)
        for t in range(T):
            prod = A[t] @ prod
        St = prod @ inp.s0[0, 0].astype(np.float64)
        for t in range(T):
            tail = np.eye(dk)
            for s in range(t + 1, T):
                tail = A[s] @ tail
            St = St + tail @ (bb[t] * np.outer(kk[t], vv[t]))
        np.testing.assert_allclose(St.T @ qq[T - 1], o[0, T - 1, 0], rtol=1e-12, atol=1e-13)
        if T == 8:
            np.testing.assert_allclose(St, S[0, 0], rtol=1e-12, atol=1e-13)


def test_exact_rational_brute_force():
    """Exact rational evaluation of Eq. (1) on the exact binary inputs (and fp64 alpha)."""
    inp = make_inputs(1, 5, 1, 1, 3, 2, dtype="bf16", s0_std=1.0, seed=20)
    o, S = oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, s0=inp.s0)
    F = lambda x: Fraction(float(x))
    Sx = [[F(inp.s0[0, 0, i, j]) for j in range(2)] for i in range(3)]
    for t in range(5):
        k = [F(x) for x in inp.k[0, t, 0]]
        q = [F(x) for x in inp.q[0, t, 0]]
        v = [F(x) for x in inp.v[0, t, 0]]
        b = F(inp.beta[0, t, 0])
        a = Fraction(math.exp(float(inp.g[0, t, 0])))
        # M = alpha (I - beta k k^T);  S = M S + beta k v^T
        M = [[a * ((1 if i == r else 0) - b * k[i] * k[r]) for r in range(3)] for i in range(3)]
        Sx = [[sum(M[i][r] * Sx[r][j] for r in range(3)) + b * k[i] * v[j] for j in range(2)]
              for i in range(3)]
        ox = [sum(q[i] * Sx[i][j] for i in range(3)) for j in range(2)]
        for j in range(2):
            assert abs(float(ox[j]) - o[0, t, 0, j]) <= 4e-16 * max(1.0, abs(float(ox[j])))
    for i in range(3):
        for j in range(2):
            assert abs(float(Sx[i][j]) - S[0, 0, i, j]) <= 4e-16 * max(1.0, abs(float(Sx[i][j])))


# ---------------------------------------------------------------- P10: grouped heads
def test_grouped_heads_equal_repeated_heads():
    inp = make_inputs(2, 19, 2, 6, 8, 8, dtype="bf16", s0_std=0.1, seed=21)
    o, S = oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, s0=inp.s0)
    qr = np.repeat(inp.q, 3, axis=2)     # value head hv uses q/k head hv // 3
    kr = np.repeat(inp.k, 3, axis=2)
    o2, S2 = oracle.run(qr, kr, inp.v, inp.beta, inp.g, s0=inp.s0)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(S2, S)
    # chain selection returns the same rows
    ch = [0, 5, 7, 11]
    o3, S3 = oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, s0=inp.s0, chains=ch)
    for n, c in enumerate(ch):
        np.testing.assert_array_equal(o3[n], o[c // 6, :, c % 6])
        np.testing.assert_array_equal(S3[n], S[c // 6, c % 6])


# ---------------------------------------------------------------- P11: norm bound
def test_spectral_norm_bound():
    inp = make_inputs(1, 30, 1, 1, 8, 8, dtype="f32", s0_std=1.0, seed=22)
    st = inp.s0.astype(np.float64).copy()
    prev = np.linalg.norm(st[0, 0], 2)
    for t in range(30):
        oracle.decode_step(inp.q[:, t], inp.k[:, t], inp.v[:, t], inp.beta[:, t], inp.g[:, t], st)
        a = math.exp(float(inp.g[0, t, 0]))
        bound = a * prev + float(inp.beta[0, t, 0]) * np.linalg.norm(inp.v[0, t, 0].astype(np.float64))
        cur = np.linalg.norm(st[0, 0], 2)
        assert cur <= bound * (1 + 1e-6) + 1e-12
        prev = cur


# ---------------------------------------------------------------- P12/P13: decode step
def test_decode_identity_and_equivalence():
    inp = make_inputs(3, 6, 2, 4, 8, 8, dtype="bf16", s0_std=0.2, seed=23)
    o_run, S_run = oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, s0=inp.s0, scale=0.5)
    st = inp.s0.astype(np.float64).copy()
    for t in range(6):
        S_prev = st.copy()
        ot = oracle.decode_step(inp.q[:, t], inp.k[:, t], inp.v[:, t], inp.beta[:, t],
                                inp.g[:, t], st, scale=0.5)
        np.testing.assert_array_equal(ot, o_run[:, t])
        # o = scale (alpha f + (k^T q) w), w = beta (v - alpha e), e = S^T k, f = S^T q
        qh = np.repeat(inp.q[:, t], 2, axis=1).astype(np.float64)
        kh = np.repeat(inp.k[:, t], 2, axis=1).astype(np.float64)
        e = np.einsum("bhi,bhij->bhj", kh, S_prev)
        f = np.einsum("bhi,bhij->bhj", qh, S_prev)
        a = np.exp(inp.g[:, t].astype(np.float64))[..., None]
        w = inp.beta[:, t, :, None] * (inp.v[:, t] - a * e)
        kq = np.einsum("bhi,bhi->bh", kh, qh)[..., None]
        np.testing.assert_allclose(ot, 0.5 * (a * f + kq * w), rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(st, S_run)


# ---------------------------------------------------------------- degenerate sizes
def test_empty_sequence_returns_initial_state():
    inp = make_inputs(2, 3, 1, 2, 4, 4, dtype="f32", s0_std=1.0, seed=25)
    o, S = oracle.run(inp.q[:, :0], inp.k[:, :0], inp.v[:, :0], inp.beta[:, :0], inp.g[:, :0], s0=inp.s0)
    assert o.shape == (2, 0, 2, 4)
    np.testing.assert_array_equal(S, inp.s0)
    o, S = oracle.run(inp.q[:, :0], inp.k[:, :0], inp.v[:, :0], inp.beta[:, :0], inp.g[:, :0])
    assert not S.any()


def test_bad_arguments_raise():
    inp = make_inputs(1, 3, 2, 2, 4, 4, dtype="f32", seed=26)
    with pytest.raises(RuntimeError):
        oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, chains=[4])


def test_bf16_rounding_helper():
    x = np.array([1.0, 1.00390625, 1.005859375, -3.0e-3, 65504.0], np.float32)
    r = round_to_bf16(x)
    bits = r.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to even (1.0)
    assert r[1] == 1.0
    np.testing.assert_allclose(r, x, rtol=2 ** -8)


# ------------------------------------------------------------------ packed sequences and prologue
def _packed(lengths, Hk=2, Hv=4, dk=16, dv=8, seed=900, s0_std=0.3):
    """Random packed inputs: the rows of len(lengths) sequences back to back."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T, N = int(sum(lengths)), len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    q = rng.standard_normal((T, Hk, dk)).astype(np.float32)
    k = rng.standard_normal((T, Hk, dk)).astype(np.float32)
    v = rng.standard_normal((T, Hv, dv)).astype(np.float32)
    beta = rng.uniform(0.05, 0.95, (T, Hv)).astype(np.float32)
    g = -rng.uniform(0.01, 0.3, (T, Hv)).astype(np.float32)
    s0 = rng.standard_normal((N, Hv, dk, dv)) * s0_std
    return dict(q=q, k=k, v=v, beta=beta, g=g, cu=cu, s0=s0)


def test_packed_reduces_to_separate_sequences():
    """Without a prologue, each packed sequence is exactly a run of the plain recurrence
    over its own rows from its own state (including an empty one and a single token)."""
    p = _packed([5, 0, 17, 1, 33])
    o, sT = oracle.run_packed(p["q"], p["k"], p["v"], p["beta"], p["g"], p["cu"], s0=p["s0"],
                              scale=0.7)
    cu = p["cu"]
    for i in range(len(cu) - 1):
        a, b = cu[i], cu[i + 1]
        oi, si = oracle.run(p["q"][None, a:b], p["k"][None, a:b], p["v"][None, a:b],
                            p["beta"][None, a:b], p["g"][None, a:b], s0=p["s0"][i:i + 1],
                            scale=0.7)
        np.testing.assert_array_equal(o[a:b], oi[0])
        np.testing.assert_array_equal(sT[i], si[0])


def test_l2norm_prologue_is_scale_invariant_and_normalises():
    """GDN_QK_L2NORM: (i) scaling a token's q or k by a power of two changes nothing (bitwise);
    (ii) it equals the plain recurrence on q/||q||, k/||k|| formed independently in numpy."""
    p = _packed([9, 14], seed=901)
    o1, s1 = oracle.run_packed(p["q"], p["k"], p["v"], p["beta"], p["g"], p["cu"], s0=p["s0"],
                               flags=oracle.QK_L2NORM)
    rng = np.random.Generator(np.random.PCG64(902))
    fq = (2.0 ** rng.integers(-6, 7, (p["q"].shape[0], p["q"].shape[1], 1))).astype(np.float32)
    fk = (2.0 ** rng.integers(-6, 7, (p["k"].shape[0], p["k"].shape[1], 1))).astype(np.float32)
    o2, s2 = oracle.run_packed(p["q"] * fq, p["k"] * fk, p["v"], p["beta"], p["g"], p["cu"],
                               s0=p["s0"], flags=oracle.QK_L2NORM)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)
    qn = p["q"].astype(np.float64)
    qn /= np.linalg.norm(qn, axis=-1, keepdims=True)
    kn = p["k"].astype(np.float64)
    kn /= np.linalg.norm(kn, axis=-1, keepdims=True)
    o3, s3 = oracle.run_packed(qn.astype(np.float32), kn.astype(np.float32), p["v"], p["beta"],
                               p["g"], p["cu"], s0=p["s0"])
    # the only difference: numpy's normalised values rounded to fp32 (u = 6e-8)
    assert np.abs(o1 - o3).max() <= 1e-6 * np.abs(o1).max()
    assert np.abs(s1 - s3).max() <= 1e-6 * np.abs(s1).max()


def test_l2norm_epsilon_clamp():
    """GDN_QK_L2NORM divides by max(||x||, 1e-6): (i) a zero key makes its token a pure decay
    (bitwise the same as beta = 0 there), (ii) a zero query reads out exactly 0, (iii) a row
    of norm 1e-8 is scaled by 1e6 (to norm 0.01) -- the same as feeding x * 1e6 without the
    prologue, and a hundredth of what plain normalisation would give."""
    p = _packed([12], Hk=1, Hv=2, seed=905)
    q, k, beta = p["q"].copy(), p["k"].copy(), p["beta"].copy()
    # (i) zero key at token 4 vs beta = 0 at token 4
    kz = k.copy()
    kz[4] = 0.0
    bz = beta.copy()
    bz[4] = 0.0
    oa, sa = oracle.run_packed(q, kz, p["v"], beta, p["g"], p["cu"], s0=p["s0"], flags=oracle.QK_L2NORM)
    ob, sb = oracle.run_packed(q, k, p["v"], bz, p["g"], p["cu"], s0=p["s0"], flags=oracle.QK_L2NORM)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(sa, sb)
    # (ii) zero query at token 6
    qz = q.copy()
    qz[6] = 0.0
    oc, _ = oracle.run_packed(qz, k, p["v"], beta, p["g"], p["cu"], s0=p["s0"], flags=oracle.QK_L2NORM)
    assert not oc[6].any()
    # (iii) rows below the epsilon: query at token 3, key at token 8
    tiny_q, tiny_k = q.copy(), k.copy()
    tiny_q[3] *= np.float32(1e-8) / np.linalg.norm(tiny_q[3].astype(np.float64), axis=-1, keepdims=True).astype(np.float32)
    tiny_k[8] *= np.float32(1e-8) / np.linalg.norm(tiny_k[8].astype(np.float64), axis=-1, keepdims=True).astype(np.float32)
    od, sd = oracle.run_packed(tiny_q, tiny_k, p["v"], beta, p["g"], p["cu"], s0=p["s0"],
                               flags=oracle.QK_L2NORM)
    qn = q.astype(np.float64) / np.linalg.norm(q.astype(np.float64), axis=-1, keepdims=True)
    kn = k.astype(np.float64) / np.linalg.norm(k.astype(np.float64), axis=-1, keepdims=True)
    qn[3] = tiny_q[3].astype(np.float64) / 1e-6
    kn[8] = tiny_k[8].astype(np.float64) / 1e-6
    oe, se = oracle.run_packed(qn.astype(np.float32), kn.astype(np.float32), p["v"], beta, p["g"],
                               p["cu"], s0=p["s0"])
    assert np.abs(od - oe).max() <= 1e-6 * np.abs(od).max()
    assert np.abs(sd - se).max() <= 1e-6 * np.abs(sd).max()
    assert abs(np.linalg.norm(qn[3], axis=-1).max() - 0.01) < 1e-6
    # plain normalisation of token 3's query would read out 100 times more
    qu = qn.copy()
    qu[3] /= np.linalg.norm(qu[3], axis=-1, keepdims=True)
    of, _ = oracle.run_packed(qu.astype(np.float32), kn.astype(np.float32), p["v"], beta, p["g"],
                              p["cu"], s0=p["s0"])
    np.testing.assert_allclose(od[3] * 100.0, of[3], rtol=1e-5, atol=1e-9)


def test_beta_logit_zero_is_one_half():
    """GDN_BETA_LOGIT with logits 0 is exactly beta = 1/2 (sigmoid(0) = 1/2 in any precision)."""
    p = _packed([11, 6], seed=903)
    z = np.zeros_like(p["beta"])
    o1, s1 = oracle.run_packed(p["q"], p["k"], p["v"], z, p["g"], p["cu"], s0=p["s0"],
                               flags=oracle.BETA_LOGIT)
    o2, s2 = oracle.run_packed(p["q"], p["k"], p["v"], z + 0.5, p["g"], p["cu"], s0=p["s0"])
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_g_logit_pure_decay_closed_form():
    """GDN_G_LOGIT with beta = 0: every state decays by the product of sigmoid(x_t), and
    o_t = (prod_{s<=t} sigmoid(x_s)) S0^T q_t (the closed form of Eq. (1) at beta = 0)."""
    p = _packed([7, 12], Hk=1, Hv=2, dk=8, dv=4, seed=904)
    rng = np.random.Generator(np.random.PCG64(905))
    x = rng.uniform(-4, 6, p["g"].shape).astype(np.float32)
    zero = np.zeros_like(p["beta"])
    o, sT = oracle.run_packed(p["q"], p["k"], p["v"], zero, x, p["cu"], s0=p["s0"],
                              flags=oracle.G_LOGIT)
    sig = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
    cu = p["cu"]
    for i in range(len(cu) - 1):
        a, b = cu[i], cu[i + 1]
        for h in range(2):
            decay = np.cumprod(sig[a:b, h])
            np.testing.assert_allclose(sT[i, h], decay[-1] * p["s0"][i, h], rtol=1e-12, atol=0)
            ref = decay[:, None] * (p["q"][a:b, 0].astype(np.float64) @ p["s0"][i, h])
            np.testing.assert_allclose(o[a:b, h], ref, rtol=1e-12, atol=1e-300)
    # a very large logit means alpha = 1 to within rounding: no decay at all
    o1, s1 = oracle.run_packed(p["q"], p["k"], p["v"], p["beta"], np.full_like(x, 60.0),
                               p["cu"], s0=p["s0"], flags=oracle.G_LOGIT)
    o2, s2 = oracle.run_packed(p["q"], p["k"], p["v"], p["beta"], np.zeros_like(x), p["cu"],
                               s0=p["s0"])
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(s1, s2, rtol=1e-13, atol=1e-15)


def test_packed_rejects_bad_offsets():
    p = _packed([3, 4], seed=906)
    for cu in ([0, 5, 6], [1, 3, 7], [0, 4, 3, 7][:3]):
        with pytest.raises(RuntimeError):
            oracle.run_packed(p["q"], p["k"], p["v"], p["beta"], p["g"], cu)


# ------------------------------------------------------------------ backward
def _torch_forward(q, k, v, beta, g, s0, scale):
    """Plain float64 torch loop of Eq. (1), used only to get reference gradients from autograd
    (an independent derivation of the backward)."""
    import torch
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    G = Hv // Hk
    outs, finals = [], []
    for b in range(B):
        ob, fb = [], []
        for hv in range(Hv):
            S = s0[b, hv]
            ot = []
            for t in range(T):
                kt, qt, vt = k[b, t, hv // G], q[b, t, hv // G], v[b, t, hv]
                a, bt = torch.exp(g[b, t, hv]), beta[b, t, hv]
                S = a * (S - bt * torch.outer(kt, kt @ S)) + bt * torch.outer(kt, vt)
                ot.append(scale * (S.T @ qt))
            ob.append(torch.stack(ot))
            fb.append(S)
        outs.append(torch.stack(ob, dim=1))
        finals.append(torch.stack(fb))
    return torch.stack(outs), torch.stack(finals)


@pytest.mark.parametrize("B,T,Hk,Hv,dk,dv", [(1, 5, 1, 1, 4, 3), (2, 7, 1, 2, 3, 5)])
def test_backward_matches_autograd(B, T, Hk, Hv, dk, dv):
    """Every gradient of the oracle's backward against torch autograd (float64) through a
    plain forward loop, with random upstream gradients of the outputs and the final state."""
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(950 + T))
    q = rng.standard_normal((B, T, Hk, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, Hk, dk)).astype(np.float32) * 0.5
    v = rng.standard_normal((B, T, Hv, dv)).astype(np.float32)
    beta = rng.uniform(0.1, 0.9, (B, T, Hv)).astype(np.float32)
    g = -rng.uniform(0.01, 0.5, (B, T, Hv)).astype(np.float32)
    s0 = rng.standard_normal((B, Hv, dk, dv))
    dO = rng.standard_normal((B, T, Hv, dv))
    dST = rng.standard_normal((B, Hv, dk, dv))
    scale = 0.75
    ref = oracle.backward(q, k, v, beta, g, dO, s0=s0, dST=dST, scale=scale)
    tt = {n: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
          for n, a in (("q", q), ("k", k), ("v", v), ("beta", beta), ("g", g), ("s0", s0))}
    o, sT = _torch_forward(tt["q"], tt["k"], tt["v"], tt["beta"], tt["g"], tt["s0"], scale)
    loss = (o * torch.tensor(dO)).sum() + (sT * torch.tensor(dST)).sum()
    loss.backward()
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("beta", "dbeta"), ("g", "dg"),
                      ("s0", "dS0")):
        np.testing.assert_allclose(ref[key], tt[name].grad.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=key)


def test_backward_pure_readout_closed_form():
    """beta = 0 and g = 0 keep the state fixed: o_t = scale S0^T q_t, so dS0 = dST +
    scale sum_t q_t dO_t^T, dq_t = scale S0 dO_t, and dk = dv = dbeta-free terms vanish."""
    rng = np.random.Generator(np.random.PCG64(960))
    B, T, H, dk, dv = 1, 6, 1, 4, 3
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    zero = np.zeros((B, T, H), dtype=np.float32)
    s0 = rng.standard_normal((B, H, dk, dv))
    dO = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((B, H, dk, dv))
    r = oracle.backward(q, k, v, zero, zero, dO, s0=s0, dST=dST, scale=2.0)
    qd = q.astype(np.float64)[0, :, 0]
    np.testing.assert_allclose(r["dS0"][0, 0], dST[0, 0] + 2.0 * qd.T @ dO[0, :, 0], rtol=1e-13)
    np.testing.assert_allclose(r["dq"][0, :, 0], 2.0 * dO[0, :, 0] @ s0[0, 0].T, rtol=1e-13)
    np.testing.assert_array_equal(r["dk"], 0.0)
    np.testing.assert_array_equal(r["dv"], 0.0)
