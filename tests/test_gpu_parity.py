"""GPU parity: libgdn.so (through its C ABI) against the fp64 oracle on the same seeded inputs.

Bars (tests/parity.py): fp32 inputs eps <= 1e-5 max(1, M); bf16 inputs eps <= 2e-3 M, with
eps = max|X - R|, M = max|R| per output tensor (o, final state).
"""
import os

import numpy as np
import pytest

import oracle
from gdn_inputs import CONFIGS, config_inputs, make_inputs
from parity import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_token_gdn_amd as gdn
    gdn.load_library()


def gdn_mod():
    import linear_attention_token_gdn_amd as gdn
    return gdn


def run_prefill(inp, chunk, scale=1.0, use_init=True, want_state=True, out_dtype=None,
                in_place=False):
    gdn = gdn_mod()
    t = inp.to_torch(DEV)
    s0 = t["s0"] if use_init else None
    kw = {}
    if in_place:
        assert s0 is not None
        kw["final_state"] = s0
    o, sT = gdn.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["g"], initial_state=s0,
                          output_final_state=want_state, chunk=chunk, scale=scale,
                          out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return (o.float().cpu().numpy(),
            None if sT is None else sT.cpu().numpy())


def oracle_prefill(inp, scale=1.0, use_init=True, chains=None):
    return oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g,
                      s0=inp.s0 if use_init else None, scale=scale, chains=chains)


def check_prefill(inp, chunk, scale=1.0, use_init=True, tag=""):
    o, sT = run_prefill(inp, chunk, scale=scale, use_init=use_init)
    ro, rS = oracle_prefill(inp, scale=scale, use_init=use_init)
    e1 = check(o, ro, inp.dtype, "o " + tag)
    e2 = check(sT, rS, inp.dtype, "final state " + tag)
    print("%s: o err %.2e (max %.2e), S err %.2e (max %.2e)" % (tag, e1[0], e1[1], e2[0], e2[1]))


# ------------------------------------------------------------------ prefill
def test_config0_tiny_fp32():
    c = CONFIGS[0]
    check_prefill(config_inputs(0), c["chunk"], tag=c["name"])


@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 32), (32, 16), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_head_sizes(dk, dv, dtype):
    inp = make_inputs(2, 45, 1, 2, dk, dv, dtype=dtype, s0_std=0.02, seed=100 + dk + dv)
    check_prefill(inp, 16, tag="dk%d dv%d %s" % (dk, dv, dtype))


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunks_and_ragged_tail(chunk):
    # T = 157 spans several chunks of every size and ends in a partial chunk
    inp = make_inputs(1, 157, 2, 4, 128, 128, dtype="bf16", s0_std=0.02, seed=200 + chunk)
    check_prefill(inp, chunk, scale=0.5, tag="chunk %d ragged" % chunk)


def test_grouped_heads_and_zero_state():
    inp = make_inputs(2, 130, 2, 8, 128, 128, dtype="bf16", seed=301)
    check_prefill(inp, 64, use_init=False, tag="gqa g=4 zero init")


def test_long_memory_gates():
    inp = make_inputs(1, 640, 2, 2, 128, 128, dtype="bf16", g_range=(0.0001, 0.02), seed=302)
    check_prefill(inp, 64, tag="long memory")


def test_t1_and_t0():
    gdn = gdn_mod()
    inp = make_inputs(2, 1, 2, 2, 64, 64, dtype="bf16", s0_std=0.1, seed=303)
    check_prefill(inp, 64, tag="T=1")
    t = inp.to_torch(DEV)
    empty = {n: t[n][:, :0].contiguous() for n in ("q", "k", "v", "beta", "g")}
    o, sT = gdn.chunk_fwd(empty["q"], empty["k"], empty["v"], empty["beta"], empty["g"],
                          initial_state=t["s0"], chunk=64)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, 64)
    assert torch.equal(sT, t["s0"])
    o, sT = gdn.chunk_fwd(empty["q"], empty["k"], empty["v"], empty["beta"], empty["g"], chunk=64)
    torch.cuda.synchronize()
    assert not sT.any()


def test_in_place_state_and_optional_outputs():
    inp = make_inputs(1, 100, 1, 2, 128, 128, dtype="bf16", s0_std=0.02, seed=304)
    ro, rS = oracle_prefill(inp)
    o, sT = run_prefill(inp, 64, in_place=True)
    check(o, ro, "bf16", "o in-place")
    check(sT, rS, "bf16", "S in-place")
    o2, none = run_prefill(inp, 64, want_state=False)
    assert none is None
    np.testing.assert_array_equal(o2, o)


def test_bf16_output():
    inp = make_inputs(1, 80, 1, 1, 64, 64, dtype="bf16", s0_std=0.02, seed=305)
    o, _ = run_prefill(inp, 32, out_dtype=torch.bfloat16)
    ro, _ = oracle_prefill(inp)
    # bf16 storage of o adds up to 2^-9 relative rounding on top of the fp32 result
    eps = np.abs(o - ro).max()
    assert eps <= (2e-3 + 2 ** -8) * np.abs(ro).max()


def test_deterministic():
    inp = make_inputs(1, 200, 2, 2, 128, 128, dtype="bf16", s0_std=0.02, seed=306)
    a = run_prefill(inp, 64)
    b = run_prefill(inp, 64)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ------------------------------------------------------------------ decode
def run_decode_steps(inp, steps, scale=1.0, out_dtype=None):
    gdn = gdn_mod()
    t = inp.to_torch(DEV)
    state = t["s0"].clone()
    outs = []
    for s in range(steps):
        o = gdn.decode_step(t["q"][:, s].contiguous(), t["k"][:, s].contiguous(),
                            t["v"][:, s].contiguous(), t["beta"][:, s].contiguous(),
                            t["g"][:, s].contiguous(), state, scale=scale, out_dtype=out_dtype)
        outs.append(o.float())
    torch.cuda.synchronize()
    return torch.stack(outs, 1).cpu().numpy(), state.cpu().numpy()


@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 128), (128, 16), (64, 32), (128, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_head_sizes(dk, dv, dtype):
    inp = make_inputs(3, 5, 2, 4, dk, dv, dtype=dtype, s0_std=0.02, seed=400 + dk + 3 * dv)
    o, S = run_decode_steps(inp, 5, scale=0.75)
    ro, rS = oracle_prefill(inp, scale=0.75)
    check(o, ro, dtype, "decode o")
    check(S, rS, dtype, "decode state")


def test_decode_config4_sampled():
    """The full decode workload (B=256, H=32, d=128, 64 chained steps) on the GPU; every
    output and state of 48 sampled (b, h) chains checked against the oracle."""
    c = CONFIGS[4]
    inp = config_inputs(4)
    o, S = run_decode_steps(inp, c["T"])
    rng = np.random.Generator(np.random.PCG64(4))
    chains = np.sort(rng.choice(c["B"] * c["Hv"], 48, replace=False))
    ro, rS = oracle_prefill(inp, chains=chains)
    b, h = chains // c["Hv"], chains % c["Hv"]
    check(o[b, :, h], ro, "bf16", "config4 decode o")
    check(S[b, h], rS, "bf16", "config4 decode state")


def test_decode_matches_prefill_path():
    """T decode steps equal one prefill over the same T tokens (same operator)."""
    inp = make_inputs(2, 9, 2, 2, 128, 128, dtype="bf16", s0_std=0.02, seed=401)
    od, Sd = run_decode_steps(inp, 9)
    op, Sp = run_prefill(inp, 64)
    M = np.abs(op).max()
    assert np.abs(od - op).max() <= 2e-3 * M
    assert np.abs(Sd - Sp).max() <= 2e-3 * np.abs(Sp).max()


# ------------------------------------------------------------------ chunk-parallel variants
@pytest.mark.parametrize("variant", ["fused", "split", "segmented"])
@pytest.mark.parametrize("d,chunk", [(128, 64), (128, 32), (64, 64), (64, 32)])
def test_chunk_variants(variant, d, chunk, monkeypatch):
    """The chunk-parallel plans (single pass; prep + scan through a workspace; segments of two
    chunks run in parallel) against the oracle, with grouped heads, an initial state, a scale
    and a ragged last chunk."""
    monkeypatch.setenv("GDN_FORCE_VARIANT", variant)
    monkeypatch.setenv("GDN_SEG_CHUNKS", "2")
    inp = make_inputs(2, 157, 2, 4, d, d, dtype="bf16", s0_std=0.02, seed=500 + d + chunk)
    check_prefill(inp, chunk, scale=0.8, tag="%s d%d c%d" % (variant, d, chunk))


def test_variants_agree_and_are_deterministic(monkeypatch):
    inp = make_inputs(1, 300, 1, 2, 128, 128, dtype="bf16", s0_std=0.02, seed=510)
    res = {}
    monkeypatch.setenv("GDN_SEG_CHUNKS", "2")
    for variant in ("fused", "split", "segmented"):
        monkeypatch.setenv("GDN_FORCE_VARIANT", variant)
        a = run_prefill(inp, 64)
        b = run_prefill(inp, 64)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])
        res[variant] = a
    M = np.abs(res["fused"][0]).max()
    assert np.abs(res["fused"][0] - res["split"][0]).max() <= 2e-3 * M
    assert np.abs(res["fused"][0] - res["segmented"][0]).max() <= 2e-3 * M


# ------------------------------------------------------------------ the workloads, full size
def _full_config_check(idx, block):
    """Run a prefill workload at its full size through the default dispatch and compare every
    output and final state of every (b, hv) chain with the oracle, `block` chains per oracle
    call (the bar applies to the whole tensor: eps and M are maxima over all chains)."""
    c = CONFIGS[idx]
    inp = config_inputs(idx)
    o, sT = run_prefill(inp, c["chunk"])
    nch = c["B"] * c["Hv"]
    eo = Mo = eS = MS = 0.0
    for c0 in range(0, nch, block):
        chains = np.arange(c0, min(nch, c0 + block))
        ro, rS = oracle_prefill(inp, chains=chains, use_init=inp.s0 is not None)
        for j, ch in enumerate(chains):
            b, h = ch // c["Hv"], ch % c["Hv"]
            eo = max(eo, float(np.abs(o[b, :, h] - ro[j]).max()))
            Mo = max(Mo, float(np.abs(ro[j]).max()))
            eS = max(eS, float(np.abs(sT[b, h] - rS[j]).max()))
            MS = max(MS, float(np.abs(rS[j]).max()))
        del ro, rS
    print("%s: all %d chains, o err %.2e (max %.2e), S err %.2e (max %.2e)"
          % (c["name"], nch, eo, Mo, eS, MS))
    assert np.isfinite(o).all() and np.isfinite(sT).all()
    assert eo <= 2e-3 * Mo, "%s o: %.3e > 2e-3 * %.3e" % (c["name"], eo, Mo)
    assert eS <= 2e-3 * MS, "%s final state: %.3e > 2e-3 * %.3e" % (c["name"], eS, MS)


def test_config1_full():
    _full_config_check(1, 16)


def test_config2_full():
    _full_config_check(2, 64)


def test_config3_full():
    """The 262,144-token workload: all 16 chains (about 620 GFLOP of fp64 on the host)."""
    _full_config_check(3, 16)


# ------------------------------------------------------------------ several tokens per decode call
def run_decode_tokens(inp, scale=1.0, in_place=True, use_init=True):
    gdn = gdn_mod()
    t = inp.to_torch(DEV)
    s_in = t["s0"].clone() if use_init else None
    shape = (inp.q.shape[0], inp.v.shape[2], inp.q.shape[3], inp.v.shape[3])
    s_out = None if in_place else torch.full(shape, float("nan"), device=DEV)
    o, s_out = gdn.decode_tokens(t["q"], t["k"], t["v"], t["beta"], t["g"], s_in,
                                 state_out=s_out, scale=scale)
    torch.cuda.synchronize()
    return o.cpu().numpy(), s_out.cpu().numpy(), (None if s_in is None else s_in.cpu().numpy())


@pytest.mark.parametrize("T", [1, 2, 5, 8])
@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 32), (128, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_tokens_matches_oracle(T, dk, dv, dtype):
    inp = make_inputs(3, T, 2, 4, dk, dv, dtype=dtype, s0_std=0.02, seed=600 + 7 * T + dk + dv)
    o, S, s_in = run_decode_tokens(inp, scale=0.9, in_place=False)
    ro, rS = oracle_prefill(inp, scale=0.9)
    check(o, ro, dtype, "decode_tokens o T=%d" % T)
    check(S, rS, dtype, "decode_tokens state T=%d" % T)
    np.testing.assert_array_equal(s_in, inp.s0)  # the input state is left as it was


def test_decode_tokens_equals_repeated_decode_steps():
    """Below the matrix-core form's threshold (T < 5) one call over T tokens performs exactly
    the arithmetic of T single-token calls."""
    inp = make_inputs(4, 3, 2, 4, 128, 128, dtype="bf16", s0_std=0.02, seed=610)
    o1, S1 = run_decode_steps(inp, 3, scale=0.7)
    o2, S2, _ = run_decode_tokens(inp, scale=0.7, in_place=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def test_decode_tokens_zero_state_and_zero_tokens():
    gdn = gdn_mod()
    inp = make_inputs(2, 3, 1, 2, 64, 64, dtype="bf16", seed=611)
    o, S, _ = run_decode_tokens(inp, use_init=False, in_place=False)
    ro, rS = oracle_prefill(inp, use_init=False)
    check(o, ro, "bf16", "decode_tokens o, zero state")
    check(S, rS, "bf16", "decode_tokens state, zero state")
    t = inp.to_torch(DEV)
    e = {n: t[n][:, :0].contiguous() for n in ("q", "k", "v", "beta", "g")}
    s_in = torch.randn((2, 2, 64, 64), device=DEV)
    s_out = torch.full_like(s_in, 7.0)
    o, s_out = gdn.decode_tokens(e["q"], e["k"], e["v"], e["beta"], e["g"], s_in,
                                 state_out=s_out)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, 64)
    assert torch.equal(s_out, s_in)


def test_decode_tokens_workload_sampled():
    """The decode workload's sizes (B=256, 32 heads, d=128) with T=8 tokens per call;
    every output and final state of 32 sampled chains against the oracle."""
    c = CONFIGS[4]
    inp = make_inputs(c["B"], 8, c["Hk"], c["Hv"], c["dk"], c["dv"], dtype="bf16",
                      s0_std=0.02, seed=612)
    o, S, _ = run_decode_tokens(inp, in_place=True)
    rng = np.random.Generator(np.random.PCG64(612))
    chains = np.sort(rng.choice(c["B"] * c["Hv"], 32, replace=False))
    ro, rS = oracle_prefill(inp, chains=chains)
    b, h = chains // c["Hv"], chains % c["Hv"]
    check(o[b, :, h], ro, "bf16", "decode_tokens workload o")
    check(S[b, h], rS, "bf16", "decode_tokens workload state")
