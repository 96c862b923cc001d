"""GPU parity of the segmented prefill plan against the fp64 oracle.

The plan cuts every chain into segments of chunks and runs them in parallel: a transition pass
gives each segment's affine map of the state (S_out = M S_in + N: the gated delta rule of the
explainer page "論文解説: Qwen3.8-Next の設計", ta-paperlens.web.app, section "GDNの中身",
Eq. (1), is affine in the state), a combine pass chains those maps into every segment's entry
state, and the single-pass kernel then runs all segments from their entry states.

The cases make the transitions matter: long-memory gates (g close to 0), an initial state of
the values' order, and segments as short as one chunk (GDN_SEG_CHUNKS), so that an error in M,
in the combine, or at a segment boundary shows in the outputs.  Bars (tests/parity.py): bf16
inputs eps <= 2e-3 M, eps = max|X - R|, M = max|R|.
"""
import numpy as np
import pytest

import oracle
from gdn_inputs import make_inputs
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


def _run(inp, chunk=64, s0=True, in_place=False, final=True, out_dtype=None):
    import linear_attention_token_gdn_amd as gdn
    t = inp.to_torch(DEV)
    init = t["s0"].clone() if (s0 and t["s0"] is not None) else None
    kw = {}
    if in_place:
        kw["final_state"] = init
    o, sT = gdn.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["g"], initial_state=init,
                          output_final_state=final, chunk=chunk, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return (o.double().cpu().numpy(),
            None if sT is None else sT.double().cpu().numpy())


def _plan(inp, chunk=64):
    import linear_attention_token_gdn_amd as gdn
    B, T, Hk, dk = inp.q.shape
    return gdn.gdn_chunk_fwd_plan(B, T, Hk, inp.v.shape[2], dk, inp.v.shape[3], chunk,
                                  gdn.GDN_BF16)


def _long_memory(B, T, Hk, Hv, d, seed, s0_std=0.5):
    # gates close to 0 and an initial state of the values' order: the state entering a
    # segment shapes its outputs, so every transition and entry state is exercised
    return make_inputs(B, T, Hk, Hv, d, d, dtype="bf16", s0_std=s0_std, seed=seed,
                       g_range=(1e-5, 1e-3))


def _tm_mode(tm, monkeypatch):
    # "records": the transition pass stores every chunk's (I + A)^-1 and the output pass reads
    # it (the default when the workspace holds the records); "formed": both passes form it
    if tm == "formed":
        monkeypatch.setenv("GDN_SEG_NO_TM", "1")


@pytest.mark.parametrize("tm", ["records", "formed"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("seg_chunks", [1, 3])
def test_segmented_matches_oracle(d, chunk, seg_chunks, tm, monkeypatch):
    monkeypatch.setenv("GDN_FORCE_VARIANT", "segmented")
    monkeypatch.setenv("GDN_SEG_CHUNKS", str(seg_chunks))
    _tm_mode(tm, monkeypatch)
    inp = _long_memory(2, 1000, 1, 2, d, seed=1100 + d + chunk + seg_chunks)
    assert _plan(inp, chunk) == "segmented"
    o, sT = _run(inp, chunk)
    ro, rS = oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, s0=inp.s0)
    tag = "segmented d%d C%d L%d %s" % (d, chunk, seg_chunks, tm)
    check(o, ro, "bf16", tag + " o")
    check(sT, rS, "bf16", tag + " final state")


@pytest.mark.parametrize("tm", ["records", "formed"])
@pytest.mark.parametrize("T", [129, 192, 4 * 64, 4 * 64 + 1])
def test_segment_boundaries(T, tm, monkeypatch):
    # two or more segments of two chunks; a last segment of one (possibly partial) chunk
    monkeypatch.setenv("GDN_FORCE_VARIANT", "segmented")
    monkeypatch.setenv("GDN_SEG_CHUNKS", "2")
    _tm_mode(tm, monkeypatch)
    inp = _long_memory(1, T, 2, 2, 128, seed=1200 + T)
    assert _plan(inp) == "segmented"
    o, sT = _run(inp)
    ro, rS = oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, s0=inp.s0)
    check(o, ro, "bf16", "T=%d o" % T)
    check(sT, rS, "bf16", "T=%d final state" % T)


def test_in_place_zero_state_no_final_and_bf16_output(monkeypatch):
    monkeypatch.setenv("GDN_FORCE_VARIANT", "segmented")
    monkeypatch.setenv("GDN_SEG_CHUNKS", "2")
    inp = _long_memory(1, 700, 2, 4, 128, seed=1300)
    ro, rS = oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, s0=inp.s0)
    o, sT = _run(inp, in_place=True)  # the final state overwrites the initial one
    check(o, ro, "bf16", "in place o")
    check(sT, rS, "bf16", "in place final state")
    o, sT = _run(inp, final=False, out_dtype=torch.bfloat16)
    assert sT is None
    # bf16 storage of o adds up to 2^-9 relative rounding on top of the fp32 result
    assert np.abs(o - ro).max() <= (2e-3 + 2 ** -8) * np.abs(ro).max()
    ro0, rS0 = oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g)
    o, sT = _run(inp, s0=False)
    check(o, ro0, "bf16", "zero state o")
    check(sT, rS0, "bf16", "zero state final")


def test_prologue_flags(monkeypatch):
    import linear_attention_token_gdn_amd as gdn
    monkeypatch.setenv("GDN_FORCE_VARIANT", "segmented")
    monkeypatch.setenv("GDN_SEG_CHUNKS", "2")
    flags = gdn.GDN_QK_L2NORM | gdn.GDN_BETA_LOGIT | gdn.GDN_G_LOGIT
    rng = np.random.default_rng(1400)
    B, T, H, d = 1, 600, 2, 128
    raw = {"q": rng.standard_normal((B, T, H, d)) * 3.0,
           "k": rng.standard_normal((B, T, H, d)) * 0.3,
           "v": rng.standard_normal((B, T, H, d)),
           "beta": rng.standard_normal((B, T, H)),
           "g": rng.standard_normal((B, T, H)) + 6.0}  # log sigmoid: gates near 1
    bf = {n: torch.from_numpy(x.astype(np.float32)).bfloat16() for n, x in raw.items()}
    s0 = (rng.standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
    t = {n: x.to(DEV) for n, x in bf.items()}
    o, sT = gdn.chunk_fwd_varlen(t["q"], t["k"], t["v"], t["beta"], t["g"],
                                 initial_state=torch.from_numpy(s0).to(DEV), flags=flags)
    torch.cuda.synchronize()
    f64 = {n: x.float().numpy().astype(np.float64) for n, x in bf.items()}
    ro, rS = oracle.run_packed(f64["q"][0], f64["k"][0], f64["v"][0], f64["beta"][0],
                               f64["g"][0], np.array([0, T], dtype=np.int32), s0=s0,
                               flags=flags)
    check(o.double().cpu().numpy()[0], ro, "bf16", "prologue o")
    check(sT.double().cpu().numpy(), rS, "bf16", "prologue final state")


def test_default_plan_few_long_chains_every_chain():
    # the default geometry on 16 chains x 8192 tokens: 16 segments of 8 chunks per chain
    inp = _long_memory(1, 8192, 16, 16, 128, seed=1500, s0_std=0.02)
    assert _plan(inp) == "segmented"
    o, sT = _run(inp)
    ro, rS = oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, s0=inp.s0)
    check(o, ro, "bf16", "default geometry o")
    check(sT, rS, "bf16", "default geometry final state")


def test_deterministic(monkeypatch):
    monkeypatch.setenv("GDN_FORCE_VARIANT", "segmented")
    monkeypatch.setenv("GDN_SEG_CHUNKS", "2")
    inp = _long_memory(1, 900, 2, 2, 128, seed=1600)
    a = _run(inp)
    b = _run(inp)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def _packed_inputs(lens, Hk, Hv, d, seed, flags):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    q = rng.standard_normal((T, Hk, d))
    k = rng.standard_normal((T, Hk, d))
    if not flags:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, Hv, d))
    bl = rng.standard_normal((T, Hv))
    beta = bl if flags else 1 / (1 + np.exp(-bl))
    al = rng.uniform(5.0, 9.0, (T, Hv))  # gates close to 1: the transitions matter
    g = al if flags else -np.log1p(np.exp(-al))
    from gdn_inputs import round_to
    x = {n: round_to(a, "bf16") for n, a in (("q", q), ("k", k), ("v", v), ("beta", beta),
                                            ("g", g))}
    s0 = (rng.standard_normal((len(lens), Hv, d, d)) * 0.5).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return x, s0, cu


@pytest.mark.parametrize("tm", ["records", "formed"])
@pytest.mark.parametrize("flags", [0, 1 | 2 | 4])
def test_packed_sequences(flags, tm, monkeypatch):
    """Packed sequences through the segmented plan: every (sequence, head) chain in the same
    number of segments, each of ceil(its chunks / segments) chunks formed on the device --
    long and short sequences, a one-token and an empty one (final state = initial state, every
    segment empty)."""
    import linear_attention_token_gdn_amd as gdn
    monkeypatch.setenv("GDN_FORCE_VARIANT", "segmented")
    _tm_mode(tm, monkeypatch)
    lens = [1500, 0, 1, 700, 65, 2300]
    x, s0, cu = _packed_inputs(lens, 1, 2, 128, seed=1700 + flags, flags=flags)
    t = {n: torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(torch.bfloat16)
         for n, a in x.items()}
    cu_t = torch.from_numpy(cu.astype(np.int32)).to(DEV)
    o, sT = gdn.chunk_fwd_varlen(t["q"], t["k"], t["v"], t["beta"], t["g"], cu_seqlens=cu_t,
                                 initial_state=torch.from_numpy(s0).to(DEV), flags=flags)
    torch.cuda.synchronize()
    o, sT = o.double().cpu().numpy(), sT.double().cpu().numpy()
    np.testing.assert_array_equal(sT[1], s0[1])  # the empty sequence
    ro, rS = oracle.run_packed(x["q"], x["k"], x["v"], x["beta"], x["g"], cu, s0=s0,
                               flags=flags)
    check(o, ro, "bf16", "packed segmented o")
    check(sT, rS, "bf16", "packed segmented state")


def test_packed_default_plan_long_sequences():
    """Few long packed sequences take the segmented plan by default (judged on the mean
    length); the workspace query agrees with the dense call of the same sizes' plan."""
    import linear_attention_token_gdn_amd as gdn
    N, T, H = 2, 2 * 16384, 4  # 8 chains: 32 segments of 8 chunks per chain
    wsz = gdn.gdn_chunk_fwd_varlen_workspace_size(N, T, H, H, 128, 128, 64, gdn.GDN_BF16, 1, 0)
    # the maps and entry states, then one (I + A)^-1 record (10 fp16 16 x 16 blocks) per chunk
    # slot and head, T / 64 + N slots
    assert wsz == (2 * 31 + 32) * N * H * 128 * 128 * 4 + H * (T // 64 + N) * 10 * 512
    x, s0, cu = _packed_inputs([16384, 16384], H, H, 128, seed=1800, flags=0)
    t = {n: torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(torch.bfloat16)
         for n, a in x.items()}
    cu_t = torch.from_numpy(cu.astype(np.int32)).to(DEV)
    o, sT = gdn.chunk_fwd_varlen(t["q"], t["k"], t["v"], t["beta"], t["g"], cu_seqlens=cu_t,
                                 initial_state=torch.from_numpy(s0).to(DEV))
    torch.cuda.synchronize()
    ro, rS = oracle.run_packed(x["q"], x["k"], x["v"], x["beta"], x["g"], cu, s0=s0)
    check(o.double().cpu().numpy(), ro, "bf16", "packed default o")
    check(sT.double().cpu().numpy(), rS, "bf16", "packed default state")
