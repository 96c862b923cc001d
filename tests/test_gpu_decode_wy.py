"""The multi-token decode on the matrix cores (gdn_decode_tokens with bf16 inputs, T >= 5 and
dk = dv in {64, 128}: the T tokens as chunks of up to 16 in the chunk form of Eq. (1) of the
explainer page "論文解説: Qwen3.8-Next の設計", section "GDNの中身") against the fp64 oracle:
ragged and multi-chunk T, both head sizes, grouped heads, both output dtypes, the input
prologue (L2 normalisation and both gates as logits), a separate output state, and the
fallback to the token-by-token kernel when q or k is not 16-byte aligned.

Bar (tests/parity.py): bf16 inputs eps <= 2e-3 max|ref| per output tensor.
"""
import numpy as np
import pytest

import oracle
from gdn_inputs import make_inputs, round_to
from parity import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_token_gdn_amd as m
    m.load_library()
    return m


def _run(gdn, x, s0, flags=0, scale=1.0, out_dtype=None, separate=True):
    t = {n: torch.from_numpy(np.ascontiguousarray(x[n], dtype=np.float32)).to(DEV).to(torch.bfloat16)
         for n in ("q", "k", "v", "beta", "g")}
    s_in = torch.from_numpy(np.ascontiguousarray(s0, dtype=np.float32)).to(DEV)
    s_out = torch.full_like(s_in, float("nan")) if separate else s_in
    o, s_out = gdn.decode_tokens(t["q"], t["k"], t["v"], t["beta"], t["g"], s_in,
                                 state_out=s_out, scale=scale, out_dtype=out_dtype, flags=flags)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), s_out.double().cpu().numpy(), s_in.cpu().numpy()


@pytest.mark.parametrize("T", [5, 9, 16, 17, 37])
@pytest.mark.parametrize("d", [64, 128])
def test_matches_oracle(gdn, T, d):
    inp = make_inputs(3, T, 2, 4, d, d, dtype="bf16", s0_std=0.05, seed=1200 + T + d)
    x = {n: getattr(inp, n) for n in ("q", "k", "v", "beta", "g")}
    o, S, s_in = _run(gdn, x, inp.s0, scale=0.8)
    ro, rS = oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, s0=inp.s0, scale=0.8)
    check(o, ro, "bf16", "decode WY o T=%d d=%d" % (T, d))
    check(S, rS, "bf16", "decode WY state T=%d d=%d" % (T, d))
    np.testing.assert_array_equal(s_in, inp.s0)  # the input state is left as it was


@pytest.mark.parametrize("T", [5, 16, 23])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_prologue_flags(gdn, T, d, out):
    """q, k normalised inside, beta and g given as logits (GDN_QK_L2NORM | GDN_BETA_LOGIT |
    GDN_G_LOGIT), against the oracle's packed form over the same B sequences.  A bf16 o adds
    up to 2^-9 relative rounding of its own on top of the fp32 result."""
    rng = np.random.default_rng(1300 + T + d)
    B, Hk, Hv = 2, 2, 4
    x = {"q": rng.standard_normal((B, T, Hk, d)) * 3.0,
         "k": rng.standard_normal((B, T, Hk, d)) * 0.5,
         "v": rng.standard_normal((B, T, Hv, d)),
         "beta": rng.standard_normal((B, T, Hv)),
         "g": rng.uniform(2.0, 6.0, (B, T, Hv))}
    x = {n: round_to(a, "bf16") for n, a in x.items()}
    s0 = (rng.standard_normal((B, Hv, d, d)) * 0.1).astype(np.float32)
    flags = gdn.GDN_QK_L2NORM | gdn.GDN_BETA_LOGIT | gdn.GDN_G_LOGIT
    o, S, _ = _run(gdn, x, s0, flags=flags,
                   out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    cu = np.arange(B + 1, dtype=np.int64) * T
    flat = {n: a.reshape((B * T,) + a.shape[2:]) for n, a in x.items()}
    ro, rS = oracle.run_packed(flat["q"], flat["k"], flat["v"], flat["beta"], flat["g"], cu,
                               s0=s0, flags=flags)
    o = o.reshape(ro.shape)
    if out == "f32":
        check(o, ro, "bf16", "decode WY prologue o T=%d d=%d" % (T, d))
    else:
        eps = np.abs(o - ro).max()
        assert eps <= (2e-3 + 2 ** -8) * np.abs(ro).max(), eps
    check(S, rS, "bf16", "decode WY prologue state T=%d d=%d" % (T, d))


def test_in_place_equals_separate_state(gdn):
    inp = make_inputs(4, 12, 2, 2, 128, 128, dtype="bf16", s0_std=0.05, seed=1400)
    x = {n: getattr(inp, n) for n in ("q", "k", "v", "beta", "g")}
    o1, S1, _ = _run(gdn, x, inp.s0, separate=True)
    o2, S2, _ = _run(gdn, x, inp.s0, separate=False)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def test_unaligned_inputs_take_the_token_kernel(gdn):
    """q and k one element past a 16-byte boundary (the matrix-core form needs q, k and v
    16-byte aligned): the call runs the token-by-token kernel
    (exactly T repeated single-token steps) and still meets the bar."""
    inp = make_inputs(2, 6, 2, 4, 128, 128, dtype="bf16", s0_std=0.05, seed=1500)
    t = inp.to_torch(DEV)
    qs = torch.empty(inp.q.size + 1, dtype=torch.bfloat16, device=DEV)
    ks = torch.empty_like(qs)
    qv = qs[1:].view(inp.q.shape)
    kv = ks[1:].view(inp.k.shape)
    qv.copy_(t["q"])
    kv.copy_(t["k"])
    assert qv.data_ptr() % 16 != 0
    s = t["s0"].clone()
    o, s = gdn.decode_tokens(qv, kv, t["v"], t["beta"], t["g"], s)
    s1 = t["s0"].clone()
    outs = []
    for i in range(6):
        outs.append(gdn.decode_step(*[t[n][:, i].contiguous() for n in ("q", "k", "v", "beta", "g")],
                                    s1))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o.cpu().numpy(), torch.stack(outs, 1).cpu().numpy())
    np.testing.assert_array_equal(s.cpu().numpy(), s1.cpu().numpy())
    ro, rS = oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, s0=inp.s0)
    check(o.double().cpu().numpy(), ro, "bf16", "unaligned o")
    check(s.double().cpu().numpy(), rS, "bf16", "unaligned state")
