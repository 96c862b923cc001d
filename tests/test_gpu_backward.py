"""GPU parity of the backward (gdn_backward, through its C ABI) against the fp64 oracle's
reverse recurrence (itself pinned to torch autograd and a closed form on the CPU).  Head sizes
in {64, 128} run the chunk-parallel kernels by default; GDN_BWD=token pins the token-recurrent
path, and both are tested.

Bars (tests/parity.py), per gradient tensor: fp32 inputs eps <= 1e-5 max(1, M); bf16 inputs
eps <= 2e-3 M.  fp32 inputs are computed in fp32 throughout; for bf16 inputs the chunk-parallel
path rounds its per-chunk records and matrix-core operands to fp16 (fp32 accumulation, fp32
states), which is where their error comes from.
"""
import numpy as np
import pytest

import oracle
from gdn_inputs import config_inputs, make_inputs
from parity import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GRADS = (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dbeta", "dbeta"), ("dg", "dg"),
         ("d_initial_state", "dS0"))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_token_gdn_amd as gdn
    gdn.load_library()


def run_case(inp, seed, scale=1.0, with_dST=True, dout_bf16=False):
    import linear_attention_token_gdn_amd as gdn
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, Hv, dv = inp.v.shape
    dk = inp.q.shape[3]
    dO = rng.standard_normal((B, T, Hv, dv)).astype(np.float32)
    if dout_bf16:
        from gdn_inputs import round_to_bf16
        dO = round_to_bf16(dO)
    dST = (rng.standard_normal((B, Hv, dk, dv)).astype(np.float32) * 0.1) if with_dST else None
    t = inp.to_torch(DEV)
    d_o = torch.from_numpy(dO).to(DEV)
    if dout_bf16:
        d_o = d_o.to(torch.bfloat16)
    got = gdn.backward(t["q"], t["k"], t["v"], t["beta"], t["g"], d_o,
                       initial_state=t["s0"],
                       d_final_state=None if dST is None else torch.from_numpy(dST).to(DEV),
                       scale=scale)
    torch.cuda.synchronize()
    ref = oracle.backward(inp.q, inp.k, inp.v, inp.beta, inp.g, dO, s0=inp.s0, dST=dST,
                          scale=scale)
    return {n: got[n].cpu().numpy() for n, _ in GRADS}, ref


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 16), (16, 64), (64, 128), (128, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_head_sizes(dk, dv, dtype):
    inp = make_inputs(2, 45, 1, 2, dk, dv, dtype=dtype, s0_std=0.02, seed=800 + dk + dv)
    got, ref = run_case(inp, 801 + dk, scale=0.9)
    for n, r in GRADS:
        check(got[n], ref[r], dtype, "%s dk%d dv%d %s" % (n, dk, dv, dtype))


@pytest.mark.parametrize("variant", ["chunk", "token"])
def test_backward_long_ragged_grouped(variant, monkeypatch):
    """T = 157 (three checkpoint blocks / chunks, the last one partial), grouped heads
    (Hv = 2 Hk), no initial state, bf16 gradient of the output."""
    if variant == "token":
        monkeypatch.setenv("GDN_BWD", "token")
    inp = make_inputs(1, 157, 2, 4, 128, 128, dtype="bf16", seed=810)
    got, ref = run_case(inp, 811, dout_bf16=True)
    for n, r in GRADS:
        check(got[n], ref[r], "bf16", n + " T=157 gqa " + variant)


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (64, 128), (128, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_chunked_against_token(dk, dv, dtype, monkeypatch):
    """The two paths against the oracle on one longer ragged case (T = 300: five chunks), with
    an initial state and a final-state gradient."""
    inp = make_inputs(1, 300, 1, 2, dk, dv, dtype=dtype, s0_std=0.02, seed=840 + dk + dv)
    got, ref = run_case(inp, 841, scale=0.8)
    monkeypatch.setenv("GDN_BWD", "token")
    tok, _ = run_case(inp, 841, scale=0.8)
    for n, r in GRADS:
        check(got[n], ref[r], dtype, "%s chunk dk%d dv%d %s" % (n, dk, dv, dtype))
        check(tok[n], ref[r], dtype, "%s token dk%d dv%d %s" % (n, dk, dv, dtype))


@pytest.mark.parametrize("T", [0, 1, 64, 65])
def test_backward_edge_lengths(T):
    inp = make_inputs(2, T, 1, 1, 64, 64, dtype="bf16", s0_std=0.05, seed=820 + T)
    got, ref = run_case(inp, 821 + T, with_dST=(T != 1))
    for n, r in GRADS:
        if got[n].size:
            check(got[n], ref[r], "bf16", "%s T=%d" % (n, T))


def test_backward_deterministic():
    inp = make_inputs(1, 100, 1, 2, 128, 128, dtype="bf16", s0_std=0.02, seed=830)
    a, _ = run_case(inp, 831)
    b, _ = run_case(inp, 831)
    for n, _ in GRADS:
        np.testing.assert_array_equal(a[n], b[n])


def test_backward_prefill_workload_full():
    """The backward at the size the benchmark times (B=1, T=4096, 16 heads, d=128, bf16
    inputs, an fp32 gradient of o, no initial state): every gradient of every chain against
    the oracle."""
    inp = config_inputs(1)
    got, ref = run_case(inp, 850, with_dST=False)
    for n, r in GRADS:
        e = check(got[n], ref[r], "bf16", n + " T=4096 H=16")
        print("%s: err %.2e (max %.2e)" % (n, e[0], e[1]))
