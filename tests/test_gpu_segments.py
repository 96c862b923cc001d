"""The split plan in segments of chunks.  Its workspace holds the per-chunk records of a
segment (at most 2 GiB of them; the environment variable GDN_SPLIT_RECORD_BYTES lowers the cap,
here to force several segments on short inputs), and longer sequences run segment after
segment with the state, its scale and its norm bound carried between them.  Every segmented
result must equal the one-pass result bit for bit, and meet the oracle's bar (bf16 inputs:
eps <= 2e-3 M): dense and packed sequences (chunks straddling segment boundaries, an empty
sequence), with and without an initial state, without a final state, in place, with the input
prologue, both head sizes and both chunk sizes.
"""
import numpy as np
import pytest

import oracle
from gdn_inputs import make_inputs, round_to
from parity import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ALL = 1 | 2 | 4  # GDN_QK_L2NORM | GDN_BETA_LOGIT | GDN_G_LOGIT
REC = {(128, 64): 73728 + 128, (128, 32): 36864 + 128, (64, 64): 40960 + 128,
       (64, 32): 18432 + 128}  # bytes per record (chunk of one unit)


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_token_gdn_amd as m
    m.load_library()
    return m


def _dense(gdn, inp, chunk, s0=True, want_state=True, in_place=False):
    t = inp.to_torch(DEV)
    init = t["s0"].clone() if s0 else None
    kw = {"final_state": init} if in_place else {}
    o, sT = gdn.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["g"], initial_state=init,
                          output_final_state=want_state, chunk=chunk, **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), None if sT is None else sT.cpu().numpy()


@pytest.mark.parametrize("d,chunk", [(128, 64), (128, 32), (64, 64)])
@pytest.mark.parametrize("slots", [1, 3])
def test_dense_segments_equal_one_pass(gdn, monkeypatch, d, chunk, slots):
    B, T, H = 1, 700, 4  # 11 or 22 chunks per chain: many segments, a ragged last chunk
    inp = make_inputs(B, T, 2, H, d, d, dtype="bf16", s0_std=0.05, seed=1600 + d + chunk)
    assert gdn.gdn_chunk_fwd_plan(B, T, 2, H, d, d, chunk, gdn.GDN_BF16) == "split"
    one = _dense(gdn, inp, chunk)
    one_in_place = _dense(gdn, inp, chunk, in_place=True)
    monkeypatch.setenv("GDN_SPLIT_RECORD_BYTES", str(slots * B * H * REC[(d, chunk)]))
    seg = _dense(gdn, inp, chunk)
    for a, b in zip(one, seg):
        np.testing.assert_array_equal(a, b)
    for a, b in zip(one_in_place, _dense(gdn, inp, chunk, in_place=True)):
        np.testing.assert_array_equal(a, b)
    o_only, none = _dense(gdn, inp, chunk, want_state=False)
    assert none is None
    np.testing.assert_array_equal(o_only, one[0])
    zero = _dense(gdn, inp, chunk, s0=False)
    monkeypatch.delenv("GDN_SPLIT_RECORD_BYTES")
    for a, b in zip(_dense(gdn, inp, chunk, s0=False), zero):
        np.testing.assert_array_equal(a, b)
    ro, rS = oracle.run(inp.q, inp.k, inp.v, inp.beta, inp.g, s0=inp.s0)
    check(seg[0], ro, "bf16", "segments o")
    check(seg[1], rS, "bf16", "segments state")


def _packed(gdn, x, cu, s0, flags, chunk):
    t = {n: torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(torch.bfloat16)
         for n, a in x.items()}
    cu_t = torch.from_numpy(cu.astype(np.int32)).to(DEV)
    init = torch.from_numpy(s0).to(DEV)
    o, sT = gdn.chunk_fwd_varlen(t["q"], t["k"], t["v"], t["beta"], t["g"], cu_seqlens=cu_t,
                                 initial_state=init, flags=flags, chunk=chunk)
    torch.cuda.synchronize()
    return o.cpu().numpy(), sT.cpu().numpy()


@pytest.mark.parametrize("flags", [0, ALL])
@pytest.mark.parametrize("slots", [1, 4])
def test_packed_segments_equal_one_pass(gdn, monkeypatch, flags, slots):
    """Five sequences of 0 to 300 tokens packed into one tensor: their record slots straddle
    the segment boundaries, one sequence is empty (final state = initial state)."""
    rng = np.random.default_rng(1700 + flags + slots)
    lens = [130, 0, 300, 65, 217]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, Hk, Hv, d, chunk = int(cu[-1]), 2, 4, 128, 64
    q = rng.standard_normal((T, Hk, d))
    k = rng.standard_normal((T, Hk, d))
    if not flags:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, Hv, d))
    bl = rng.standard_normal((T, Hv))
    beta = bl if flags else 1 / (1 + np.exp(-bl))
    al = rng.uniform(2.0, 6.0, (T, Hv))
    g = al if flags else -np.log1p(np.exp(-al))
    x = {n: round_to(a, "bf16") for n, a in (("q", q), ("k", k), ("v", v), ("beta", beta),
                                            ("g", g))}
    s0 = (rng.standard_normal((len(lens), Hv, d, d)) * 0.05).astype(np.float32)
    one = _packed(gdn, x, cu, s0, flags, chunk)
    monkeypatch.setenv("GDN_SPLIT_RECORD_BYTES", str(slots * Hv * REC[(d, chunk)]))
    seg = _packed(gdn, x, cu, s0, flags, chunk)
    for a, b in zip(one, seg):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(seg[1][1], s0[1])  # the empty sequence
    ro, rS = oracle.run_packed(x["q"], x["k"], x["v"], x["beta"], x["g"], cu, s0=s0, flags=flags)
    check(seg[0], ro, "bf16", "packed segments o")
    check(seg[1], rS, "bf16", "packed segments state")
