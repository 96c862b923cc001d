"""GPU parity of the input prologue and packed sequences (gdn_chunk_fwd_varlen, and the flags of
gdn_decode_tokens) against the fp64 oracle's packed entry point, on seeded raw inputs: q and k
not normalised, beta and alpha as logits where the flags say so.

Bars (tests/parity.py): fp32 inputs eps <= 1e-5 max(1, M); bf16 inputs eps <= 2e-3 M.
"""
import numpy as np
import pytest

import oracle
from gdn_inputs import round_to
from parity import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ALL = 1 | 2 | 4  # GDN_QK_L2NORM | GDN_BETA_LOGIT | GDN_G_LOGIT


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_token_gdn_amd as gdn
    gdn.load_library()


def gdn_mod():
    import linear_attention_token_gdn_amd as gdn
    return gdn


def raw_inputs(lead, Hk, Hv, dk, dv, flags, dtype, seed, s0_shape=None):
    """Raw stored inputs with leading dims `lead` (q, k unnormalised when the prologue
    normalises them; gate logits when the flags say so), rounded to the storage dtype."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal(lead + (Hk, dk)).astype(np.float32)
    k = rng.standard_normal(lead + (Hk, dk)).astype(np.float32)
    if not flags & 1:  # plain path: unit keys and queries, as the caller would provide
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    else:  # any scale: the library normalises
        q *= rng.uniform(0.2, 5.0, lead + (Hk, 1)).astype(np.float32)
        k *= rng.uniform(0.2, 5.0, lead + (Hk, 1)).astype(np.float32)
    v = rng.standard_normal(lead + (Hv, dv)).astype(np.float32)
    blog = rng.standard_normal(lead + (Hv,)).astype(np.float32)
    beta = blog if flags & 2 else 1.0 / (1.0 + np.exp(-blog))
    # alpha in (0.88, 0.998) either as a logit or as log alpha
    alog = rng.uniform(2.0, 6.0, lead + (Hv,)).astype(np.float32)
    g = alog if flags & 4 else -np.log1p(np.exp(-alog.astype(np.float64)))
    s0 = None if s0_shape is None else (rng.standard_normal(s0_shape) * 0.02).astype(np.float32)
    return {n: round_to(x, dtype) for n, x in (("q", q), ("k", k), ("v", v), ("beta", beta),
                                                 ("g", g))}, s0


def to_dev(d, dtype):
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    return {n: torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(td) for n, x in d.items()}


LENGTHS = [64, 1, 0, 130, 63, 65, 200, 17]


@pytest.mark.parametrize("flags", [0, ALL, 1, 6, ALL | 8])
@pytest.mark.parametrize("variant", ["default", "fused", "recurrent"])
def test_packed_bf16(flags, variant, monkeypatch):
    """The default for these 32 (sequence, head) chains is the split plan; flag 8 is the plan
    hint GDN_PREFER_SPLIT (split here anyway unless a variant is forced)."""
    if variant != "default":
        monkeypatch.setenv("GDN_FORCE_VARIANT", variant)
    gdn = gdn_mod()
    Hk, Hv, d = 2, 4, 128
    cu = np.concatenate([[0], np.cumsum(LENGTHS)]).astype(np.int64)
    T, N = int(cu[-1]), len(LENGTHS)
    if variant == "default":
        assert gdn.gdn_chunk_fwd_plan(N, T, Hk, Hv, d, d, 64, gdn.GDN_BF16) == "split"
    x, s0 = raw_inputs((T,), Hk, Hv, d, d, flags, "bf16", 700 + flags, (N, Hv, d, d))
    t = to_dev(x, "bf16")
    cu_t = torch.from_numpy(cu.astype(np.int32)).to(DEV)
    s0_t = torch.from_numpy(s0).to(DEV)
    o, sT = gdn.chunk_fwd_varlen(t["q"], t["k"], t["v"], t["beta"], t["g"], cu_seqlens=cu_t,
                                 initial_state=s0_t, chunk=64, scale=0.9, flags=flags)
    torch.cuda.synchronize()
    ro, rS = oracle.run_packed(x["q"], x["k"], x["v"], x["beta"], x["g"], cu, s0=s0,
                               scale=0.9, flags=flags)
    check(o.cpu().numpy(), ro, "bf16", "packed o flags=%d %s" % (flags, variant))
    check(sT.cpu().numpy(), rS, "bf16", "packed state flags=%d %s" % (flags, variant))


@pytest.mark.parametrize("flags", [0, ALL])
def test_packed_fp32_and_small_heads(flags):
    """fp32 inputs (the recurrent path, IEEE fp32 throughout) and dk != dv."""
    gdn = gdn_mod()
    Hk, Hv, dk, dv = 1, 2, 32, 16
    lengths = [3, 0, 40, 1, 19]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T, N = int(cu[-1]), len(lengths)
    x, s0 = raw_inputs((T,), Hk, Hv, dk, dv, flags, "f32", 710 + flags, (N, Hv, dk, dv))
    t = to_dev(x, "f32")
    cu_t = torch.from_numpy(cu.astype(np.int32)).to(DEV)
    o, sT = gdn.chunk_fwd_varlen(t["q"], t["k"], t["v"], t["beta"], t["g"], cu_seqlens=cu_t,
                                 initial_state=torch.from_numpy(s0).to(DEV), chunk=16,
                                 flags=flags)
    torch.cuda.synchronize()
    ro, rS = oracle.run_packed(x["q"], x["k"], x["v"], x["beta"], x["g"], cu, s0=s0,
                               flags=flags)
    check(o.cpu().numpy(), ro, "f32", "packed fp32 o flags=%d" % flags)
    check(sT.cpu().numpy(), rS, "f32", "packed fp32 state flags=%d" % flags)


def test_packed_without_states_and_all_empty():
    gdn = gdn_mod()
    cu = np.array([0, 0, 50, 50], dtype=np.int64)
    x, _ = raw_inputs((50,), 1, 1, 64, 64, ALL, "bf16", 720)
    t = to_dev(x, "bf16")
    o, sT = gdn.chunk_fwd_varlen(t["q"], t["k"], t["v"], t["beta"], t["g"],
                                 cu_seqlens=torch.from_numpy(cu.astype(np.int32)).to(DEV),
                                 flags=ALL)
    torch.cuda.synchronize()
    ro, rS = oracle.run_packed(x["q"], x["k"], x["v"], x["beta"], x["g"], cu, flags=ALL)
    check(o.cpu().numpy(), ro, "bf16", "packed o, zero states")
    check(sT.cpu().numpy(), rS, "bf16", "packed state, zero states")
    assert not sT[0].any() and not sT[2].any()  # empty sequences keep the zero state


@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("variant", ["fused", "split", "hint"])
def test_packed_many_sequences(variant, chunk, monkeypatch):
    """More than 64 sequences (the split prep finds a slot's sequence 64 offsets at a time),
    many of them empty or of one token, bf16 outputs, a given initial state.  "hint": no forced
    variant, the plan hint GDN_PREFER_SPLIT instead."""
    if variant != "hint":
        monkeypatch.setenv("GDN_FORCE_VARIANT", variant)
    gdn = gdn_mod()
    rng = np.random.default_rng(750 + chunk)
    lengths = rng.choice([0, 1, 2, chunk - 1, chunk, chunk + 1, 3 * chunk + 5], size=70)
    lengths[:3] = 0  # leading empty sequences
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    # 140 chains: the fused kernel by default, split only when forced or hinted
    T, N, Hk, Hv, d = int(cu[-1]), len(lengths), 1, 2, 64
    x, s0 = raw_inputs((T,), Hk, Hv, d, d, ALL, "bf16", 751 + chunk, (N, Hv, d, d))
    t = to_dev(x, "bf16")
    run = lambda flags: gdn.chunk_fwd_varlen(
        t["q"], t["k"], t["v"], t["beta"], t["g"],
        cu_seqlens=torch.from_numpy(cu.astype(np.int32)).to(DEV),
        initial_state=torch.from_numpy(s0).to(DEV), chunk=chunk, scale=1.1, flags=flags,
        out_dtype=torch.bfloat16)
    o, sT = run(ALL | (gdn.GDN_PREFER_SPLIT if variant == "hint" else 0))
    torch.cuda.synchronize()
    if variant == "hint":  # the hint runs exactly the split plan
        monkeypatch.setenv("GDN_FORCE_VARIANT", "split")
        o2, s2 = run(ALL)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(sT, s2)
    ro, rS = oracle.run_packed(x["q"], x["k"], x["v"], x["beta"], x["g"], cu, s0=s0, scale=1.1,
                               flags=ALL)
    # bf16 storage of o adds up to 2^-9 relative rounding on top of the fp32 result
    oe = np.abs(o.float().cpu().numpy() - ro).max()
    assert oe <= (2e-3 + 2 ** -8) * np.abs(ro).max(), ("many packed o " + variant, oe)
    check(sT.cpu().numpy(), rS, "bf16", "many packed state " + variant)
    empty = np.flatnonzero(lengths == 0)
    assert torch.equal(sT[empty].cpu(), torch.from_numpy(s0[empty]))  # final = initial


@pytest.mark.parametrize("variant", ["split", "fused", "recurrent"])
def test_dense_with_prologue(variant, monkeypatch):
    """cu_seqlens = NULL: dense batches with the prologue, on every plan (split is the
    default for these few chains)."""
    monkeypatch.setenv("GDN_FORCE_VARIANT", variant)
    gdn = gdn_mod()
    B, T, Hk, Hv, d = 2, 157, 2, 4, 128
    x, s0 = raw_inputs((B, T), Hk, Hv, d, d, ALL, "bf16", 730, (B, Hv, d, d))
    t = to_dev(x, "bf16")
    o, sT = gdn.chunk_fwd_varlen(t["q"], t["k"], t["v"], t["beta"], t["g"],
                                 initial_state=torch.from_numpy(s0).to(DEV), chunk=64,
                                 scale=0.8, flags=ALL)
    torch.cuda.synchronize()
    cu = np.arange(B + 1, dtype=np.int64) * T
    flat = {n: a.reshape((B * T,) + a.shape[2:]) for n, a in x.items()}
    ro, rS = oracle.run_packed(flat["q"], flat["k"], flat["v"], flat["beta"], flat["g"], cu,
                               s0=s0, scale=0.8, flags=ALL)
    check(o.cpu().numpy().reshape(B * T, Hv, d), ro, "bf16", "dense+prologue o " + variant)
    check(sT.cpu().numpy(), rS, "bf16", "dense+prologue state " + variant)


@pytest.mark.parametrize("variant", ["fused", "split"])
def test_packed_equals_dense_when_lengths_are_equal(variant):
    """Equal lengths: the packed call and the dense call run the same arithmetic per chain."""
    gdn = gdn_mod()
    B, T, Hk, Hv, d = 3, 100, 2, 4, 64
    x, s0 = raw_inputs((B, T), Hk, Hv, d, d, ALL, "bf16", 740, (B, Hv, d, d))
    t = to_dev(x, "bf16")
    s0_t = torch.from_numpy(s0).to(DEV)
    import os
    os.environ["GDN_FORCE_VARIANT"] = variant
    try:
        od, Sd = gdn.chunk_fwd_varlen(t["q"], t["k"], t["v"], t["beta"], t["g"],
                                      initial_state=s0_t, chunk=32, flags=ALL)
        cu = torch.arange(B + 1, dtype=torch.int32, device=DEV) * T
        flat = {n: a.reshape((B * T,) + tuple(a.shape[2:])) for n, a in t.items()}
        op, Sp = gdn.chunk_fwd_varlen(flat["q"], flat["k"], flat["v"], flat["beta"], flat["g"],
                                      cu_seqlens=cu, initial_state=s0_t, chunk=32, flags=ALL)
        torch.cuda.synchronize()
    finally:
        del os.environ["GDN_FORCE_VARIANT"]
    assert torch.equal(od.reshape(B * T, Hv, d), op)
    assert torch.equal(Sd, Sp)


@pytest.mark.parametrize("T", [1, 4])
@pytest.mark.parametrize("flags", [ALL, 1, 2])
def test_decode_tokens_with_prologue(T, flags):
    gdn = gdn_mod()
    B, Hk, Hv, d = 3, 2, 4, 128
    x, s0 = raw_inputs((B, T), Hk, Hv, d, d, flags, "bf16", 750 + T + flags, (B, Hv, d, d))
    t = to_dev(x, "bf16")
    state = torch.from_numpy(s0).to(DEV)
    o, S = gdn.decode_tokens(t["q"], t["k"], t["v"], t["beta"], t["g"], state, flags=flags,
                             scale=1.1)
    torch.cuda.synchronize()
    cu = np.arange(B + 1, dtype=np.int64) * T
    flat = {n: a.reshape((B * T,) + a.shape[2:]) for n, a in x.items()}
    ro, rS = oracle.run_packed(flat["q"], flat["k"], flat["v"], flat["beta"], flat["g"], cu,
                               s0=s0, scale=1.1, flags=flags)
    check(o.cpu().numpy().reshape(B * T, Hv, d), ro, "bf16", "decode prologue o T=%d" % T)
    check(S.cpu().numpy(), rS, "bf16", "decode prologue state T=%d" % T)


@pytest.mark.parametrize("variant", ["split", "fused", "recurrent"])
def test_malformed_offsets_stay_in_bounds(variant, monkeypatch):
    """Offsets that decrease or leave [0, T] are clamped on the device: the call succeeds, every
    access stays inside the tensors (and the split plan's record slots inside the workspace).
    The per-chain kernels give each sequence the recurrence over its clamped range
    a = clamp(cu[i], 0, T), b = min(max(cu[i+1], a), T).  The split plan's record slots of
    overlapping sequences coincide (sequences 1 and 3 here), so there only sequence 0, whose
    slots no other sequence claims, is checked.  Clamped ranges overlap, so the rows of o
    (written by several sequences) are only checked to be finite."""
    monkeypatch.setenv("GDN_FORCE_VARIANT", variant)
    gdn = gdn_mod()
    T, Hk, Hv, d = 300, 1, 2, 64
    cu = np.array([0, 120, 80, 400, -5, 300], dtype=np.int64)
    N = len(cu) - 1
    x, s0 = raw_inputs((T,), Hk, Hv, d, d, ALL, "bf16", 760, (N, Hv, d, d))
    t = to_dev(x, "bf16")
    o, sT = gdn.chunk_fwd_varlen(t["q"], t["k"], t["v"], t["beta"], t["g"],
                                 cu_seqlens=torch.from_numpy(cu.astype(np.int32)).to(DEV),
                                 initial_state=torch.from_numpy(s0).to(DEV), chunk=64, flags=ALL)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    for i in (range(1) if variant == "split" else range(N)):
        a = min(max(int(cu[i]), 0), T)
        b = min(max(int(cu[i + 1]), a), T)
        sl = {n: arr[a:b] for n, arr in x.items()}
        _, rS = oracle.run_packed(sl["q"], sl["k"], sl["v"], sl["beta"], sl["g"],
                                  np.array([0, b - a]), s0=s0[i:i + 1], flags=ALL)
        check(sT[i:i + 1].cpu().numpy(), rS, "bf16", "clamped sequence %d state %s" % (i, variant))
