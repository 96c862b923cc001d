"""GPU check of gdn_chunk_fwd_noalloc (the prefill for callers that cannot allocate, whose
workspace is the library's static scratch) against gdn_chunk_fwd with a caller workspace, both
through the C ABI on the same inputs: bit-identical outputs and final states, two calls in a
row (the second smaller, so the scratch still holds the first call's records), a plan without a
workspace, the segmented plan (transitions, entry states and per-chunk (I + A)^-1 records in
the scratch; and, where the records do not fit, the same plan forming that inverse in both
passes, as gdn_chunk_fwd does under GDN_SEG_NO_TM), and a split-plan
input whose records exceed the scratch, which runs in two segments there and in one with the
caller's workspace.  The outputs are also held to the oracle's bar (bf16
inputs: eps <= 2e-3 M).
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


def _call(inp, noalloc, chunk=64):
    import linear_attention_token_gdn_amd as gdn
    t = inp.to_torch(DEV)
    B, T, Hk, dk = inp.q.shape
    Hv, dv = inp.v.shape[2], inp.v.shape[3]
    o = torch.full((B, T, Hv, dv), float("nan"), device=DEV)
    sT = torch.full((B, Hv, dk, dv), float("nan"), device=DEV)
    s0 = t["s0"]
    stream = torch.cuda.current_stream().cuda_stream
    ptr = lambda x: None if x is None else x.data_ptr()
    args = [ptr(t[n]) for n in ("q", "k", "v", "beta", "g")] + [ptr(s0), o.data_ptr(),
                                                                 sT.data_ptr()]
    dims = [B, T, Hk, Hv, dk, dv, chunk, 1.0, gdn.GDN_BF16, gdn.GDN_F32]
    if noalloc:
        st = gdn.gdn_chunk_fwd_noalloc(*args, *dims, stream)
    else:
        need = gdn.gdn_chunk_fwd_workspace_size(B, T, Hk, Hv, dk, dv, chunk, gdn.GDN_BF16)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
        st = gdn.gdn_chunk_fwd(*args, *dims, ws.data_ptr() if need else None, need, stream)
    torch.cuda.synchronize()
    return st, o.cpu().numpy(), sT.cpu().numpy()


def _same(inp, plan):
    import linear_attention_token_gdn_amd as gdn
    B, T, Hk, dk = inp.q.shape
    assert gdn.gdn_chunk_fwd_plan(B, T, Hk, inp.v.shape[2], dk, inp.v.shape[3], 64,
                                  gdn.GDN_BF16) == plan
    st1, o1, s1 = _call(inp, noalloc=True)
    st2, o2, s2 = _call(inp, noalloc=False)
    assert st1 == gdn.GDN_OK and st2 == gdn.GDN_OK, (st1, st2)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)
    return o1, s1


def test_noalloc_equals_the_workspace_entry_point(monkeypatch):
    import linear_attention_token_gdn_amd as gdn
    # 1: the 4096-token, 16-head prefill (split plan, 72 MiB of the 80 MiB scratch)
    big = make_inputs(1, 4096, 16, 16, 128, 128, dtype="bf16", seed=990)
    o, s = _same(big, "split")
    chains = np.array([0, 7, 15])
    ro, rS = oracle.run(big.q, big.k, big.v, big.beta, big.g, chains=chains)
    check(o[0][:, chains].transpose(1, 0, 2), ro, "bf16", "noalloc o (T=4096)")
    check(s[0][chains], rS, "bf16", "noalloc state (T=4096)")
    # 2: right after, a smaller call with an initial state and a ragged tail: the scratch
    #    still holds the first call's records and progress words
    small = make_inputs(2, 1000, 2, 4, 128, 128, dtype="bf16", s0_std=0.02, seed=991)
    o, s = _same(small, "split")
    ro, rS = oracle.run(small.q, small.k, small.v, small.beta, small.g, s0=small.s0)
    check(o, ro, "bf16", "noalloc o (T=1000)")
    check(s, rS, "bf16", "noalloc state (T=1000)")
    # 3: a plan without a workspace (many chains: the single-pass kernel)
    many = make_inputs(1, 200, 64, 128, 64, 64, dtype="bf16", s0_std=0.02, seed=992)
    _same(many, "fused")
    # 4: the segmented plan (8192 tokens, 16 heads: 16 segments of 8 chunks per chain; its
    #    transitions and entry states in 46 MiB of the scratch)
    huge = make_inputs(1, 8192, 16, 16, 128, 128, dtype="bf16", s0_std=0.02, seed=993)
    o, s = _same(huge, "segmented")
    chains = np.array([3, 12])
    ro, rS = oracle.run(huge.q, huge.k, huge.v, huge.beta, huge.g, s0=huge.s0, chains=chains)
    check(o[0][:, chains].transpose(1, 0, 2), ro, "bf16", "noalloc segmented o (T=8192)")
    check(s[0][chains], rS, "bf16", "noalloc segmented state (T=8192)")
    # 4b: the segmented plan where the per-chunk (I + A)^-1 records do not fit beside the maps
    #     in the scratch (32,768 tokens, 16 heads: 46 MiB of maps + 42 MiB of records): both
    #     passes form the inverse instead -- bit for bit gdn_chunk_fwd with GDN_SEG_NO_TM
    long_ = make_inputs(1, 32768, 16, 16, 128, 128, dtype="bf16", s0_std=0.02, seed=994)
    need = gdn.gdn_chunk_fwd_workspace_size(1, 32768, 16, 16, 128, 128, 64, gdn.GDN_BF16)
    assert need > gdn.GDN_NOALLOC_SCRATCH_BYTES
    st1, o1, s1 = _call(long_, noalloc=True)
    monkeypatch.setenv("GDN_SEG_NO_TM", "1")
    assert gdn.gdn_chunk_fwd_workspace_size(1, 32768, 16, 16, 128, 128, 64, gdn.GDN_BF16) \
        <= gdn.GDN_NOALLOC_SCRATCH_BYTES
    st2, o2, s2 = _call(long_, noalloc=False)
    monkeypatch.delenv("GDN_SEG_NO_TM")
    assert st1 == gdn.GDN_OK and st2 == gdn.GDN_OK, (st1, st2)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)
    lc = np.array([5])
    rlo, rlS = oracle.run(long_.q, long_.k, long_.v, long_.beta, long_.g, s0=long_.s0, chains=lc)
    check(o1[0][:, lc].transpose(1, 0, 2), rlo, "bf16", "noalloc segmented o (T=32768)")
    check(s1[0][lc], rlS, "bf16", "noalloc segmented state (T=32768)")
    # 5: split records beyond the scratch (the same input: 144 MiB in one pass): two segments
    #    of chunks in the scratch, bit for bit the one-pass result
    monkeypatch.setenv("GDN_FORCE_VARIANT", "split")
    assert (gdn.gdn_chunk_fwd_workspace_size(1, 8192, 16, 16, 128, 128, 64, gdn.GDN_BF16)
            > gdn.GDN_NOALLOC_SCRATCH_BYTES)
    o, s = _same(huge, "split")
    check(o[0][:, chains].transpose(1, 0, 2), ro, "bf16", "noalloc o (T=8192)")
    check(s[0][chains], rS, "bf16", "noalloc state (T=8192)")
