"""GPU parity of the QSA compressed indexer (gdn_qsa_index, through its C ABI) against the fp64
oracle (oracle/qsa.py) on seeded inputs.

What is unique is compared exactly: which blocks are eligible, how many are kept, their order,
the -1 padding, and -- where the definition leaves no room for rounding (equal keys, zero
queries) -- the kept set itself.  Elsewhere the kept set depends on fp32 importance values that
differ from the fp64 ones by rounding, so it is checked for validity: no kept block may be
beaten by a dropped one by more than the error bound below, and the kernel's selection must be
exactly the top-nsel (ties to the lower index) of the importance values it reports.

Error bound of an importance value (derived from the arithmetic, not fitted): the scores are
products of fp16 copies (unit roundoff 2^-11, power-of-two scaled, so relative) of the rotated
queries and pooled keys with fp32 accumulation, so |ds| <= scale * sum_i |q_i k_i| * e_s with
e_s = 2^-10 + d 2^-24 + 2^-20.  A softmax shifts by at most the largest score error of its row,
so each head's probability moves by a factor of at most exp(2 M_h + e_f), M_h the largest
|ds| of that head's row and e_f = n 2^-24 + 2^-19 the fp32 sum, exp2 and log2 error.
"""
import math

import numpy as np
import pytest

from oracle import qsa as oq

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


def inputs(B, T, d, dtype, seed):
    """Indexer activations stand-in: q, k ~ N(0, 1), rounded to the storage dtype."""
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.standard_normal((B, T, 4, d)).astype(np.float32)
    k = g.standard_normal((B, T, d)).astype(np.float32)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    qt = torch.from_numpy(q).to(td)
    kt = torch.from_numpy(k).to(td)
    return qt.float().numpy().astype(np.float64), kt.float().numpy().astype(np.float64), \
        qt.to(DEV), kt.to(DEV)


def tolerance(q, k, r, rope_dims, base, scale, rows=None):
    """Per (b, row, block) bound on |importance_kernel - importance_oracle| (module docstring)."""
    B, T, Hq, d = q.shape
    rows = np.arange(T) if rows is None else np.asarray(rows)
    kb = oq.rope(oq.pool_keys(k, r), np.arange(-(-T // r)) * r, rope_dims, base)
    qr = oq.rope(q[:, rows], rows[None, :, None], rope_dims, base)
    es = 2.0 ** -10 + d * 2.0 ** -24 + 2.0 ** -20
    E = np.einsum("bthd,bjd->bthj", np.abs(qr), np.abs(kb)) * abs(scale) * es
    imp_h = []
    _, elig = oq.importance(q[:, :, :1], k, r, rope_dims, base, scale, rows=rows)
    M = np.where(elig[None, :, None, :], E, 0.0).max(axis=-1, keepdims=True)   # [B, n, Hq, 1]
    n = elig.sum(axis=1)[None, :, None, None]
    ef = n * 2.0 ** -24 + 2.0 ** -19
    for h in range(Hq):
        p, _ = oq.importance(q[:, :, h:h + 1], k, r, rope_dims, base, scale, rows=rows)
        imp_h.append(p * (np.exp(2 * M[:, :, h] + ef[:, :, 0]) - 1.0))
    return sum(imp_h)


def exact_topk(imp_row, elig_row, nsel):
    """Top-nsel eligible indices of one row (larger first, ties to the lower index), ascending."""
    cand = np.nonzero(elig_row)[0]
    order = cand[np.lexsort((cand, -imp_row[cand]))]
    return np.sort(order[:nsel])


def check_rows(sel, imp_o, elig, tol, nsel, where, imp_k=None):
    """Compare one batch of rows: sel [n, nsel] from the kernel, the oracle's importance and
    eligibility, the bound; imp_k (the kernel's importance) when it was requested."""
    for i in range(sel.shape[0]):
        row = sel[i]
        ne = int(elig[i].sum())
        cnt = min(nsel, ne)
        kept = row[:cnt]
        assert (row[cnt:] == -1).all(), "%s row %d: padding" % (where, i)
        assert (np.diff(kept) > 0).all(), "%s row %d: not ascending" % (where, i)
        assert elig[i, kept].all() if cnt else True, "%s row %d: ineligible block" % (where, i)
        if cnt < ne:
            dropped = np.setdiff1d(np.nonzero(elig[i])[0], kept)
            lo = (imp_o[i, kept] + tol[i, kept]).min()
            hi = (imp_o[i, dropped] - tol[i, dropped]).max()
            assert lo >= hi, "%s row %d: kept %.9g (+tol) < dropped %.9g (-tol)" % (where, i, lo, hi)
        if imp_k is not None:
            assert np.array_equal(kept, exact_topk(imp_k[i], elig[i], nsel)), \
                "%s row %d: selection is not the top-nsel of its own importance" % (where, i)


def run_and_check(B, T, d, dtype, r, nsel, rope_dims, seed, base=10000.0, scale=None):
    gdn = gdn_mod()
    q, k, qt, kt = inputs(B, T, d, dtype, seed)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    sel, imp = gdn.qsa_index(qt, kt, r=r, nsel=nsel, rope_dims=rope_dims, rope_base=base,
                             scale=sc, want_importance=True)
    torch.cuda.synchronize()
    sel, imp = sel.cpu().numpy(), imp.cpu().numpy().astype(np.float64)
    imp_o, elig = oq.importance(q, k, r, rope_dims, base, sc)
    tol = tolerance(q, k, r, rope_dims, base, sc)
    # importance: zero where not eligible (exactly), within the bound elsewhere
    assert (imp[:, ~elig] == 0).all()
    err = np.abs(imp - imp_o)
    assert (err <= tol).all(), "importance error %.3g > bound (worst ratio %.3g)" % (
        err.max(), (err / np.maximum(tol, 1e-300)).max())
    for b in range(B):
        check_rows(sel[b], imp_o[b], elig, tol[b], nsel, "b=%d" % b, imp_k=imp[b])
    return sel, imp, imp_o


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_qsa_matches_oracle(d, dtype):
    """Several 16-query tiles and block tiles, ragged tails (T = 333 with r = 4)."""
    run_and_check(B=2, T=333, d=d, dtype=dtype, r=4, nsel=9, rope_dims=d // 2, seed=800 + d)


@pytest.mark.parametrize("r,nsel,rope_dims", [(1, 5, 128), (3, 17, 0), (8, 1, 64), (4, 64, 32),
                                              (2, 200, 64)])
def test_qsa_shapes(r, nsel, rope_dims):
    run_and_check(B=1, T=517, d=128, dtype="bf16", r=r, nsel=nsel, rope_dims=rope_dims,
                  seed=810 + r + nsel)


def test_qsa_large_budget():
    """More kept blocks than one wavefront holds eleven times over (nsel = 700 of up to 1500):
    rows that finish by ranking a few gathered keys merge them into long kept lists."""
    run_and_check(B=1, T=1500, d=64, dtype="bf16", r=1, nsel=700, rope_dims=64, seed=815)


@pytest.mark.parametrize("T", [1, 3, 4, 15, 16, 17])
def test_qsa_tiny_lengths(T):
    """Fewer tokens than a block or a query tile: the last token sees the short last block."""
    sel, imp, _ = run_and_check(B=2, T=T, d=64, dtype="bf16", r=4, nsel=2, rope_dims=32,
                                seed=820 + T)
    if T <= 4:  # one (short) block, eligible for the last token only
        assert (sel[:, T - 1] == [0, -1]).all() and (sel[:, :T - 1] == -1).all()


def test_qsa_zero_queries_keep_the_first_blocks():
    """Zero queries: every eligible block has the same importance, so ties decide: the first
    nsel eligible blocks, exactly."""
    gdn = gdn_mod()
    T, r, nsel = 700, 4, 37
    _, _, qt, kt = inputs(1, T, 128, "bf16", 830)
    qt.zero_()
    sel, imp = gdn.qsa_index(qt, kt, r=r, nsel=nsel, want_importance=True)
    sel = sel.cpu().numpy()[0]
    for t in range(T):
        n = (t + 1) // r if t < T - 1 else -(-T // r)
        want = list(range(min(n, nsel))) + [-1] * (nsel - min(n, nsel))
        assert sel[t].tolist() == want, t


def test_qsa_equal_keys_tie_to_the_lower_index():
    """All pooled keys equal and no rotation: equal importance in every row, bit for bit."""
    gdn = gdn_mod()
    T, r, nsel = 300, 2, 11
    _, _, qt, kt = inputs(2, T, 64, "bf16", 840)
    kt[:] = kt[:, :1]
    sel, imp = gdn.qsa_index(qt, kt, r=r, nsel=nsel, rope_dims=0, want_importance=True)
    sel = sel.cpu().numpy()
    assert (sel[:, T - 1] == np.arange(nsel)).all()
    assert (sel[:, 2 * nsel + 5] == np.arange(nsel)).all()


def test_qsa_is_deterministic():
    gdn = gdn_mod()
    _, _, qt, kt = inputs(1, 2000, 128, "bf16", 850)
    a, ia = gdn.qsa_index(qt, kt, r=4, nsel=40, want_importance=True)
    b, ib = gdn.qsa_index(qt, kt, r=4, nsel=40, want_importance=True)
    assert torch.equal(a, b) and torch.equal(ia, ib)


def test_qsa_full_size_sampled():
    """B = 1, T = 65536, r = 4, 512 blocks (2048 tokens) kept, d = 128, 64 rotated dims: the
    configuration the benchmark times.  Every row is checked for the properties that hold at any
    size (count, order, eligibility, padding); sampled rows against the oracle."""
    gdn = gdn_mod()
    B, T, d, r, nsel = 1, 65536, 128, 4, 512
    q, k, qt, kt = inputs(B, T, d, "bf16", 860)
    sel, _ = gdn.qsa_index(qt, kt, r=r, nsel=nsel, rope_dims=64)
    torch.cuda.synchronize()
    # all rows, on the GPU: kept count = min(nsel, eligible), ascending, eligible, -1 padded
    t = torch.arange(T, device=DEV)
    ne = torch.where(t == T - 1, torch.full_like(t, -(-T // r)), (t + 1) // r)
    cnt = torch.clamp(ne, max=nsel)
    s = sel[0].long()
    pos = torch.arange(nsel, device=DEV)[None, :]
    valid = pos < cnt[:, None]
    assert bool(((s >= 0) == valid).all())
    assert bool((~valid | (s < ne[:, None])).all())
    assert bool((((s[:, 1:] - s[:, :-1]) > 0) | ~valid[:, 1:]).all())
    rows = np.array([0, 3, 4, 2047, 2048, 2051, 5000, 20001, 40000, 65534, 65535])
    imp_o, elig = oq.importance(q, k, r, 64, 10000.0, 1 / math.sqrt(d), rows=rows)
    tol = tolerance(q, k, r, 64, 10000.0, 1 / math.sqrt(d), rows=rows)
    check_rows(sel[0].cpu().numpy()[rows], imp_o[0], elig, tol[0], nsel, "full")
