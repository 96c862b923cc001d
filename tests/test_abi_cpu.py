"""CPU-side checks of the C ABI: the built library loads, exports every function that
include/gdn.h declares, and rejects bad arguments on the host before launching anything
(no call here reaches a kernel, so no GPU is needed)."""
import ctypes
import os
import re

import pytest

import linear_attention_token_gdn_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        from linear_attention_token_gdn_amd import build
        build.build()
    return gdn.load_library()


def test_header_declares_the_abi():
    assert declared_functions() == sorted(gdn.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr), name


def test_version_and_status_strings(lib):
    with open(os.path.join(ROOT, "include", "gdn.h")) as f:
        declared = int(re.search(r"#define GDN_ABI_VERSION (\d+)", f.read()).group(1))
    assert gdn.gdn_abi_version() == declared == gdn.ABI_VERSION
    assert gdn.gdn_status_string(0) == "GDN_OK"
    assert gdn.gdn_status_string(1) == "GDN_ERR_INVALID_ARG"
    assert gdn.gdn_status_string(2) == "GDN_ERR_UNSUPPORTED"
    assert gdn.gdn_status_string(3) == "GDN_ERR_HIP"
    assert gdn.gdn_status_string(4).startswith("GDN_ERR_SCRATCH_TOO_SMALL")
    assert gdn.gdn_status_string(99) == "GDN_ERR_UNKNOWN"


def _tm_records(B, T, Hv, chunk, packed=False):
    # one (I + A)^-1 record per chunk slot and value head: the NR (NR + 1) / 2 lower 16 x 16
    # fp16 blocks (512 B each, NR = chunk / 16); ceil(rows / chunk) + B slots per head
    rows = T if packed else B * T
    nr = chunk // 16
    return Hv * (-(-rows // chunk) + B) * nr * (nr + 1) // 2 * 512


def test_workspace_of_the_segmented_plan(lib, monkeypatch):
    # per chain and segment: the fp32 transition M and state N of every segment but the last,
    # and the entry state of every segment (d x d floats each); 256 / chains segments; then
    # the per-chunk (I + A)^-1 records (GDN_SEG_NO_TM: none)
    D2 = 128 * 128 * 4
    for B, T, H, nseg in ((1, 262144, 16, 16), (1, 8192, 16, 16), (4, 4096, 16, 4),
                          (1, 1 << 20, 2, 128)):
        chains = B * H
        maps = (2 * (nseg - 1) + nseg) * chains * D2
        assert gdn.gdn_chunk_fwd_workspace_size(B, T, H, H, 128, 128, 64, gdn.GDN_BF16) == (
            maps + _tm_records(B, T, H, 64))
        monkeypatch.setenv("GDN_SEG_NO_TM", "1")
        assert gdn.gdn_chunk_fwd_workspace_size(B, T, H, H, 128, 128, 64, gdn.GDN_BF16) == maps
        monkeypatch.delenv("GDN_SEG_NO_TM")
    # records beyond 2 GiB (16 heads x 8 M tokens: 10 GiB): the maps alone, both passes form Tm
    maps = (2 * 15 + 16) * 16 * D2
    assert _tm_records(1, 1 << 23, 16, 64) > 2 << 30
    assert gdn.gdn_chunk_fwd_workspace_size(1, 1 << 23, 16, 16, 128, 128, 64, gdn.GDN_BF16) == maps
    # the largest maps: 256 units at d = 128 fit the allocation-free entry point's scratch (it
    # runs without the records when they do not fit beside them)
    monkeypatch.setenv("GDN_SEG_NO_TM", "1")
    assert gdn.gdn_chunk_fwd_workspace_size(1, 1 << 20, 1, 2, 128, 128, 64, gdn.GDN_BF16) \
        <= gdn.GDN_NOALLOC_SCRATCH_BYTES
    monkeypatch.delenv("GDN_SEG_NO_TM")
    # a pinned segment length (tests): one chunk per segment
    monkeypatch.setenv("GDN_SEG_CHUNKS", "1")
    monkeypatch.setenv("GDN_FORCE_VARIANT", "segmented")
    assert gdn.gdn_chunk_fwd_plan(1, 200, 2, 2, 64, 64, 64, gdn.GDN_BF16) == "segmented"
    assert gdn.gdn_chunk_fwd_workspace_size(1, 200, 2, 2, 64, 64, 64, gdn.GDN_BF16) == (
        (2 * 3 + 4) * 2 * 64 * 64 * 4 + _tm_records(1, 200, 2, 64))
    # one chunk in all: nothing to cut, the default plan
    assert gdn.gdn_chunk_fwd_plan(1, 64, 2, 2, 64, 64, 64, gdn.GDN_BF16) == "split"


def test_workspace_of_the_segmented_plan_packed(lib):
    # packed sequences: 256 / chains segments per chain whatever their lengths (formed on the
    # device); the plan is taken when the mean sequence has >= 8 chunks per segment
    ws = gdn.gdn_chunk_fwd_varlen_workspace_size
    D2 = 128 * 128 * 4
    assert ws(2, 2 * 16384, 4, 4, 128, 128, 64, gdn.GDN_BF16, 1) == (
        (2 * 31 + 32) * 8 * D2 + _tm_records(2, 2 * 16384, 4, 64, packed=True))
    assert ws(1, 262144, 16, 16, 128, 128, 64, gdn.GDN_BF16, 1) == (
        (2 * 15 + 16) * 16 * D2 + _tm_records(1, 262144, 16, 64, packed=True))
    # short on average: the split plan's records (one 72 KiB + 128 B record per chunk slot)
    short = ws(8, 8 * 512, 4, 4, 128, 128, 64, gdn.GDN_BF16, 1)
    assert short != (2 * 7 + 8) * 32 * D2 and short >= 4 * (4096 // 64 + 8) * (73728 + 128)
    # the plan hint keeps the split plan
    assert ws(1, 262144, 16, 16, 128, 128, 64, gdn.GDN_BF16, 1, gdn.GDN_PREFER_SPLIT) > 1 << 30


def test_workspace_size_of_the_chunk_kernels(lib):
    # few chains: the prep + scan form needs a workspace; one float32 path needs none
    assert gdn.gdn_chunk_fwd_workspace_size(1, 4096, 16, 16, 128, 128, 64, gdn.GDN_BF16) > 16 * 64 * 65536
    assert gdn.gdn_chunk_fwd_workspace_size(1, 64, 2, 2, 16, 16, 16, gdn.GDN_F32) == 0
    assert gdn.gdn_chunk_fwd_workspace_size(1, 0, 2, 2, 128, 128, 64, gdn.GDN_BF16) == 0


def test_plan(lib):
    assert gdn.gdn_chunk_fwd_plan(1, 4096, 16, 16, 128, 128, 64, gdn.GDN_BF16) == "split"
    # few long chains: segments of >= 8 chunks, at most 256 (chain, segment) units
    assert gdn.gdn_chunk_fwd_plan(1, 8192, 16, 16, 128, 128, 64, gdn.GDN_BF16) == "segmented"
    assert gdn.gdn_chunk_fwd_plan(1, 262144, 16, 16, 128, 128, 64, gdn.GDN_BF16) == "segmented"
    assert gdn.gdn_chunk_fwd_plan(4, 4096, 16, 16, 128, 128, 64, gdn.GDN_BF16) == "segmented"
    assert gdn.gdn_chunk_fwd_plan(1, 262144, 16, 16, 128, 128, 64, gdn.GDN_F32) == "recurrent"
    assert gdn.gdn_chunk_fwd_plan(8, 8192, 16, 32, 128, 128, 64, gdn.GDN_BF16) == "fused"
    assert gdn.gdn_chunk_fwd_plan(1, 64, 2, 2, 16, 16, 16, gdn.GDN_F32) == "recurrent"
    assert gdn.gdn_chunk_fwd_plan(1, 64, 2, 2, 16, 32, 16, gdn.GDN_BF16) == "recurrent"
    assert gdn.gdn_chunk_fwd_plan(1, 64, 2, 3, 16, 16, 16, gdn.GDN_BF16) == "invalid"


def test_workspace_size_rejects_bad_sizes(lib):
    assert gdn.gdn_chunk_fwd_workspace_size(1, 64, 2, 3, 16, 16, 16, gdn.GDN_BF16) == 0
    assert gdn.gdn_chunk_fwd_workspace_size(1, 64, 2, 2, 48, 16, 16, gdn.GDN_BF16) == 0
    assert gdn.gdn_chunk_fwd_workspace_size(1, 64, 2, 2, 16, 16, 24, gdn.GDN_BF16) == 0
    assert gdn.gdn_chunk_fwd_workspace_size(0, 64, 2, 2, 16, 16, 16, gdn.GDN_BF16) == 0


# fake, well-aligned, non-overlapping device addresses: validation must reject the call
# before anything dereferences them
BASE = 1 << 40
P = {n: BASE + i * (1 << 32)
     for i, n in enumerate(["q", "k", "v", "beta", "g", "s0", "o", "sT", "cu", "ws"])}


def prefill(**kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], beta=P["beta"], g=P["g"], initial_state=P["s0"],
             o=P["o"], final_state=P["sT"], B=1, T=64, Hk=2, Hv=2, dk=16, dv=16, chunk=16,
             scale=1.0, in_dtype=gdn.GDN_BF16, out_dtype=gdn.GDN_F32, workspace=None,
             workspace_bytes=0, stream=None)
    a.update(kw)
    return gdn.gdn_chunk_fwd(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(Hv=3), gdn.GDN_ERR_INVALID_ARG),
    (dict(B=-1), gdn.GDN_ERR_INVALID_ARG),
    (dict(T=-5), gdn.GDN_ERR_INVALID_ARG),
    (dict(Hk=0), gdn.GDN_ERR_INVALID_ARG),
    (dict(dk=48), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dv=256), gdn.GDN_ERR_UNSUPPORTED),
    (dict(chunk=24), gdn.GDN_ERR_UNSUPPORTED),
    (dict(in_dtype=7), gdn.GDN_ERR_UNSUPPORTED),
    (dict(out_dtype=7), gdn.GDN_ERR_UNSUPPORTED),
    (dict(q=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(o=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(g=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(q=P["q"] + 2), gdn.GDN_ERR_INVALID_ARG),         # misaligned
    (dict(initial_state=P["s0"] + 4), gdn.GDN_ERR_INVALID_ARG),
    (dict(o=P["q"] + 64), gdn.GDN_ERR_INVALID_ARG),        # o overlaps q
    (dict(o=P["s0"]), gdn.GDN_ERR_INVALID_ARG),            # o overlaps a state
    (dict(final_state=P["s0"] + 1024), gdn.GDN_ERR_INVALID_ARG),  # partial state overlap
])
def test_prefill_validation(lib, kw, status):
    assert prefill(**kw) == status


def test_prefill_empty_batch_is_noop(lib):
    assert prefill(B=0, q=None, k=None, v=None, beta=None, g=None, o=None) == gdn.GDN_OK


def prefill_noalloc(**kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], beta=P["beta"], g=P["g"], initial_state=P["s0"],
             o=P["o"], final_state=P["sT"], B=1, T=64, Hk=2, Hv=2, dk=16, dv=16, chunk=16,
             scale=1.0, in_dtype=gdn.GDN_BF16, out_dtype=gdn.GDN_F32, stream=None)
    a.update(kw)
    return gdn.gdn_chunk_fwd_noalloc(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(Hv=3), gdn.GDN_ERR_INVALID_ARG),
    (dict(dk=48), gdn.GDN_ERR_UNSUPPORTED),
    (dict(q=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(o=P["q"] + 64), gdn.GDN_ERR_INVALID_ARG),
])
def test_noalloc_validation(lib, kw, status):
    assert prefill_noalloc(**kw) == status


def test_noalloc_scratch_holds_the_smallest_split_workspace(lib, monkeypatch):
    """The split plan runs in segments of as many chunks as the scratch holds: its smallest
    workspace (one chunk per segment) fits 80 MiB even at the largest chain count the plan
    takes (127 chains at d = 128), so no size the plans run is refused for its length."""
    monkeypatch.setenv("GDN_SPLIT_RECORD_BYTES", "1")
    monkeypatch.setenv("GDN_FORCE_VARIANT", "split")  # dense sizes like these run segmented
    least = gdn.gdn_chunk_fwd_workspace_size(1, 1 << 20, 1, 127, 128, 128, 64, gdn.GDN_BF16)
    assert gdn.gdn_chunk_fwd_plan(1, 1 << 20, 1, 127, 128, 128, 64, gdn.GDN_BF16) == "split"
    assert 0 < least <= gdn.GDN_NOALLOC_SCRATCH_BYTES // 4
    assert prefill_noalloc(B=0, q=None, k=None, v=None, beta=None, g=None, o=None) == gdn.GDN_OK


def test_noalloc_scratch_size_matches_the_header(lib):
    text = open(HEADER).read()
    m = re.search(r"#define GDN_NOALLOC_SCRATCH_BYTES \((\d+)ull << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == gdn.GDN_NOALLOC_SCRATCH_BYTES


def decode(**kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], beta=P["beta"], g=P["g"], state=P["s0"], o=P["o"],
             B=4, Hk=2, Hv=4, dk=16, dv=32, scale=1.0, in_dtype=gdn.GDN_BF16,
             out_dtype=gdn.GDN_F32, stream=None)
    a.update(kw)
    return gdn.gdn_decode_step(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(Hv=3), gdn.GDN_ERR_INVALID_ARG),
    (dict(B=-1), gdn.GDN_ERR_INVALID_ARG),
    (dict(dk=8), gdn.GDN_ERR_UNSUPPORTED),
    (dict(in_dtype=5), gdn.GDN_ERR_UNSUPPORTED),
    (dict(state=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(state=P["s0"] + 8), gdn.GDN_ERR_INVALID_ARG),
    (dict(o=P["v"]), gdn.GDN_ERR_INVALID_ARG),
    (dict(state=P["q"]), gdn.GDN_ERR_INVALID_ARG),
])
def test_decode_validation(lib, kw, status):
    assert decode(**kw) == status


def test_decode_empty_batch_is_noop(lib):
    assert decode(B=0) == gdn.GDN_OK


def decode_tokens(**kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], beta=P["beta"], g=P["g"], state_in=P["s0"],
             state_out=P["s0"], o=P["o"], B=2, T=2, Hk=2, Hv=4, dk=16, dv=32, scale=1.0,
             flags=0, in_dtype=gdn.GDN_BF16, out_dtype=gdn.GDN_F32, stream=None)
    a.update(kw)
    return gdn.gdn_decode_tokens(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), gdn.GDN_ERR_INVALID_ARG),
    (dict(flags=8), gdn.GDN_ERR_INVALID_ARG),  # the plan hint is for the prefill only
    (dict(Hv=3), gdn.GDN_ERR_INVALID_ARG),
    (dict(dv=48), gdn.GDN_ERR_UNSUPPORTED),
    (dict(out_dtype=7), gdn.GDN_ERR_UNSUPPORTED),
    (dict(state_out=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(state_in=P["s0"] + 16), gdn.GDN_ERR_INVALID_ARG),  # partial state overlap
    (dict(state_out=P["s0"] + 4), gdn.GDN_ERR_INVALID_ARG),  # misaligned
    (dict(q=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(o=P["k"]), gdn.GDN_ERR_INVALID_ARG),               # o overlaps k
    (dict(state_in=P["s0"], state_out=P["sT"], o=P["s0"]), gdn.GDN_ERR_INVALID_ARG),
    (dict(flags=8), gdn.GDN_ERR_INVALID_ARG),                # unknown prologue flag
])
def test_decode_tokens_validation(lib, kw, status):
    assert decode_tokens(**kw) == status


def test_decode_tokens_empty_batch_is_noop(lib):
    assert decode_tokens(B=0) == gdn.GDN_OK


def test_missing_library_fails_loudly(tmp_path):
    saved = gdn._lib
    gdn._lib = None
    try:
        with pytest.raises(RuntimeError, match="not built"):
            gdn.load_library(str(tmp_path / "missing.so"))
    finally:
        gdn._lib = saved


def prefill_varlen(**kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], beta=P["beta"], g=P["g"], initial_state=P["s0"],
             o=P["o"], final_state=P["sT"], cu_seqlens=P["cu"], num_seqs=3, T=100, Hk=2, Hv=4,
             dk=64, dv=64, chunk=64, scale=1.0, flags=gdn.GDN_QK_L2NORM | gdn.GDN_BETA_LOGIT,
             in_dtype=gdn.GDN_BF16, out_dtype=gdn.GDN_F32, workspace=None, workspace_bytes=0,
             stream=None)
    a.update(kw)
    return gdn.gdn_chunk_fwd_varlen(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(flags=16), gdn.GDN_ERR_INVALID_ARG),
    (dict(num_seqs=0), gdn.GDN_ERR_INVALID_ARG),           # packed needs >= 1 sequence
    (dict(cu_seqlens=P["cu"] + 2), gdn.GDN_ERR_INVALID_ARG),  # misaligned offsets
    (dict(dk=48), gdn.GDN_ERR_UNSUPPORTED),
    (dict(chunk=128), gdn.GDN_ERR_UNSUPPORTED),
    (dict(q=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(o=P["q"] + 128), gdn.GDN_ERR_INVALID_ARG),       # o overlaps q
])
def test_prefill_varlen_validation(lib, kw, status):
    assert prefill_varlen(**kw) == status


def split_fixed(chains, d):
    """The split plan's workspace beside its records: progress words, carried states and the
    carried bound and scale of every 16-column tile."""
    scales = chains * (d // 16) * 2 * 4
    return chains * 256 + chains * d * d * 4 + (scales + 255) // 256 * 256


def test_split_workspace_is_bounded(lib, monkeypatch):
    """The split plan keeps at most 2 GiB of records (segments of chunks): the workspace of a
    sequence of a million tokens is that of about 1,800 chunks, not of 16,384; the environment
    cap lowers it, down to one chunk per segment."""
    rec = 73728 + 128
    monkeypatch.setenv("GDN_FORCE_VARIANT", "split")  # the default for these is segmented
    big = gdn.gdn_chunk_fwd_workspace_size(1, 1 << 20, 16, 16, 128, 128, 64, gdn.GDN_BF16)
    L = (2 << 30) // (16 * rec)
    assert big == L * 16 * rec + split_fixed(16, 128)
    short = gdn.gdn_chunk_fwd_workspace_size(1, 4096, 16, 16, 128, 128, 64, gdn.GDN_BF16)
    assert short == 64 * 16 * rec + split_fixed(16, 128)  # all 64 chunks fit: one segment
    monkeypatch.setenv("GDN_SPLIT_RECORD_BYTES", str(20 * 16 * rec))
    assert gdn.gdn_chunk_fwd_workspace_size(1, 4096, 16, 16, 128, 128, 64, gdn.GDN_BF16) == (
        20 * 16 * rec + split_fixed(16, 128))
    monkeypatch.setenv("GDN_SPLIT_RECORD_BYTES", "1")
    assert gdn.gdn_chunk_fwd_workspace_size(1, 4096, 16, 16, 128, 128, 64, gdn.GDN_BF16) == (
        16 * rec + split_fixed(16, 128))


def test_varlen_workspace(lib):
    ws = gdn.gdn_chunk_fwd_varlen_workspace_size
    # dense = gdn_chunk_fwd's
    assert (ws(1, 4096, 16, 16, 128, 128, 64, gdn.GDN_BF16, 0)
            == gdn.gdn_chunk_fwd_workspace_size(1, 4096, 16, 16, 128, 128, 64, gdn.GDN_BF16))
    # many chains: the single-pass kernel, no workspace, packed or not
    assert gdn.gdn_chunk_fwd_plan(16, 4096, 16, 16, 128, 128, 64, gdn.GDN_BF16) == "fused"
    assert ws(16, 4096, 16, 16, 128, 128, 64, gdn.GDN_BF16, 1) == 0
    # few chains, packed: the split plan (the segmented plan takes dense inputs only);
    # packed sequences take one record slot per sequence and head beyond the chunks of the
    # total length (records of 72 KiB + one 128-byte line of scalars at d = 128, C = 64), plus
    # per chain a 256-byte progress word, the fp32 state carried between segments and two
    # floats per 16-column tile (padded to 256 B)
    slots = 16 * (4096 // 64 + 4)
    assert ws(4, 4096, 16, 16, 128, 128, 64, gdn.GDN_BF16, 1) == (
        slots * (73728 + 128) + split_fixed(4 * 16, 128))
    assert ws(0, 4096, 16, 16, 128, 128, 64, gdn.GDN_BF16, 1) == 0
    # the plan hint: split for many chains too, with the same slot layout
    slots = 16 * (4096 // 64 + 16)
    assert ws(16, 4096, 16, 16, 128, 128, 64, gdn.GDN_BF16, 1, gdn.GDN_PREFER_SPLIT) == (
        slots * (73728 + 128) + split_fixed(16 * 16, 128))
    assert ws(2, 4096, 16, 16, 128, 128, 64, gdn.GDN_F32, 1, gdn.GDN_PREFER_SPLIT) == 0
    assert ws(2, 4096, 16, 16, 128, 128, 64, gdn.GDN_F32, 1) == 0  # fp32: recurrent


def backward_call(**kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], beta=P["beta"], g=P["g"], initial_state=P["s0"],
             d_o=P["o"], d_final_state=None, dq=P["sT"], dk=P["sT"] + (1 << 28),
             dv=P["sT"] + (2 << 28), dbeta=P["sT"] + (3 << 28), dg=P["cu"],
             d_initial_state=P["cu"] + (1 << 28), B=2, T=8, Hk=1, Hv=2, dk_dim=16, dv_dim=16,
             scale=1.0, in_dtype=gdn.GDN_BF16, dout_dtype=gdn.GDN_F32, workspace=None,
             workspace_bytes=0, stream=None)
    a.update(kw)
    return gdn.gdn_backward(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(Hv=3), gdn.GDN_ERR_INVALID_ARG),
    (dict(dk_dim=24), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dout_dtype=9), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dq=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(dq=P["q"]), gdn.GDN_ERR_INVALID_ARG),              # output overlaps an input
    (dict(dk=P["sT"] + 64), gdn.GDN_ERR_INVALID_ARG),        # outputs overlap each other
    (dict(), gdn.GDN_ERR_INVALID_ARG),                        # no workspace given
])
def test_backward_validation(lib, kw, status):
    assert backward_call(**kw) == status


def test_backward_workspace_size(lib):
    n = gdn.gdn_backward_workspace_size(1, 4096, 16, 16, 128, 128)
    # checkpoints + one block per chain, then the parts of dq, dk (8 slices of 16 columns)
    # and of dbeta, dg
    assert n == ((16 * 64 + 16 * 65) * 128 * 128 + 2 * 4096 * 16 * 8 * 128
                 + 2 * 4096 * 16 * 8) * 4
    assert gdn.gdn_backward_workspace_size(1, 64, 2, 2, 32, 16) == (2 * 1 + 2 * 65) * 32 * 16 * 4
    assert gdn.gdn_backward_workspace_size(1, 100, 1, 2, 64, 64) > 0
    assert gdn.gdn_backward_workspace_size(0, 100, 1, 2, 64, 64) == 0
    assert backward_call(B=0) == gdn.GDN_OK


def qsa_call(**kw):
    a = dict(q=P["q"], k=P["k"], sel=P["sT"], importance=None, B=2, T=64, Hq=4, d=128, r=4,
             nsel=8, rope_dims=64, rope_base=10000.0, scale=0.088, in_dtype=gdn.GDN_BF16,
             workspace=P["ws"], workspace_bytes=1 << 30, stream=None)
    a.update(kw)
    return gdn.gdn_qsa_index(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=2), gdn.GDN_ERR_UNSUPPORTED),
    (dict(d=96), gdn.GDN_ERR_UNSUPPORTED),
    (dict(in_dtype=7), gdn.GDN_ERR_UNSUPPORTED),
    (dict(r=0), gdn.GDN_ERR_INVALID_ARG),
    (dict(nsel=0), gdn.GDN_ERR_INVALID_ARG),
    (dict(rope_dims=63), gdn.GDN_ERR_INVALID_ARG),
    (dict(rope_dims=130), gdn.GDN_ERR_INVALID_ARG),
    (dict(rope_base=0.0), gdn.GDN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), gdn.GDN_ERR_INVALID_ARG),
    (dict(scale=float("inf")), gdn.GDN_ERR_INVALID_ARG),
    (dict(sel=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(sel=P["q"]), gdn.GDN_ERR_INVALID_ARG),               # output overlaps an input
    (dict(importance=P["sT"] + 64), gdn.GDN_ERR_INVALID_ARG),  # outputs overlap each other
    (dict(workspace=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(workspace_bytes=1024), gdn.GDN_ERR_INVALID_ARG),
    (dict(workspace=P["ws"] + 64), gdn.GDN_ERR_INVALID_ARG),   # misaligned workspace
])
def test_qsa_validation(lib, kw, status):
    assert qsa_call(**kw) == status


def test_qsa_workspace_and_empty_calls(lib):
    n = gdn.gdn_qsa_workspace_size(1, 65536, 4, 128, 4)
    # q16 + qinv + qnorm + kbar fp32 + kbar fp16 + partial maxima (2 floats) + batch stats
    assert n == 65536 * 4 * 128 * 2 + 2 * 65536 * 4 * 4 + 16384 * 128 * (4 + 2) + 2048 + 256
    assert gdn.gdn_qsa_workspace_size(1, 64, 2, 128, 4) == 0
    assert gdn.gdn_qsa_workspace_size(0, 64, 4, 128, 4) == 0
    assert qsa_call(B=0) == gdn.GDN_OK
    assert qsa_call(T=0) == gdn.GDN_OK


def test_calibration_library():
    """libgdn_calib.so (the benchmark's attainable-peak kernels) exports what gdn_calib.h
    declares and rejects bad arguments before launching anything."""
    path = os.path.join(gdn.PKG_DIR, "libgdn_calib.so")
    if not os.path.exists(path):
        from linear_attention_token_gdn_amd import build
        build.build()
    cal = ctypes.CDLL(path)
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "gdn_calib.h")).read(),
                  flags=re.S)
    names = sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))
    assert names == ["gdn_calib_copy", "gdn_calib_mfma", "gdn_calib_mfma_clock",
                     "gdn_calib_wall_clock_khz"]
    for n in names:
        assert isinstance(getattr(cal, n), ctypes._CFuncPtr), n
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    cal.gdn_calib_copy.argtypes = [vp, vp, sz, i, i, vp]
    cal.gdn_calib_mfma.argtypes = [vp, i, i, vp]
    assert cal.gdn_calib_copy(None, None, 32768, 64, 0, None) == 1
    assert cal.gdn_calib_copy(1 << 20, 1 << 30, 16384, 64, 0, None) == 1   # not a multiple
    assert cal.gdn_calib_copy(1 << 20, (1 << 20) + 32768, 65536, 64, 0, None) == 1  # overlap
    assert cal.gdn_calib_copy(1 << 20, 1 << 30, 32768, 64, 5, None) == 1   # no such variant
    assert cal.gdn_calib_copy(1 << 20, 1 << 30, 32768, 64, 4, None) == 1   # slices uneven
    assert cal.gdn_calib_copy(1 << 20, 1 << 30, 32768, 64, 3, None) == 1   # in place: src == dst
    assert cal.gdn_calib_mfma(None, 64, 16, None) == 1
    assert cal.gdn_calib_mfma(1 << 20, 64, 0, None) == 1
    cal.gdn_calib_mfma_clock.argtypes = [vp, vp, i, i, i, vp]
    assert cal.gdn_calib_mfma_clock(1 << 20, None, 64, 16, 0, None) == 1
    assert cal.gdn_calib_mfma_clock(1 << 20, 1 << 30, 64, 16, 2, None) == 1  # no such form
    assert cal.gdn_calib_mfma_clock(1 << 20, 1 << 30, 0, 16, 0, None) == 1
