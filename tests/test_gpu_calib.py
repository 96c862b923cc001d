"""The benchmark's attainable-peak kernels (libgdn_calib.so) do the work they are timed for: every
copy variant copies exactly, and the MFMA loop's per-lane sums equal the product it claims to
accumulate (computed here in numpy from the documented operand layout of a 16x16x32 MFMA:
lane l supplies A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16] and holds
D[4 (l / 16) + i][l % 16]; of a 32x32x16 one: A[l % 32][8 (l / 32) + e], B[8 (l / 32) + e][l % 32],
and D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32] in accumulator register r)."""
import ctypes
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def cal():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_token_gdn_amd as gdn
    path = os.path.join(os.path.dirname(gdn.LIB_PATH), "libgdn_calib.so")
    lib = ctypes.CDLL(path)
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.gdn_calib_copy.argtypes = [vp, vp, sz, i, i, vp]
    lib.gdn_calib_mfma.argtypes = [vp, i, i, vp]
    lib.gdn_calib_mfma_clock.argtypes = [vp, vp, i, i, i, vp]
    lib.gdn_calib_wall_clock_khz.restype = i
    return lib


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4])
def test_copy_variants(cal, variant):
    n = 8 << 20  # floats: 32 MiB
    g = torch.Generator(device=DEV)
    g.manual_seed(40 + variant)
    src = torch.randn(n, device=DEV, generator=g)
    ref = src.clone()
    dst = src if variant == 3 else torch.zeros_like(src)
    rc = cal.gdn_calib_copy(src.data_ptr(), dst.data_ptr(), 4 * n, 64, variant,
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(dst, ref) and torch.equal(src, ref)


def test_mfma_loop_result(cal):
    blocks, iters = 4, 16
    out = torch.full((blocks * 256,), -1.0, device=DEV)
    rc = cal.gdn_calib_mfma(out.data_ptr(), blocks, iters, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    lanes = np.arange(64)
    a = np.array([[((l + e) & 7) / 1024.0 for e in range(8)] for l in lanes])
    b = np.array([[((3 * l + e) & 7) / 1024.0 for e in range(8)] for l in lanes])
    A = np.zeros((16, 32))
    B = np.zeros((32, 16))
    for l in lanes:
        A[l % 16, 8 * (l // 16): 8 * (l // 16) + 8] = a[l]
        B[8 * (l // 16): 8 * (l // 16) + 8, l % 16] = b[l]
    D = A @ B  # exact: multiples of 2^-20 well inside fp32
    want = np.array([8 * iters * sum(D[4 * (l // 16) + i, l % 16] for i in range(4)) for l in lanes])
    got = out.cpu().numpy().reshape(blocks * 4, 64)
    assert np.array_equal(got, np.broadcast_to(want.astype(np.float32), got.shape))


def _operands(lanes):
    a = np.array([[((l + e) & 7) / 1024.0 for e in range(8)] for l in lanes])
    b = np.array([[((3 * l + e) & 7) / 1024.0 for e in range(8)] for l in lanes])
    return a, b


@pytest.mark.parametrize("form", [0, 1])
def test_mfma_clock_loop(cal, form):
    """The clocked loop computes the documented products (exactly) and records a plausible
    engine clock: shader-clock cycles over wall-clock ticks times the wall-clock rate."""
    blocks, iters = 8, 32
    out = torch.full((blocks * 256,), -1.0, device=DEV)
    clk = torch.zeros(2 * blocks, dtype=torch.int64, device=DEV)
    rc = cal.gdn_calib_mfma_clock(out.data_ptr(), clk.data_ptr(), blocks, iters, form,
                                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    lanes = np.arange(64)
    a, b = _operands(lanes)
    n = 16 if form == 0 else 32
    A = np.zeros((n, 64 // n * 8))
    B = np.zeros((64 // n * 8, n))
    for l in lanes:
        A[l % n, 8 * (l // n): 8 * (l // n) + 8] = a[l]
        B[8 * (l // n): 8 * (l // n) + 8, l % n] = b[l]
    D = A @ B  # exact: multiples of 2^-20 well inside fp32
    if form == 0:
        want = [8 * iters * sum(D[4 * (l // 16) + i, l % 16] for i in range(4)) for l in lanes]
    else:
        want = [4 * iters * sum(D[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32] for r in range(16))
                for l in lanes]
    got = out.cpu().numpy().reshape(blocks * 4, 64)
    assert np.array_equal(got, np.broadcast_to(np.array(want, dtype=np.float32), got.shape))
    c = clk.view(blocks, 2).cpu().numpy().astype(np.float64)
    assert (c > 0).all()
    khz = cal.gdn_calib_wall_clock_khz()
    assert khz > 0
    mhz = c[:, 0] / c[:, 1] * khz / 1e3
    assert ((mhz > 300) & (mhz < 4000)).all(), mhz


def test_mfma_clock_rejects(cal):
    out = torch.zeros(256, device=DEV)
    clk = torch.zeros(2, dtype=torch.int64, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    assert cal.gdn_calib_mfma_clock(out.data_ptr(), clk.data_ptr(), 1, 4, 2, st) == 1
    assert cal.gdn_calib_mfma_clock(out.data_ptr(), None, 1, 4, 0, st) == 1
    assert cal.gdn_calib_mfma_clock(out.data_ptr(), clk.data_ptr(), 1, 0, 0, st) == 1
