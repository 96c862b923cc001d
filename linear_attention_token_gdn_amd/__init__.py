"""MI355X-native Gated DeltaNet token mixer: Python face of libgdn.so.

The gated delta rule (explainer page "論文解説: Qwen3.8-Next の設計", ta-paperlens.web.app,
section "GDNの中身: 足すのではなく、消してから書く", Eq. (1)):

    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = scale * S_t^T q_t

with g_t = log(alpha_t).  Every step runs in the HIP kernels of ``libgdn.so`` (built with
``python -m linear_attention_token_gdn_amd.build``); this module only checks tensor
properties, allocates outputs with torch and passes raw pointers and the current torch
stream through ctypes.  There is no CPU fallback: without the built library every call raises.

The C entry points are exposed unchanged as ``gdn_chunk_fwd``, ``gdn_decode_step``,
``gdn_decode_tokens``, ``gdn_chunk_fwd_varlen``, ``gdn_chunk_fwd_varlen_workspace_size``,
``gdn_backward``, ``gdn_backward_workspace_size``, ``gdn_chunk_fwd_workspace_size``,
``gdn_qsa_index``, ``gdn_qsa_workspace_size``,
``gdn_chunk_fwd_plan``, ``gdn_chunk_fwd_noalloc``,
``gdn_status_string`` and ``gdn_abi_version``.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# GDN_LIBRARY: another build of the library (the sanitizer test loads an instrumented one)
LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(PKG_DIR, "libgdn.so")

ABI_VERSION = 5  # the GDN_ABI_VERSION of include/gdn.h that these signatures follow
GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_HIP = 0, 1, 2, 3
GDN_ERR_SCRATCH_TOO_SMALL = 4
GDN_NOALLOC_SCRATCH_BYTES = 80 << 20  # static scratch of gdn_chunk_fwd_noalloc
GDN_F32, GDN_BF16 = 0, 1
GDN_QK_L2NORM, GDN_BETA_LOGIT, GDN_G_LOGIT = 1, 2, 4  # input prologue flags
GDN_PREFER_SPLIT = 8  # plan hint of the prefill with packed sequences
EXPORTED_SYMBOLS = ("gdn_abi_version", "gdn_status_string", "gdn_chunk_fwd_workspace_size",
                    "gdn_chunk_fwd_plan", "gdn_chunk_fwd", "gdn_decode_step", "gdn_decode_tokens",
                    "gdn_chunk_fwd_varlen", "gdn_chunk_fwd_varlen_workspace_size",
                    "gdn_backward", "gdn_backward_workspace_size", "gdn_qsa_workspace_size",
                    "gdn_qsa_index", "gdn_chunk_fwd_noalloc")

_lib = None


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s failed: %s" % (where, status_string(status)))
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgdn.so and declare the C signatures.  Raises if the library is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libgdn.so is not built (%s); run "
                           "`python -m linear_attention_token_gdn_amd.build`" % path)
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.gdn_abi_version.argtypes = []
    lib.gdn_abi_version.restype = i
    lib.gdn_status_string.argtypes = [i]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_chunk_fwd_workspace_size.argtypes = [i, i, i, i, i, i, i, i]
    lib.gdn_chunk_fwd_workspace_size.restype = sz
    lib.gdn_chunk_fwd_plan.argtypes = [i, i, i, i, i, i, i, i]
    lib.gdn_chunk_fwd_plan.restype = ctypes.c_char_p
    lib.gdn_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i,
                                  vp, sz, vp]
    lib.gdn_chunk_fwd.restype = i
    lib.gdn_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f,
                                          i, i, vp]
    lib.gdn_chunk_fwd_noalloc.restype = i
    lib.gdn_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.gdn_decode_step.restype = i
    u = ctypes.c_uint
    lib.gdn_decode_tokens.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, u, i, i,
                                      vp]
    lib.gdn_decode_tokens.restype = i
    lib.gdn_chunk_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f,
                                         u, i, i, vp, sz, vp]
    lib.gdn_chunk_fwd_varlen.restype = i
    lib.gdn_chunk_fwd_varlen_workspace_size.argtypes = [i, i, i, i, i, i, i, i, i, ctypes.c_uint]
    lib.gdn_chunk_fwd_varlen_workspace_size.restype = sz
    lib.gdn_backward_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.gdn_backward_workspace_size.restype = sz
    lib.gdn_backward.argtypes = [vp] * 14 + [i] * 6 + [f, i, i, vp, sz, vp]
    lib.gdn_backward.restype = i
    lib.gdn_qsa_workspace_size.argtypes = [i, i, i, i, i]
    lib.gdn_qsa_workspace_size.restype = sz
    lib.gdn_qsa_index.argtypes = [vp, vp, vp, vp] + [i] * 7 + [f, f, i, vp, sz, vp]
    lib.gdn_qsa_index.restype = i
    if lib.gdn_abi_version() != ABI_VERSION:
        raise RuntimeError("libgdn.so has ABI version %d, this binding expects %d; rebuild it "
                           "with `python -m linear_attention_token_gdn_amd.build`"
                           % (lib.gdn_abi_version(), ABI_VERSION))
    _lib = lib
    return lib


# ------------------------------------------------------------------ raw C entry points
def gdn_abi_version() -> int:
    return int(load_library().gdn_abi_version())


def gdn_status_string(status: int) -> str:
    return load_library().gdn_status_string(int(status)).decode()


status_string = gdn_status_string


def gdn_chunk_fwd_workspace_size(B, T, Hk, Hv, dk, dv, chunk, in_dtype) -> int:
    return int(load_library().gdn_chunk_fwd_workspace_size(B, T, Hk, Hv, dk, dv, chunk, in_dtype))


def gdn_chunk_fwd_plan(B, T, Hk, Hv, dk, dv, chunk, in_dtype) -> str:
    return load_library().gdn_chunk_fwd_plan(B, T, Hk, Hv, dk, dv, chunk, in_dtype).decode()


def gdn_chunk_fwd(q, k, v, beta, g, initial_state, o, final_state, B, T, Hk, Hv, dk, dv, chunk,
                  scale, in_dtype, out_dtype, workspace, workspace_bytes, stream) -> int:
    """Raw call: pointer arguments are ints (device addresses) or None."""
    return int(load_library().gdn_chunk_fwd(q, k, v, beta, g, initial_state, o, final_state, B, T,
                                            Hk, Hv, dk, dv, chunk, scale, in_dtype, out_dtype,
                                            workspace, workspace_bytes, stream))


def gdn_chunk_fwd_noalloc(q, k, v, beta, g, initial_state, o, final_state, B, T, Hk, Hv, dk, dv,
                          chunk, scale, in_dtype, out_dtype, stream) -> int:
    """Raw call: pointer arguments are ints (device addresses) or None.  Uses the library's
    static scratch instead of a workspace (nothing is allocated)."""
    return int(load_library().gdn_chunk_fwd_noalloc(q, k, v, beta, g, initial_state, o,
                                                    final_state, B, T, Hk, Hv, dk, dv, chunk,
                                                    scale, in_dtype, out_dtype, stream))


def gdn_decode_step(q, k, v, beta, g, state, o, B, Hk, Hv, dk, dv, scale, in_dtype, out_dtype,
                    stream) -> int:
    """Raw call: pointer arguments are ints (device addresses) or None."""
    return int(load_library().gdn_decode_step(q, k, v, beta, g, state, o, B, Hk, Hv, dk, dv, scale,
                                              in_dtype, out_dtype, stream))


def gdn_decode_tokens(q, k, v, beta, g, state_in, state_out, o, B, T, Hk, Hv, dk, dv, scale,
                      flags, in_dtype, out_dtype, stream) -> int:
    """Raw call: pointer arguments are ints (device addresses) or None."""
    return int(load_library().gdn_decode_tokens(q, k, v, beta, g, state_in, state_out, o, B, T,
                                                Hk, Hv, dk, dv, scale, flags, in_dtype,
                                                out_dtype, stream))


def gdn_chunk_fwd_varlen(q, k, v, beta, g, initial_state, o, final_state, cu_seqlens, num_seqs,
                         T, Hk, Hv, dk, dv, chunk, scale, flags, in_dtype, out_dtype, workspace,
                         workspace_bytes, stream) -> int:
    """Raw call: pointer arguments are ints (device addresses) or None."""
    return int(load_library().gdn_chunk_fwd_varlen(
        q, k, v, beta, g, initial_state, o, final_state, cu_seqlens, num_seqs, T, Hk, Hv, dk, dv,
        chunk, scale, flags, in_dtype, out_dtype, workspace, workspace_bytes, stream))


def gdn_qsa_workspace_size(B, T, Hq, d, r) -> int:
    return int(load_library().gdn_qsa_workspace_size(B, T, Hq, d, r))


def gdn_qsa_index(q, k, sel, importance, B, T, Hq, d, r, nsel, rope_dims, rope_base, scale,
                  in_dtype, workspace, workspace_bytes, stream) -> int:
    """Raw call: pointer arguments are ints (device addresses) or None."""
    return int(load_library().gdn_qsa_index(q, k, sel, importance, B, T, Hq, d, r, nsel,
                                            rope_dims, rope_base, scale, in_dtype, workspace,
                                            workspace_bytes, stream))


def gdn_chunk_fwd_varlen_workspace_size(num_seqs, T, Hk, Hv, dk, dv, chunk, in_dtype,
                                        packed, flags=0) -> int:
    return int(load_library().gdn_chunk_fwd_varlen_workspace_size(num_seqs, T, Hk, Hv, dk, dv,
                                                                  chunk, in_dtype, packed, flags))


def gdn_backward_workspace_size(B, T, Hk, Hv, dk, dv) -> int:
    return int(load_library().gdn_backward_workspace_size(B, T, Hk, Hv, dk, dv))


def gdn_backward(q, k, v, beta, g, initial_state, d_o, d_final_state, dq, dk, dv, dbeta, dg,
                 d_initial_state, B, T, Hk, Hv, dk_dim, dv_dim, scale, in_dtype, dout_dtype,
                 workspace, workspace_bytes, stream) -> int:
    """Raw call: pointer arguments are ints (device addresses) or None."""
    return int(load_library().gdn_backward(
        q, k, v, beta, g, initial_state, d_o, d_final_state, dq, dk, dv, dbeta, dg,
        d_initial_state, B, T, Hk, Hv, dk_dim, dv_dim, scale, in_dtype, dout_dtype, workspace,
        workspace_bytes, stream))


# ------------------------------------------------------------------ torch-facing wrappers
def _dtype_code(t):
    import torch
    if t == torch.float32:
        return GDN_F32
    if t == torch.bfloat16:
        return GDN_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(t, name, shape, dtype, device):
    if t.shape != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (name, dtype, t.dtype))
    if t.device != device:
        raise ValueError("%s: expected device %s, got %s" % (name, device, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def chunk_fwd(q, k, v, beta, g, initial_state=None, output_final_state=True, chunk=64,
              scale=1.0, out_dtype=None, final_state=None, o=None, workspace=None):
    """Prefill over T tokens.

    q, k: [B,T,Hk,dk]; v: [B,T,Hv,dv]; beta, g: [B,T,Hv] (all float32 or all bfloat16, same
    device); initial_state: [B,Hv,dk,dv] float32 or None.  ``final_state`` may be passed (it
    may be ``initial_state`` itself for an in-place update).  Returns (o, final_state or None);
    o is float32 unless ``out_dtype`` says otherwise.
    """
    import torch
    lib = load_library()
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev, dt = q.device, q.dtype
    for t, n, s in ((q, "q", (B, T, Hk, dk)), (k, "k", (B, T, Hk, dk)), (v, "v", (B, T, Hv, dv)),
                    (beta, "beta", (B, T, Hv)), (g, "g", (B, T, Hv))):
        _check(t, n, s, dt, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (B, Hv, dk, dv), torch.float32, dev)
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=out_dtype, device=dev)
    else:
        _check(o, "o", (B, T, Hv, dv), out_dtype, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check(final_state, "final_state", (B, Hv, dk, dv), torch.float32, dev)
    in_code, out_code = _dtype_code(dt), _dtype_code(out_dtype)
    need = int(lib.gdn_chunk_fwd_workspace_size(B, T, Hk, Hv, dk, dv, chunk, in_code))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(initial_state),
                           _ptr(o), _ptr(final_state), B, T, Hk, Hv, dk, dv, chunk, float(scale),
                           in_code, out_code, _ptr(workspace), ws_bytes, stream)
    if st != GDN_OK:
        raise GdnError(st, "gdn_chunk_fwd")
    return o, final_state


def decode_step(q, k, v, beta, g, state, scale=1.0, out_dtype=None, o=None):
    """One token per sequence.  q, k: [B,Hk,dk]; v: [B,Hv,dv]; beta, g: [B,Hv];
    state: [B,Hv,dk,dv] float32, updated in place.  Returns o [B,Hv,dv]."""
    import torch
    lib = load_library()
    B, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    dev, dt = q.device, q.dtype
    for t, n, s in ((q, "q", (B, Hk, dk)), (k, "k", (B, Hk, dk)), (v, "v", (B, Hv, dv)),
                    (beta, "beta", (B, Hv)), (g, "g", (B, Hv))):
        _check(t, n, s, dt, dev)
    _check(state, "state", (B, Hv, dk, dv), torch.float32, dev)
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, Hv, dv), dtype=out_dtype, device=dev)
    else:
        _check(o, "o", (B, Hv, dv), out_dtype, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(state), _ptr(o),
                             B, Hk, Hv, dk, dv, float(scale), _dtype_code(dt),
                             _dtype_code(out_dtype), stream)
    if st != GDN_OK:
        raise GdnError(st, "gdn_decode_step")
    return o


def decode_tokens(q, k, v, beta, g, state, state_out=None, scale=1.0, out_dtype=None, o=None,
                  flags=0):
    """T tokens per sequence in one pass over the state.  q, k: [B,T,Hk,dk]; v: [B,T,Hv,dv];
    beta, g: [B,T,Hv]; state: [B,Hv,dk,dv] float32 (or None for zeros).  The state after the
    T tokens goes to ``state_out`` (default: ``state`` itself, updated in place).  ``flags``:
    the input prologue (GDN_QK_L2NORM | GDN_BETA_LOGIT | GDN_G_LOGIT).  Returns
    (o [B,T,Hv,dv], state_out)."""
    import torch
    lib = load_library()
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev, dt = q.device, q.dtype
    for t, n, s in ((q, "q", (B, T, Hk, dk)), (k, "k", (B, T, Hk, dk)), (v, "v", (B, T, Hv, dv)),
                    (beta, "beta", (B, T, Hv)), (g, "g", (B, T, Hv))):
        _check(t, n, s, dt, dev)
    if state is not None:
        _check(state, "state", (B, Hv, dk, dv), torch.float32, dev)
    if state_out is None:
        state_out = state if state is not None else torch.empty((B, Hv, dk, dv),
                                                                 dtype=torch.float32, device=dev)
    _check(state_out, "state_out", (B, Hv, dk, dv), torch.float32, dev)
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=out_dtype, device=dev)
    else:
        _check(o, "o", (B, T, Hv, dv), out_dtype, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.gdn_decode_tokens(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(state),
                               _ptr(state_out), _ptr(o), B, T, Hk, Hv, dk, dv, float(scale),
                               int(flags), _dtype_code(dt), _dtype_code(out_dtype), stream)
    if st != GDN_OK:
        raise GdnError(st, "gdn_decode_tokens")
    return o, state_out


def chunk_fwd_varlen(q, k, v, beta, g, cu_seqlens=None, initial_state=None,
                     output_final_state=True, chunk=64, scale=1.0, flags=0, out_dtype=None,
                     final_state=None, o=None, workspace=None):
    """Prefill with the input prologue and, optionally, packed sequences.

    Packed (``cu_seqlens`` an int32 device tensor of N+1 offsets): q, k: [T,Hk,dk]; v: [T,Hv,dv];
    beta, g: [T,Hv]; states [N,Hv,dk,dv].  Dense (``cu_seqlens`` None): the shapes of
    ``chunk_fwd``.  ``flags``: GDN_QK_L2NORM | GDN_BETA_LOGIT | GDN_G_LOGIT, and the plan hint
    GDN_PREFER_SPLIT for packed batches of very uneven lengths.  Returns
    (o, final_state or None)."""
    import torch
    lib = load_library()
    dev, dt = q.device, q.dtype
    if cu_seqlens is None:
        B, T, Hk, dk = q.shape
        Hv, dv = v.shape[2], v.shape[3]
        lead = (B, T)
        nseq = B
    else:
        T, Hk, dk = q.shape
        Hv, dv = v.shape[1], v.shape[2]
        lead = (T,)
        nseq = cu_seqlens.numel() - 1
        _check(cu_seqlens, "cu_seqlens", (nseq + 1,), torch.int32, dev)
    for t, n, s_ in ((q, "q", lead + (Hk, dk)), (k, "k", lead + (Hk, dk)),
                     (v, "v", lead + (Hv, dv)), (beta, "beta", lead + (Hv,)),
                     (g, "g", lead + (Hv,))):
        _check(t, n, s_, dt, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (nseq, Hv, dk, dv), torch.float32, dev)
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty(lead + (Hv, dv), dtype=out_dtype, device=dev)
    else:
        _check(o, "o", lead + (Hv, dv), out_dtype, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((nseq, Hv, dk, dv), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check(final_state, "final_state", (nseq, Hv, dk, dv), torch.float32, dev)
    in_code, out_code = _dtype_code(dt), _dtype_code(out_dtype)
    need = int(lib.gdn_chunk_fwd_varlen_workspace_size(nseq, T, Hk, Hv, dk, dv, chunk, in_code,
                                                       int(cu_seqlens is not None), int(flags)))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.gdn_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                  _ptr(initial_state), _ptr(o), _ptr(final_state),
                                  _ptr(cu_seqlens), nseq, T, Hk, Hv, dk, dv, chunk, float(scale),
                                  int(flags), in_code, out_code, _ptr(workspace), ws_bytes, stream)
    if st != GDN_OK:
        raise GdnError(st, "gdn_chunk_fwd_varlen")
    return o, final_state


def backward(q, k, v, beta, g, d_o, initial_state=None, d_final_state=None, scale=1.0,
             want_d_initial_state=True, workspace=None):
    """Gradients of ``chunk_fwd``'s outputs.  Shapes as ``chunk_fwd``; d_o: [B,T,Hv,dv]
    (float32 or bfloat16); d_final_state: [B,Hv,dk,dv] float32 or None.  Returns a dict of
    float32 tensors dq, dk [B,T,Hk,dk], dv [B,T,Hv,dv], dbeta, dg [B,T,Hv] and
    d_initial_state [B,Hv,dk,dv] (or None)."""
    import torch
    lib = load_library()
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev, dt = q.device, q.dtype
    for t, n, s_ in ((q, "q", (B, T, Hk, dk)), (k, "k", (B, T, Hk, dk)),
                     (v, "v", (B, T, Hv, dv)), (beta, "beta", (B, T, Hv)), (g, "g", (B, T, Hv))):
        _check(t, n, s_, dt, dev)
    _check(d_o, "d_o", (B, T, Hv, dv), d_o.dtype, dev)
    for st, n in ((initial_state, "initial_state"), (d_final_state, "d_final_state")):
        if st is not None:
            _check(st, n, (B, Hv, dk, dv), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dq": torch.empty((B, T, Hk, dk), **f32), "dk": torch.empty((B, T, Hk, dk), **f32),
           "dv": torch.empty((B, T, Hv, dv), **f32), "dbeta": torch.empty((B, T, Hv), **f32),
           "dg": torch.empty((B, T, Hv), **f32),
           "d_initial_state": torch.empty((B, Hv, dk, dv), **f32) if want_d_initial_state else None}
    need = int(lib.gdn_backward_workspace_size(B, T, Hk, Hv, dk, dv))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.gdn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(initial_state),
                          _ptr(d_o), _ptr(d_final_state), _ptr(out["dq"]), _ptr(out["dk"]),
                          _ptr(out["dv"]), _ptr(out["dbeta"]), _ptr(out["dg"]),
                          _ptr(out["d_initial_state"]), B, T, Hk, Hv, dk, dv, float(scale),
                          _dtype_code(dt), _dtype_code(d_o.dtype), _ptr(workspace), ws_bytes,
                          stream)
    if st != GDN_OK:
        raise GdnError(st, "gdn_backward")
    return out


def qsa_index(q, k, r=4, nsel=512, rope_dims=64, rope_base=10000.0, scale=None,
              want_importance=False, sel=None, workspace=None):
    """QSA compressed indexer.  q: [B,T,4,d], k: [B,T,d] (bfloat16 or float32, d in {64,128}).
    Returns (sel [B,T,nsel] int32: the kept block indices of each query, ascending, -1 padded;
    importance [B,T,ceil(T/r)] float32 or None).  ``scale`` defaults to 1/sqrt(d)."""
    import torch
    lib = load_library()
    B, T, Hq, d = q.shape
    dev, dt = q.device, q.dtype
    _check(q, "q", (B, T, Hq, d), dt, dev)
    _check(k, "k", (B, T, d), dt, dev)
    scale = 1.0 / float(d) ** 0.5 if scale is None else float(scale)
    nb = (T + r - 1) // r
    if sel is None:
        sel = torch.empty((B, T, nsel), dtype=torch.int32, device=dev)
    else:
        _check(sel, "sel", (B, T, nsel), torch.int32, dev)
    imp = torch.empty((B, T, nb), dtype=torch.float32, device=dev) if want_importance else None
    need = int(lib.gdn_qsa_workspace_size(B, T, Hq, d, r))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.gdn_qsa_index(_ptr(q), _ptr(k), _ptr(sel), _ptr(imp), B, T, Hq, d, r, nsel,
                           rope_dims, float(rope_base), scale, _dtype_code(dt), _ptr(workspace),
                           ws_bytes, stream)
    if st != GDN_OK:
        raise GdnError(st, "gdn_qsa_index")
    return sel, imp
