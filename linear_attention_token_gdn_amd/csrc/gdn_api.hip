// gdn_api.hip -- the C ABI of libgdn.so (declared in include/gdn.h): host-side argument
// validation and dispatch to the kernels.  Nothing here allocates device memory or
// synchronises the host.  The only state is the per-device address of the static scratch
// buffer of gdn_chunk_fwd_noalloc, looked up once per device.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "gdn_internal.h"

// Scratch of gdn_chunk_fwd_noalloc (its workspace), for callers that cannot allocate: one copy
// in every GPU's memory, held from the library's load until the process ends.  Host code uses
// it only through the device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

bool dim_supported(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool dtype_known(gdn_dtype_t t) { return t == GDN_F32 || t == GDN_BF16; }
size_t dtype_bytes(gdn_dtype_t t) { return t == GDN_F32 ? 4 : 2; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Half-open byte ranges [p, p + n) overlap.
bool overlap(const void *p, size_t n, const void *r, size_t m) {
    if (p == nullptr || r == nullptr || n == 0 || m == 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(r);
    return a < b + m && b < a + n;
}

// Prefill variants.  GDN_FORCE_VARIANT=recurrent|fused|split|segmented pins one for A/B
// measurements (a variant that does not support the sizes falls back to the default choice).
enum class Variant { Recurrent, Fused, Split, Segmented };

// Below this many (b, hv) chains the single-pass kernel leaves most compute units idle; long
// chains are then cut into segments run in parallel, shorter ones take the two-kernel form
// (parallel over chunks).
constexpr long kSplitBelowChains = 128;

bool segmented_supported(const gdn::PrefillArgs &a) {
    if (!gdn::chunk_mfma_supports(a)) return false;
    gdn::PrefillArgs s = a;
    s.seg = true;
    return gdn::seg_geometry(s).nseg > 1;
}

// The default choice for few chains: segments of at least kSegMinChunks chunks (or a length
// pinned by GDN_SEG_CHUNKS).  Packed sequences: judged on the mean length, T / num_seqs (the
// host does not read the offsets).
bool segmented_preferred(const gdn::PrefillArgs &a) {
    if (!segmented_supported(a)) return false;
    gdn::PrefillArgs s = a;
    s.seg = true;
    const gdn::SegGeom sg = gdn::seg_geometry(s);
    if (a.cu != nullptr) {
        const long mean_chunks = static_cast<long>(a.T) / a.B / a.chunk;
        return mean_chunks >= gdn::kSegMinChunks * sg.nseg;
    }
    const char *env = getenv("GDN_SEG_CHUNKS");
    return (env != nullptr && atol(env) > 0) || sg.seg_chunks >= gdn::kSegMinChunks;
}

Variant choose_variant(const gdn::PrefillArgs &a) {
    const char *env = getenv("GDN_FORCE_VARIANT");
    if (env != nullptr) {
        if (strcmp(env, "recurrent") == 0) return Variant::Recurrent;
        if (strcmp(env, "fused") == 0 && gdn::chunk_mfma_supports(a)) return Variant::Fused;
        if (strcmp(env, "split") == 0 && gdn::chunk_split_supports(a)) return Variant::Split;
        if (strcmp(env, "segmented") == 0 && segmented_supported(a)) return Variant::Segmented;
    }
    const long chains = static_cast<long>(a.B) * a.Hv;
    const bool few = chains < kSplitBelowChains;
    if (gdn::chunk_split_supports(a) && (a.flags & GDN_PREFER_SPLIT)) return Variant::Split;
    if (few && segmented_preferred(a)) return Variant::Segmented;
    if (few && gdn::chunk_split_supports(a)) return Variant::Split;
    if (gdn::chunk_mfma_supports(a)) return Variant::Fused;
    return Variant::Recurrent;
}

// The arguments with the plan's own switches set.
gdn::PrefillArgs for_plan(const gdn::PrefillArgs &a, Variant var) {
    gdn::PrefillArgs r = a;
    r.seg = var == Variant::Segmented;
    return r;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char *gdn_status_string(gdn_status_t s) {
    switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
    case GDN_ERR_SCRATCH_TOO_SMALL:
        return "GDN_ERR_SCRATCH_TOO_SMALL (the sizes need more workspace than the "
               "GDN_NOALLOC_SCRATCH_BYTES of gdn_chunk_fwd_noalloc's static scratch)";
    default: break;
    }
    return "GDN_ERR_UNKNOWN";
}

static gdn_status_t check_prefill(const gdn::PrefillArgs &a) {
    if (a.B < 0 || a.T < 0 || a.Hk <= 0 || a.Hv <= 0 || a.dk <= 0 || a.dv <= 0)
        return GDN_ERR_INVALID_ARG;
    if (a.Hv % a.Hk != 0) return GDN_ERR_INVALID_ARG;
    if (!dtype_known(a.in_dt) || !dtype_known(a.out_dt)) return GDN_ERR_UNSUPPORTED;
    if (!dim_supported(a.dk) || !dim_supported(a.dv)) return GDN_ERR_UNSUPPORTED;
    if (a.chunk != 16 && a.chunk != 32 && a.chunk != 64) return GDN_ERR_UNSUPPORTED;
    if (a.flags & ~(GDN_QK_L2NORM | GDN_BETA_LOGIT | GDN_G_LOGIT | GDN_PREFER_SPLIT))
        return GDN_ERR_INVALID_ARG;
    const size_t B = a.B, T = a.T, Hk = a.Hk, Hv = a.Hv, dk = a.dk, dv = a.dv;
    const size_t rows = a.cu ? T : B * T;  // token rows of the q, k, v, beta, g, o tensors
    const size_t ib = dtype_bytes(a.in_dt), ob = dtype_bytes(a.out_dt);
    const size_t nq = rows * Hk * dk * ib, nv = rows * Hv * dv * ib, ng = rows * Hv * ib;
    const size_t no = rows * Hv * dv * ob, ns = B * Hv * dk * dv * sizeof(float);
    if (a.cu && (B == 0 || !aligned(a.cu, 4))) return GDN_ERR_INVALID_ARG;
    if (rows > 0) {
        if (!a.q || !a.k || !a.v || !a.beta || !a.g || !a.o) return GDN_ERR_INVALID_ARG;
        if (!aligned(a.q, 16) || !aligned(a.k, 16) || !aligned(a.v, 16) || !aligned(a.o, 16))
            return GDN_ERR_INVALID_ARG;
        if (!aligned(a.beta, ib) || !aligned(a.g, ib)) return GDN_ERR_INVALID_ARG;
        if (overlap(a.o, no, a.q, nq) || overlap(a.o, no, a.k, nq) || overlap(a.o, no, a.v, nv) ||
            overlap(a.o, no, a.beta, ng) || overlap(a.o, no, a.g, ng) ||
            overlap(a.o, no, a.s0, ns) || overlap(a.o, no, a.sT, ns))
            return GDN_ERR_INVALID_ARG;
    }
    if ((a.s0 && !aligned(a.s0, 16)) || (a.sT && !aligned(a.sT, 16))) return GDN_ERR_INVALID_ARG;
    if (a.sT && a.sT != a.s0 && overlap(a.sT, ns, a.s0, ns)) return GDN_ERR_INVALID_ARG;
    if (a.sT && rows > 0 &&
        (overlap(a.sT, ns, a.q, nq) || overlap(a.sT, ns, a.k, nq) || overlap(a.sT, ns, a.v, nv)))
        return GDN_ERR_INVALID_ARG;
    return GDN_OK;
}

// Workspace bytes the plan `var` needs for a validated prefill with tokens: the size the
// workspace-size queries return, or (least) the smallest it runs with.
static size_t plan_workspace(const gdn::PrefillArgs &a, Variant var, bool least = false) {
    return var == Variant::Split ? gdn::chunk_split_workspace(a, least)
           : var == Variant::Fused || var == Variant::Segmented
               ? gdn::chunk_mfma_workspace(for_plan(a, var), least)
               : 0;
}

// The whole prefill: validation, the T = 0 case, workspace check and dispatch.  least: the
// workspace only has to hold the plan's smallest size (the allocation-free entry point).
static gdn_status_t run_prefill(gdn::PrefillArgs &a, bool least = false) {
    gdn_status_t st = check_prefill(a);
    if (st != GDN_OK) return st;
    if (a.B == 0) return GDN_OK;
    if (a.T == 0) {  // no tokens at all: final = initial
        if (!a.sT) return GDN_OK;
        const size_t n = static_cast<size_t>(a.B) * a.Hv * a.dk * a.dv;
        return gdn::launch_state_init(a.s0, a.sT, n, a.stream) == hipSuccess ? GDN_OK
                                                                              : GDN_ERR_HIP;
    }
    const Variant var = choose_variant(a);
    const size_t need = plan_workspace(a, var, least);
    if (need > 0 && (a.ws == nullptr || a.ws_bytes < need)) return GDN_ERR_INVALID_ARG;
    if (need > 0 && !aligned(a.ws, 256)) return GDN_ERR_INVALID_ARG;
    hipError_t e = var == Variant::Split ? gdn::launch_chunk_split(a)
                   : var == Variant::Fused || var == Variant::Segmented
                       ? gdn::launch_chunk_mfma(for_plan(a, var))
                       : gdn::launch_recurrent(a);
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}


const char *gdn_chunk_fwd_plan(int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                               gdn_dtype_t in_dtype) {
    gdn::PrefillArgs a = {};
    a.B = B; a.T = T; a.Hk = Hk; a.Hv = Hv; a.dk = dk; a.dv = dv; a.chunk = chunk;
    a.in_dt = in_dtype; a.out_dt = GDN_F32;
    if (B < 0 || T < 0 || Hk <= 0 || Hv <= 0 || Hv % Hk != 0 || !dim_supported(dk) ||
        !dim_supported(dv) || (chunk != 16 && chunk != 32 && chunk != 64) || !dtype_known(in_dtype))
        return "invalid";
    switch (choose_variant(a)) {
    case Variant::Split: return "split";
    case Variant::Fused: return "fused";
    case Variant::Segmented: return "segmented";
    default: return "recurrent";
    }
}

// Workspace bytes of the plan these sizes run; packed: offsets given (their values do not
// matter: the bound on the record slots holds for any offsets).
static size_t prefill_workspace(int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                                gdn_dtype_t in_dtype, bool packed, unsigned flags) {
    static const int32_t kPackedTag = 0;  // a.cu only marks packed sequences here; never read
    gdn::PrefillArgs a = {};
    a.B = B; a.T = T; a.Hk = Hk; a.Hv = Hv; a.dk = dk; a.dv = dv; a.chunk = chunk;
    a.in_dt = in_dtype; a.out_dt = GDN_F32;
    a.cu = packed ? &kPackedTag : nullptr;
    a.flags = flags & GDN_PREFER_SPLIT;
    if (B < 0 || T < 0 || Hk <= 0 || Hv <= 0 || Hv % Hk != 0 || !dim_supported(dk) ||
        !dim_supported(dv) || (chunk != 16 && chunk != 32 && chunk != 64) || !dtype_known(in_dtype))
        return 0;
    if (B == 0 || T == 0) return 0;
    const Variant var = choose_variant(a);
    switch (var) {
    case Variant::Split: return gdn::chunk_split_workspace(a);
    case Variant::Fused:
    case Variant::Segmented: return gdn::chunk_mfma_workspace(for_plan(a, var));
    default: return 0;
    }
}

size_t gdn_chunk_fwd_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                                    gdn_dtype_t in_dtype) {
    return prefill_workspace(B, T, Hk, Hv, dk, dv, chunk, in_dtype, false, 0u);
}

gdn_status_t gdn_chunk_fwd(const void *q, const void *k, const void *v, const void *beta,
                           const void *g, const float *initial_state, void *o,
                           float *final_state, int B, int T, int Hk, int Hv, int dk, int dv,
                           int chunk, float scale, gdn_dtype_t in_dtype, gdn_dtype_t out_dtype,
                           void *workspace, size_t workspace_bytes, void *stream) {
    return gdn_chunk_fwd_varlen(q, k, v, beta, g, initial_state, o, final_state, nullptr, B, T,
                                Hk, Hv, dk, dv, chunk, scale, 0u, in_dtype, out_dtype, workspace,
                                workspace_bytes, stream);
}

gdn_status_t gdn_chunk_fwd_varlen(const void *q, const void *k, const void *v, const void *beta,
                                  const void *g, const float *initial_state, void *o,
                                  float *final_state, const int32_t *cu_seqlens, int num_seqs,
                                  int T, int Hk, int Hv, int dk, int dv, int chunk, float scale,
                                  unsigned flags, gdn_dtype_t in_dtype, gdn_dtype_t out_dtype,
                                  void *workspace, size_t workspace_bytes, void *stream) {
    gdn::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = g;
    a.s0 = initial_state; a.o = o; a.sT = final_state;
    a.B = num_seqs; a.T = T; a.Hk = Hk; a.Hv = Hv; a.dk = dk; a.dv = dv; a.chunk = chunk;
    a.cu = cu_seqlens; a.flags = flags;
    a.scale = scale; a.in_dt = in_dtype; a.out_dt = out_dtype;
    a.ws = workspace; a.ws_bytes = workspace_bytes;
    a.stream = static_cast<hipStream_t>(stream);
    return run_prefill(a);
}

}  // extern "C"

namespace {

// Device address of `scratch` on each device, looked up once per device (with that device
// current) and kept until the process ends.
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void *g_scratch_addr[kMaxDevices];

// The scratch address on the device that runs `stream` (the current device for the null
// stream).
hipError_t scratch_address(hipStream_t stream, void **addr) {
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    dev = cur;
    if (stream != nullptr) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_addr[dev] == nullptr) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

gdn_status_t gdn_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const void *beta,
                                   const void *g, const float *initial_state, void *o,
                                   float *final_state, int B, int T, int Hk, int Hv, int dk,
                                   int dv, int chunk, float scale, gdn_dtype_t in_dtype,
                                   gdn_dtype_t out_dtype, void *stream) {
    gdn::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = g;
    a.s0 = initial_state; a.o = o; a.sT = final_state;
    a.B = B; a.T = T; a.Hk = Hk; a.Hv = Hv; a.dk = dk; a.dv = dv; a.chunk = chunk;
    a.cu = nullptr; a.flags = 0u;
    a.scale = scale; a.in_dt = in_dtype; a.out_dt = out_dtype;
    a.ws = nullptr; a.ws_bytes = 0;
    a.stream = static_cast<hipStream_t>(stream);
    const gdn_status_t st = check_prefill(a);
    if (st != GDN_OK) return st;
    if (a.B > 0 && a.T > 0) {
        // the split plan runs in segments of as many chunks as the scratch holds
        const size_t need = plan_workspace(a, choose_variant(a), true);
        if (need > GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_SCRATCH_TOO_SMALL;
        if (need > 0) {
            // whatever a kernel must find zeroed it clears itself (the split plan's prep kernel
            // resets the scan's progress words), so no memset is needed
            if (scratch_address(a.stream, &a.ws) != hipSuccess) return GDN_ERR_HIP;
            a.ws_bytes = GDN_NOALLOC_SCRATCH_BYTES;
        }
    }
    return run_prefill(a, true);
}

size_t gdn_chunk_fwd_varlen_workspace_size(int num_seqs, int T, int Hk, int Hv, int dk, int dv,
                                           int chunk, gdn_dtype_t in_dtype, int packed,
                                           unsigned flags) {
    return prefill_workspace(num_seqs, T, Hk, Hv, dk, dv, chunk, in_dtype, packed != 0, flags);
}

gdn_status_t gdn_decode_tokens(const void *q, const void *k, const void *v, const void *beta,
                               const void *g, const float *state_in, float *state_out, void *o,
                               int B, int T, int Hk, int Hv, int dk, int dv, float scale,
                               unsigned flags, gdn_dtype_t in_dtype, gdn_dtype_t out_dtype,
                               void *stream) {
    if (B < 0 || T < 0 || Hk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hk != 0)
        return GDN_ERR_INVALID_ARG;
    if (flags & ~(GDN_QK_L2NORM | GDN_BETA_LOGIT | GDN_G_LOGIT)) return GDN_ERR_INVALID_ARG;
    if (!dtype_known(in_dtype) || !dtype_known(out_dtype)) return GDN_ERR_UNSUPPORTED;
    if (!dim_supported(dk) || !dim_supported(dv)) return GDN_ERR_UNSUPPORTED;
    if (B == 0) return GDN_OK;
    if (!state_out) return GDN_ERR_INVALID_ARG;
    if (T > 0 && (!q || !k || !v || !beta || !g || !o)) return GDN_ERR_INVALID_ARG;
    const size_t ib = dtype_bytes(in_dtype), ob = dtype_bytes(out_dtype);
    if (!aligned(state_out, 16) || (state_in && !aligned(state_in, 16))) return GDN_ERR_INVALID_ARG;
    const size_t ns = size_t(B) * Hv * dk * dv * sizeof(float);
    // the input state is either the output state itself (in place) or disjoint from it
    if (state_in != state_out && overlap(state_in, ns, state_out, ns)) return GDN_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (T == 0)
        return gdn::launch_state_init(state_in, state_out, size_t(B) * Hv * dk * dv, st) == hipSuccess
                   ? GDN_OK
                   : GDN_ERR_HIP;
    if (!aligned(q, ib) || !aligned(k, ib) || !aligned(v, ib) || !aligned(beta, ib) ||
        !aligned(g, ib) || !aligned(o, ob))
        return GDN_ERR_INVALID_ARG;
    const size_t nq = size_t(B) * T * Hk * dk * ib, nv = size_t(B) * T * Hv * dv * ib;
    const size_t ng = size_t(B) * T * Hv * ib, no = size_t(B) * T * Hv * dv * ob;
    if (overlap(o, no, q, nq) || overlap(o, no, k, nq) || overlap(o, no, v, nv) ||
        overlap(o, no, beta, ng) || overlap(o, no, g, ng) || overlap(o, no, state_out, ns) ||
        overlap(o, no, state_in, ns) || overlap(state_out, ns, q, nq) ||
        overlap(state_out, ns, k, nq) || overlap(state_out, ns, v, nv) ||
        overlap(state_out, ns, beta, ng) || overlap(state_out, ns, g, ng))
        return GDN_ERR_INVALID_ARG;
    gdn::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = g;
    a.state_in = state_in; a.state = state_out; a.o = o;
    a.B = B; a.T = T; a.Hk = Hk; a.Hv = Hv; a.dk = dk; a.dv = dv; a.scale = scale;
    a.flags = flags; a.in_dt = in_dtype; a.out_dt = out_dtype;
    a.stream = st;
    return gdn::launch_decode(a) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status_t gdn_decode_step(const void *q, const void *k, const void *v, const void *beta,
                             const void *g, float *state, void *o, int B, int Hk, int Hv,
                             int dk, int dv, float scale, gdn_dtype_t in_dtype,
                             gdn_dtype_t out_dtype, void *stream) {
    if (B > 0 && !state) return GDN_ERR_INVALID_ARG;  // the state is required here
    return gdn_decode_tokens(q, k, v, beta, g, state, state, o, B, 1, Hk, Hv, dk, dv, scale, 0u,
                             in_dtype, out_dtype, stream);
}

size_t gdn_backward_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv) {
    if (B <= 0 || T < 0 || Hk <= 0 || Hv <= 0 || Hv % Hk != 0 || !dim_supported(dk) ||
        !dim_supported(dv))
        return 0;
    return gdn::backward_workspace(B, T, Hk, Hv, dk, dv);
}

gdn_status_t gdn_backward(const void *q, const void *k, const void *v, const void *beta,
                          const void *g, const float *initial_state, const void *d_o,
                          const float *d_final_state, float *dq, float *dk, float *dv,
                          float *dbeta, float *dg, float *d_initial_state, int B, int T, int Hk,
                          int Hv, int dk_dim, int dv_dim, float scale, gdn_dtype_t in_dtype,
                          gdn_dtype_t dout_dtype, void *workspace, size_t workspace_bytes,
                          void *stream) {
    if (B < 0 || T < 0 || Hk <= 0 || Hv <= 0 || dk_dim <= 0 || dv_dim <= 0 || Hv % Hk != 0)
        return GDN_ERR_INVALID_ARG;
    if (!dtype_known(in_dtype) || !dtype_known(dout_dtype)) return GDN_ERR_UNSUPPORTED;
    if (!dim_supported(dk_dim) || !dim_supported(dv_dim)) return GDN_ERR_UNSUPPORTED;
    if (B == 0) return GDN_OK;
    const size_t BT = size_t(B) * T;
    const size_t ib = dtype_bytes(in_dtype), db = dtype_bytes(dout_dtype);
    const size_t nq = BT * Hk * dk_dim, nv = BT * Hv * dv_dim, ng = BT * Hv;
    const size_t ns = size_t(B) * Hv * dk_dim * dv_dim;
    if (T > 0) {
        if (!q || !k || !v || !beta || !g || !d_o || !dq || !dk || !dv || !dbeta || !dg)
            return GDN_ERR_INVALID_ARG;
        if (!aligned(q, ib) || !aligned(k, ib) || !aligned(v, ib) || !aligned(beta, ib) ||
            !aligned(g, ib) || !aligned(d_o, db) || !aligned(dv, 16))
            return GDN_ERR_INVALID_ARG;
        // every output is disjoint from every input and from the other outputs
        const void *in[] = {q, k, v, beta, g, d_o, initial_state, d_final_state};
        const size_t inb[] = {nq * ib, nq * ib, nv * ib, ng * ib, ng * ib, nv * db, ns * 4, ns * 4};
        float *out[] = {dq, dk, dv, dbeta, dg, d_initial_state};
        const size_t outb[] = {nq * 4, nq * 4, nv * 4, ng * 4, ng * 4, ns * 4};
        for (int i = 0; i < 6; ++i) {
            for (int j = 0; j < 8; ++j)
                if (overlap(out[i], outb[i], in[j], inb[j])) return GDN_ERR_INVALID_ARG;
            for (int j = i + 1; j < 6; ++j)
                if (overlap(out[i], outb[i], out[j], outb[j])) return GDN_ERR_INVALID_ARG;
        }
    }
    if ((initial_state && !aligned(initial_state, 16)) ||
        (d_final_state && !aligned(d_final_state, 16)) ||
        (d_initial_state && !aligned(d_initial_state, 16)))
        return GDN_ERR_INVALID_ARG;
    const size_t need = gdn::backward_workspace(B, T, Hk, Hv, dk_dim, dv_dim);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
        return GDN_ERR_INVALID_ARG;
    gdn::BackwardArgs a;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = g; a.s0 = initial_state;
    a.dO = d_o; a.dST = d_final_state;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dbeta = dbeta; a.dg = dg; a.dS0 = d_initial_state;
    a.B = B; a.T = T; a.Hk = Hk; a.Hv = Hv; a.dk_ = dk_dim; a.dv_ = dv_dim; a.scale = scale;
    a.in_dt = in_dtype; a.dout_dt = dout_dtype;
    a.ws = workspace;
    a.stream = static_cast<hipStream_t>(stream);
    return gdn::launch_backward(a) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

size_t gdn_qsa_workspace_size(int B, int T, int Hq, int d, int r) {
    if (B <= 0 || T <= 0 || Hq != 4 || (d != 64 && d != 128) || r < 1) return 0;
    return gdn::qsa_workspace(B, T, d, r);
}

gdn_status_t gdn_qsa_index(const void *q, const void *k, int32_t *sel, float *importance, int B,
                           int T, int Hq, int d, int r, int nsel, int rope_dims, float rope_base,
                           float scale, gdn_dtype_t in_dtype, void *workspace,
                           size_t workspace_bytes, void *stream) {
    if (B < 0 || T < 0 || Hq <= 0 || d <= 0 || r < 1 || nsel < 1) return GDN_ERR_INVALID_ARG;
    if (rope_dims < 0 || rope_dims > d || rope_dims % 2 != 0) return GDN_ERR_INVALID_ARG;
    if (!(scale == scale) || scale - scale != 0.f) return GDN_ERR_INVALID_ARG;  // NaN or Inf
    if (rope_dims > 0 && !(rope_base > 0.f && rope_base - rope_base == 0.f))
        return GDN_ERR_INVALID_ARG;
    if (!dtype_known(in_dtype)) return GDN_ERR_UNSUPPORTED;
    if (Hq != 4 || (d != 64 && d != 128)) return GDN_ERR_UNSUPPORTED;
    if (B == 0 || T == 0) return GDN_OK;
    const size_t ib = dtype_bytes(in_dtype);
    const size_t BT = size_t(B) * T, nb = (size_t(T) + r - 1) / r;
    const size_t qb = BT * Hq * d * ib, kb = BT * d * ib, sb = BT * nsel * 4, mb = BT * nb * 4;
    if (!q || !k || !sel) return GDN_ERR_INVALID_ARG;
    if (!aligned(q, ib) || !aligned(k, ib) || !aligned(sel, 4) ||
        (importance && !aligned(importance, 4)))
        return GDN_ERR_INVALID_ARG;
    const size_t need = gdn::qsa_workspace(B, T, d, r);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return GDN_ERR_INVALID_ARG;
    // outputs are disjoint from the inputs, from each other and from the workspace
    const void *ro[] = {q, k, workspace};
    const size_t rob[] = {qb, kb, need};
    for (int j = 0; j < 3; ++j)
        if (overlap(sel, sb, ro[j], rob[j]) || overlap(importance, mb, ro[j], rob[j]))
            return GDN_ERR_INVALID_ARG;
    if (overlap(sel, sb, importance, mb)) return GDN_ERR_INVALID_ARG;
    gdn::QsaArgs a;
    a.q = q; a.k = k; a.sel = sel; a.imp = importance;
    a.B = B; a.T = T; a.d = d; a.r = r; a.nsel = nsel; a.rope_dims = rope_dims;
    a.rope_base = rope_base; a.scale = scale; a.in_dt = in_dtype;
    a.ws = workspace;
    a.stream = static_cast<hipStream_t>(stream);
    return gdn::launch_qsa(a) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"
