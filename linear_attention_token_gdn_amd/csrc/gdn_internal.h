// gdn_internal.h -- launch interfaces and small device helpers shared by the kernels of
// libgdn.so.  Not part of the public ABI (include/gdn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gdn.h"

namespace gdn {

struct PrefillArgs {
    const void *q, *k, *v, *beta, *g;
    const float *s0;  // may be null (zero state)
    void *o;
    float *sT;        // may be null (not written); may equal s0
    // B sequences.  Dense: sequence b is rows b*T .. b*T+T-1.  Packed (cu != null, device
    // memory): sequence b is rows cu[b] .. cu[b+1]-1 of T rows in all.
    int B, T, Hk, Hv, dk, dv, chunk;
    const int32_t *cu;
    unsigned flags;   // GDN_QK_L2NORM | GDN_BETA_LOGIT | GDN_G_LOGIT
    float scale;
    gdn_dtype_t in_dt, out_dt;
    void *ws;
    size_t ws_bytes;
    hipStream_t stream;
    bool seg = false;  // the single-pass kernel runs the segmented plan (chunk_mfma.hip)
};

struct DecodeArgs {
    const void *q, *k, *v, *beta, *g;
    const float *state_in;  // may equal state, or be null for a zero state
    float *state;           // written with the state after the T tokens
    void *o;
    int B, T, Hk, Hv, dk, dv;
    unsigned flags;
    float scale;
    gdn_dtype_t in_dt, out_dt;
    hipStream_t stream;
};

struct BackwardArgs {
    const void *q, *k, *v, *beta, *g;  // the forward inputs (in_dt)
    const float *s0;                    // may be null (zero initial state)
    const void *dO;                     // [B,T,Hv,dv] (dout_dt)
    const float *dST;                   // may be null (zero)
    float *dq, *dk, *dv, *dbeta, *dg, *dS0;  // dS0 may be null
    int B, T, Hk, Hv, dk_, dv_;               // dk_, dv_: head sizes
    float scale;
    gdn_dtype_t in_dt, dout_dt;
    void *ws;
    hipStream_t stream;
};
// The reverse recurrence (csrc/backward.hip) and the workspace it needs.
size_t backward_workspace(int B, int T, int Hk, int Hv, int dk, int dv);
hipError_t launch_backward(const BackwardArgs &a);
// The chunk-parallel form (csrc/backward_chunk.hip), for dk, dv in {64, 128}.
bool backward_chunk_supports(const BackwardArgs &a);
size_t backward_chunk_workspace(int B, int T, int Hk, int Hv, int dk, int dv);
hipError_t launch_backward_chunk(const BackwardArgs &a);
// out[r][h][i] = sum_j part[((r H + h) M + j) W + i] for i < W, n = rows * H * W outputs
hipError_t launch_part_sum(const float *part, float *out, size_t n, int M, int W,
                           hipStream_t st);

struct QsaArgs {
    const void *q, *k;   // [B, T, 4, d] and [B, T, d] (in_dt)
    int32_t *sel;        // [B, T, nsel]
    float *imp;          // [B, T, ceil(T/r)] or null
    int B, T, d, r, nsel, rope_dims;
    float rope_base, scale;
    gdn_dtype_t in_dt;
    void *ws;
    hipStream_t stream;
};
// The QSA compressed indexer (csrc/qsa.hip) and its workspace.
size_t qsa_workspace(int B, int T, int d, int r);
hipError_t launch_qsa(const QsaArgs &a);

// Token-by-token kernel: every (dk, dv) in {16,32,64,128}^2, both dtypes.  It is the fp32
// path and the fallback of the chunked kernel.
hipError_t launch_recurrent(const PrefillArgs &a);

// Chunk-parallel MFMA kernel for bf16 inputs.  supports() says whether the sizes are handled.
// With a.seg, the segmented plan: every chain is cut into nseg segments of seg_chunks chunks
// (packed sequences: seg_chunks = 0, each chain's segments of ceil(its chunks / nseg) chunks,
// formed on the device), run in parallel -- a transition pass (each segment's affine map of
// the state), a sequential combine of those maps into every segment's entry state, then the
// single-pass kernel over all segments.  Its workspace holds the maps and the entry states,
// then (when it has room for them) every chunk's (I + A)^-1, which the transition pass stores
// and the single pass reads instead of forming it.
struct SegGeom {
    int nseg, seg_chunks;
};
constexpr long kSegTargetUnits = 256;  // (chain, segment) units at most: MI355X's CUs
// Segments shorter than this many chunks lose to the two-kernel form (measured: 16 chains of
// 4,096 tokens run in 4-chunk segments at 0.115 ms against 0.098 ms; of 8,192 tokens in 8-chunk
// segments at 0.171 ms against 0.186 ms)
constexpr long kSegMinChunks = 8;
SegGeom seg_geometry(const PrefillArgs &a);
bool chunk_mfma_supports(const PrefillArgs &a);
// The segmented plan's workspace: the maps and entry states, plus (least = false) the per-chunk
// (I + A)^-1 records that spare the output pass forming them; with only the former it runs
// without the records.
size_t chunk_mfma_workspace(const PrefillArgs &a, bool least = false);
hipError_t launch_chunk_mfma(const PrefillArgs &a);

// Two-kernel chunk-parallel form (a fully parallel prep kernel and a per-chain scan kernel
// through a workspace) for shapes with fewer chains than compute units.  The workspace holds
// the records of a segment of chunks; longer sequences run segment after segment, as many
// chunks at a time as a.ws_bytes holds.  chunk_split_workspace: the size that keeps the
// records to at most 2 GiB (smallest = false), or the least the plan runs with (one chunk
// per segment).
bool chunk_split_supports(const PrefillArgs &a);
size_t chunk_split_workspace(const PrefillArgs &a, bool smallest = false);
hipError_t launch_chunk_split(const PrefillArgs &a);

// One streaming pass over the decode state.
hipError_t launch_decode(const DecodeArgs &a);

// final_state = initial_state (or zeros) -- the whole result of a T = 0 prefill.
hipError_t launch_state_init(const float *s0, float *sT, size_t n, hipStream_t stream);

// ---------------------------------------------------------------------------------------
// device helpers

typedef uint16_t bf16_t;  // raw bf16 storage

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round to nearest even; NaN stays NaN (quiet bit set).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ float load_f32(const T *p);
template <> __device__ __forceinline__ float load_f32<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float load_f32<bf16_t>(const bf16_t *p) {
    return bf16_to_f32(*p);
}

// ---- where a sequence's tokens are (see PrefillArgs): first row and length.  Packed
//      offsets are clamped into [0, T] and made nondecreasing, so malformed offsets can only
//      give wrong lengths, never accesses outside the tensors.
__device__ __forceinline__ void seq_range(const int32_t *cu, int T, int seq, size_t &base,
                                          int &len) {
    if (cu == nullptr) {
        base = static_cast<size_t>(seq) * T;
        len = T;
    } else {
        const int a = min(max(cu[seq], 0), T);
        const int b = min(max(cu[seq + 1], a), T);
        base = static_cast<size_t>(a);
        len = b - a;
    }
}

// ---- the input prologue (flags of gdn_chunk_fwd_varlen / gdn_decode_tokens)
__device__ __forceinline__ float beta_from_input(float x, unsigned flags) {
    return (flags & GDN_BETA_LOGIT) ? 1.f / (1.f + expf(-x)) : x;
}
// log alpha; from a logit x: log sigmoid(x) = -log(1 + e^-x), evaluated without overflow
__device__ __forceinline__ float log_alpha_from_input(float x, unsigned flags) {
    if (!(flags & GDN_G_LOGIT)) return x;
    return x >= 0.f ? -log1pf(expf(-x)) : x - log1pf(expf(x));
}
// 1 / max(||x||_2, eps) for the L2 normalisation of q and k
constexpr float kNormEps = 1e-6f;
__device__ __forceinline__ float inv_norm_from_sumsq(float ss) {
    return 1.f / fmaxf(sqrtf(ss), kNormEps);
}

// ---- power-of-two operand scaling for the fp16 matrix-core operands.  The value side of the
//      rule (v, U, Delta, the state S and the output) is linear in (v, S0), and every value
//      column j evolves on its own, so the fp16 copies of a column may carry any power of two
//      sigma_j: products of scaled operands are exactly sigma_j times the unscaled ones, and
//      multiplying fp32 results by sigma_j or 1/sigma_j is exact.  Given m = max |x| over the
//      values to convert, pow2_scale returns sigma with m * sigma in [2^8, 2^9): far from
//      fp16's overflow (65504) and from its subnormals (below 2^-14), whatever the magnitude
//      of v and S0.  sigma = 1 for m = 0, Inf or NaN; the exponent is clamped to +-100 so that
//      sigma and 1/sigma stay normal fp32 numbers.
__device__ __forceinline__ void pow2_scale(float m, float &sigma, float &inv_sigma) {
    const int eb = static_cast<int>((__float_as_uint(m) >> 23) & 0xffu);  // biased exponent
    // m in [2^(eb-127), 2^(eb-126))  ->  m * 2^e in [2^8, 2^9) for e = 135 - eb; arithmetic
    // selects only (no branch on the value)
    const int ok = static_cast<int>(static_cast<unsigned>(eb - 1) < 254u);  // not 0, Inf, NaN
    const int e = ok * min(max(135 - eb, -100), 100);
    sigma = __uint_as_float(static_cast<uint32_t>(127 + e) << 23);
    inv_sigma = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
}

// Maximum over the four lanes l mod 16 + 16 r (r = 0..3) of a wavefront -- the four lanes of a
// column in the 16x16 MFMA accumulator and B-operand layouts -- with two VALU lane swaps:
// permlane16_swap exchanges rows 1, 3 of its first operand with rows 0, 2 of its second (a
// row being 16 lanes), permlane32_swap the upper half of the first with the lower half of
// the second; given the same value twice, the maximum of the two results is the maximum over
// row pairs (0, 1), (2, 3), and then over halves.  No LDS round trip (ds_bpermute) involved.
__device__ __forceinline__ float max_over_rows(float x) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const unsigned w = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <typename T> __device__ __forceinline__ void store_f32(T *p, float x);
template <> __device__ __forceinline__ void store_f32<float>(float *p, float x) { *p = x; }
template <> __device__ __forceinline__ void store_f32<bf16_t>(bf16_t *p, float x) {
    *p = f32_to_bf16(x);
}

}  // namespace gdn
