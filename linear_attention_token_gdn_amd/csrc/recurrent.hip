// recurrent.hip -- token-by-token prefill of the gated delta rule (explainer page
// "論文解説: Qwen3.8-Next の設計", ta-paperlens.web.app, section "GDNの中身", Eq. (1)).
//
// This is the fp32-input path (every operation in IEEE fp32) and the fallback for sizes the
// chunked MFMA kernel does not take.  One workgroup per (b, hv) chain; thread j owns column j
// of the dk x dv state in registers, so both dk-reductions of a token (e = S^T k and the
// read-out S^T q) are thread-local and a token needs no barrier.  Per token:
//     w = beta (v_j - alpha e_j),  S[:, j] = alpha S[:, j] + k w,  o_j = scale * S[:, j]^T q.
// The sequence loop is sequential, so this kernel is latency-bound: it is meant for the fp32
// workloads and odd shapes, not for throughput.
#include "gdn_internal.h"

namespace gdn {
namespace {

template <int DK, int DV, typename TI, typename TO>
__global__ void __launch_bounds__((DV < 64 ? 64 : DV))
recurrent_kernel(const TI *__restrict__ q, const TI *__restrict__ k, const TI *__restrict__ v,
                 const TI *__restrict__ beta, const TI *__restrict__ g,
                 const float *__restrict__ s0, TO *__restrict__ o, float *__restrict__ sT,
                 int T, const int32_t *__restrict__ cu, unsigned flags, int Hk, int Hv,
                 float scale) {
    const int head = blockIdx.x;  // b * Hv + hv
    const int b = head / Hv, hv = head - b * Hv;
    const int hq = hv / (Hv / Hk);
    const int j = threadIdx.x;
    if (j >= DV) return;
    const size_t sbase = static_cast<size_t>(head) * DK * DV;
    size_t base;
    int len;
    seq_range(cu, T, b, base, len);
    const bool norm = (flags & GDN_QK_L2NORM) != 0;

    float S[DK];
#pragma unroll
    for (int i = 0; i < DK; ++i) S[i] = s0 ? s0[sbase + static_cast<size_t>(i) * DV + j] : 0.f;

    for (int t = 0; t < len; ++t) {
        const size_t bt = base + t;
        const TI *kt = k + (bt * Hk + hq) * DK;
        const TI *qt = q + (bt * Hk + hq) * DK;
        const float alpha = expf(log_alpha_from_input(load_f32(g + bt * Hv + hv), flags));
        const float bet = beta_from_input(load_f32(beta + bt * Hv + hv), flags);
        const float vj = load_f32(v + (bt * Hv + hv) * DV + j);
        float kv[DK];
        float kss = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) {
            kv[i] = load_f32(kt + i);
            kss += kv[i] * kv[i];
        }
        if (norm) {  // (every thread forms the same norms: no exchange needed)
            const float r = inv_norm_from_sumsq(kss);
#pragma unroll
            for (int i = 0; i < DK; ++i) kv[i] *= r;
        }
        float e = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) e += kv[i] * S[i];
        const float w = bet * (vj - alpha * e);
        float f = 0.f, qss = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) {
            S[i] = alpha * S[i] + kv[i] * w;
            const float qi = load_f32(qt + i);
            f += qi * S[i];
            qss += qi * qi;
        }
        if (norm) f *= inv_norm_from_sumsq(qss);  // the read-out is linear in q
        store_f32(o + (bt * Hv + hv) * DV + j, scale * f);
    }
    if (sT) {
#pragma unroll
        for (int i = 0; i < DK; ++i) sT[sbase + static_cast<size_t>(i) * DV + j] = S[i];
    }
}

template <int DK, int DV, typename TI, typename TO>
hipError_t launch_typed(const PrefillArgs &a) {
    const unsigned nblk = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hv);
    hipLaunchKernelGGL((recurrent_kernel<DK, DV, TI, TO>), dim3(nblk), dim3(DV < 64 ? 64 : DV), 0,
                       a.stream, static_cast<const TI *>(a.q), static_cast<const TI *>(a.k),
                       static_cast<const TI *>(a.v), static_cast<const TI *>(a.beta),
                       static_cast<const TI *>(a.g), a.s0, static_cast<TO *>(a.o), a.sT, a.T, a.cu,
                       a.flags, a.Hk, a.Hv, a.scale);
    return hipGetLastError();
}

template <int DK, int DV> hipError_t launch_dims(const PrefillArgs &a) {
    if (a.in_dt == GDN_BF16)
        return a.out_dt == GDN_F32 ? launch_typed<DK, DV, bf16_t, float>(a)
                                   : launch_typed<DK, DV, bf16_t, bf16_t>(a);
    return a.out_dt == GDN_F32 ? launch_typed<DK, DV, float, float>(a)
                               : launch_typed<DK, DV, float, bf16_t>(a);
}

template <int DK> hipError_t launch_dk(const PrefillArgs &a) {
    switch (a.dv) {
    case 16: return launch_dims<DK, 16>(a);
    case 32: return launch_dims<DK, 32>(a);
    case 64: return launch_dims<DK, 64>(a);
    case 128: return launch_dims<DK, 128>(a);
    }
    return hipErrorInvalidValue;
}

__global__ void state_init_kernel(const float *__restrict__ s0, float *__restrict__ sT, size_t n) {
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        sT[i] = s0 ? s0[i] : 0.f;
}

}  // namespace

hipError_t launch_recurrent(const PrefillArgs &a) {
    if (a.B == 0) return hipSuccess;
    switch (a.dk) {
    case 16: return launch_dk<16>(a);
    case 32: return launch_dk<32>(a);
    case 64: return launch_dk<64>(a);
    case 128: return launch_dk<128>(a);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_state_init(const float *s0, float *sT, size_t n, hipStream_t stream) {
    if (n == 0 || sT == s0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(state_init_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       s0, sT, n);
    return hipGetLastError();
}

}  // namespace gdn
