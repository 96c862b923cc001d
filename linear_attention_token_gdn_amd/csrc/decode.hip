// decode.hip -- one decode step of the gated delta rule as a single streaming pass over the
// fp32 state (explainer page "論文解説: Qwen3.8-Next の設計", ta-paperlens.web.app, section
// "GDNの中身", Eq. (1), applied to one new token per sequence).
//
// With e = S^T k and f = S^T q taken from the OLD state, one token of Eq. (1) is
//     w  = beta (v - alpha e)
//     S' = alpha S + k w^T
//     o  = scale S'^T q = scale (alpha f + (k^T q) w)
// so both dk-reductions come from one read of S, and S' is written while the slice is still
// in registers: exactly one read and one write of every state byte.
//
// One workgroup per (b, hv) state.  Thread (rg, cg) holds float4 column group cg of the rows
// rg, rg + R, rg + 2R, ... (R row groups): every load and store instruction of a wavefront
// covers whole 512-byte rows.  The state is read with ordinary loads and written with
// non-temporal stores (it is not read again in this step); on MI355X this pairing streams
// ~6.2 TB/s for the 1 GiB read+write of a 256 x 32 x 128 x 128 state, as fast as a plain
// read-modify-write kernel, while non-temporal loads cost ~15%.
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DK, int DV> struct DecodeShape {
    static constexpr int CG = DV / 4;                                  // float4 groups per row
    static constexpr int RPT = (DK * DV / 1024) > 0 ? DK * DV / 1024 : 1;  // rows per thread
    static constexpr int R = DK / RPT;                                 // row groups
    static constexpr int NT = CG * R;                                  // threads (64..256)
    static constexpr int NW = NT / 64;                                 // wavefronts
    static_assert(NT % 64 == 0 && NT <= 256, "decode block shape");
};

template <int DK, int DV, typename TI, typename TO>
__global__ void __launch_bounds__((DecodeShape<DK, DV>::NT))
decode_kernel(const TI *__restrict__ q, const TI *__restrict__ k, const TI *__restrict__ v,
              const TI *__restrict__ beta, const TI *__restrict__ g, float *__restrict__ state,
              TO *__restrict__ o, int Hk, int Hv, float scale) {
    using Sh = DecodeShape<DK, DV>;
    __shared__ float red_e[Sh::NW][DV];
    __shared__ float red_f[Sh::NW][DV];
    __shared__ float red_kq[Sh::NW];
    __shared__ __attribute__((aligned(16))) float w_sh[DV];

    const int head = blockIdx.x;  // b * Hv + hv
    const int b = head / Hv, hv = head - b * Hv;
    const int hq = hv / (Hv / Hk);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % Sh::CG, rg = tid / Sh::CG;

    f32x4 *S = reinterpret_cast<f32x4 *>(state + static_cast<size_t>(head) * DK * DV);
    const TI *kp = k + (static_cast<size_t>(b) * Hk + hq) * DK;
    const TI *qp = q + (static_cast<size_t>(b) * Hk + hq) * DK;

    f32x4 s[Sh::RPT];
#pragma unroll
    for (int m = 0; m < Sh::RPT; ++m)
        s[m] = S[(rg + Sh::R * m) * Sh::CG + cg];
    float kr[Sh::RPT], qr[Sh::RPT];
#pragma unroll
    for (int m = 0; m < Sh::RPT; ++m) {
        kr[m] = load_f32(kp + rg + Sh::R * m);
        qr[m] = load_f32(qp + rg + Sh::R * m);
    }

    f32x4 e = {0.f, 0.f, 0.f, 0.f}, f = e;
    float kq = 0.f;
#pragma unroll
    for (int m = 0; m < Sh::RPT; ++m) {
        e.x += kr[m] * s[m].x; e.y += kr[m] * s[m].y; e.z += kr[m] * s[m].z; e.w += kr[m] * s[m].w;
        f.x += qr[m] * s[m].x; f.y += qr[m] * s[m].y; f.z += qr[m] * s[m].z; f.w += qr[m] * s[m].w;
        kq += kr[m] * qr[m];
    }
    if (cg != 0) kq = 0.f;  // every row counted once
    // reduce over the row groups held by this wavefront (lanes CG apart share columns)
#pragma unroll
    for (int off = Sh::CG; off < 64; off <<= 1) {
        e.x += __shfl_xor(e.x, off); e.y += __shfl_xor(e.y, off);
        e.z += __shfl_xor(e.z, off); e.w += __shfl_xor(e.w, off);
        f.x += __shfl_xor(f.x, off); f.y += __shfl_xor(f.y, off);
        f.z += __shfl_xor(f.z, off); f.w += __shfl_xor(f.w, off);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) kq += __shfl_xor(kq, off);
    if (lane < Sh::CG) {
        red_e[wave][4 * cg + 0] = e.x; red_e[wave][4 * cg + 1] = e.y;
        red_e[wave][4 * cg + 2] = e.z; red_e[wave][4 * cg + 3] = e.w;
        red_f[wave][4 * cg + 0] = f.x; red_f[wave][4 * cg + 1] = f.y;
        red_f[wave][4 * cg + 2] = f.z; red_f[wave][4 * cg + 3] = f.w;
    }
    if (lane == 0) red_kq[wave] = kq;
    __syncthreads();

    const size_t gi = static_cast<size_t>(head);
    const float alpha = expf(load_f32(g + gi));
    const float bt = load_f32(beta + gi);
    if (tid < DV) {
        float ej = 0.f, fj = 0.f, kqs = 0.f;
#pragma unroll
        for (int w = 0; w < Sh::NW; ++w) {
            ej += red_e[w][tid];
            fj += red_f[w][tid];
            kqs += red_kq[w];
        }
        const float vj = load_f32(v + gi * DV + tid);
        const float wj = bt * (vj - alpha * ej);
        w_sh[tid] = wj;
        store_f32(o + gi * DV + tid, scale * (alpha * fj + kqs * wj));
    }
    __syncthreads();

    const f32x4 w4 = reinterpret_cast<const f32x4 *>(w_sh)[cg];
#pragma unroll
    for (int m = 0; m < Sh::RPT; ++m) {
        f32x4 x = s[m];
        x.x = alpha * x.x + kr[m] * w4.x;
        x.y = alpha * x.y + kr[m] * w4.y;
        x.z = alpha * x.z + kr[m] * w4.z;
        x.w = alpha * x.w + kr[m] * w4.w;
        __builtin_nontemporal_store(x, &S[(rg + Sh::R * m) * Sh::CG + cg]);
    }
}

template <int DK, int DV, typename TI, typename TO>
hipError_t launch_typed(const DecodeArgs &a) {
    using Sh = DecodeShape<DK, DV>;
    const unsigned nblk = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hv);
    hipLaunchKernelGGL((decode_kernel<DK, DV, TI, TO>), dim3(nblk), dim3(Sh::NT), 0, a.stream,
                       static_cast<const TI *>(a.q), static_cast<const TI *>(a.k),
                       static_cast<const TI *>(a.v), static_cast<const TI *>(a.beta),
                       static_cast<const TI *>(a.g), a.state, static_cast<TO *>(a.o), a.Hk, a.Hv,
                       a.scale);
    return hipGetLastError();
}

template <int DK, int DV> hipError_t launch_dims(const DecodeArgs &a) {
    if (a.in_dt == GDN_BF16)
        return a.out_dt == GDN_F32 ? launch_typed<DK, DV, bf16_t, float>(a)
                                   : launch_typed<DK, DV, bf16_t, bf16_t>(a);
    return a.out_dt == GDN_F32 ? launch_typed<DK, DV, float, float>(a)
                               : launch_typed<DK, DV, float, bf16_t>(a);
}

template <int DK> hipError_t launch_dk(const DecodeArgs &a) {
    switch (a.dv) {
    case 16: return launch_dims<DK, 16>(a);
    case 32: return launch_dims<DK, 32>(a);
    case 64: return launch_dims<DK, 64>(a);
    case 128: return launch_dims<DK, 128>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a) {
    if (a.B == 0) return hipSuccess;
    switch (a.dk) {
    case 16: return launch_dk<16>(a);
    case 32: return launch_dk<32>(a);
    case 64: return launch_dk<64>(a);
    case 128: return launch_dk<128>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
