// decode.hip -- decode steps of the gated delta rule as a single streaming pass over the
// fp32 state (explainer page "論文解説: Qwen3.8-Next の設計", ta-paperlens.web.app, section
// "GDNの中身", Eq. (1), applied to T = 1 .. 16 new tokens per sequence: T = 1 is the plain
// decode step; T > 1 applies several tokens, e.g. drafted ones being verified, with one read
// and one write of the state for all of them).
//
// With e = S^T k and f = S^T q taken from the OLD state, one token of Eq. (1) is
//     w  = beta (v - alpha e)
//     S' = alpha S + k w^T
//     o  = scale S'^T q = scale (alpha f + (k^T q) w)
// so both dk-reductions come from one read of S, and S' is written while the slice is still
// in registers: exactly one read and one write of every state byte per call, whatever T.
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

// Workgroup barrier that orders LDS only: it does not wait for this thread's global loads
// or stores (a __syncthreads would wait for every token's output stores).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int DK, int DV> struct DecodeShape {
    static constexpr int CG = DV / 4;                                  // float4 groups per row
    static constexpr int RPT = (DK * DV / 1024) > 0 ? DK * DV / 1024 : 1;  // rows per thread
    static constexpr int R = DK / RPT;                                 // row groups
    static constexpr int NT = CG * R;                                  // threads (64..256)
    static constexpr int NW = NT / 64;                                 // wavefronts
    static_assert(NT % 64 == 0 && NT <= 256, "decode block shape");
};

// Tokens whose inputs are staged in LDS together (one burst of loads per block of tokens).
constexpr int kTokBlock = 8;

template <int DK, int DV, typename TI, typename TO, bool MULTI>
__global__ void __launch_bounds__((DecodeShape<DK, DV>::NT))
decode_kernel(const TI *__restrict__ q, const TI *__restrict__ k, const TI *__restrict__ v,
              const TI *__restrict__ beta, const TI *__restrict__ g, const float *state_in,
              float *state_out, TO *__restrict__ o, int T, int Hk, int Hv, float scale,
              unsigned flags) {
    using Sh = DecodeShape<DK, DV>;
    // per-wavefront partial sums, double-buffered by token parity: each thread forms w for
    // its own four columns from them, so one barrier per token suffices (token t + 2 reuses a
    // buffer only after every thread has passed token t + 1's barrier, i.e. finished reading)
    __shared__ __attribute__((aligned(16))) float red_e[2][Sh::NW][DV];
    __shared__ __attribute__((aligned(16))) float red_f[2][Sh::NW][DV];
    __shared__ float red_kq[2][Sh::NW];
    // the current block of tokens' inputs, fp32
    __shared__ __attribute__((aligned(16))) float t_k[kTokBlock][DK], t_q[kTokBlock][DK],
        t_v[kTokBlock][DV];
    __shared__ float t_alpha[kTokBlock], t_beta[kTokBlock];

    const int head = blockIdx.x;  // b * Hv + hv
    const int b = head / Hv, hv = head - b * Hv;
    const int hq = hv / (Hv / Hk);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % Sh::CG, rg = tid / Sh::CG;

    // token t of sequence b: q/k row (b*T + t)*Hk + hq, v/o row (b*T + t)*Hv + hv
    const size_t tok0 = static_cast<size_t>(b) * T;

    // the state tile of this thread; every element is read before any is written, so the
    // update may be in place (state_out == state_in)
    f32x4 s[Sh::RPT];
    const size_t sbase = static_cast<size_t>(head) * DK * DV;
    if (state_in != nullptr) {
        const f32x4 *Si = reinterpret_cast<const f32x4 *>(state_in + sbase);
#pragma unroll
        for (int m = 0; m < Sh::RPT; ++m) s[m] = Si[(rg + Sh::R * m) * Sh::CG + cg];
    } else {
#pragma unroll
        for (int m = 0; m < Sh::RPT; ++m) s[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int t0 = 0; t0 < T; t0 += kTokBlock) {
        const int nt = MULTI ? min(kTokBlock, T - t0) : 1;
        // a single token reads its inputs straight into registers (no staging barrier)
        float kr1[Sh::RPT], qr1[Sh::RPT], a1 = 0.f, b1 = 0.f;
        f32x4 v1 = {0.f, 0.f, 0.f, 0.f};  // columns 4 cg .. 4 cg + 3
        if constexpr (!MULTI) {
#pragma unroll
            for (int m = 0; m < Sh::RPT; ++m) {
                const size_t off = (tok0 * Hk + hq) * DK + rg + Sh::R * m;
                kr1[m] = load_f32(k + off);
                qr1[m] = load_f32(q + off);
            }
            const size_t gi = tok0 * Hv + hv;
            a1 = expf(log_alpha_from_input(load_f32(g + gi), flags));
            b1 = beta_from_input(load_f32(beta + gi), flags);
#pragma unroll
            for (int c = 0; c < 4; ++c) v1[c] = load_f32(v + gi * DV + 4 * cg + c);
        }
        // ---- stage the block's inputs (all loads of the block in flight together)
        if constexpr (MULTI) {
        if (t0 > 0) lds_barrier();  // the previous block's last token is done reading t_*
        for (int i = tid; i < nt * DK; i += Sh::NT) {
            const int tt = i / DK, c = i - tt * DK;
            const size_t off = ((tok0 + t0 + tt) * Hk + hq) * DK + c;
            t_k[tt][c] = load_f32(k + off);
            t_q[tt][c] = load_f32(q + off);
        }
        for (int i = tid; i < nt * DV; i += Sh::NT) {
            const int tt = i / DV, c = i - tt * DV;
            t_v[tt][c] = load_f32(v + ((tok0 + t0 + tt) * Hv + hv) * DV + c);
        }
        if (tid < nt) {
            const size_t gi = (tok0 + t0 + tid) * Hv + hv;
            t_alpha[tid] = expf(log_alpha_from_input(load_f32(g + gi), flags));
            t_beta[tid] = beta_from_input(load_f32(beta + gi), flags);
        }
        lds_barrier();
        if (flags & GDN_QK_L2NORM) {
            // normalise the staged k and q rows: 16 threads per row
            const int grp = tid >> 4, l16 = tid & 15;
            for (int pr = grp; pr < 2 * nt; pr += Sh::NT / 16) {
                float *row = (pr & 1) ? t_q[pr >> 1] : t_k[pr >> 1];
                float ss = 0.f;
                for (int i = l16; i < DK; i += 16) ss += row[i] * row[i];
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) ss += __shfl_xor(ss, off);
                const float r = inv_norm_from_sumsq(ss);
                for (int i = l16; i < DK; i += 16) row[i] *= r;
            }
            lds_barrier();
        }
        }

        for (int tt = 0; tt < nt; ++tt) {
            float kr[Sh::RPT], qr[Sh::RPT];
#pragma unroll
            for (int m = 0; m < Sh::RPT; ++m) {
                kr[m] = MULTI ? t_k[tt][rg + Sh::R * m] : kr1[m];
                qr[m] = MULTI ? t_q[tt][rg + Sh::R * m] : qr1[m];
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
            const int pb = (t0 + tt) & 1;
            if (lane < Sh::CG) {
                *reinterpret_cast<f32x4 *>(&red_e[pb][wave][4 * cg]) = e;
                *reinterpret_cast<f32x4 *>(&red_f[pb][wave][4 * cg]) = f;
            }
            if (lane == 0) red_kq[pb][wave] = kq;
            lds_barrier();

            // w for this thread's columns (every row group forms the same values)
            const float alpha = MULTI ? t_alpha[tt] : a1;
            const float bt = MULTI ? t_beta[tt] : b1;
            const f32x4 vv = MULTI ? *reinterpret_cast<const f32x4 *>(&t_v[tt][4 * cg]) : v1;
            f32x4 ej = {0.f, 0.f, 0.f, 0.f}, fj = ej;
            float kqs = 0.f;
#pragma unroll
            for (int w = 0; w < Sh::NW; ++w) {
                ej += *reinterpret_cast<const f32x4 *>(&red_e[pb][w][4 * cg]);
                fj += *reinterpret_cast<const f32x4 *>(&red_f[pb][w][4 * cg]);
                kqs += red_kq[pb][w];
            }
            f32x4 w4;
#pragma unroll
            for (int c = 0; c < 4; ++c) w4[c] = bt * (vv[c] - alpha * ej[c]);
            if (rg == 0) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    store_f32(o + ((tok0 + t0 + tt) * Hv + hv) * DV + 4 * cg + c,
                              scale * (alpha * fj[c] + kqs * w4[c]));
            }
#pragma unroll
            for (int m = 0; m < Sh::RPT; ++m) {
                s[m].x = alpha * s[m].x + kr[m] * w4.x;
                s[m].y = alpha * s[m].y + kr[m] * w4.y;
                s[m].z = alpha * s[m].z + kr[m] * w4.z;
                s[m].w = alpha * s[m].w + kr[m] * w4.w;
            }
        }
    }
    f32x4 *So = reinterpret_cast<f32x4 *>(state_out + sbase);
#pragma unroll
    for (int m = 0; m < Sh::RPT; ++m)
        __builtin_nontemporal_store(s[m], &So[(rg + Sh::R * m) * Sh::CG + cg]);
}

template <int DK, int DV, typename TI, typename TO>
hipError_t launch_typed(const DecodeArgs &a) {
    using Sh = DecodeShape<DK, DV>;
    const unsigned nblk = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hv);
    // one token without normalisation reads its inputs into registers; otherwise through LDS
    const bool staged = a.T > 1 || (a.flags & GDN_QK_L2NORM);
    auto kern = staged ? decode_kernel<DK, DV, TI, TO, true> : decode_kernel<DK, DV, TI, TO, false>;
    hipLaunchKernelGGL(kern, dim3(nblk), dim3(Sh::NT), 0, a.stream,
                       static_cast<const TI *>(a.q), static_cast<const TI *>(a.k),
                       static_cast<const TI *>(a.v), static_cast<const TI *>(a.beta),
                       static_cast<const TI *>(a.g), a.state_in, a.state, static_cast<TO *>(a.o),
                       a.T, a.Hk, a.Hv, a.scale, a.flags);
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
    if (a.B == 0 || a.Hv == 0) return hipSuccess;
    switch (a.dk) {
    case 16: return launch_dk<16>(a);
    case 32: return launch_dk<32>(a);
    case 64: return launch_dk<64>(a);
    case 128: return launch_dk<128>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
