// backward.hip -- gradients of the gated delta rule (explainer page "論文解説: Qwen3.8-Next
// の設計", ta-paperlens.web.app, section "GDNの中身", Eq. (1)), token by token in reverse.
//
// Forward, per token:  X = S_{t-1},  e = X^T k,  S_t = alpha X + k (beta (v - alpha e))^T,
// o_t = scale S_t^T q.  Reverse, with dS the gradient w.r.t. S_t:
//     dq_t = scale S_t dO_t ;   dS += scale q dO_t^T ;   u = dS^T k ;   w = v - alpha e
//     dv_t = beta u ;   dbeta_t = u . w ;   dg_t = alpha (<dS, X> - beta u . e)
//     dk_t = beta dS w - alpha beta X u ;   dS_{t-1} = alpha (dS - beta k u^T)
// (dg is the gradient w.r.t. g = log alpha.)
//
// One workgroup per (b, hv) chain, the state's layout as in the decode kernel: thread
// (rg, cg) holds float4 column group cg of rows rg, rg + R, ...  The reverse walk needs every
// S_{t-1}: a forward pass stores the state every kBlk tokens (checkpoints), then, block by block
// from the end, the block's states are recomputed into a workspace buffer and walked back.
// Each thread stores and reloads only its own elements, so these buffers need no barrier.
// Per token one LDS-only barrier publishes the column partials (double-buffered by token
// parity).  dq and dk of a grouped q/k head are written per value head and summed afterwards
// by a second kernel (no atomics: deterministic).
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlk = 64;  // tokens between checkpoints

__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) {
    return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

template <int DK, int DV> struct BwdShape {
    static constexpr int CG = DV / 4;                                  // float4 groups per row
    static constexpr int RPT = (DK * DV / 1024) > 0 ? DK * DV / 1024 : 1;  // rows per thread
    static constexpr int R = DK / RPT;                                 // row groups
    static constexpr int NT = CG * R;                                  // threads
    static constexpr int NW = NT / 64;                                 // wavefronts
    static_assert(NT % 64 == 0 && NT <= 256 && CG <= 32, "backward block shape");
};

template <int DK, int DV, typename TI, typename TD>
__global__ void __launch_bounds__((BwdShape<DK, DV>::NT))
backward_kernel(const TI *__restrict__ q, const TI *__restrict__ k, const TI *__restrict__ v,
                const TI *__restrict__ beta, const TI *__restrict__ g,
                const float *__restrict__ s0, const TD *__restrict__ dO,
                const float *__restrict__ dST, float *__restrict__ dq_part,
                float *__restrict__ dk_part, float *__restrict__ dv_out,
                float *__restrict__ dbeta, float *__restrict__ dg, float *__restrict__ dS0,
                float *__restrict__ ckpt, float *__restrict__ hist, int T, int Hk, int Hv,
                float scale) {
    using Sh = BwdShape<DK, DV>;
    constexpr int RPT = Sh::RPT, R = Sh::R, CG = Sh::CG, NW = Sh::NW;
    __shared__ float red_a[2][NW][DV], red_b[2][NW][DV], red_s[2][NW];

    const int chain = blockIdx.x;  // b * Hv + hv
    const int b = chain / Hv, hv = chain - b * Hv, hq = hv / (Hv / Hk);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % CG, rg = tid / CG;
    const int nblk = (T + kBlk - 1) / kBlk;
    constexpr size_t SS = static_cast<size_t>(DK) * DV;  // floats per state
    auto elem = [&](int m) { return (rg + R * m) * CG + cg; };  // f32x4 index in a state
    f32x4 *ck = reinterpret_cast<f32x4 *>(ckpt + static_cast<size_t>(chain) * nblk * SS);
    f32x4 *hs = reinterpret_cast<f32x4 *>(hist + static_cast<size_t>(chain) * (kBlk + 1) * SS);
    int par = 0;

    // sum of v over the lanes of this wavefront that hold the same columns (lanes CG apart)
    auto col_reduce = [&](f32x4 x) {
#pragma unroll
        for (int off = CG; off < 64; off <<= 1) {
            x.x += __shfl_xor(x.x, off); x.y += __shfl_xor(x.y, off);
            x.z += __shfl_xor(x.z, off); x.w += __shfl_xor(x.w, off);
        }
        return x;
    };
    // sum over the CG lanes that hold one row
    auto row_reduce = [&](float x) {
#pragma unroll
        for (int off = 1; off < CG; off <<= 1) x += __shfl_xor(x, off);
        return x;
    };
    // the whole-column sums of two partials, through LDS (one barrier)
    auto publish = [&](f32x4 a, f32x4 c, float s, f32x4 &ra, f32x4 &rc, float &rs) {
        a = col_reduce(a);
        c = col_reduce(c);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) s += __shfl_xor(s, off);
        if (lane < CG) {
            *reinterpret_cast<f32x4 *>(&red_a[par][wave][4 * cg]) = a;
            *reinterpret_cast<f32x4 *>(&red_b[par][wave][4 * cg]) = c;
        }
        if (lane == 0) red_s[par][wave] = s;
        lds_barrier();
        ra = rc = f32x4{0.f, 0.f, 0.f, 0.f};
        rs = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            ra += *reinterpret_cast<const f32x4 *>(&red_a[par][w][4 * cg]);
            rc += *reinterpret_cast<const f32x4 *>(&red_b[par][w][4 * cg]);
            rs += red_s[par][w];
        }
        par ^= 1;  // the other buffer next time: a slow wave may still be reading this one
    };

    f32x4 s[RPT];
    if (s0 != nullptr) {
        const f32x4 *S0 = reinterpret_cast<const f32x4 *>(s0 + chain * SS);
#pragma unroll
        for (int m = 0; m < RPT; ++m) s[m] = S0[elem(m)];
    } else {
#pragma unroll
        for (int m = 0; m < RPT; ++m) s[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // one forward token: s = alpha s + k (beta (v - alpha s^T k))^T
    auto forward_token = [&](int t) {
        const size_t bt = static_cast<size_t>(b) * T + t;
        const TI *kt = k + (bt * Hk + hq) * DK;
        float kr[RPT];
        f32x4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            kr[m] = load_f32(kt + rg + R * m);
            e += kr[m] * s[m];
        }
        const float alpha = expf(load_f32(g + bt * Hv + hv)), bt_ = load_f32(beta + bt * Hv + hv);
        const TI *vt = v + (bt * Hv + hv) * DV + 4 * cg;
        const f32x4 v4 = {load_f32(vt), load_f32(vt + 1), load_f32(vt + 2), load_f32(vt + 3)};
        f32x4 ea, unused;
        float us;
        publish(e, f32x4{0.f, 0.f, 0.f, 0.f}, 0.f, ea, unused, us);
        const f32x4 w4 = bt_ * (v4 - alpha * ea);
#pragma unroll
        for (int m = 0; m < RPT; ++m) s[m] = alpha * s[m] + kr[m] * w4;
    };

    // ---- forward pass: checkpoints at the start of every block
    for (int blk = 0; blk < nblk; ++blk) {
#pragma unroll
        for (int m = 0; m < RPT; ++m) ck[static_cast<size_t>(blk) * (SS / 4) + elem(m)] = s[m];
        const int t1 = min(T, (blk + 1) * kBlk);
        for (int t = blk * kBlk; t < t1; ++t) forward_token(t);
    }

    // ---- reverse pass
    f32x4 d[RPT];
    if (dST != nullptr) {
        const f32x4 *D = reinterpret_cast<const f32x4 *>(dST + chain * SS);
#pragma unroll
        for (int m = 0; m < RPT; ++m) d[m] = D[elem(m)];
    } else {
#pragma unroll
        for (int m = 0; m < RPT; ++m) d[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int blk = nblk - 1; blk >= 0; --blk) {
        const int t0 = blk * kBlk, len = min(kBlk, T - t0);
        // recompute the block's states H[0 .. len] (H[i] = state before token t0 + i)
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            s[m] = ck[static_cast<size_t>(blk) * (SS / 4) + elem(m)];
            hs[elem(m)] = s[m];
        }
        for (int i = 0; i < len; ++i) {
            forward_token(t0 + i);
#pragma unroll
            for (int m = 0; m < RPT; ++m) hs[static_cast<size_t>(i + 1) * (SS / 4) + elem(m)] = s[m];
        }
        // s = H[len] = S after the block's last token
        for (int i = len - 1; i >= 0; --i) {
            const int t = t0 + i;
            const size_t bt = static_cast<size_t>(b) * T + t;
            f32x4 X[RPT];
#pragma unroll
            for (int m = 0; m < RPT; ++m) X[m] = hs[static_cast<size_t>(i) * (SS / 4) + elem(m)];
            const TI *kt = k + (bt * Hk + hq) * DK;
            const TI *qt = q + (bt * Hk + hq) * DK;
            float kr[RPT], qr[RPT];
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                kr[m] = load_f32(kt + rg + R * m);
                qr[m] = load_f32(qt + rg + R * m);
            }
            const float alpha = expf(load_f32(g + bt * Hv + hv)), bt_ = load_f32(beta + bt * Hv + hv);
            const TI *vt = v + (bt * Hv + hv) * DV + 4 * cg;
            const TD *dot_ = dO + (bt * Hv + hv) * DV + 4 * cg;
            const f32x4 v4 = {load_f32(vt), load_f32(vt + 1), load_f32(vt + 2), load_f32(vt + 3)};
            const f32x4 o4 = {load_f32(dot_), load_f32(dot_ + 1), load_f32(dot_ + 2), load_f32(dot_ + 3)};
            float *dqo = dq_part + (bt * Hv + hv) * DK;
            float *dko = dk_part + (bt * Hv + hv) * DK;
            // dq_t = scale S_t dO_t (S_t = s), then the read-out's share of dS
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const float r = row_reduce(dot4(s[m], o4));
                if (cg == 0) dqo[rg + R * m] = scale * r;
                d[m] += (scale * qr[m]) * o4;
            }
            // column sums e = X^T k, u = dS^T k and the full sum <dS, X>
            f32x4 e = {0.f, 0.f, 0.f, 0.f}, u = e;
            float dsx = 0.f;
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                e += kr[m] * X[m];
                u += kr[m] * d[m];
                dsx += dot4(d[m], X[m]);
            }
            f32x4 ea, ua;
            float dsxa;
            publish(e, u, dsx, ea, ua, dsxa);
            const f32x4 w4 = v4 - alpha * ea;
            // dk_t = beta dS w - alpha beta X u
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const float r1 = row_reduce(dot4(d[m], w4));
                const float r2 = row_reduce(dot4(X[m], ua));
                if (cg == 0) dko[rg + R * m] = bt_ * r1 - alpha * bt_ * r2;
            }
            // dv, dbeta, dg from the lanes of row group 0 (one copy of every column)
            if (rg == 0) {
                *reinterpret_cast<f32x4 *>(dv_out + (bt * Hv + hv) * DV + 4 * cg) = bt_ * ua;
                const float ub = row_reduce(dot4(ua, w4)), ue = row_reduce(dot4(ua, ea));
                if (cg == 0) {
                    dbeta[bt * Hv + hv] = ub;
                    dg[bt * Hv + hv] = alpha * (dsxa - bt_ * ue);
                }
            }
            // dS_{t-1} = alpha (dS - beta k u^T); the state walks back one token
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                d[m] = alpha * (d[m] - (bt_ * kr[m]) * ua);
                s[m] = X[m];
            }
        }
    }
    if (dS0 != nullptr) {
        f32x4 *D0 = reinterpret_cast<f32x4 *>(dS0 + chain * SS);
#pragma unroll
        for (int m = 0; m < RPT; ++m) D0[elem(m)] = d[m];
    }
}

// dq, dk of q/k head hq = the sum of the per-value-head parts of its G value heads
__global__ void group_sum_kernel(const float *__restrict__ part, float *__restrict__ out,
                                 size_t rows, int Hk, int G, int DK) {
    const size_t n = rows * Hk * DK;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x) {
        const size_t r = i / (static_cast<size_t>(Hk) * DK);
        const size_t rem = i - r * Hk * DK;
        const int hq = static_cast<int>(rem / DK), c = static_cast<int>(rem - static_cast<size_t>(hq) * DK);
        float acc = 0.f;
        for (int j = 0; j < G; ++j)
            acc += part[((r * Hk + hq) * G + j) * DK + c];
        out[i] = acc;
    }
}

template <int DK, int DV, typename TI, typename TD> hipError_t launch_typed(const BackwardArgs &a) {
    using Sh = BwdShape<DK, DV>;
    const int G = a.Hv / a.Hk;
    const size_t chains = static_cast<size_t>(a.B) * a.Hv;
    const int nblk = (a.T + kBlk - 1) / kBlk;
    const size_t SS = static_cast<size_t>(DK) * DV;
    unsigned char *ws = static_cast<unsigned char *>(a.ws);
    float *ckpt = reinterpret_cast<float *>(ws);
    float *hist = ckpt + chains * nblk * SS;
    float *dq_part = G == 1 ? a.dq : hist + chains * (kBlk + 1) * SS;
    float *dk_part = G == 1 ? a.dk : dq_part + static_cast<size_t>(a.B) * a.T * a.Hv * DK;
    hipLaunchKernelGGL((backward_kernel<DK, DV, TI, TD>), dim3(static_cast<unsigned>(chains)),
                       dim3(Sh::NT), 0, a.stream, static_cast<const TI *>(a.q),
                       static_cast<const TI *>(a.k), static_cast<const TI *>(a.v),
                       static_cast<const TI *>(a.beta), static_cast<const TI *>(a.g), a.s0,
                       static_cast<const TD *>(a.dO), a.dST, dq_part, dk_part, a.dv, a.dbeta,
                       a.dg, a.dS0, ckpt, hist, a.T, a.Hk, a.Hv, a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || G == 1) return e;
    const size_t rows = static_cast<size_t>(a.B) * a.T, n = rows * a.Hk * DK;
    const size_t nb0 = (n + 255) / 256;
    const unsigned nb = static_cast<unsigned>(nb0 < 4096 ? nb0 : 4096);
    hipLaunchKernelGGL(group_sum_kernel, dim3(nb), dim3(256), 0, a.stream, dq_part, a.dq, rows,
                       a.Hk, G, DK);
    hipLaunchKernelGGL(group_sum_kernel, dim3(nb), dim3(256), 0, a.stream, dk_part, a.dk, rows,
                       a.Hk, G, DK);
    return hipGetLastError();
}

template <int DK, int DV> hipError_t launch_dims(const BackwardArgs &a) {
    if (a.in_dt == GDN_BF16)
        return a.dout_dt == GDN_F32 ? launch_typed<DK, DV, bf16_t, float>(a)
                                    : launch_typed<DK, DV, bf16_t, bf16_t>(a);
    return a.dout_dt == GDN_F32 ? launch_typed<DK, DV, float, float>(a)
                                : launch_typed<DK, DV, float, bf16_t>(a);
}

template <int DK> hipError_t launch_dk(const BackwardArgs &a) {
    switch (a.dv_) {
    case 16: return launch_dims<DK, 16>(a);
    case 32: return launch_dims<DK, 32>(a);
    case 64: return launch_dims<DK, 64>(a);
    case 128: return launch_dims<DK, 128>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t backward_workspace(int B, int T, int Hk, int Hv, int dk, int dv) {
    const size_t chains = static_cast<size_t>(B) * Hv;
    const size_t nblk = (static_cast<size_t>(T) + kBlk - 1) / kBlk;
    const size_t SS = static_cast<size_t>(dk) * dv;
    size_t bytes = (chains * nblk * SS + chains * (kBlk + 1) * SS) * sizeof(float);
    if (Hv != Hk) bytes += 2 * static_cast<size_t>(B) * T * Hv * dk * sizeof(float);
    return bytes;
}

hipError_t launch_backward(const BackwardArgs &a) {
    if (a.B == 0) return hipSuccess;
    switch (a.dk_) {
    case 16: return launch_dk<16>(a);
    case 32: return launch_dk<32>(a);
    case 64: return launch_dk<64>(a);
    case 128: return launch_dk<128>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
