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
// Both recurrences act on the state column by column (S_t's column j depends only on column j
// of S_{t-1}; dS_{t-1}'s column j only on column j of dS), so every (b, hv) chain is split into
// slices of SW <= 16 state columns, one workgroup each.  Only per-token scalars and row vectors
// need sums over all columns: each slice writes its parts of dq, dk (rows of S dO, dS w and
// X u), dbeta (u . w) and dg (<dS, X>, u . e), and a second kernel adds the slices (and the
// value heads of a grouped q/k head) up -- no atomics, so the results are deterministic.
//
// In a slice, thread (rg, cg) holds float4 column group cg of rows rg, rg + R, ...  The
// reverse walk needs every S_{t-1}: a forward pass stores the state every kBlk tokens
// (checkpoints), then, block by block from the end, the block's states are recomputed into a
// workspace buffer and walked back.  Each thread stores and reloads only its own elements, so
// these buffers need no barrier.  Per token one LDS-only barrier publishes the column sums
// (double-buffered by token parity).  Every token's inputs are loaded one token ahead, and the
// token loops have no branches (masked stores go through buffer resources whose range check
// drops them), so those loads stay in flight while the previous token is processed.
#include <stdlib.h>
#include <string.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlk = 64;                 // tokens between checkpoints
constexpr unsigned kOob = 0x7ffffff0u;   // a buffer offset past any range: the store is dropped

__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) {
    return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, size_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0,
                                             static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ void store1(float x, __amdgpu_buffer_rsrc_t r, unsigned off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, static_cast<int>(off), 0, 0);
}

template <int DK, int DV> struct BwdShape {
    static constexpr int SW = DV < 16 ? DV : 16;                 // state columns per slice
    static constexpr int NS = DV / SW;                           // slices per chain
    static constexpr int CG = SW / 4;                            // float4 groups per row
    static constexpr int R = DK < 256 / CG ? DK : 256 / CG;      // row groups
    static constexpr int RPT = DK / R;                           // rows per thread
    static constexpr int NT = CG * R;                            // threads
    static constexpr int NW = NT / 64;                           // wavefronts
    static_assert(NT % 64 == 0 && NT <= 256 && RPT * R == DK, "backward block shape");
};

// One token's inputs, in their stored types (converted where they are used, so that the loads
// of the next token stay in flight).
template <int RPT, typename TI, typename TD> struct TokIn {
    TI kr[RPT], qr[RPT];
    TI v4[4];
    TD o4[4];
    TI g, beta;
    f32x4 X[RPT];
};

template <typename T> __device__ __forceinline__ float cvt(T x);
template <> __device__ __forceinline__ float cvt<float>(float x) { return x; }
template <> __device__ __forceinline__ float cvt<bf16_t>(bf16_t x) { return bf16_to_f32(x); }

template <int DK, int DV, typename TI, typename TD>
__global__ void __launch_bounds__((BwdShape<DK, DV>::NT))
backward_kernel(const TI *__restrict__ q, const TI *__restrict__ k, const TI *__restrict__ v,
                const TI *__restrict__ beta, const TI *__restrict__ g,
                const float *__restrict__ s0, const TD *__restrict__ dO,
                const float *__restrict__ dST, float *__restrict__ dq_part,
                float *__restrict__ dk_part, float *__restrict__ dv_out,
                float *__restrict__ db_part, float *__restrict__ dg_part,
                float *__restrict__ dS0, float *__restrict__ ckpt, float *__restrict__ hist,
                int T, int Hk, int Hv, float scale) {
    using Sh = BwdShape<DK, DV>;
    constexpr int RPT = Sh::RPT, R = Sh::R, CG = Sh::CG, NW = Sh::NW, SW = Sh::SW, NS = Sh::NS;
    __shared__ f32x4 red_a[2][NW][64], red_b[2][NW][64];
    __shared__ float red_s[2][NW][64];

    const int chain = blockIdx.x / NS, sl = blockIdx.x - chain * NS;  // chain = b * Hv + hv
    const int b = chain / Hv, hv = chain - b * Hv, hq = hv / (Hv / Hk);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % CG, rg = tid / CG;
    const int nblk = (T + kBlk - 1) / kBlk;
    constexpr size_t SS = static_cast<size_t>(DK) * SW;  // floats per slice state
    auto elem = [&](int m) { return (rg + R * m) * CG + cg; };                 // in the slice
    auto gelem = [&](int m) { return ((rg + R * m) * DV + SW * sl) / 4 + cg; };  // full state
    f32x4 *ck = reinterpret_cast<f32x4 *>(ckpt + static_cast<size_t>(blockIdx.x) * nblk * SS);
    f32x4 *hs = reinterpret_cast<f32x4 *>(hist + static_cast<size_t>(blockIdx.x) * (kBlk + 1) * SS);
    const int col0 = SW * sl + 4 * cg;  // first state column of this thread
    int par = 0;

    // sum over the lanes of this wavefront that hold the same columns (lanes CG apart)
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
    // the whole-column sums of one or two partials (and of one scalar), through LDS: every
    // lane writes its own slot, lane cg's slot of each wavefront is read back (one barrier)
    auto publish = [&](f32x4 a, f32x4 c, float s, f32x4 &ra, f32x4 &rc, float &rs, bool two) {
        a = col_reduce(a);
        red_a[par][wave][lane] = a;
        if (two) {
            c = col_reduce(c);
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) s += __shfl_xor(s, off);
            red_b[par][wave][lane] = c;
            red_s[par][wave][lane] = s;
        }
        lds_barrier();
        ra = rc = f32x4{0.f, 0.f, 0.f, 0.f};
        rs = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            ra += red_a[par][w][cg];
            if (two) {
                rc += red_b[par][w][cg];
                rs += red_s[par][w][0];
            }
        }
        par ^= 1;  // the other buffer next time: a slow wave may still be reading this one
    };

    using Tok = TokIn<RPT, TI, TD>;
    // inputs of token t (X from hist row i when rev)
    auto fetch = [&](Tok &o, int t, int i, bool rev) {
        const size_t bt = static_cast<size_t>(b) * T + t;
        const TI *kt = k + (bt * Hk + hq) * DK;
        const TI *qt = q + (bt * Hk + hq) * DK;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            o.kr[m] = kt[rg + R * m];
            if (rev) o.qr[m] = qt[rg + R * m];
        }
        const TI *vt = v + (bt * Hv + hv) * DV + col0;
#pragma unroll
        for (int j = 0; j < 4; ++j) o.v4[j] = vt[j];
        if (rev) {
            const TD *ot = dO + (bt * Hv + hv) * DV + col0;
#pragma unroll
            for (int j = 0; j < 4; ++j) o.o4[j] = ot[j];
#pragma unroll
            for (int m = 0; m < RPT; ++m) o.X[m] = hs[static_cast<size_t>(i) * (SS / 4) + elem(m)];
        }
        o.g = g[bt * Hv + hv];
        o.beta = beta[bt * Hv + hv];
    };

    f32x4 s[RPT];
    if (s0 != nullptr) {
        const f32x4 *S0 = reinterpret_cast<const f32x4 *>(s0 + chain * static_cast<size_t>(DK) * DV);
#pragma unroll
        for (int m = 0; m < RPT; ++m) s[m] = S0[gelem(m)];
    } else {
#pragma unroll
        for (int m = 0; m < RPT; ++m) s[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // one forward token: s = alpha s + k (beta (v - alpha s^T k))^T
    auto forward_token = [&](const Tok &o) {
        float kr[RPT];
        f32x4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            kr[m] = cvt(o.kr[m]);
            e += kr[m] * s[m];
        }
        const float alpha = expf(cvt(o.g)), bt_ = cvt(o.beta);
        const f32x4 v4 = {cvt(o.v4[0]), cvt(o.v4[1]), cvt(o.v4[2]), cvt(o.v4[3])};
        f32x4 ea, unused;
        float us;
        publish(e, e, 0.f, ea, unused, us, false);
        const f32x4 w4 = bt_ * (v4 - alpha * ea);
#pragma unroll
        for (int m = 0; m < RPT; ++m) s[m] = alpha * s[m] + kr[m] * w4;
    };
    // tokens t0 .. t1-1 forward, prefetching one token ahead; after each, store(i, s)
    auto forward_run = [&](int t0, int t1, auto &&store) {
        Tok cur, nxt;
        fetch(nxt, t0, 0, false);
        for (int t = t0; t < t1; ++t) {
            cur = nxt;
            fetch(nxt, min(t + 1, t1 - 1), 0, false);
            __builtin_amdgcn_sched_barrier(0);  // keep the next token's loads here
            forward_token(cur);
            store(t - t0, s);
        }
    };

    // ---- forward pass: checkpoints at the start of every block
    for (int blk = 0; blk < nblk; ++blk) {
#pragma unroll
        for (int m = 0; m < RPT; ++m) ck[static_cast<size_t>(blk) * (SS / 4) + elem(m)] = s[m];
        forward_run(blk * kBlk, min(T, (blk + 1) * kBlk), [](int, const f32x4 *) {});
    }

    // ---- reverse pass
    f32x4 d[RPT];
    if (dST != nullptr) {
        const f32x4 *D = reinterpret_cast<const f32x4 *>(dST + chain * static_cast<size_t>(DK) * DV);
#pragma unroll
        for (int m = 0; m < RPT; ++m) d[m] = D[gelem(m)];
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
        forward_run(t0, t0 + len, [&](int i, const f32x4 *st) {
#pragma unroll
            for (int m = 0; m < RPT; ++m) hs[static_cast<size_t>(i + 1) * (SS / 4) + elem(m)] = st[m];
        });
        // this block's output rows, through buffer resources (masked lanes are dropped)
        const size_t row0 = (static_cast<size_t>(b) * T + t0) * Hv + hv;  // (b, t0, hv)
        const __amdgpu_buffer_rsrc_t rq = rsrc(dq_part + (row0 * NS + sl) * DK,
                                               static_cast<size_t>(len) * Hv * NS * DK * 4);
        const __amdgpu_buffer_rsrc_t rk = rsrc(dk_part + (row0 * NS + sl) * DK,
                                               static_cast<size_t>(len) * Hv * NS * DK * 4);
        const __amdgpu_buffer_rsrc_t rv = rsrc(dv_out + row0 * DV + SW * sl,
                                               static_cast<size_t>(len) * Hv * DV * 4);
        const __amdgpu_buffer_rsrc_t rb = rsrc(db_part + row0 * NS + sl,
                                               static_cast<size_t>(len) * Hv * NS * 4);
        const __amdgpu_buffer_rsrc_t rgr = rsrc(dg_part + row0 * NS + sl,
                                                static_cast<size_t>(len) * Hv * NS * 4);
        // s = H[len] = S after the block's last token; walk back, inputs one token ahead
        Tok cur, nxt;
        fetch(nxt, t0 + len - 1, len - 1, true);
        for (int i = len - 1; i >= 0; --i) {
            cur = nxt;
            fetch(nxt, t0 + max(i - 1, 0), max(i - 1, 0), true);
            __builtin_amdgcn_sched_barrier(0);  // keep the next token's loads here
            float kr[RPT], qr[RPT];
#pragma unroll
            for (int m = 0; m < RPT; ++m) { kr[m] = cvt(cur.kr[m]); qr[m] = cvt(cur.qr[m]); }
            const float alpha = expf(cvt(cur.g)), bt_ = cvt(cur.beta);
            const f32x4 v4 = {cvt(cur.v4[0]), cvt(cur.v4[1]), cvt(cur.v4[2]), cvt(cur.v4[3])};
            const f32x4 o4 = {cvt(cur.o4[0]), cvt(cur.o4[1]), cvt(cur.o4[2]), cvt(cur.o4[3])};
            const unsigned tq = static_cast<unsigned>(i) * Hv * NS * DK;  // token i's dq/dk row
            const unsigned tb = static_cast<unsigned>(i) * Hv * NS;       // its dbeta/dg entry
            // dq_t = scale S_t dO_t (S_t = s), then the read-out's share of dS
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const float r = row_reduce(dot4(s[m], o4));
                store1(scale * r, rq, cg == 0 ? (tq + rg + R * m) * 4u : kOob);
                d[m] += (scale * qr[m]) * o4;
            }
            // column sums e = X^T k, u = dS^T k and the full sum <dS, X>
            f32x4 e = {0.f, 0.f, 0.f, 0.f}, u = e;
            float dsx = 0.f;
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                e += kr[m] * cur.X[m];
                u += kr[m] * d[m];
                dsx += dot4(d[m], cur.X[m]);
            }
            f32x4 ea, ua;
            float dsxa;
            publish(e, u, dsx, ea, ua, dsxa, true);
            const f32x4 w4 = v4 - alpha * ea;
            // dk_t = beta dS w - alpha beta X u
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const float r1 = row_reduce(dot4(d[m], w4));
                const float r2 = row_reduce(dot4(cur.X[m], ua));
                store1(bt_ * r1 - alpha * bt_ * r2, rk, cg == 0 ? (tq + rg + R * m) * 4u : kOob);
            }
            // dv, dbeta, dg (this slice's columns) from the lanes of row group 0
            const f32x4 dv4 = bt_ * ua;
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, dv4), rv,
                static_cast<int>(rg == 0 ? (static_cast<unsigned>(i) * Hv * DV + 4 * cg) * 4u : kOob),
                0, 0);
            const float ub = row_reduce(dot4(ua, w4)), ue = row_reduce(dot4(ua, ea));
            const bool one = rg == 0 && cg == 0;
            store1(ub, rb, one ? tb * 4u : kOob);
            store1(alpha * (dsxa - bt_ * ue), rgr, one ? tb * 4u : kOob);
            // dS_{t-1} = alpha (dS - beta k u^T); the state walks back one token
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                d[m] = alpha * (d[m] - (bt_ * kr[m]) * ua);
                s[m] = cur.X[m];
            }
        }
    }
    if (dS0 != nullptr) {
        f32x4 *D0 = reinterpret_cast<f32x4 *>(dS0 + chain * static_cast<size_t>(DK) * DV);
#pragma unroll
        for (int m = 0; m < RPT; ++m) D0[gelem(m)] = d[m];
    }
}

// out[r][h][i] = sum_j part[((r H + h) M + j) W + i]: the M = (value heads per q/k head) x
// (slices) parts of dq and dk (W = dk), or the slices of dbeta and dg (W = 1)
__global__ void part_sum_kernel(const float *__restrict__ part, float *__restrict__ out,
                                size_t n, int M, int W) {
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x) {
        const size_t rh = i / W, c = i - rh * W;
        const float *p = part + rh * M * W + c;
        float acc = 0.f;
        for (int j = 0; j < M; ++j) acc += p[static_cast<size_t>(j) * W];
        out[i] = acc;
    }
}

}  // namespace

hipError_t launch_part_sum(const float *part, float *out, size_t n, int M, int W,
                           hipStream_t st) {
    if (n == 0) return hipSuccess;  // T = 0: nothing to sum (and no empty grid)
    const size_t nb0 = (n + 255) / 256;
    const unsigned nb = static_cast<unsigned>(nb0 < 8192 ? nb0 : 8192);
    hipLaunchKernelGGL(part_sum_kernel, dim3(nb), dim3(256), 0, st, part, out, n, M, W);
    return hipGetLastError();
}

namespace {

// workspace: checkpoints, block history, then (when a sum is needed) the parts of dq, dk
// (rows x Hv x NS x dk) and of dbeta, dg (rows x Hv x NS)
struct BwdLayout {
    size_t ckpt, hist, dq, dk, db, dg, total;
};
BwdLayout bwd_layout(int B, int T, int Hk, int Hv, int dk, int dv) {
    const int NS = dv < 16 ? 1 : dv / 16;
    const size_t chains = static_cast<size_t>(B) * Hv;
    const size_t nblk = (static_cast<size_t>(T) + kBlk - 1) / kBlk;
    const size_t SS = static_cast<size_t>(dk) * dv;  // all slices of a chain
    const size_t rows = static_cast<size_t>(B) * T;
    BwdLayout L;
    size_t o = 0;
    L.ckpt = o; o += chains * nblk * SS * 4;
    L.hist = o; o += chains * (kBlk + 1) * SS * 4;
    L.dq = L.dk = L.db = L.dg = 0;
    if (NS * (Hv / Hk) > 1) {
        L.dq = o; o += rows * Hv * NS * dk * 4;
        L.dk = o; o += rows * Hv * NS * dk * 4;
    }
    if (NS > 1) {
        L.db = o; o += rows * Hv * NS * 4;
        L.dg = o; o += rows * Hv * NS * 4;
    }
    L.total = o;
    return L;
}

template <int DK, int DV, typename TI, typename TD> hipError_t launch_typed(const BackwardArgs &a) {
    using Sh = BwdShape<DK, DV>;
    constexpr int NS = Sh::NS;
    const int G = a.Hv / a.Hk;
    const size_t chains = static_cast<size_t>(a.B) * a.Hv;
    const BwdLayout L = bwd_layout(a.B, a.T, a.Hk, a.Hv, DK, DV);
    unsigned char *ws = static_cast<unsigned char *>(a.ws);
    float *ckpt = reinterpret_cast<float *>(ws + L.ckpt);
    float *hist = reinterpret_cast<float *>(ws + L.hist);
    const bool qsum = NS * G > 1, bsum = NS > 1;
    float *dq_part = qsum ? reinterpret_cast<float *>(ws + L.dq) : a.dq;
    float *dk_part = qsum ? reinterpret_cast<float *>(ws + L.dk) : a.dk;
    float *db_part = bsum ? reinterpret_cast<float *>(ws + L.db) : a.dbeta;
    float *dg_part = bsum ? reinterpret_cast<float *>(ws + L.dg) : a.dg;
    hipLaunchKernelGGL((backward_kernel<DK, DV, TI, TD>), dim3(static_cast<unsigned>(chains * NS)),
                       dim3(Sh::NT), 0, a.stream, static_cast<const TI *>(a.q),
                       static_cast<const TI *>(a.k), static_cast<const TI *>(a.v),
                       static_cast<const TI *>(a.beta), static_cast<const TI *>(a.g), a.s0,
                       static_cast<const TD *>(a.dO), a.dST, dq_part, dk_part, a.dv, db_part,
                       dg_part, a.dS0, ckpt, hist, a.T, a.Hk, a.Hv, a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t rows = static_cast<size_t>(a.B) * a.T;
    if (qsum) {
        e = launch_part_sum(dq_part, a.dq, rows * a.Hk * DK, NS * G, DK, a.stream);
        if (e == hipSuccess) e = launch_part_sum(dk_part, a.dk, rows * a.Hk * DK, NS * G, DK, a.stream);
    }
    if (e == hipSuccess && bsum) {
        e = launch_part_sum(db_part, a.dbeta, rows * a.Hv, NS, 1, a.stream);
        if (e == hipSuccess) e = launch_part_sum(dg_part, a.dg, rows * a.Hv, NS, 1, a.stream);
    }
    return e;
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
    const size_t tok = bwd_layout(B, T, Hk, Hv, dk, dv).total;
    if ((dk == 64 || dk == 128) && (dv == 64 || dv == 128)) {
        const size_t ch = backward_chunk_workspace(B, T, Hk, Hv, dk, dv);
        return ch > tok ? ch : tok;  // enough for either path
    }
    return tok;
}

// GDN_BWD=token pins the token-recurrent path (for comparisons); otherwise the chunk-parallel
// path runs wherever it supports the sizes.
hipError_t launch_backward(const BackwardArgs &a) {
    if (a.B == 0) return hipSuccess;
    const char *env = getenv("GDN_BWD");
    const bool token = env != nullptr && strcmp(env, "token") == 0;
    if (!token && backward_chunk_supports(a)) return launch_backward_chunk(a);
    switch (a.dk_) {
    case 16: return launch_dk<16>(a);
    case 32: return launch_dk<32>(a);
    case 64: return launch_dk<64>(a);
    case 128: return launch_dk<128>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
