// backward_chunk.hip -- chunk-parallel gradients of the gated delta rule (explainer page
// "論文解説: Qwen3.8-Next の設計", ta-paperlens.web.app, section "GDNの中身", Eq. (1)).
//
// The chunked (WY/UT) form of the forward over a chunk of C tokens, with gamma = the cumulative
// sum of g inside the chunk, Gm = e^gamma, D_rs = e^(gamma_r - gamma_s) (s <= r):
//   A = strictly_lower(diag(beta) (K K^T o D)),  Tm = (I + A)^-1
//   U = Tm diag(beta) V,   W = Tm diag(beta Gm) K,   Delta = U - W S0
//   O = scale (diag(Gm) Q S0 + P Delta),  P = lower(Q K^T) o D
//   S_L = e^gamma_last S0 + Kt^T Delta,   Kt = diag(e^(gamma_last - gamma)) K
// Its reverse, with dS_L the gradient of the state at the chunk's end and dO' = scale dO:
//   dDelta = P^T dO' + Kt dS_L
//   dS0    = e^gamma_last dS_L + (Gm Q)^T dO' - W^T dDelta          (the chain over chunks)
// and, inside a chunk, the chain rule through every term above (dU = dDelta, dW = -dDelta S0^T,
// dTm = dU (beta V)^T + dW (beta Gm K)^T, dA = -strictly_lower(Tm^T dTm Tm^T), the decay
// matrices through gamma, gamma through a reverse cumulative sum into dg).
//
// Four kernels, all in fp32:
//   bprep_kernel  per (chain, chunk): Tm, U, W, Kt, Gm Q, P, e^gamma_last -> records
//   bscan_kernel  per (chain, 16 state columns): the forward chain of chunk-start states and,
//                 in the other half of the grid, the reverse chain of chunk-end gradients dS
//                 (the two are independent); both act on the state column by column
//   bgrad_kernel  per (chain, chunk): every input gradient of the chunk, the value dimension
//                 walked in slices of 32 columns, then the terms through Tm, the decays and
//                 gamma
// Padded rows of the last chunk (zero q, k, v, beta, g) contribute nothing, so every chunk
// uses the full-size formulas.  No atomics: deterministic.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kC = 64;    // tokens per chunk
constexpr int kNT = 256;  // threads per workgroup

__device__ __forceinline__ void bar() { __syncthreads(); }
// Workgroup barrier that waits only for LDS traffic, not for global loads still in flight
// (__syncthreads also waits for those, which would defeat a prefetch).
__device__ __forceinline__ void lds_bar() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// A uniform fp32 load through a buffer resource: a vector-memory load, so a load in flight
// does not hold up the LDS-only barrier (which also counts scalar loads).
__device__ __forceinline__ float vload1(const float *p) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p), 0, 4,
                                                                       0x00020000);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, 0));
}

// Register-tile product: acc[i][j] += sum_k A(row_i, k) B(k, col_j), row_i = ty + i NY,
// col_j = tx + j NX with (ty, tx) = (tid / NX, tid % NX) and NY = 256 / NX.  A(r, k) = A[r ar
// + k ak], B(k, c) = B[k bk + c bc] (strides allow transposed operands).
template <int TM, int TN, int NX>
__device__ __forceinline__ void mm(float (&acc)[TM][TN], const float *A, int ar, int ak,
                                   const float *B, int bk, int bc, int K) {
    constexpr int NY = kNT / NX;
    const int tid = threadIdx.x, ty = tid / NX, tx = tid % NX;
    const float *a0 = A + ty * ar;
    const float *b0 = B + tx * bc;
#pragma unroll 4
    for (int k = 0; k < K; ++k) {
        float a[TM], b[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = a0[i * NY * ar + k * ak];
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = b0[k * bk + j * NX * bc];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
}
template <int TM, int TN> __device__ __forceinline__ void zero(float (&a)[TM][TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) a[i][j] = 0.f;
}
// sum over the NX consecutive lanes of a tile row
template <int NX> __device__ __forceinline__ float row_sum(float x) {
#pragma unroll
    for (int off = 1; off < NX; off <<= 1) x += __shfl_xor(x, off);
    return x;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One 16 x 16 output block on the matrix cores in fp32: acc += A(16 x K) B(K x 16), with A(m, k)
// = A[m ar + k ak] and B(k, n) = B[k bk + n bc] (pointers already at the block's origin).
// Lane l supplies A(l%16, k + l/16) and B(k + l/16, l%16) and holds D(4 (l/16) + i, l%16).
__device__ __forceinline__ f32x4 mfma_blk(f32x4 acc, const float *A, int ar, int ak,
                                          const float *B, int bk, int bc, int K) {
    const int lane = threadIdx.x & 63, mi = lane & 15, kq = lane >> 4;
    const float *a = A + mi * ar + kq * ak;
    const float *b = B + kq * bk + mi * bc;
#pragma unroll 8
    for (int k = 0; k < K; k += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[k * ak], b[k * bk], acc, 0, 0, 0);
    return acc;
}

template <int DK, int DV> struct CB {
    // records per (chain, chunk), fp32, row-major
    static constexpr size_t OFF_W = 0;                          // [C][DK]
    static constexpr size_t OFF_U = OFF_W + kC * DK;            // [C][DV]
    static constexpr size_t OFF_KT = OFF_U + kC * DV;           // [C][DK]
    static constexpr size_t OFF_GQ = OFF_KT + kC * DK;          // [C][DK]
    static constexpr size_t OFF_P = OFF_GQ + kC * DK;           // [C][C]
    static constexpr size_t OFF_T = OFF_P + kC * kC;            // [C][C]
    static constexpr size_t OFF_EL = OFF_T + kC * kC;           // e^gamma_last
    static constexpr size_t REC = OFF_EL + 4;
    static constexpr int LK = DK + 1, LV = DV + 1, LC = kC + 1;  // padded LDS strides
    // 64 x DK register tiles
    static constexpr int NXK = DK / 4, TMK = kC / (kNT / NXK);
    static_assert((DK == 64 || DK == 128) && (DV == 64 || DV == 128), "chunked backward sizes");
};

// inclusive prefix sum over one wavefront (64 lanes)
__device__ __forceinline__ float wave_scan(float x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// Bulk copies with every load in flight before the first LDS store: a ROWS x COLS tile (COLS a
// multiple of 4) of a row-major fp32 matrix with row stride sld, as float4 per thread.
template <int ROWS, int COLS> struct Tile4 {
    static constexpr int N = ROWS * COLS / 4 / kNT;  // float4 per thread
    static_assert(N * 4 * kNT == ROWS * COLS, "tile must split evenly over the threads");
    float4 v[N];
    __device__ __forceinline__ void load(const float *src, int sld, float mul = 1.f) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = (i * kNT + threadIdx.x) * 4, r = idx / COLS, c = idx - r * COLS;
            v[i] = *reinterpret_cast<const float4 *>(src + static_cast<size_t>(r) * sld + c);
            v[i].x *= mul; v[i].y *= mul; v[i].z *= mul; v[i].w *= mul;
        }
    }
    // rows of a [.., H, D] input tensor (any stored type) at head h; zero past L
    template <typename TI>
    __device__ __forceinline__ void load_in(const TI *src, size_t row0, int H, int h, int c0,
                                            int D, int L, float mul = 1.f) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = (i * kNT + threadIdx.x) * 4, r = idx / COLS, c = idx - r * COLS;
            const TI *p = src + ((row0 + min(r, L - 1)) * H + h) * D + c0 + c;
            float4 x = load4(p);
            const float m = r < L ? mul : 0.f;
            v[i] = make_float4(m * x.x, m * x.y, m * x.z, m * x.w);
        }
    }
    __device__ __forceinline__ void store(float *dst, int ld) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = (i * kNT + threadIdx.x) * 4, r = idx / COLS, c = idx - r * COLS;
            float *d = dst + r * ld + c;
            d[0] = v[i].x; d[1] = v[i].y; d[2] = v[i].z; d[3] = v[i].w;
        }
    }
    __device__ static __forceinline__ float4 load4(const float *p) {
        return *reinterpret_cast<const float4 *>(p);
    }
    __device__ static __forceinline__ float4 load4(const bf16_t *p) {
        const uint2 u = *reinterpret_cast<const uint2 *>(p);
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
    }
};

// ---------------------------------------------------------------------------------------
template <int DK, int DV, typename TI>
__global__ void __launch_bounds__(kNT)
bprep_kernel(const TI *__restrict__ q, const TI *__restrict__ k, const TI *__restrict__ v,
             const TI *__restrict__ beta, const TI *__restrict__ g, float *__restrict__ rec,
             int T, int Hk, int Hv, int nch) {
    using F = CB<DK, DV>;
    constexpr int LK = F::LK, LV = F::LV, LC = F::LC;
    __shared__ float sK[kC * LK], sQ[kC * LK], sV[kC * LV], sA[kC * LC], sT[kC * LC];
    __shared__ float sgam[kC], sbeta[kC];
    const int chain = blockIdx.x / nch, c = blockIdx.x - chain * nch;
    const int b = chain / Hv, hv = chain - b * Hv, hq = hv / (Hv / Hk);
    const int t0 = c * kC, L = min(kC, T - t0);
    const size_t row0 = static_cast<size_t>(b) * T + t0;
    const int tid = threadIdx.x;
    float *R = rec + (static_cast<size_t>(chain) * nch + c) * F::REC;

    {
        Tile4<kC, DK> tk, tq;
        Tile4<kC, DV> tv;
        tk.load_in(k, row0, Hk, hq, 0, DK, L);
        tq.load_in(q, row0, Hk, hq, 0, DK, L);
        tv.load_in(v, row0, Hv, hv, 0, DV, L);
        float gg = 0.f, bb = 0.f;
        if (tid < 64 && tid < L) {
            gg = load_f32(g + (row0 + tid) * Hv + hv);
            bb = load_f32(beta + (row0 + tid) * Hv + hv);
        }
        tk.store(sK, LK);
        tq.store(sQ, LK);
        tv.store(sV, LV);
        if (tid < 64) {
            sgam[tid] = wave_scan(gg, tid);
            sbeta[tid] = bb;
        }
    }
    bar();
    const float glast = sgam[kC - 1];
    // K K^T and Q K^T (64 x 64 tiles), A and P
    {
        float kk[4][4], qk[4][4];
        zero(kk);
        zero(qk);
        mm<4, 4, 16>(kk, sK, LK, 1, sK, 1, LK, DK);
        mm<4, 4, 16>(qk, sQ, LK, 1, sK, 1, LK, DK);
        const int ty = tid / 16, tx = tid % 16;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = ty + 16 * i, s = tx + 16 * j;
                const float d = s <= r ? __expf(sgam[r] - sgam[s]) : 0.f;
                sA[r * LC + s] = s < r ? sbeta[r] * kk[i][j] * d : 0.f;
                R[F::OFF_P + r * kC + s] = qk[i][j] * d;
            }
    }
    bar();
    // Tm = (I + A)^-1 by forward substitution, one column per thread (rows in order)
    if (tid < kC) {
        const int j = tid;
        for (int r = 0; r < kC; ++r) {
            float x = r == j ? 1.f : 0.f;
            for (int s = j; s < r; ++s) x -= sA[r * LC + s] * sT[s * LC + j];
            sT[r * LC + j] = r >= j ? x : 0.f;
        }
    }
    // Gm Q and Kt to the records; then sQ <- beta Gm K (W's right factor), sV <- beta V
    for (int i = tid; i < kC * DK; i += kNT) {
        const int r = i / DK, cc = i - r * DK;
        R[F::OFF_GQ + i] = __expf(sgam[r]) * sQ[r * LK + cc];
        R[F::OFF_KT + i] = __expf(glast - sgam[r]) * sK[r * LK + cc];
    }
    bar();
    for (int i = tid; i < kC * DK; i += kNT) {
        const int r = i / DK, cc = i - r * DK;
        sQ[r * LK + cc] = sbeta[r] * __expf(sgam[r]) * sK[r * LK + cc];
    }
    for (int i = tid; i < kC * DV; i += kNT) {
        const int r = i / DV, cc = i - r * DV;
        sV[r * LV + cc] *= sbeta[r];
    }
    bar();
    // U = Tm (beta V), W = Tm (beta Gm K)
    {
        constexpr int NXV = DV / 4, TMV = kC / (kNT / NXV);
        float u[TMV][4];
        zero(u);
        mm<TMV, 4, NXV>(u, sT, LC, 1, sV, LV, 1, kC);
        const int ty = tid / NXV, tx = tid % NXV;
#pragma unroll
        for (int i = 0; i < TMV; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                R[F::OFF_U + (ty + i * (kNT / NXV)) * DV + tx + j * NXV] = u[i][j];
    }
    {
        float w[F::TMK][4];
        zero(w);
        mm<F::TMK, 4, F::NXK>(w, sT, LC, 1, sQ, LK, 1, kC);
        const int ty = tid / F::NXK, tx = tid % F::NXK;
#pragma unroll
        for (int i = 0; i < F::TMK; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                R[F::OFF_W + (ty + i * (kNT / F::NXK)) * DK + tx + j * F::NXK] = w[i][j];
    }
    for (int i = tid; i < kC * kC; i += kNT) R[F::OFF_T + i] = sT[(i / kC) * LC + (i % kC)];
    if (tid == 0) R[F::OFF_EL] = __expf(glast);
}

// ---------------------------------------------------------------------------------------
// bscan_kernel: blocks [0, chains * NSL) run the forward state chain, the rest the reverse
// gradient chain; one block per (chain, 16-column slice).  The per-chunk products run on the
// matrix cores (fp32), each wavefront owning whole 16 x 16 output blocks; the LDS row strides
// are chosen per operand orientation so that a product's 64 lanes read 64 different banks
// (stride = 4 mod 64 floats where a lane group walks rows, 16 mod 64 where it walks columns).
template <int DK, int DV, typename TD>
__global__ void __launch_bounds__(kNT)
bscan_kernel(const float *__restrict__ rec, const TD *__restrict__ dO,
             const float *__restrict__ s0, const float *__restrict__ dST,
             float *__restrict__ Sc, float *__restrict__ dSe, float *__restrict__ dS0, int T,
             int Hv, int nch, int chains, float scale) {
    using F = CB<DK, DV>;
    constexpr int NSL = DV / 16;
    constexpr int L4 = DK + 4, L16 = DK + 16, LP = kC + 16;  // strides (see above)
    constexpr int NRB = DK / 16 / 4;                          // DK-row blocks per wavefront
    __shared__ float sM1[kC * L16], sM2[kC * L16], sM3[kC * L16], sP[kC * LP];
    __shared__ float sS[DK * 16], sD[kC * 16], sO[kC * 16];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, mi = lane & 15, kq = lane >> 4;
    const bool fwd = blockIdx.x < chains * NSL;
    const int idx = fwd ? blockIdx.x : blockIdx.x - chains * NSL;
    const int chain = idx / NSL, sl = idx - chain * NSL, col0 = 16 * sl;
    const int b = chain / Hv, hv = chain - b * Hv;
    const size_t SS = static_cast<size_t>(DK) * DV;
    const float *init = fwd ? s0 : dST;
    for (int i = tid; i < DK * 16; i += kNT) {
        const int r = i / 16, cc = i % 16;
        sS[i] = init ? init[chain * SS + r * DV + col0 + cc] : 0.f;
    }
    auto save_state = [&](float *dst) {
        for (int i = tid; i < DK * 16; i += kNT) {
            const int r = i / 16, cc = i % 16;
            dst[r * DV + col0 + cc] = sS[i];
        }
    };
    auto recp = [&](int c) { return rec + (static_cast<size_t>(chain) * nch + c) * F::REC; };
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    // The next chunk's operands are loaded into registers while this chunk is computed, then
    // written to LDS: the sequential chain never waits for a record fetch.
    if (fwd) {
        Tile4<kC, DK> nW, nK;
        Tile4<kC, 16> nU;
        auto fetch = [&](int c) {
            const float *R = recp(c);
            nW.load(R + F::OFF_W, DK);
            nK.load(R + F::OFF_KT, DK);
            nU.load(R + F::OFF_U + col0, DV);
        };
        auto put = [&]() {
            nW.store(sM1, L4);   // A, rows walked by lanes
            nK.store(sM2, L16);  // A transposed
            nU.store(sO, 16);
        };
        fetch(0);
        float el = vload1(recp(0) + F::OFF_EL);
        put();
        for (int c = 0; c < nch; ++c) {
            lds_bar();
            save_state(Sc + (static_cast<size_t>(chain) * nch + c) * SS);
            fetch(min(c + 1, nch - 1));
            const float eln = vload1(recp(min(c + 1, nch - 1)) + F::OFF_EL);
            // Delta = U - W S: wavefront w, rows 16w..16w+15
            {
                const f32x4 d = mfma_blk(z4, sM1 + 16 * w * L4, L4, 1, sS, 16, 1, DK);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int o = (16 * w + 4 * kq + i) * 16 + mi;
                    sD[o] = sO[o] - d[i];
                }
            }
            lds_bar();
            // S <- e^gamma_last S + Kt^T Delta: row blocks w, w + 4, ...
#pragma unroll
            for (int j = 0; j < NRB; ++j) {
                const int m0 = 16 * (w + 4 * j);
                const f32x4 u = mfma_blk(z4, sM2 + m0, 1, L16, sD, 16, 1, kC);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float &x = sS[(m0 + 4 * kq + i) * 16 + mi];
                    x = el * x + u[i];
                }
            }
            lds_bar();
            put();
            el = eln;
        }
    } else {
        Tile4<kC, kC> nP;
        Tile4<kC, DK> nK, nG, nW;
        Tile4<kC, 16> nO;
        auto fetch = [&](int c) {
            const float *R = recp(c);
            nP.load(R + F::OFF_P, kC);
            nK.load(R + F::OFF_KT, DK);
            nG.load(R + F::OFF_GQ, DK);
            nW.load(R + F::OFF_W, DK);
            nO.load_in(dO, static_cast<size_t>(b) * T + c * kC, Hv, hv, col0, DV,
                       min(kC, T - c * kC), scale);
        };
        auto put = [&]() {
            nP.store(sP, LP);    // A transposed
            nK.store(sM1, L4);   // A
            nG.store(sM2, L16);  // A transposed
            nW.store(sM3, L16);  // A transposed
            nO.store(sO, 16);
        };
        fetch(nch - 1);
        float el = vload1(recp(nch - 1) + F::OFF_EL);
        put();
        for (int c = nch - 1; c >= 0; --c) {
            lds_bar();
            save_state(dSe + (static_cast<size_t>(chain) * nch + c) * SS);
            fetch(max(c - 1, 0));
            const float eln = vload1(recp(max(c - 1, 0)) + F::OFF_EL);
            // dDelta = P^T dO' + Kt dS: wavefront w, rows 16w..
            {
                f32x4 d = mfma_blk(z4, sP + 16 * w, 1, LP, sO, 16, 1, kC);
                d = mfma_blk(d, sM1 + 16 * w * L4, L4, 1, sS, 16, 1, DK);
#pragma unroll
                for (int i = 0; i < 4; ++i) sD[(16 * w + 4 * kq + i) * 16 + mi] = d[i];
            }
            lds_bar();
            // dS <- e^gamma_last dS + (Gm Q)^T dO' - W^T dDelta
#pragma unroll
            for (int j = 0; j < NRB; ++j) {
                const int m0 = 16 * (w + 4 * j);
                const f32x4 u = mfma_blk(z4, sM2 + m0, 1, L16, sO, 16, 1, kC);
                const f32x4 x = mfma_blk(z4, sM3 + m0, 1, L16, sD, 16, 1, kC);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float &y = sS[(m0 + 4 * kq + i) * 16 + mi];
                    y = el * y + u[i] - x[i];
                }
            }
            lds_bar();
            put();
            el = eln;
        }
        bar();
        if (dS0 != nullptr) save_state(dS0 + chain * SS);
    }
}

// ---------------------------------------------------------------------------------------
template <int DK, int DV, typename TI, typename TD>
__global__ void __launch_bounds__(kNT)
bgrad_kernel(const TI *__restrict__ q, const TI *__restrict__ k, const TI *__restrict__ v,
             const TI *__restrict__ beta, const TI *__restrict__ g, const TD *__restrict__ dO,
             const float *__restrict__ rec, const float *__restrict__ Sc,
             const float *__restrict__ dSe, float *__restrict__ dq_part,
             float *__restrict__ dk_part, float *__restrict__ dv_out,
             float *__restrict__ dbeta, float *__restrict__ dg, int T, int Hk, int Hv, int nch,
             float scale) {
    using F = CB<DK, DV>;
    constexpr int LK = F::LK, LC = F::LC, SW = 32, LS = SW + 1, NSL = DV / SW;
    constexpr int NXK = F::NXK, TMK = F::TMK, NYK = kNT / NXK;
    // phase 1: W, P, Tm + one value slice; phase 2 reuses the slice area and W for K, Q, ...
    constexpr int PH1 = kC * LK + 2 * DK * LS + 4 * kC * LS;       // W + slice buffers
    constexpr int PH2 = 3 * kC * LK + kC * LC;                     // K, Q, X + Y
    constexpr int BIG = PH1 > PH2 ? PH1 : PH2;
    __shared__ float smem[BIG + 2 * kC * LC];
    __shared__ float sgam[kC], sbeta[kC], sv[8][kC];
    float *sP = smem + BIG, *sT = sP + kC * LC;
    float *sW = smem, *sS0 = sW + kC * LK, *sSe = sS0 + DK * LS, *sO = sSe + DK * LS;
    float *sVv = sO + kC * LS, *sD = sVv + kC * LS, *sdD = sD + kC * LS;

    const int chain = blockIdx.x / nch, c = blockIdx.x - chain * nch;
    const int b = chain / Hv, hv = chain - b * Hv, hq = hv / (Hv / Hk);
    const int t0 = c * kC, L = min(kC, T - t0);
    const size_t row0 = static_cast<size_t>(b) * T + t0;
    const int tid = threadIdx.x, lane = tid & 63;
    const float *R = rec + (static_cast<size_t>(chain) * nch + c) * F::REC;
    const size_t SS = static_cast<size_t>(DK) * DV;
    const float *S0 = Sc + (static_cast<size_t>(chain) * nch + c) * SS;
    const float *DSE = dSe + (static_cast<size_t>(chain) * nch + c) * SS;

    {
        Tile4<kC, DK> tw;
        Tile4<kC, kC> tp, tt;
        tw.load(R + F::OFF_W, DK);
        tp.load(R + F::OFF_P, kC);
        tt.load(R + F::OFF_T, kC);
        float gg = 0.f, bb = 0.f;
        if (tid < 64 && tid < L) {
            gg = load_f32(g + (row0 + tid) * Hv + hv);
            bb = load_f32(beta + (row0 + tid) * Hv + hv);
        }
        tw.store(sW, LK);
        tp.store(sP, LC);
        tt.store(sT, LC);
        if (tid < 64) {
            sgam[tid] = wave_scan(gg, tid);
            sbeta[tid] = bb;
        }
    }

    // accumulators over the value slices
    float dGQ[TMK][4], dKt[TMK][4], dW[TMK][4], dP[4][4], dTv[4][4];
    zero(dGQ); zero(dKt); zero(dW); zero(dP); zero(dTv);
    float dglast = 0.f, dbv[4] = {0.f, 0.f, 0.f, 0.f};
    const int ty16 = tid / 16, tx16 = tid % 16;            // 64 x 64 and 64 x 32 tiles
    const int tyk = tid / NXK, txk = tid % NXK;            // 64 x DK tiles

    for (int j = 0; j < NSL; ++j) {
        const int cj = SW * j;
        bar();  // the previous slice's buffers are free
        {
            Tile4<DK, SW> t0s, tes;
            Tile4<kC, SW> tos, tvs;
            t0s.load(S0 + cj, DV);
            tes.load(DSE + cj, DV);
            tos.load_in(dO, row0, Hv, hv, cj, DV, L, scale);
            tvs.load_in(v, row0, Hv, hv, cj, DV, L);
            t0s.store(sS0, LS);
            tes.store(sSe, LS);
            tos.store(sO, LS);
            tvs.store(sVv, LS);
        }
        bar();
        // Delta = U - W S0 ; dDelta = P^T dO' + Kt dSe  (64 x 32 tiles)
        {
            float d[4][2], e[4][2];
            zero(d);
            zero(e);
            mm<4, 2, 16>(d, sW, LK, 1, sS0, LS, 1, DK);
            mm<4, 2, 16>(e, sP, 1, LC, sO, LS, 1, kC);
            mm<4, 2, 16>(e, R + F::OFF_KT, DK, 1, sSe, LS, 1, DK);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int r = ty16 + 16 * i, cc = tx16 + 16 * jj;
                    sD[r * LS + cc] = R[F::OFF_U + r * DV + cj + cc] - d[i][jj];
                    sdD[r * LS + cc] = e[i][jj];
                }
        }
        for (int i = tid; i < DK * SW; i += kNT) dglast += sS0[(i / SW) * LS + i % SW] * sSe[(i / SW) * LS + i % SW];
        bar();
        // dBv = Tm^T dDelta -> dv = beta dBv, dbeta += rowsum(dBv o V)
        {
            float x[4][2];
            zero(x);
            mm<4, 2, 16>(x, sT, 1, LC, sdD, LS, 1, kC);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = ty16 + 16 * i;
                float rs = 0.f;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int cc = tx16 + 16 * jj;
                    rs += x[i][jj] * sVv[r * LS + cc];
                    if (r < L) dv_out[((row0 + r) * Hv + hv) * DV + cj + cc] = sbeta[r] * x[i][jj];
                }
                dbv[i] += row_sum<16>(rs);
            }
        }
        // the partial sums over this slice's value columns
        mm<TMK, 4, NXK>(dGQ, sO, LS, 1, sS0, 1, LS, SW);    // dO' S0^T
        mm<TMK, 4, NXK>(dKt, sD, LS, 1, sSe, 1, LS, SW);    // Delta dSe^T
        mm<TMK, 4, NXK>(dW, sdD, LS, 1, sS0, 1, LS, SW);    // dDelta S0^T   (dW = minus this)
        mm<4, 4, 16>(dP, sO, LS, 1, sD, 1, LS, SW);         // dO' Delta^T
        mm<4, 4, 16>(dTv, sdD, LS, 1, sVv, 1, LS, SW);      // dDelta V^T    (times beta_col)
    }
    bar();

    // ---- phase 2: K, Q, and the terms through Tm, the decays and gamma
    float *sK = smem, *sQ = sK + kC * LK, *sX = sQ + kC * LK, *sY = sX + kC * LK;
    {
        Tile4<kC, DK> tk, tq;
        tk.load_in(k, row0, Hk, hq, 0, DK, L);
        tq.load_in(q, row0, Hk, hq, 0, DK, L);
        tk.store(sK, LK);
        tq.store(sQ, LK);
    }
#pragma unroll
    for (int i = 0; i < TMK; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sX[(tyk + NYK * i) * LK + txk + NXK * jj] = -dW[i][jj];
    bar();
    const float glast = sgam[kC - 1];
    auto Gm = [&](int r) { return __expf(sgam[r]); };
    auto Dm = [&](int r, int s) { return s <= r ? __expf(sgam[r] - sgam[s]) : 0.f; };

    float kk[4][4], qk[4][4], dT[4][4];
    zero(kk); zero(qk); zero(dT);
    mm<4, 4, 16>(kk, sK, LK, 1, sK, 1, LK, DK);
    mm<4, 4, 16>(qk, sQ, LK, 1, sK, 1, LK, DK);
    mm<4, 4, 16>(dT, sX, LK, 1, sK, 1, LK, DK);  // dW K^T  (times beta Gm of the column)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int cc = tx16 + 16 * jj;
            dT[i][jj] = sbeta[cc] * (dTv[i][jj] + Gm(cc) * dT[i][jj]);
        }
    float dBk[TMK][4];
    zero(dBk);
    mm<TMK, 4, NXK>(dBk, sT, 1, LC, sX, LK, 1, kC);  // Tm^T dW
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sY[(ty16 + 16 * i) * LC + tx16 + 16 * jj] = dT[i][jj];
    bar();
    float m1[4][4];
    zero(m1);
    mm<4, 4, 16>(m1, sT, 1, LC, sY, LC, 1, kC);  // Tm^T dTm
    bar();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sY[(ty16 + 16 * i) * LC + tx16 + 16 * jj] = m1[i][jj];
    bar();
    float dA[4][4];
    zero(dA);
    mm<4, 4, 16>(dA, sY, LC, 1, sT, 1, LC, kC);  // (Tm^T dTm) Tm^T
    // per-element terms of the 64 x 64 tiles; the row and column sums of the decay gradient
    float dKK[4][4], dQK[4][4], rE[4], rA[4], cE[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = ty16 + 16 * i;
        rE[i] = 0.f;
        rA[i] = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int s = tx16 + 16 * jj;
            const float d = Dm(r, s);
            const float a = s < r ? -dA[i][jj] : 0.f;       // dA (strictly lower)
            const float p = s <= r ? dP[i][jj] : 0.f;       // dP (lower)
            const float dGs = sbeta[r] * a;
            rA[i] += a * kk[i][jj] * d;                      // dbeta: dA o (K K^T o D)
            dKK[i][jj] = dGs * d;
            dQK[i][jj] = p * d;
            const float e = (dGs * kk[i][jj] + p * qk[i][jj]) * d;
            rE[i] += e;
            cE[jj] += e;
        }
        rE[i] = row_sum<16>(rE[i]);
        rA[i] = row_sum<16>(rA[i]);
    }
    // column sums of E over the 16 row groups: through LDS (each (ty, col) slot written once)
    bar();
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) sY[ty16 * LC + tx16 + 16 * jj] = cE[jj];
    if (tx16 == 0)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sv[0][ty16 + 16 * i] = rE[i];
            sv[1][ty16 + 16 * i] = rA[i];
            sv[2][ty16 + 16 * i] = dbv[i];
        }
    bar();
    if (tid < kC) {
        float s = 0.f;
        for (int y = 0; y < 16; ++y) s += sY[y * LC + tid];
        sv[3][tid] = s;
    }
    bar();
    // dKK + dKK^T to sX (as 64 x 64), dQK to sY
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sY[(ty16 + 16 * i) * LC + tx16 + 16 * jj] = dKK[i][jj];
    bar();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r = ty16 + 16 * i, s = tx16 + 16 * jj;
            sX[r * LC + s] = dKK[i][jj] + sY[s * LC + r];
        }
    bar();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sY[(ty16 + 16 * i) * LC + tx16 + 16 * jj] = dQK[i][jj];
    bar();
    // dK = (dKK + dKK^T) K + dQK^T Q + e^(glast - gamma) dKt + beta Gm dBk ; dQ = dQK K + Gm dGQ
    float dK[TMK][4], dQ[TMK][4];
    zero(dK);
    zero(dQ);
    mm<TMK, 4, NXK>(dK, sX, LC, 1, sK, LK, 1, kC);
    mm<TMK, 4, NXK>(dK, sY, 1, LC, sQ, LK, 1, kC);
    mm<TMK, 4, NXK>(dQ, sY, LC, 1, sK, LK, 1, kC);
    float *dqo = dq_part + (row0 * Hv + hv) * DK;  // [rows][Hv][DK] parts (G = 1: the output)
    float *dko = dk_part + (row0 * Hv + hv) * DK;
    float rq[TMK], rk[TMK], rb[TMK];
#pragma unroll
    for (int i = 0; i < TMK; ++i) {
        const int r = tyk + NYK * i;
        const float gm = Gm(r), ekt = __expf(glast - sgam[r]), bg = sbeta[r] * gm;
        float sq = 0.f, sk = 0.f, sb = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int cc = txk + NXK * jj;
            const float kv = sK[r * LK + cc], qv = sQ[r * LK + cc];
            const float dkv = dK[i][jj] + ekt * dKt[i][jj] + bg * dBk[i][jj];
            const float dqv = dQ[i][jj] + gm * dGQ[i][jj];
            sq += dGQ[i][jj] * qv;       // rowsum(dGQ o Q)
            sk += dKt[i][jj] * kv;       // rowsum(dKt o K)
            sb += dBk[i][jj] * kv;       // rowsum(dBk o K)
            if (r < L) {
                dko[static_cast<size_t>(r) * Hv * DK + cc] = dkv;
                dqo[static_cast<size_t>(r) * Hv * DK + cc] = dqv;
            }
        }
        rq[i] = row_sum<NXK>(sq) * gm;
        rk[i] = row_sum<NXK>(sk) * ekt;
        rb[i] = row_sum<NXK>(sb) * gm;
    }
    if (txk == 0)
#pragma unroll
        for (int i = 0; i < TMK; ++i) {
            const int r = tyk + NYK * i;
            sv[4][r] = rq[i];
            sv[5][r] = rk[i];
            sv[6][r] = rb[i];
        }
    // <dSe, S0> summed over the workgroup
    float dl = dglast;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) dl += __shfl_xor(dl, off);
    if (lane == 0) sv[7][tid >> 6] = dl;
    bar();
    if (tid < kC) {
        const int r = tid;
        float tsum = sv[5][r];
        for (int off = 1; off < 64; off <<= 1) tsum += __shfl_xor(tsum, off);
        const float dsx = sv[7][0] + sv[7][1] + sv[7][2] + sv[7][3];
        const float bt = sbeta[r];
        float dgam = sv[4][r] - sv[5][r] + bt * sv[6][r] + sv[0][r] - sv[3][r];
        if (r == kC - 1) dgam += __expf(glast) * dsx + tsum;
        const float db = sv[2][r] + sv[1][r] + sv[6][r];
        // dg = reverse cumulative sum of dgamma within the chunk
        float tot = dgam;
        for (int off = 1; off < 64; off <<= 1) tot += __shfl_xor(tot, off);
        const float incl = wave_scan(dgam, r);
        const float dgs = tot - incl + dgam;
        if (r < L) {
            dbeta[(row0 + r) * Hv + hv] = db;
            dg[(row0 + r) * Hv + hv] = dgs;
        }
    }
}

}  // namespace

// 16-byte aligned q, k, v and dO (their rows are read four elements at a time)
bool backward_chunk_supports(const BackwardArgs &a) {
    auto al = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    return (a.dk_ == 64 || a.dk_ == 128) && (a.dv_ == 64 || a.dv_ == 128) && a.T > 0 &&
           al(a.q) && al(a.k) && al(a.v) && al(a.dO);
}

size_t backward_chunk_workspace(int B, int T, int Hk, int Hv, int dk, int dv) {
    const size_t chains = static_cast<size_t>(B) * Hv;
    const size_t nch = (static_cast<size_t>(T) + kC - 1) / kC;
    const size_t rec = static_cast<size_t>(kC) * (3 * dk + dv + 2 * kC) + 4;
    size_t bytes = chains * nch * (rec + 2 * static_cast<size_t>(dk) * dv) * 4;
    if (Hv != Hk) bytes += 2 * static_cast<size_t>(B) * T * Hv * dk * 4;
    return bytes;
}

namespace {
template <int DK, int DV, typename TI, typename TD>
hipError_t launch_chunk_typed(const BackwardArgs &a) {
    using F = CB<DK, DV>;
    const int G = a.Hv / a.Hk;
    const int nch = (a.T + kC - 1) / kC;
    const size_t chains = static_cast<size_t>(a.B) * a.Hv;
    float *rec = static_cast<float *>(a.ws);
    float *Sc = rec + chains * nch * F::REC;
    float *dSe = Sc + chains * nch * DK * DV;
    float *dq_part = G == 1 ? a.dq : dSe + chains * nch * DK * DV;
    float *dk_part = G == 1 ? a.dk : dq_part + static_cast<size_t>(a.B) * a.T * a.Hv * DK;
    const unsigned grid = static_cast<unsigned>(chains * nch);
    hipLaunchKernelGGL((bprep_kernel<DK, DV, TI>), dim3(grid), dim3(kNT), 0, a.stream,
                       static_cast<const TI *>(a.q), static_cast<const TI *>(a.k),
                       static_cast<const TI *>(a.v), static_cast<const TI *>(a.beta),
                       static_cast<const TI *>(a.g), rec, a.T, a.Hk, a.Hv, nch);
    hipLaunchKernelGGL((bscan_kernel<DK, DV, TD>), dim3(static_cast<unsigned>(2 * chains * (DV / 16))),
                       dim3(kNT), 0, a.stream, rec, static_cast<const TD *>(a.dO), a.s0, a.dST,
                       Sc, dSe, a.dS0, a.T, a.Hv, nch, static_cast<int>(chains), a.scale);
    hipLaunchKernelGGL((bgrad_kernel<DK, DV, TI, TD>), dim3(grid), dim3(kNT), 0, a.stream,
                       static_cast<const TI *>(a.q), static_cast<const TI *>(a.k),
                       static_cast<const TI *>(a.v), static_cast<const TI *>(a.beta),
                       static_cast<const TI *>(a.g), static_cast<const TD *>(a.dO), rec, Sc, dSe,
                       dq_part, dk_part, a.dv, a.dbeta, a.dg, a.T, a.Hk, a.Hv, nch, a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || G == 1) return e;
    const size_t n = static_cast<size_t>(a.B) * a.T * a.Hk * DK;
    e = launch_part_sum(dq_part, a.dq, n, G, DK, a.stream);
    if (e == hipSuccess) e = launch_part_sum(dk_part, a.dk, n, G, DK, a.stream);
    return e;
}

template <int DK, int DV> hipError_t launch_chunk_dims(const BackwardArgs &a) {
    if (a.in_dt == GDN_BF16)
        return a.dout_dt == GDN_F32 ? launch_chunk_typed<DK, DV, bf16_t, float>(a)
                                    : launch_chunk_typed<DK, DV, bf16_t, bf16_t>(a);
    return a.dout_dt == GDN_F32 ? launch_chunk_typed<DK, DV, float, float>(a)
                                : launch_chunk_typed<DK, DV, float, bf16_t>(a);
}
}  // namespace

hipError_t launch_backward_chunk(const BackwardArgs &a) {
    if (a.dk_ == 128) return a.dv_ == 128 ? launch_chunk_dims<128, 128>(a) : launch_chunk_dims<128, 64>(a);
    return a.dv_ == 128 ? launch_chunk_dims<64, 128>(a) : launch_chunk_dims<64, 64>(a);
}

}  // namespace gdn
