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
// Three kernels.  fp32 inputs compute in fp32 throughout (fp32 matrix-core products); bf16
// inputs keep the per-chunk records in fp16 and take fp16 operands with fp32 accumulation on
// the matrix cores, while the states, e^gamma_last and every sum stay fp32:
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

#include <type_traits>

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

typedef _Float16 f16x8h __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4h __attribute__((ext_vector_type(4)));

// The same 16 x 16 output block with fp16 operands (rounded from the fp32 values in LDS) and
// fp32 accumulation: one v_mfma_f32_16x16x32_f16 per 32 k (16x16x16 for K = 16), holding the
// same D(4 (l/16) + i, l%16) as the fp32 form.  The order of k inside one product is free as
// long as A and B agree: lane l supplies either the 8 consecutive k + 8 (l/16) + e (IL false:
// wide LDS reads where operands are contiguous in k) or k + l/16 + 4e (IL true: the same
// addresses per instruction as the fp32 form, hence the same LDS banks, for which the row
// strides were chosen).  Which is faster was measured per kernel.  Used for bf16 inputs only.
template <bool IL, typename TA, typename TB>
__device__ __forceinline__ f32x4 mfma_blk_h(f32x4 acc, const TA *A, int ar, int ak,
                                            const TB *B, int bk, int bc, int K) {
    const int lane = threadIdx.x & 63, mi = lane & 15, kq = lane >> 4;
    if (K % 32 == 0) {
        constexpr int ks = IL ? 4 : 1;  // step between a lane's k
        const TA *a = A + mi * ar + (IL ? kq : 8 * kq) * ak;
        const TB *b = B + (IL ? kq : 8 * kq) * bk + mi * bc;
#pragma unroll 4
        for (int k = 0; k < K; k += 32) {
            f16x8h af, bf;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                af[e] = static_cast<_Float16>(a[(k + ks * e) * ak]);
                bf[e] = static_cast<_Float16>(b[(k + ks * e) * bk]);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, acc, 0, 0, 0);
        }
        return acc;
    }
    if (K == 16) {
        const TA *a = A + mi * ar + (IL ? kq : 4 * kq) * ak;
        const TB *b = B + (IL ? kq : 4 * kq) * bk + mi * bc;
        f16x4h af, bf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            af[e] = static_cast<_Float16>(a[(IL ? 4 * e : e) * ak]);
            bf[e] = static_cast<_Float16>(b[(IL ? 4 * e : e) * bk]);
        }
        return __builtin_amdgcn_mfma_f32_16x16x16f16(af, bf, acc, 0, 0, 0);
    }
    // any other K (none is used): fp32 operands, four k at a time
    const TA *a = A + mi * ar + kq * ak;
    const TB *b = B + kq * bk + mi * bc;
    for (int k = 0; k < K; k += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(static_cast<float>(a[k * ak]),
                                                   static_cast<float>(b[k * bk]), acc, 0, 0, 0);
    return acc;
}
// fp16 operands (H, k order IL) or fp32 operands
template <bool H, bool IL = false, typename TA, typename TB>
__device__ __forceinline__ f32x4 mfma_p(f32x4 acc, const TA *A, int ar, int ak,
                                        const TB *B, int bk, int bc, int K) {
    if constexpr (H)
        return mfma_blk_h<IL>(acc, A, ar, ak, B, bk, bc, K);
    else
        return mfma_blk(acc, A, ar, ak, B, bk, bc, K);
}

// One lane's A-operand values of a 16 x K block (A(m, k) = A[m ar + k], K a multiple of 32),
// loaded once where the same block enters several products: in the order mfma_p<H> (IL false)
// reads them -- k + 8 (l/16) + e, fp16, for H; k + l/16 in steps of 4, fp32, otherwise.
template <bool H, int K> struct AFrag {
    static constexpr int N = H ? K / 32 : K / 4;
    typename std::conditional<H, f16x8h, float>::type v[N];
    template <typename TA> __device__ __forceinline__ void load(const TA *A, int ar) {
        const int lane = threadIdx.x & 63, mi = lane & 15, kq = lane >> 4;
        if constexpr (H) {
            const TA *a = A + mi * ar + 8 * kq;
#pragma unroll
            for (int n = 0; n < N; ++n)
#pragma unroll
                for (int e = 0; e < 8; ++e) v[n][e] = static_cast<_Float16>(a[32 * n + e]);
        } else {
            const TA *a = A + mi * ar + kq;
#pragma unroll
            for (int n = 0; n < N; ++n) v[n] = static_cast<float>(a[4 * n]);
        }
    }
};
// acc += A B with A from registers (AFrag) and B(k, n) = B[k bk + n bc], as mfma_p<H>
template <bool H, int K, typename TB>
__device__ __forceinline__ f32x4 mfma_pre(f32x4 acc, const AFrag<H, K> &a, const TB *B, int bk,
                                          int bc) {
    const int lane = threadIdx.x & 63, mi = lane & 15, kq = lane >> 4;
    if constexpr (H) {
        const TB *b = B + 8 * kq * bk + mi * bc;
#pragma unroll
        for (int n = 0; n < AFrag<H, K>::N; ++n) {
            f16x8h bf;
#pragma unroll
            for (int e = 0; e < 8; ++e) bf[e] = static_cast<_Float16>(b[(32 * n + e) * bk]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v[n], bf, acc, 0, 0, 0);
        }
    } else {
        const TB *b = B + kq * bk + mi * bc;
#pragma unroll
        for (int n = 0; n < AFrag<H, K>::N; ++n)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[n], static_cast<float>(b[4 * n * bk]),
                                                       acc, 0, 0, 0);
    }
    return acc;
}

// Record element type: fp16 for bf16 inputs (the matrix cores take fp16 operands there), fp32
// otherwise.  e^gamma_last is an fp32 value in either case (at OFF_EL, 4-byte aligned).
template <bool H> using RecT = typename std::conditional<H, _Float16, float>::type;
template <typename RT> __device__ __forceinline__ RT *rec_at(float *base, size_t idx, size_t rec) {
    return reinterpret_cast<RT *>(base) + idx * rec;
}
template <typename RT>
__device__ __forceinline__ const RT *rec_at(const float *base, size_t idx, size_t rec) {
    return reinterpret_cast<const RT *>(base) + idx * rec;
}

template <int DK, int DV> struct CB {
    // records per (chain, chunk), row-major, in elements of the record type
    static constexpr size_t OFF_W = 0;                          // [C][DK]
    static constexpr size_t OFF_U = OFF_W + kC * DK;            // [C][DV]
    static constexpr size_t OFF_KT = OFF_U + kC * DV;           // [C][DK]
    static constexpr size_t OFF_GQ = OFF_KT + kC * DK;          // [C][DK]
    static constexpr size_t OFF_P = OFF_GQ + kC * DK;           // [C][C]
    static constexpr size_t OFF_T = OFF_P + kC * kC;            // [C][C]
    static constexpr size_t OFF_EL = OFF_T + kC * kC;           // e^gamma_last
    static constexpr size_t REC = OFF_EL + 8;  // a multiple of 8: 16-byte aligned records
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
    // the same from an fp16 matrix (8-byte loads)
    __device__ __forceinline__ void load(const _Float16 *src, int sld, float mul = 1.f) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = (i * kNT + threadIdx.x) * 4, r = idx / COLS, c = idx - r * COLS;
            const f16x4h h = *reinterpret_cast<const f16x4h *>(src + static_cast<size_t>(r) * sld + c);
            v[i] = make_float4(mul * float(h[0]), mul * float(h[1]), mul * float(h[2]),
                               mul * float(h[3]));
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
    // to LDS rows of stride ld, a multiple of 4 (16-byte writes)
    __device__ __forceinline__ void store4(float *dst, int ld) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = (i * kNT + threadIdx.x) * 4, r = idx / COLS, c = idx - r * COLS;
            *reinterpret_cast<float4 *>(dst + r * ld + c) = v[i];
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

// Rows of a [.., H, D] input tensor kept in registers as loaded (fp32 or bf16 bits) with their
// row masks, converted only when written to LDS: nothing waits for the loads until then.
template <int ROWS, int COLS, typename TI> struct InTile {
    static constexpr int N = ROWS * COLS / 4 / kNT;
    static_assert(N * 4 * kNT == ROWS * COLS, "tile must split evenly over the threads");
    using Raw = typename std::conditional<std::is_same<TI, float>::value, float4, uint2>::type;
    Raw x[N];
    float m[N];
    __device__ __forceinline__ void load(const TI *src, size_t row0, int H, int h, int c0, int D,
                                         int L, float mul) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = (i * kNT + threadIdx.x) * 4, r = idx / COLS, c = idx - r * COLS;
            x[i] = *reinterpret_cast<const Raw *>(src + ((row0 + min(r, L - 1)) * H + h) * D + c0 + c);
            m[i] = r < L ? mul : 0.f;
        }
    }
    __device__ __forceinline__ void store4(float *dst, int ld) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = (i * kNT + threadIdx.x) * 4, r = idx / COLS, c = idx - r * COLS;
            float4 f;
            if constexpr (std::is_same<TI, float>::value) {
                f = x[i];
            } else {
                f = make_float4(__uint_as_float(x[i].x << 16), __uint_as_float(x[i].x & 0xffff0000u),
                                __uint_as_float(x[i].y << 16), __uint_as_float(x[i].y & 0xffff0000u));
            }
            *reinterpret_cast<float4 *>(dst + r * ld + c) =
                make_float4(m[i] * f.x, m[i] * f.y, m[i] * f.z, m[i] * f.w);
        }
    }
};

// A ROWS x COLS tile of a row-major record matrix kept in registers as stored (fp16 or fp32),
// 4 elements per 8- or 16-byte load, written to LDS as fp32.
template <int ROWS, int COLS, typename RT, int E = 4> struct TileR {  // E elements per load
    static constexpr int N = ROWS * COLS / E / kNT;
    static_assert(N * E * kNT == ROWS * COLS, "tile must split evenly over the threads");
    static_assert(E == 4 || (E == 8 && !std::is_same<RT, float>::value), "8 per load: fp16");
    using V = typename std::conditional<std::is_same<RT, float>::value, f32x4,
              typename std::conditional<E == 8, f16x8h, f16x4h>::type>::type;
    V v[N];
    __device__ __forceinline__ void load(const RT *src, int sld) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = (i * kNT + threadIdx.x) * E, r = idx / COLS, c = idx - r * COLS;
            v[i] = *reinterpret_cast<const V *>(src + static_cast<size_t>(r) * sld + c);
        }
    }
    // as stored (no conversion): one LDS write of E elements (8 or 16 bytes)
    __device__ __forceinline__ void store_raw(RT *dst, int ld) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = (i * kNT + threadIdx.x) * E, r = idx / COLS, c = idx - r * COLS;
            *reinterpret_cast<V *>(dst + r * ld + c) = v[i];
        }
    }
    // ld and dst 16-byte aligned: one 16-byte LDS write per 4 elements
    __device__ __forceinline__ void store(float *dst, int ld) const {
        static_assert(E == 4, "converting store: 4 elements per load");
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = (i * kNT + threadIdx.x) * 4, r = idx / COLS, c = idx - r * COLS;
            *reinterpret_cast<f32x4 *>(dst + r * ld + c) =
                f32x4{static_cast<float>(v[i][0]), static_cast<float>(v[i][1]),
                      static_cast<float>(v[i][2]), static_cast<float>(v[i][3])};
        }
    }
};

// ---------------------------------------------------------------------------------------
// bprep_kernel: one workgroup per (chain, chunk).  The products on the matrix cores (fp32),
// wavefront w owning row block w; Tm by forward substitution, one column per thread.
template <int DK, int DV, typename TI>
// one workgroup per compute unit (LDS), so every wavefront may use the whole register file
__global__ void __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(1, 1)))
bprep_kernel(const TI *__restrict__ q, const TI *__restrict__ k, const TI *__restrict__ v,
             const TI *__restrict__ beta, const TI *__restrict__ g, float *__restrict__ rec,
             int T, int Hk, int Hv, int nch) {
    using F = CB<DK, DV>;
    constexpr bool HP = std::is_same<TI, bf16_t>::value;  // fp16 operands for bf16 inputs
    constexpr int LK4 = DK + 4, LV16 = DV + 16, LC4 = kC + 4, LC1 = kC + 1;
    __shared__ __attribute__((aligned(16))) float sK[kC * LK4], sQ[kC * LK4], sV[kC * LV16],
        sT[kC * LC4];
    __shared__ float sA[kC * LC1], sgam[kC], sbeta[kC], sX[4][16 * 17];
    const int chain = blockIdx.x / nch, c = blockIdx.x - chain * nch;
    const int b = chain / Hv, hv = chain - b * Hv, hq = hv / (Hv / Hk);
    const int t0 = c * kC, L = min(kC, T - t0);
    const size_t row0 = static_cast<size_t>(b) * T + t0;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, mi = lane & 15, kq = lane >> 4;
    const int rb = 16 * w + 4 * kq;
    using RT = RecT<HP>;
    RT *R = rec_at<RT>(rec, static_cast<size_t>(chain) * nch + c, F::REC);
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};

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
        tk.store(sK, LK4);
        tq.store(sQ, LK4);
        tv.store(sV, LV16);
        if (tid < 64) {
            sgam[tid] = wave_scan(gg, tid);
            sbeta[tid] = bb;
        }
    }
    bar();
    const float glast = sgam[kC - 1];
    // K K^T and Q K^T (row block w), then A (strictly lower) and P (lower) with the decays
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
        const f32x4 kk = mfma_p<HP>(z4, sK + 16 * w * LK4, LK4, 1, sK + 16 * bj * LK4, 1, LK4, DK);
        const f32x4 qk = mfma_p<HP>(z4, sQ + 16 * w * LK4, LK4, 1, sK + 16 * bj * LK4, 1, LK4, DK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rb + i, s = 16 * bj + mi;
            const float d = s <= r ? __expf(sgam[r] - sgam[s]) : 0.f;
            sA[r * LC1 + s] = s < r ? sbeta[r] * kk[i] * d : 0.f;
            R[F::OFF_P + r * kC + s] = static_cast<RT>(qk[i] * d);
        }
    }
    bar();
    // Tm = (I + A)^-1 (A strictly lower) by 16 x 16 blocks: the four diagonal blocks by forward
    // substitution, one column per thread; then block rows 1..3 in order on the matrix cores,
    // T_ij = -T_ii sum_{j <= k < i} A_ik T_kj, wavefront w forming block column w.
    for (int i = tid; i < kC * LC4; i += kNT) sT[i] = 0.f;
    bar();
    if (tid < kC) {
        // column j of the inverse of diagonal block o, in registers: x_r = [r == j] -
        // sum_{s<r} A_rs x_s (x_s = 0 for s < j, so the terms below j add nothing); the block's
        // entries of A are read as broadcasts, independently of x
        const int o = 16 * (tid >> 4), j = tid & 15;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = r == j ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < r; ++s) acc -= sA[(o + r) * LC1 + o + s] * x[s];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[(o + r) * LC4 + o + j] = x[r];
    }
    bar();
    for (int bi = 1; bi < 4; ++bi) {
        if (w < bi) {
            f32x4 x = z4;
            for (int bk = w; bk < bi; ++bk)
                x = mfma_p<HP>(x, sA + 16 * bi * LC1 + 16 * bk, LC1, 1, sT + 16 * bk * LC4 + 16 * w,
                             LC4, 1, 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) sX[w][(4 * kq + i) * 17 + mi] = x[i];
            // the same wavefront reads its block back: LDS operations of a wavefront are in order
            const f32x4 t = mfma_p<HP>(z4, sT + 16 * bi * LC4 + 16 * bi, LC4, 1, sX[w], 17, 1, 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) sT[(16 * bi + 4 * kq + i) * LC4 + 16 * w + mi] = -t[i];
        }
        bar();
    }
    // Gm Q and Kt to the records; then sQ <- beta Gm K (W's right factor), sV <- beta V
    for (int i = tid; i < kC * DK; i += kNT) {
        const int r = i / DK, cc = i - r * DK;
        R[F::OFF_GQ + i] = static_cast<RT>(__expf(sgam[r]) * sQ[r * LK4 + cc]);
        R[F::OFF_KT + i] = static_cast<RT>(__expf(glast - sgam[r]) * sK[r * LK4 + cc]);
    }
    bar();
    for (int i = tid; i < kC * DK; i += kNT) {
        const int r = i / DK, cc = i - r * DK;
        sQ[r * LK4 + cc] = sbeta[r] * __expf(sgam[r]) * sK[r * LK4 + cc];
    }
    for (int i = tid; i < kC * DV; i += kNT) {
        const int r = i / DV, cc = i - r * DV;
        sV[r * LV16 + cc] *= sbeta[r];
    }
    bar();
    // U = Tm (beta V), W = Tm (beta Gm K)  (row block w)
#pragma unroll
    for (int bj = 0; bj < DV / 16; ++bj) {
        const f32x4 u = mfma_p<HP>(z4, sT + 16 * w * LC4, LC4, 1, sV + 16 * bj, LV16, 1, kC);
#pragma unroll
        for (int i = 0; i < 4; ++i) R[F::OFF_U + (rb + i) * DV + 16 * bj + mi] = static_cast<RT>(u[i]);
    }
#pragma unroll
    for (int bj = 0; bj < DK / 16; ++bj) {
        const f32x4 x = mfma_p<HP>(z4, sT + 16 * w * LC4, LC4, 1, sQ + 16 * bj, LK4, 1, kC);
#pragma unroll
        for (int i = 0; i < 4; ++i) R[F::OFF_W + (rb + i) * DK + 16 * bj + mi] = static_cast<RT>(x[i]);
    }
    for (int i = tid; i < kC * kC; i += kNT) R[F::OFF_T + i] = static_cast<RT>(sT[(i / kC) * LC4 + (i % kC)]);
    if (tid == 0) *reinterpret_cast<float *>(R + F::OFF_EL) = __expf(glast);
}

// ---------------------------------------------------------------------------------------
// bscan_kernel: blocks [0, chains * NSL) run the forward state chain, the rest the reverse
// gradient chain; one block per (chain, 16-column slice).  The per-chunk products run on the
// matrix cores, each wavefront owning whole 16 x 16 output blocks.  The record operands sit in
// LDS as stored (fp16 for bf16 inputs, else fp32); their row strides are chosen per operand
// orientation so that a product's 64 lanes read 64 different banks: 4 mod 64 floats (or
// 8 mod 128 halves: lanes kq, kq + 1 share a dword) where a lane group walks rows, 16 mod 64
// floats (or halves) where it walks columns.
template <int DK, int DV, typename TD, bool HP>
// one workgroup per compute unit (LDS), so every wavefront may use the whole register file
__global__ void __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(1, 1)))
bscan_kernel(const float *__restrict__ rec, const TD *__restrict__ dO,
             const float *__restrict__ s0, const float *__restrict__ dST,
             float *__restrict__ Sc, float *__restrict__ dSe, float *__restrict__ dS0, int T,
             int Hv, int nch, int chains, float scale) {
    using F = CB<DK, DV>;
    constexpr int NSL = DV / 16;
    using RE = RecT<HP>;                                       // record element type
    constexpr int L4 = HP ? DK + 8 : DK + 4, L16 = DK + 16, LP = kC + 16;  // element strides
    constexpr int NRB = DK / 16 / 4;                          // DK-row blocks per wavefront
    __shared__ __attribute__((aligned(16))) RE sM1[kC * L16], sM2[kC * L16], sM3[kC * L16],
        sP[kC * LP];
    __shared__ __attribute__((aligned(16))) float sS[DK * 16], sD[kC * 16], sO[kC * 16];
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
    using RT = RecT<HP>;
    auto recp = [&](int c) { return rec_at<RT>(rec, static_cast<size_t>(chain) * nch + c, F::REC); };
    auto elp = [&](int c) { return reinterpret_cast<const float *>(recp(c) + F::OFF_EL); };
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    // The operands of the next three chunks are in registers (three sets in rotation) while
    // chunk c is computed: the next chunk's set waits to be written to LDS at the end of the
    // step, the one after is in flight, and the third is being loaded -- in three parts, at
    // three points of the step, so that no wavefront stalls on a long burst of load issues.
    // The sequential chain waits for no record fetch as long as a fetch takes under two steps.
    if (fwd) {
        struct Set {
            TileR<kC, DK, RT, HP ? 8 : 4> W, K;  // 16-byte loads for fp16 records
            TileR<kC, 16, RT> U;
            float el;
        } s0, s1, s2;
        // chunk c's loads in three parts, issued at three points of an earlier chunk's step
        auto fetch_part = [&](Set &x, int c, int part) {
            c = min(c, nch - 1);
            const RT *R = recp(c);
            if (part == 0) {
                x.U.load(R + F::OFF_U + col0, DV);
                x.el = vload1(elp(c));
            } else if (part == 1) {
                x.K.load(R + F::OFF_KT, DK);
            } else {
                x.W.load(R + F::OFF_W, DK);
            }
        };
        auto fetch = [&](Set &x, int c) {
            fetch_part(x, c, 0);
            fetch_part(x, c, 1);
            fetch_part(x, c, 2);
        };
        float el = 0.f;
        auto put = [&](const Set &x) {
            x.W.store_raw(sM1, L4);   // A, rows walked by lanes
            x.K.store_raw(sM2, L16);  // A transposed
            x.U.store(sO, 16);
            el = x.el;
        };
        // step c, loading chunk c + 3 into the free set `ld` on the way
        auto step = [&](int c, Set &ld) {
            lds_bar();
            save_state(Sc + (static_cast<size_t>(chain) * nch + c) * SS);
            fetch_part(ld, c + 3, 0);
            // Delta = U - W S: wavefront w, rows 16w..16w+15
            {
                const f32x4 d = mfma_p<HP, true>(z4, sM1 + 16 * w * L4, L4, 1, sS, 16, 1, DK);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int o = (16 * w + 4 * kq + i) * 16 + mi;
                    sD[o] = sO[o] - d[i];
                }
            }
            fetch_part(ld, c + 3, 1);
            lds_bar();
            // S <- e^gamma_last S + Kt^T Delta: row blocks w, w + 4, ...
#pragma unroll
            for (int j = 0; j < NRB; ++j) {
                const int m0 = 16 * (w + 4 * j);
                const f32x4 u = mfma_p<HP, true>(z4, sM2 + m0, 1, L16, sD, 16, 1, kC);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float &x = sS[(m0 + 4 * kq + i) * 16 + mi];
                    x = el * x + u[i];
                }
            }
            fetch_part(ld, c + 3, 2);
            lds_bar();
        };
        // three sets in rotation, as in the reverse chain below
        fetch(s0, 0);
        put(s0);
        fetch(s1, 1);
        fetch(s2, 2);
        for (int c = 0; c < nch; c += 3) {
            step(c, s0);
            put(s1);  // chunk c + 1
            if (c + 1 < nch) {
                step(c + 1, s1);
                put(s2);  // chunk c + 2
            }
            if (c + 2 < nch) {
                step(c + 2, s2);
                put(s0);  // chunk c + 3
            }
        }
    } else {
        struct Set {
            TileR<kC, kC, RT, HP ? 8 : 4> P;  // 16-byte loads for fp16 records
            TileR<kC, DK, RT, HP ? 8 : 4> K, G, W;
            InTile<kC, 16, TD> O;
            float el;
        } s0, s1, s2;
        // chunk c's loads in three parts, issued at three points of an earlier chunk's step so
        // that the wavefronts never stall on a long burst of load issues
        auto fetch_part = [&](Set &x, int c, int part) {
            c = max(c, 0);
            const RT *R = recp(c);
            if (part == 0) {
                x.P.load(R + F::OFF_P, kC);
                x.O.load(dO, static_cast<size_t>(b) * T + c * kC, Hv, hv, col0, DV,
                         min(kC, T - c * kC), scale);
                x.el = vload1(elp(c));
            } else if (part == 1) {
                x.K.load(R + F::OFF_KT, DK);
                x.G.load(R + F::OFF_GQ, DK);
            } else {
                x.W.load(R + F::OFF_W, DK);
            }
        };
        auto fetch = [&](Set &x, int c) {
            fetch_part(x, c, 0);
            fetch_part(x, c, 1);
            fetch_part(x, c, 2);
        };
        float el = 0.f;
        auto put = [&](const Set &x) {
            x.P.store_raw(sP, LP);    // A transposed
            x.K.store_raw(sM1, L4);   // A
            x.G.store_raw(sM2, L16);  // A transposed
            x.W.store_raw(sM3, L16);  // A transposed
            x.O.store4(sO, 16);
            el = x.el;
        };
        // step c, loading chunk c - 3 into the free set `ld` on the way
        auto step = [&](int c, Set &ld) {
            lds_bar();
            save_state(dSe + (static_cast<size_t>(chain) * nch + c) * SS);
            fetch_part(ld, c - 3, 0);
            // dDelta = P^T dO' + Kt dS: wavefront w, rows 16w..
            {
                f32x4 d = mfma_p<HP, true>(z4, sP + 16 * w, 1, LP, sO, 16, 1, kC);
                d = mfma_p<HP, true>(d, sM1 + 16 * w * L4, L4, 1, sS, 16, 1, DK);
#pragma unroll
                for (int i = 0; i < 4; ++i) sD[(16 * w + 4 * kq + i) * 16 + mi] = d[i];
            }
            fetch_part(ld, c - 3, 1);
            lds_bar();
            // dS <- e^gamma_last dS + (Gm Q)^T dO' - W^T dDelta
#pragma unroll
            for (int j = 0; j < NRB; ++j) {
                const int m0 = 16 * (w + 4 * j);
                const f32x4 u = mfma_p<HP, true>(z4, sM2 + m0, 1, L16, sO, 16, 1, kC);
                const f32x4 x = mfma_p<HP, true>(z4, sM3 + m0, 1, L16, sD, 16, 1, kC);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float &y = sS[(m0 + 4 * kq + i) * 16 + mi];
                    y = el * y + u[i] - x[i];
                }
            }
            fetch_part(ld, c - 3, 2);
            lds_bar();
        };
        // Three sets in rotation: while chunk c is computed, chunk c - 1's set waits to be
        // written to LDS, chunk c - 2's loads are in flight and chunk c's set (already in LDS)
        // receives chunk c - 3.  Constant set names only (no indexed register arrays).
        fetch(s0, nch - 1);
        put(s0);
        fetch(s1, nch - 2);
        fetch(s2, nch - 3);
        for (int c = nch - 1; c >= 0; c -= 3) {
            step(c, s0);
            put(s1);  // chunk c - 1
            if (c - 1 >= 0) {
                step(c - 1, s1);
                put(s2);  // chunk c - 2
            }
            if (c - 2 >= 0) {
                step(c - 2, s2);
                put(s0);  // chunk c - 3
            }
        }
        bar();
        if (dS0 != nullptr) save_state(dS0 + chain * SS);
    }
}

// ---------------------------------------------------------------------------------------
// bgrad_kernel: one workgroup per (chain, chunk).  All products on the matrix cores (fp32):
// wavefront w owns row block w (rows 16w..16w+15) of every 64 x 64 and 64 x DK product, so its
// lane l holds rows 16w + 4 (l/16) + i, i < 4, of column 16 bj + l%16 of column block bj.
template <int DK, int DV, typename TI, typename TD>
// one workgroup per compute unit (LDS), so every wavefront may use the whole register file
__global__ void __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(1, 1)))
bgrad_kernel(const TI *__restrict__ q, const TI *__restrict__ k, const TI *__restrict__ v,
             const TI *__restrict__ beta, const TI *__restrict__ g, const TD *__restrict__ dO,
             const float *__restrict__ rec, const float *__restrict__ Sc,
             const float *__restrict__ dSe, float *__restrict__ dq_part,
             float *__restrict__ dk_part, float *__restrict__ dv_out,
             float *__restrict__ dbeta, float *__restrict__ dg, int T, int Hk, int Hv, int nch,
             float scale) {
    using F = CB<DK, DV>;
    constexpr bool HP = std::is_same<TI, bf16_t>::value;  // fp16 operands for bf16 inputs
    // value slices of SW = 32 columns (CT = 2 tiles of 16): the products summed over the
    // slice's columns run as 16x16x32 MFMAs, and a chunk takes DV / 32 slice steps
    constexpr int SW = 32, CT = SW / 16, NSL = DV / SW, NBK = DK / 16;
    constexpr int LK4 = DK + 4, LC16 = kC + 16, LC4 = kC + 4, LS = SW + 4;
    constexpr int P1 = kC * LK4 + 2 * DK * LS + 4 * kC * LS;  // W + one value slice
    constexpr int P2 = 3 * kC * LK4;                          // K, Q, dW / (dKK + dKK^T)
    constexpr int BIG = P1 > P2 ? P1 : P2;
    __shared__ __attribute__((aligned(16))) float smem[BIG + 2 * kC * LC16];
    __shared__ float sgam[kC], sbeta[kC], sv[8][kC], scol[4][kC];
    float *sPY = smem + BIG;       // P (phase 1), then a 64 x 64 scratch Y (phase 2)
    float *sT = sPY + kC * LC16;   // Tm
    float *sW = smem, *sS0 = sW + kC * LK4, *sSe = sS0 + DK * LS, *sO = sSe + DK * LS;
    float *sVv = sO + kC * LS, *sD = sVv + kC * LS, *sdD = sD + kC * LS;

    const int chain = blockIdx.x / nch, c = blockIdx.x - chain * nch;
    const int b = chain / Hv, hv = chain - b * Hv, hq = hv / (Hv / Hk);
    const int t0 = c * kC, L = min(kC, T - t0);
    const size_t row0 = static_cast<size_t>(b) * T + t0;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, mi = lane & 15, kq = lane >> 4;
    const int rb = 16 * w + 4 * kq;  // this lane's first row
    using RT = RecT<HP>;
    const RT *R = rec_at<RT>(rec, static_cast<size_t>(chain) * nch + c, F::REC);
    const size_t SS = static_cast<size_t>(DK) * DV;
    const float *S0 = Sc + (static_cast<size_t>(chain) * nch + c) * SS;
    const float *DSE = dSe + (static_cast<size_t>(chain) * nch + c) * SS;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
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
        tw.store4(sW, LK4);
        tp.store4(sPY, LC16);
        tt.store4(sT, LC16);
        if (tid < 64) {
            sgam[tid] = wave_scan(gg, tid);
            sbeta[tid] = bb;
        }
    }

    // accumulators over the value slices (row block w)
    f32x4 aGQ[NBK], aKt[NBK], aW[NBK], aP[4], aTv[4];
#pragma unroll
    for (int j = 0; j < NBK; ++j) aGQ[j] = aKt[j] = aW[j] = z4;
#pragma unroll
    for (int j = 0; j < 4; ++j) aP[j] = aTv[j] = z4;
    float dglast = 0.f, dbv[4] = {0.f, 0.f, 0.f, 0.f};

    // the value slices' tiles: slice j + 1's loads are in flight while slice j is computed
    // (the barriers below wait for LDS only, so they do not wait for those loads)
    Tile4<DK, SW> t0s, tes;
    Tile4<kC, SW> tos, tvs;
    float uf[CT][4];  // U of this lane's rows in the slice's columns 16 ct + mi
    auto fetch = [&](int j) {
        const int cj = SW * j;
        t0s.load(S0 + cj, DV);
        tes.load(DSE + cj, DV);
        tos.load_in(dO, row0, Hv, hv, cj, DV, L, scale);
        tvs.load_in(v, row0, Hv, hv, cj, DV, L);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                uf[ct][i] = static_cast<float>(R[F::OFF_U + (rb + i) * DV + cj + 16 * ct + mi]);
    };
    // Kt's row block w, the A operand of one product in every slice: read once.  With it and U
    // fetched with the tiles, no global load is waited for inside a slice except the next
    // slice's (the vector-memory counter is in order).
    AFrag<HP, DK> ktw;
    ktw.load(R + F::OFF_KT + 16 * w * DK, DK);
    fetch(0);
#pragma unroll  // constant indices everywhere: the tiles stay in registers
    for (int j = 0; j < NSL; ++j) {
        const int cj = SW * j;
        lds_bar();  // the previous slice's buffers are free
        t0s.store4(sS0, LS);
        tes.store4(sSe, LS);
        tos.store4(sO, LS);
        tvs.store4(sVv, LS);
        float u[CT][4];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) u[ct][i] = uf[ct][i];
        if (j + 1 < NSL) fetch(j + 1);
        lds_bar();
        // Delta = U - W S0 ; dDelta = P^T dO' + Kt dSe   (row block w, column tile ct)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const f32x4 d = mfma_p<HP>(z4, sW + 16 * w * LK4, LK4, 1, sS0 + 16 * ct, LS, 1, DK);
            f32x4 e = mfma_p<HP>(z4, sPY + 16 * w, 1, LC16, sO + 16 * ct, LS, 1, kC);
            e = mfma_pre<HP, DK>(e, ktw, sSe + 16 * ct, LS, 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rb + i;
                sD[r * LS + 16 * ct + mi] = u[ct][i] - d[i];
                sdD[r * LS + 16 * ct + mi] = e[i];
            }
        }
        for (int i = tid; i < DK * SW; i += kNT)
            dglast += sS0[(i / SW) * LS + i % SW] * sSe[(i / SW) * LS + i % SW];
        lds_bar();
        // dBv = Tm^T dDelta -> dv = beta dBv, dbeta += rowsum(dBv o V)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const f32x4 x = mfma_p<HP>(z4, sT + 16 * w, 1, LC16, sdD + 16 * ct, LS, 1, kC);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rb + i;
                if (r < L) dv_out[((row0 + r) * Hv + hv) * DV + cj + 16 * ct + mi] = sbeta[r] * x[i];
                dbv[i] += row_sum<16>(x[i] * sVv[r * LS + 16 * ct + mi]);
            }
        }
        // the partial sums over this slice's value columns (K = SW)
#pragma unroll
        for (int bj = 0; bj < NBK; ++bj) {
            aGQ[bj] = mfma_p<HP>(aGQ[bj], sO + 16 * w * LS, LS, 1, sS0 + 16 * bj * LS, 1, LS, SW);
            aKt[bj] = mfma_p<HP>(aKt[bj], sD + 16 * w * LS, LS, 1, sSe + 16 * bj * LS, 1, LS, SW);
            aW[bj] = mfma_p<HP>(aW[bj], sdD + 16 * w * LS, LS, 1, sS0 + 16 * bj * LS, 1, LS, SW);
        }
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            aP[bj] = mfma_p<HP>(aP[bj], sO + 16 * w * LS, LS, 1, sD + 16 * bj * LS, 1, LS, SW);
            aTv[bj] = mfma_p<HP>(aTv[bj], sdD + 16 * w * LS, LS, 1, sVv + 16 * bj * LS, 1, LS, SW);
        }
    }
    lds_bar();

    // ---- phase 2: K, Q, and the terms through Tm, the decays and gamma
    float *sK = smem, *sQ = sK + kC * LK4, *sX = sQ + kC * LK4, *sY = sPY;
    {
        Tile4<kC, DK> tk, tq;
        tk.load_in(k, row0, Hk, hq, 0, DK, L);
        tq.load_in(q, row0, Hk, hq, 0, DK, L);
        tk.store4(sK, LK4);
        tq.store4(sQ, LK4);
    }
#pragma unroll
    for (int bj = 0; bj < NBK; ++bj)
#pragma unroll
        for (int i = 0; i < 4; ++i) sX[(rb + i) * LK4 + 16 * bj + mi] = -aW[bj][i];  // dW
    lds_bar();
    const float glast = sgam[kC - 1];
    f32x4 aKK[4], aQK[4], aT[4];
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
        aKK[bj] = mfma_p<HP>(z4, sK + 16 * w * LK4, LK4, 1, sK + 16 * bj * LK4, 1, LK4, DK);
        aQK[bj] = mfma_p<HP>(z4, sQ + 16 * w * LK4, LK4, 1, sK + 16 * bj * LK4, 1, LK4, DK);
        aT[bj] = mfma_p<HP>(z4, sX + 16 * w * LK4, LK4, 1, sK + 16 * bj * LK4, 1, LK4, DK);  // dW K^T
    }
    f32x4 aBk[NBK];
#pragma unroll
    for (int bj = 0; bj < NBK; ++bj)
        aBk[bj] = mfma_p<HP>(z4, sT + 16 * w, 1, LC16, sX + 16 * bj, LK4, 1, kC);  // Tm^T dW
    // dTm = beta_col (dDelta V^T + Gm_col dW K^T) -> Y
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
        const int s = 16 * bj + mi;
        const float bs = sbeta[s], gs = __expf(sgam[s]);
#pragma unroll
        for (int i = 0; i < 4; ++i) sY[(rb + i) * LC16 + s] = bs * (aTv[bj][i] + gs * aT[bj][i]);
    }
    lds_bar();
    f32x4 aM[4];
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) aM[bj] = mfma_p<HP>(z4, sT + 16 * w, 1, LC16, sY + 16 * bj, LC16, 1, kC);
    lds_bar();
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
        for (int i = 0; i < 4; ++i) sY[(rb + i) * LC16 + 16 * bj + mi] = aM[bj][i];
    lds_bar();
    f32x4 aA[4];
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) aA[bj] = mfma_p<HP>(z4, sY + 16 * w * LC16, LC16, 1, sT + 16 * bj * LC16, 1, LC16, kC);
    // per-element terms; row and column sums of the decay gradient E = dD o D
    f32x4 aKKd[4], aQKd[4];
    float rE[4] = {0.f, 0.f, 0.f, 0.f}, rA[4] = {0.f, 0.f, 0.f, 0.f}, cE[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rb + i, s = 16 * bj + mi;
            const float d = s <= r ? __expf(sgam[r] - sgam[s]) : 0.f;
            const float a = s < r ? -aA[bj][i] : 0.f;  // dA (strictly lower)
            const float p = s <= r ? aP[bj][i] : 0.f;  // dP (lower)
            const float dGs = sbeta[r] * a;
            rA[i] += a * aKK[bj][i] * d;
            aKKd[bj][i] = dGs * d;
            aQKd[bj][i] = p * d;
            const float e = (dGs * aKK[bj][i] + p * aQK[bj][i]) * d;
            rE[i] += e;
            cE[bj] += e;
        }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        rE[i] = row_sum<16>(rE[i]);
        rA[i] = row_sum<16>(rA[i]);
    }
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
        cE[bj] += __shfl_xor(cE[bj], 16);
        cE[bj] += __shfl_xor(cE[bj], 32);
    }
    lds_bar();  // Y (M1) is no longer read
    if (kq == 0)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) scol[w][16 * bj + mi] = cE[bj];
    if (mi == 0)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sv[0][rb + i] = rE[i];
            sv[1][rb + i] = rA[i];
            sv[2][rb + i] = dbv[i];
        }
    // dKK -> Y, then (dKK + dKK^T) -> X (64 x 64, stride LC4; dW is no longer read)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
        for (int i = 0; i < 4; ++i) sY[(rb + i) * LC16 + 16 * bj + mi] = aKKd[bj][i];
    lds_bar();
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rb + i, s = 16 * bj + mi;
            sX[r * LC4 + s] = aKKd[bj][i] + sY[s * LC16 + r];
        }
    lds_bar();
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
        for (int i = 0; i < 4; ++i) sY[(rb + i) * LC16 + 16 * bj + mi] = aQKd[bj][i];
    lds_bar();
    // dK = (dKK + dKK^T) K + dQK^T Q + e^(glast - gamma) dKt + beta Gm dBk ; dQ = dQK K + Gm dGQ
    float *dqo = dq_part + (row0 * Hv + hv) * DK;  // [rows][Hv][DK] parts (G = 1: the output)
    float *dko = dk_part + (row0 * Hv + hv) * DK;
    float sq[4] = {0.f, 0.f, 0.f, 0.f}, sk[4] = {0.f, 0.f, 0.f, 0.f}, sb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int bj = 0; bj < NBK; ++bj) {
        f32x4 dk4 = mfma_p<HP>(z4, sX + 16 * w * LC4, LC4, 1, sK + 16 * bj, LK4, 1, kC);
        dk4 = mfma_p<HP>(dk4, sY + 16 * w, 1, LC16, sQ + 16 * bj, LK4, 1, kC);
        const f32x4 dq4 = mfma_p<HP>(z4, sY + 16 * w * LC16, LC16, 1, sK + 16 * bj, LK4, 1, kC);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rb + i, cc = 16 * bj + mi;
            const float gm = __expf(sgam[r]), ekt = __expf(glast - sgam[r]);
            const float kv = sK[r * LK4 + cc], qv = sQ[r * LK4 + cc];
            const float dkv = dk4[i] + ekt * aKt[bj][i] + sbeta[r] * gm * aBk[bj][i];
            const float dqv = dq4[i] + gm * aGQ[bj][i];
            sq[i] += aGQ[bj][i] * qv;  // rowsum(dGQ o Q)
            sk[i] += aKt[bj][i] * kv;  // rowsum(dKt o K)
            sb[i] += aBk[bj][i] * kv;  // rowsum(dBk o K)
            if (r < L) {
                dko[static_cast<size_t>(r) * Hv * DK + cc] = dkv;
                dqo[static_cast<size_t>(r) * Hv * DK + cc] = dqv;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = rb + i;
        const float gm = __expf(sgam[r]), ekt = __expf(glast - sgam[r]);
        const float a = row_sum<16>(sq[i]) * gm, bk = row_sum<16>(sk[i]) * ekt,
                    cb = row_sum<16>(sb[i]) * gm;
        if (mi == 0) {
            sv[4][r] = a;
            sv[5][r] = bk;
            sv[6][r] = cb;
        }
    }
    // <dSe, S0> summed over the workgroup
    float dl = dglast;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) dl += __shfl_xor(dl, off);
    if (lane == 0) sv[7][w] = dl;
    lds_bar();
    if (tid < kC) {
        const int r = tid;
        float tsum = sv[5][r];
        for (int off = 1; off < 64; off <<= 1) tsum += __shfl_xor(tsum, off);
        const float dsx = sv[7][0] + sv[7][1] + sv[7][2] + sv[7][3];
        const float colE = scol[0][r] + scol[1][r] + scol[2][r] + scol[3][r];
        const float bt = sbeta[r];
        float dgam = sv[4][r] - sv[5][r] + bt * sv[6][r] + sv[0][r] - colE;
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
    const size_t rec = static_cast<size_t>(kC) * (3 * dk + dv + 2 * kC) + 8;
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
    hipLaunchKernelGGL((bscan_kernel<DK, DV, TD, std::is_same<TI, bf16_t>::value>), dim3(static_cast<unsigned>(2 * chains * (DV / 16))),
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
