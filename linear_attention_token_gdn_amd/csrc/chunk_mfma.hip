// chunk_mfma.hip -- chunk-parallel prefill of the gated delta rule on gfx950 matrix cores.
//
// The rule (explainer page "論文解説: Qwen3.8-Next の設計", ta-paperlens.web.app, section
// "GDNの中身", Eq. (1)):  S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
// o_t = scale * S_t^T q_t.  Writing S_r = alpha_r S_{r-1} + k_r d_r^T with
// d_r = beta_r (v_r - alpha_r S_{r-1}^T k_r) and unrolling it over a chunk of C tokens that
// starts from state S gives an exact rewriting (no approximation):
//
//   gamma_r = sum_{s<=r} g_s (chunk-local),  D_rs = exp(gamma_r - gamma_s)  (s <= r)
//   A       = strictly_lower(diag(beta) (K K^T o D))           (o = elementwise product)
//   U       = (I + A)^-1 diag(beta) V                            } independent of S: the
//   W       = (I + A)^-1 diag(beta exp(gamma)) K                 } "WY/UT" transform
//   Delta   = U - W S                                            (rows are d_r)
//   O       = scale (diag(exp(gamma)) Q S + (lower(Q K^T) o D) Delta)
//   S_next  = exp(gamma_last) S + K^T diag(exp(gamma_last - gamma)) Delta
//
// Only ratios exp(gamma_r - gamma_s) <= 1 appear, so no factor can overflow.
//
// Design: one workgroup of D/16 wavefronts per (b, hv) chain walks the chunks in order.
//   * The D x D fp32 state lives in MFMA accumulator registers for the whole sequence;
//     wavefront w owns value columns [16w, 16w + 16).
//   * Q, K, V of the next chunk are prefetched into registers while the current chunk runs,
//     then staged in LDS as fp16 (exact for normalised q/k; v must stay inside fp16 range).
//   * KK^T and QK^T: v_mfma_f32_16x16x32_f16 on exact inputs, fp32 accumulation.
//   * (I + A)^-1 is never formed: the 16x16 diagonal blocks are inverted in fp32 by forward
//     substitution, and U, W come from a blocked forward substitution over 16-row blocks,
//     X_a = T_aa (R_a - sum_{c<a} A_ac X_c), on v_mfma_f32_16x16x16_f16 -- every wavefront
//     solves its own two 16-column panels (of diag(beta) V and diag(beta e^gamma) K), so the
//     solve needs no barrier.
//   * Derived fp32 operands (W, S, Delta, P, X) are rounded to fp16 for the MFMAs; every sum
//     accumulates in fp32 and the fp32 state itself is never rounded.
//   * The accumulator layout (lane l holds rows 4(l/16)..4(l/16)+3 of column l%16) is fed
//     straight back as a B operand, with the k index of the A operand permuted to match, so
//     the state and the solve panels never leave registers.
//   * O is staged in LDS and written with coalesced 16-byte stores at the top of the next
//     chunk, before the next prefetch is issued (the vector-memory counter is in-order).
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma_k32(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k16(f16x4 a, f16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 cat(f16x4 lo, f16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f16x4 to_f16x4(f32x4 x) {
    return f16x4{f16(x[0]), f16(x[1]), f16(x[2]), f16(x[3])};
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Workgroup barrier that waits only for this wave's LDS traffic.  __syncthreads() also waits
// for every outstanding global load and store, which would stall each chunk on the prefetch of
// the next chunk and on the output stores; nothing here reads global memory written by another
// wave, so LDS completion is all a barrier has to guarantee.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D, int C> struct Cfg {
    static constexpr int NW = D / 16;       // wavefronts: one 16-column state tile each
    static constexpr int NT = 64 * NW;
    static constexpr int NR = C / 16;       // 16-row blocks of a chunk
    static constexpr int NI = D / 16;       // 16-row tiles of the state (key index)
    static constexpr int KD = D / 32;       // 32-wide k-steps over the key index
    static constexpr int KC = C / 32;       // 32-wide k-steps over the chunk
    // padded LDS pitches (halves).  Arrays read as 16-byte A-operand rows (q, k, -W over the
    // head dimension; P, K^T over the chunk) take 16 extra halves: lanes li = 0..15 of one
    // half-wavefront then read rows li and 16-byte slots 4lg (lg = 0, 1) from distinct banks
    // (the row pitch is 8 mod 32 dwords).  v and A, read in 2- and 8-byte pieces, take 8.
    static constexpr int PQ = D + 16;
    static constexpr int PV = D + 8;
    static constexpr int PT = C + 16;
    static constexpr int PA = C + 8;
    static constexpr int PO = D + 4;        // output staging pitch (floats)
    static constexpr int NQ = C * D / 8 / NT;  // 16-byte pieces of q (or k, v) per thread
    static constexpr int NO = C * D / 4 / NT;  // 16-byte pieces of o per thread
    static_assert((D == 64 || D == 128) && (C == 32 || C == 64), "chunk kernel shape");
    static_assert(NQ >= 1 && (C * D / 8) % NT == 0 && (C * D / 4) % NT == 0, "tiling");
};

// Columns of q, k, -W (head dimension) and of P, K^T (chunk index) are stored permuted within
// each 32-wide k-step: index 16h + 4g + e (h < 2, g < 4, e < 4) sits at 8g + 4h + e.  The
// 8 values a lane (li, g) feeds one 16x16x32 MFMA -- k = 4g..4g+3 of both 16-wide halves,
// the order in which a B operand built from two accumulator tiles holds them -- are then
// contiguous: one 16-byte LDS read instead of two 8-byte ones.  QK^T and KK^T sum over the
// head dimension in the stored order on both sides, which is the same sum.
__device__ __forceinline__ constexpr int kperm(int c) {
    return (c & ~31) | (((c >> 2) & 3) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
}
__device__ __forceinline__ constexpr int kunperm(int p) {
    return (p & ~31) | (((p >> 2) & 1) << 4) | (((p >> 3) & 3) << 2) | (p & 3);
}

template <int D, int C> struct Smem {
    using F = Cfg<D, C>;
    f16 q[C][F::PQ];          // Q rows (columns permuted)
    f16 k[C][F::PQ];          // K rows (columns permuted)
    f16 kt[D][F::PT];         // K^T (columns permuted)
    f16 v[C][F::PV];          // V rows
    f16 p[C][F::PT];          // lower(Q K^T) o D (columns permuted)
    f16 wn[C][F::PQ];         // -W (columns permuted)
    f16 an[C][F::PA];         // -A, off-diagonal 16x16 blocks (lower)
    f16 td[F::NR][16][24];    // inverses of the diagonal blocks of I + A, fp16
    float ad[F::NR][16][20];  // diagonal blocks of A, fp32
    float gam[C];             // gamma (chunk-local cumulative log-gate)
    float Gam[C];             // exp(gamma)
    float dec[C];             // exp(gamma_last - gamma)
    float bet[C];             // beta
    float ost[C][F::PO];      // scaled output of the chunk, waiting to be stored
};

// Block -> chain order that keeps the G value heads sharing one q/k head on one XCD
// (blocks i and i + 8 are dispatched to the same XCD), so their q/k reads meet in its L2.
__device__ __forceinline__ int chain_of_block(int blk, int nblk, int G) {
    if (G <= 1 || nblk % (8 * G) != 0) return blk;
    const int x = blk & 7, m = blk >> 3;
    return ((m / G) * 8 + x) * G + (m % G);
}

template <typename TO> __device__ __forceinline__ void store4(TO *p, f32x4 x);
template <> __device__ __forceinline__ void store4<float>(float *p, f32x4 x) {
    *reinterpret_cast<f32x4 *>(p) = x;
}
template <> __device__ __forceinline__ void store4<bf16_t>(bf16_t *p, f32x4 x) {
    *reinterpret_cast<u16x4 *>(p) =
        u16x4{f32_to_bf16(x[0]), f32_to_bf16(x[1]), f32_to_bf16(x[2]), f32_to_bf16(x[3])};
}

template <int D, int C, typename TO>
__global__ void __launch_bounds__((Cfg<D, C>::NT))
chunk_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
             const bf16_t *__restrict__ v, const bf16_t *__restrict__ beta,
             const bf16_t *__restrict__ g, const float *__restrict__ s0, TO *__restrict__ o,
             float *__restrict__ sT, int T, const int32_t *__restrict__ cu, unsigned flags,
             int Hk, int Hv, float scale) {
    using F = Cfg<D, C>;
    constexpr int NT = F::NT, NR = F::NR;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    Smem<D, C> &sm = *reinterpret_cast<Smem<D, C> *>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;
    const int G = Hv / Hk;
    const int chain = chain_of_block(blockIdx.x, gridDim.x, G);
    const int b = chain / Hv, hv = chain - b * Hv, hq = hv / G;
    const int col = 16 * wave + li;  // the state column this lane holds
    size_t base;  // this sequence's first row and length
    int len;
    seq_range(cu, T, b, base, len);

    // ---- the state: tile it holds rows 16it + 4lg + r of column `col`
    f32x4 S[F::NI];
    const size_t sbase = static_cast<size_t>(chain) * D * D;
    if (s0 != nullptr) {  // one branch, so that all loads are in flight together
#pragma unroll
        for (int it = 0; it < F::NI; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[it][r] = s0[sbase + static_cast<size_t>(16 * it + 4 * lg + r) * D + col];
    } else {
#pragma unroll
        for (int it = 0; it < F::NI; ++it) S[it] = zero4();
    }

    // ---- raw inputs of the next chunk, prefetched into registers (rows past the end read as 0)
    u16x8 pq[F::NQ], pk[F::NQ], pv[F::NQ];
    bf16_t pg = 0, pb = 0;
    auto prefetch = [&](int cidx) {
        const int tt = cidx * C, L = min(C, len - tt);
#pragma unroll
        for (int n = 0; n < F::NQ; ++n) {
            const int idx = tid + n * NT, r = idx / (D / 8), cc = idx - r * (D / 8);
            pq[n] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
            pk[n] = pq[n];
            pv[n] = pq[n];
            if (r < L) {
                const size_t row = base + tt + r;
                const size_t oq = (row * Hk + hq) * D + cc * 8, ov = (row * Hv + hv) * D + cc * 8;
                pq[n] = *reinterpret_cast<const u16x8 *>(q + oq);
                pk[n] = *reinterpret_cast<const u16x8 *>(k + oq);
                pv[n] = *reinterpret_cast<const u16x8 *>(v + ov);
            }
        }
        pg = 0;
        pb = 0;
        if (tid < L) {
            const size_t gi = (base + tt + tid) * Hv + hv;
            pg = g[gi];
            pb = beta[gi];
        }
    };

    const int nchunks = (len + C - 1) / C;
    if (nchunks > 0) prefetch(0);
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C;
        lds_barrier();  // the previous chunk is done with every LDS buffer

        // ---- stage 0: stage this chunk in LDS, store the previous chunk's output, prefetch
#pragma unroll
        for (int n = 0; n < F::NQ; ++n) {
            const int idx = tid + n * NT, r = idx / (D / 8), cc = idx - r * (D / 8);
            float qs = 1.f, ks = 1.f;  // L2 normalisation: the D/8 consecutive lanes of a row
            if (flags & GDN_QK_L2NORM) {
                float qq = 0.f, kq = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float a = bf16_to_f32(pq[n][e]), c2 = bf16_to_f32(pk[n][e]);
                    qq += a * a;
                    kq += c2 * c2;
                }
#pragma unroll
                for (int off = 1; off < D / 8; off <<= 1) {
                    qq += __shfl_xor(qq, off);
                    kq += __shfl_xor(kq, off);
                }
                qs = inv_norm_from_sumsq(qq);
                ks = inv_norm_from_sumsq(kq);
            }
            f16x8 qh, kh, vh;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qh[e] = f16(qs * bf16_to_f32(pq[n][e]));
                kh[e] = f16(ks * bf16_to_f32(pk[n][e]));
                vh[e] = f16(bf16_to_f32(pv[n][e]));
            }
            // columns 8cc .. 8cc+7 are two runs of 4 in the permuted order
            const int c0 = kperm(cc * 8), c1 = kperm(cc * 8 + 4);
            *reinterpret_cast<f16x4 *>(&sm.q[r][c0]) = f16x4{qh[0], qh[1], qh[2], qh[3]};
            *reinterpret_cast<f16x4 *>(&sm.q[r][c1]) = f16x4{qh[4], qh[5], qh[6], qh[7]};
            *reinterpret_cast<f16x4 *>(&sm.k[r][c0]) = f16x4{kh[0], kh[1], kh[2], kh[3]};
            *reinterpret_cast<f16x4 *>(&sm.k[r][c1]) = f16x4{kh[4], kh[5], kh[6], kh[7]};
            *reinterpret_cast<f16x8 *>(&sm.v[r][cc * 8]) = vh;
        }
        if (wave == 0) {
            const int L = min(C, len - t0);  // rows past the end: g = beta = 0
            float gv = lane < L ? log_alpha_from_input(bf16_to_f32(pg), flags) : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {  // inclusive prefix sum over the chunk
                const float y = __shfl_up(gv, off);
                if (lane >= off) gv += y;
            }
            const float glast = __shfl(gv, C - 1);
            if (lane < C) {
                sm.gam[lane] = gv;
                sm.Gam[lane] = __expf(gv);
                sm.dec[lane] = __expf(glast - gv);
                sm.bet[lane] = lane < L ? beta_from_input(bf16_to_f32(pb), flags) : 0.f;
            }
        }
        if (c > 0) {
            const int tp = t0 - C;  // the previous chunk is always a full one
#pragma unroll
            for (int n = 0; n < F::NO; ++n) {
                const int idx = tid + n * NT, r = idx / (D / 4), cc = idx - r * (D / 4);
                const f32x4 x = *reinterpret_cast<const f32x4 *>(&sm.ost[r][cc * 4]);
                store4<TO>(o + ((base + tp + r) * Hv + hv) * D + cc * 4, x);
            }
        }
        if (c + 1 < nchunks) prefetch(c + 1);
        lds_barrier();

        // ---- stage 1: KK^T -> A, QK^T -> P (lower-triangular 16x16 tiles), and K^T
        for (int job = wave; job < 2 * NR; job += F::NW) {
            const bool isq = job >= NR;
            const int rt = isq ? job - NR : job;
            const f16 *arow = isq ? &sm.q[16 * rt + li][0] : &sm.k[16 * rt + li][0];
            f16x8 af[F::KD];
#pragma unroll
            for (int kk = 0; kk < F::KD; ++kk)
                af[kk] = *reinterpret_cast<const f16x8 *>(arow + 32 * kk + 8 * lg);
            float gr[4], br[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                gr[rr] = sm.gam[16 * rt + 4 * lg + rr];
                br[rr] = sm.bet[16 * rt + 4 * lg + rr];
            }
#pragma unroll
            for (int st = 0; st < NR; ++st) {
                if (st > rt) break;
                f32x4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < F::KD; ++kk)
                    acc = mma_k32(af[kk],
                                  *reinterpret_cast<const f16x8 *>(&sm.k[16 * st + li][32 * kk + 8 * lg]),
                                  acc);
                const int s = 16 * st + li;
                const float gs = sm.gam[s];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int r = 16 * rt + 4 * lg + rr;
                    const float d = (s <= r) ? __expf(gr[rr] - gs) : 0.f;
                    if (isq) {
                        sm.p[r][kperm(s)] = f16(acc[rr] * d);
                    } else {
                        const float av = (s < r) ? br[rr] * d * acc[rr] : 0.f;
                        if (st == rt)
                            sm.ad[rt][4 * lg + rr][li] = av;
                        else
                            sm.an[r][s] = f16(-av);
                    }
                }
            }
            if (isq && rt + 1 < NR) {  // the tile right of the diagonal is read by P Delta
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    sm.p[16 * rt + 4 * lg + rr][kperm(16 * (rt + 1) + li)] = f16(0.f);
            }
        }
        for (int idx = tid; idx < D * (C / 8); idx += NT) {
            const int i = idx % D, s8 = idx / D, ki = kperm(i);
            f16x8 x;  // stored positions 8 s8 .. 8 s8 + 7 of row i of K^T
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = sm.k[kunperm(s8 * 8 + e)][ki];
            *reinterpret_cast<f16x8 *>(&sm.kt[i][s8 * 8]) = x;
        }
        lds_barrier();

        // ---- stage 2: inverse of each 16x16 diagonal block of I + A (forward substitution)
        if (wave < NR && lane < 16) {
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == lane) ? 1.f : 0.f;
#pragma unroll
                for (int s = 0; s < r; ++s) acc -= sm.ad[wave][r][s] * x[s];
                x[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.td[wave][r][lane] = f16(x[r]);
        }
        lds_barrier();

        // ---- stage 3: blocked forward substitution for this wave's panels,
        //      U[:, 16w..] = (I+A)^-1 diag(beta) V[:, 16w..]  (kept in registers)
        //      W[:, 16w..] = (I+A)^-1 diag(beta e^gamma) K[:, 16w..]  (-W to LDS)
        f32x4 U[NR], Wp[NR];
#pragma unroll
        for (int a = 0; a < NR; ++a) {
            const f16x4 kv4 = *reinterpret_cast<const f16x4 *>(&sm.kt[col][kperm(16 * a + 4 * lg)]);
            f32x4 yu, yw;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = 16 * a + 4 * lg + rr;
                const float br = sm.bet[r];
                yu[rr] = br * float(sm.v[r][col]);
                yw[rr] = br * sm.Gam[r] * float(kv4[rr]);
            }
#pragma unroll
            for (int cb = 0; cb < a; ++cb) {
                const f16x4 an = *reinterpret_cast<const f16x4 *>(&sm.an[16 * a + li][16 * cb + 4 * lg]);
                yu = mma_k16(an, to_f16x4(U[cb]), yu);
                yw = mma_k16(an, to_f16x4(Wp[cb]), yw);
            }
            const f16x4 td = *reinterpret_cast<const f16x4 *>(&sm.td[a][li][4 * lg]);
            U[a] = mma_k16(td, to_f16x4(yu), zero4());
            Wp[a] = mma_k16(td, to_f16x4(yw), zero4());
        }
#pragma unroll
        for (int a = 0; a < NR; ++a)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sm.wn[16 * a + 4 * lg + rr][kperm(col)] = f16(-Wp[a][rr]);
        lds_barrier();

        // ---- stage 4 (sequential part): Delta, O, next state
        // S as fp16 B operands over the key index: slot e < 4 -> tile 2kk row 4lg+e,
        // slot e >= 4 -> tile 2kk+1 row 4lg+e-4.  A operands read the matching k indices.
        f16x8 bS[F::KD];
#pragma unroll
        for (int kk = 0; kk < F::KD; ++kk)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bS[kk][e] = f16(S[2 * kk][e]);
                bS[kk][4 + e] = f16(S[2 * kk + 1][e]);
            }
        // Delta = U + (-W) S   (accumulated onto U);  O = diag(e^gamma) Q S
        f32x4 O[NR];
#pragma unroll
        for (int rt = 0; rt < NR; ++rt) {
            O[rt] = zero4();
#pragma unroll
            for (int kk = 0; kk < F::KD; ++kk) {
                const f16x8 aw = *reinterpret_cast<const f16x8 *>(&sm.wn[16 * rt + li][32 * kk + 8 * lg]);
                const f16x8 aq = *reinterpret_cast<const f16x8 *>(&sm.q[16 * rt + li][32 * kk + 8 * lg]);
                U[rt] = mma_k32(aw, bS[kk], U[rt]);
                O[rt] = mma_k32(aq, bS[kk], O[rt]);
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) O[rt][rr] *= sm.Gam[16 * rt + 4 * lg + rr];
        }
        // Delta as fp16 B operands over the chunk index, plain and decayed to the chunk end
        f16x8 bD[F::KC], bDs[F::KC];
#pragma unroll
        for (int kk = 0; kk < F::KC; ++kk)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s0i = 32 * kk + 4 * lg + e, s1i = s0i + 16;
                const float d0 = U[2 * kk][e], d1 = U[2 * kk + 1][e];
                bD[kk][e] = f16(d0);
                bD[kk][4 + e] = f16(d1);
                bDs[kk][e] = f16(d0 * sm.dec[s0i]);
                bDs[kk][4 + e] = f16(d1 * sm.dec[s1i]);
            }
        // O += P Delta, staged for the store at the top of the next chunk
#pragma unroll
        for (int rt = 0; rt < NR; ++rt) {
#pragma unroll
            for (int kk = 0; kk < F::KC; ++kk)
                if (32 * kk <= 16 * rt + 15)
                    O[rt] = mma_k32(*reinterpret_cast<const f16x8 *>(&sm.p[16 * rt + li][32 * kk + 8 * lg]),
                                    bD[kk], O[rt]);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sm.ost[16 * rt + 4 * lg + rr][col] = scale * O[rt][rr];
        }
        // S = e^gamma_last S + K^T diag(e^(gamma_last - gamma)) Delta
        const float GC = sm.Gam[C - 1];
#pragma unroll
        for (int it = 0; it < F::NI; ++it) {
            S[it] *= GC;
#pragma unroll
            for (int kk = 0; kk < F::KC; ++kk)
                S[it] = mma_k32(*reinterpret_cast<const f16x8 *>(&sm.kt[16 * it + li][32 * kk + 8 * lg]),
                                bDs[kk], S[it]);
        }
    }

    // ---- the last chunk's output (rows past T are not stored) and the final state
    lds_barrier();
    if (nchunks > 0) {
        const int tp = (nchunks - 1) * C, L = len - tp;
#pragma unroll
        for (int n = 0; n < F::NO; ++n) {
            const int idx = tid + n * NT, r = idx / (D / 4), cc = idx - r * (D / 4);
            if (r < L) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(&sm.ost[r][cc * 4]);
                store4<TO>(o + ((base + tp + r) * Hv + hv) * D + cc * 4, x);
            }
        }
    }
    if (sT) {
#pragma unroll
        for (int it = 0; it < F::NI; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sT[sbase + static_cast<size_t>(16 * it + 4 * lg + r) * D + col] = S[it][r];
    }
}

template <int D, int C, typename TO> hipError_t launch_typed(const PrefillArgs &a) {
    auto kern = chunk_kernel<D, C, TO>;
    const size_t lds = sizeof(Smem<D, C>);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    const unsigned nblk = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hv);
    hipLaunchKernelGGL(kern, dim3(nblk), dim3(Cfg<D, C>::NT), lds, a.stream,
                       static_cast<const bf16_t *>(a.q), static_cast<const bf16_t *>(a.k),
                       static_cast<const bf16_t *>(a.v), static_cast<const bf16_t *>(a.beta),
                       static_cast<const bf16_t *>(a.g), a.s0, static_cast<TO *>(a.o), a.sT, a.T,
                       a.cu, a.flags, a.Hk, a.Hv, a.scale);
    return hipGetLastError();
}

template <int D, int C> hipError_t launch_out(const PrefillArgs &a) {
    return a.out_dt == GDN_F32 ? launch_typed<D, C, float>(a) : launch_typed<D, C, bf16_t>(a);
}

template <int D> hipError_t launch_chunk(const PrefillArgs &a) {
    return a.chunk == 64 ? launch_out<D, 64>(a) : launch_out<D, 32>(a);
}

}  // namespace

bool chunk_mfma_supports(const PrefillArgs &a) {
    return a.in_dt == GDN_BF16 && a.dk == a.dv && (a.dk == 64 || a.dk == 128) &&
           (a.chunk == 32 || a.chunk == 64);
}

size_t chunk_mfma_workspace(const PrefillArgs &) { return 0; }

hipError_t launch_chunk_mfma(const PrefillArgs &a) {
    if (!chunk_mfma_supports(a)) return hipErrorNotSupported;
    return a.dk == 128 ? launch_chunk<128>(a) : launch_chunk<64>(a);
}

}  // namespace gdn
