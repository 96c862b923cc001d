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
//   T       = (I + A)^-1                                         (unit lower triangular)
//   U       = T diag(beta) V,     W = T diag(beta exp(gamma)) K  (independent of S)
//   Delta   = U - W S                                            (rows are d_r)
//   O       = scale (diag(exp(gamma)) Q S + (lower(Q K^T) o D) Delta)
//   S_next  = exp(gamma_last) S + K^T diag(exp(gamma_last - gamma)) Delta
//
// Only ratios exp(gamma_r - gamma_s) <= 1 appear, so no factor can overflow.
//
// Design (one workgroup of 4 wavefronts per (b, hv) chain, the chunks walked in order):
//   * the dk x dv fp32 state lives in MFMA accumulator registers for the whole sequence:
//     wavefront w owns value columns [w*DV/4, (w+1)*DV/4);
//   * Q, K, V of a chunk are staged in LDS once, converted bf16 -> fp16 (exact for the
//     normalised q/k; v must stay inside the fp16 range);
//   * KK^T and QK^T use exact fp16 inputs on v_mfma_f32_16x16x32_f16 with fp32 accumulation;
//   * the unit-lower-triangular inverse is done in fp32: 16x16 diagonal blocks by forward
//     substitution, off-diagonal blocks by block substitution on v_mfma_f32_16x16x4_f32;
//   * operands derived in fp32 (T, W, S, Delta, P) are rounded to fp16 for the 16x16x32 MFMAs
//     and every sum is accumulated in fp32 -- the fp32 state itself is never rounded;
//   * the accumulator layout of S and Delta (lane l holds rows 4(l/16)..4(l/16)+3 of column
//     l%16) is fed straight back as the B operand of the next product, with the k index of
//     the A operand permuted to match, so the state never leaves registers.
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mma16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 cat(f16x4 lo, f16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

constexpr int NW = 4;     // wavefronts per workgroup
constexpr int NT = 64 * NW;

template <int DK, int DV, int C> struct Cfg {
    static constexpr int NR = C / 16;        // 16-row tiles of a chunk
    static constexpr int NI = DK / 16;       // 16-row tiles of the state (key index)
    static constexpr int NJ = DV / 16 / NW;  // 16-column state tiles per wavefront
    static constexpr int NIW = NI / NW;      // 16-column tiles of W per wavefront
    static constexpr int KD = DK / 32;       // k-steps over the key index
    static constexpr int KC = C / 32;        // k-steps over the chunk
    static constexpr int PD = DK + 8;        // padded LDS pitches (halves / floats)
    static constexpr int PV = DV + 8;
    static constexpr int PC = C + 8;
    static constexpr int PF = C + 4;
    static_assert(DK % 64 == 0 && DV % 64 == 0 && C % 32 == 0, "unsupported chunk kernel shape");
    static_assert(NJ >= 1 && NIW >= 1, "unsupported chunk kernel shape");
};

template <int DK, int DV, int C> struct Smem {
    using F = Cfg<DK, DV, C>;
    f16 q[C][F::PD];      // Q rows
    f16 k[C][F::PD];      // K rows
    f16 kt[DK][F::PC];    // K^T
    f16 v[C][F::PV];      // V rows
    f16 tb[C][F::PC];     // T diag(beta)
    f16 tbg[C][F::PC];    // T diag(beta exp(gamma))
    f16 p[C][F::PC];      // lower(Q K^T) o D
    f16 wn[C][F::PD];     // -W
    float a[C][F::PF];    // A (strict lower); then T: diagonal blocks in place, off-diagonal
                          // blocks T[r][s] (r > s) stored transposed at a[s][r]
    float gam[C];         // gamma (chunk-local cumulative log-gate)
    float Gam[C];         // exp(gamma)
    float dec[C];         // exp(gamma_last - gamma)
    float bet[C];         // beta
};

// Block -> chain order that keeps the G value heads sharing one q/k head on one XCD
// (blocks i and i + 8 are dispatched to the same XCD), so their q/k reads meet in its L2.
__device__ __forceinline__ int chain_of_block(int blk, int nblk, int G) {
    if (G <= 1 || nblk % (8 * G) != 0) return blk;
    const int x = blk & 7, m = blk >> 3;
    return ((m / G) * 8 + x) * G + (m % G);
}

template <int DK, int DV, int C, typename TO>
__global__ void __launch_bounds__(NT)
chunk_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
             const bf16_t *__restrict__ v, const bf16_t *__restrict__ beta,
             const bf16_t *__restrict__ g, const float *__restrict__ s0, TO *__restrict__ o,
             float *__restrict__ sT, int T, int Hk, int Hv, float scale) {
    using F = Cfg<DK, DV, C>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    Smem<DK, DV, C> &sm = *reinterpret_cast<Smem<DK, DV, C> *>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int G = Hv / Hk;
    const int chain = chain_of_block(blockIdx.x, gridDim.x, G);
    const int b = chain / Hv, hv = chain - b * Hv, hq = hv / G;

    // lower(QK^T) tiles above the diagonal are never written: clear them once
    for (int idx = tid; idx < C * F::PC; idx += NT) (&sm.p[0][0])[idx] = f16(0.f);

    // ---- the state: tile (it, jt) holds rows 16it + 4lg + r, column colj(jt)
    f32x4 S[F::NI][F::NJ];
    const size_t sbase = static_cast<size_t>(chain) * DK * DV;
#pragma unroll
    for (int it = 0; it < F::NI; ++it)
#pragma unroll
        for (int jt = 0; jt < F::NJ; ++jt) {
            const int col = (wave * F::NJ + jt) * 16 + li;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[it][jt][r] = s0 ? s0[sbase + static_cast<size_t>(16 * it + 4 * lg + r) * DV + col]
                                  : 0.f;
        }

    // ---- raw inputs of the next chunk, prefetched into registers while the current chunk
    // is being computed (16-byte pieces; rows past the end of the sequence read as zero)
    constexpr int NQ = C * DK / 8 / NT, NV = C * DV / 8 / NT;
    static_assert(NQ >= 1 && NV >= 1 && C * DK / 8 % NT == 0 && C * DV / 8 % NT == 0, "tiling");
    u16x8 pq[NQ], pk[NQ], pv[NV];
    float pgv = 0.f, pbv = 0.f;
    auto prefetch = [&](int cidx) {
        const int tt = cidx * C, L = min(C, T - tt);
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            const int idx = tid + n * NT, r = idx / (DK / 8), cc = idx - r * (DK / 8);
            pq[n] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
            pk[n] = pq[n];
            if (r < L) {
                const size_t off = ((static_cast<size_t>(b) * T + tt + r) * Hk + hq) * DK + cc * 8;
                pq[n] = *reinterpret_cast<const u16x8 *>(q + off);
                pk[n] = *reinterpret_cast<const u16x8 *>(k + off);
            }
        }
#pragma unroll
        for (int n = 0; n < NV; ++n) {
            const int idx = tid + n * NT, r = idx / (DV / 8), cc = idx - r * (DV / 8);
            pv[n] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
            if (r < L)
                pv[n] = *reinterpret_cast<const u16x8 *>(
                    v + ((static_cast<size_t>(b) * T + tt + r) * Hv + hv) * DV + cc * 8);
        }
        pgv = 0.f;
        pbv = 0.f;
        if (tid < L) {
            const size_t gi = (static_cast<size_t>(b) * T + tt + tid) * Hv + hv;
            pgv = bf16_to_f32(g[gi]);
            pbv = bf16_to_f32(beta[gi]);
        }
    };

    const int nchunks = (T + C - 1) / C;
    if (nchunks > 0) prefetch(0);
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C;
        const int Lc = min(C, T - t0);
        __syncthreads();  // the previous chunk is done with every LDS buffer

        // ---- stage 0: this chunk's Q, K, V rows (bf16 -> fp16) and gates into LDS
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            const int idx = tid + n * NT, r = idx / (DK / 8), cc = idx - r * (DK / 8);
            f16x8 qh, kh;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qh[e] = f16(bf16_to_f32(pq[n][e]));
                kh[e] = f16(bf16_to_f32(pk[n][e]));
            }
            *reinterpret_cast<f16x8 *>(&sm.q[r][cc * 8]) = qh;
            *reinterpret_cast<f16x8 *>(&sm.k[r][cc * 8]) = kh;
        }
#pragma unroll
        for (int n = 0; n < NV; ++n) {
            const int idx = tid + n * NT, r = idx / (DV / 8), cc = idx - r * (DV / 8);
            f16x8 vh;
#pragma unroll
            for (int e = 0; e < 8; ++e) vh[e] = f16(bf16_to_f32(pv[n][e]));
            *reinterpret_cast<f16x8 *>(&sm.v[r][cc * 8]) = vh;
        }
        if (tid < 64) {
            float gv = pgv;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {  // inclusive prefix sum over the chunk
                const float y = __shfl_up(gv, off);
                if (lane >= off) gv += y;
            }
            const float glast = __shfl(gv, C - 1);
            if (tid < C) {
                sm.gam[tid] = gv;
                sm.Gam[tid] = expf(gv);
                sm.dec[tid] = expf(glast - gv);
                sm.bet[tid] = pbv;
            }
        }
        if (c + 1 < nchunks) prefetch(c + 1);
        __syncthreads();

        // ---- stage 0b: K^T
        for (int idx = tid; idx < DK * (C / 8); idx += NT) {
            const int i = idx % DK, s8 = idx / DK;
            f16x8 x;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = sm.k[s8 * 8 + e][i];
            *reinterpret_cast<f16x8 *>(&sm.kt[i][s8 * 8]) = x;
        }

        // ---- stage 1: KK^T -> A (fp32), QK^T -> P (fp16); lower-triangular tiles only
        {
            constexpr int NTRI = F::NR * (F::NR + 1) / 2;
            for (int pidx = wave; pidx < 2 * NTRI; pidx += NW) {
                const bool isP = pidx >= NTRI;
                const int pp = isP ? pidx - NTRI : pidx;
                int rt = 0;
                while ((rt + 1) * (rt + 2) / 2 <= pp) ++rt;
                const int st = pp - rt * (rt + 1) / 2;
                const f16 *arow = isP ? &sm.q[16 * rt + li][0] : &sm.k[16 * rt + li][0];
                const f16 *brow = &sm.k[16 * st + li][0];
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < F::KD; ++kk)
                    acc = mma16(*reinterpret_cast<const f16x8 *>(arow + 32 * kk + 8 * lg),
                                *reinterpret_cast<const f16x8 *>(brow + 32 * kk + 8 * lg), acc);
                const int s = 16 * st + li;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int r = 16 * rt + 4 * lg + rr;
                    const float d = (s <= r) ? expf(sm.gam[r] - sm.gam[s]) : 0.f;
                    if (isP)
                        sm.p[r][s] = f16(acc[rr] * d);
                    else
                        sm.a[r][s] = (s < r) ? sm.bet[r] * d * acc[rr] : 0.f;
                }
            }
        }
        __syncthreads();

        // ---- stage 2a: inverse of each 16x16 diagonal block of I + A (forward substitution)
        if (wave < F::NR && lane < 16) {
            const int base = 16 * wave;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == lane) ? 1.f : 0.f;
#pragma unroll
                for (int s = 0; s < r; ++s) acc -= sm.a[base + r][base + s] * x[s];
                x[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.a[base + r][base + lane] = x[r];
        }
        __syncthreads();

        // ---- stage 2b: off-diagonal blocks, T_ab = -T_aa sum_{b<=c<a} A_ac T_cb, by distance
        for (int d = 1; d < F::NR; ++d) {
            if (wave < F::NR - d) {
                const int bb = wave, aa = wave + d;
                f32x4 X = {0.f, 0.f, 0.f, 0.f};
                for (int cc = bb; cc < aa; ++cc) {
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const int kx = 4 * ks + lg;
                        const float av = sm.a[16 * aa + li][16 * cc + kx];  // A_ac[m][k]
                        const float bv = (cc == bb) ? sm.a[16 * bb + kx][16 * bb + li]
                                                    : sm.a[16 * bb + li][16 * cc + kx];  // T_cb[k][n]
                        X = mma32(av, bv, X);
                    }
                }
                f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    Y = mma32(sm.a[16 * aa + li][16 * aa + 4 * lg + rr], X[rr], Y);  // T_aa X
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) sm.a[16 * bb + li][16 * aa + 4 * lg + rr] = -Y[rr];
            }
            __syncthreads();
        }

        // ---- stage 2c: T diag(beta) and T diag(beta exp(gamma)) in fp16
        for (int idx = tid; idx < C * C; idx += NT) {
            const int r = idx / C, s = idx - r * C;
            float tv = 0.f;
            if (s <= r) tv = ((r >> 4) == (s >> 4)) ? sm.a[r][s] : sm.a[s][r];
            const float tb = tv * sm.bet[s];
            sm.tb[r][s] = f16(tb);
            sm.tbg[r][s] = f16(tb * sm.Gam[s]);
        }
        __syncthreads();

        // ---- stage 3: U = T diag(beta) V (kept in registers), -W to LDS
        f32x4 U[F::NR][F::NJ];
#pragma unroll
        for (int rt = 0; rt < F::NR; ++rt)
#pragma unroll
            for (int jt = 0; jt < F::NJ; ++jt) U[rt][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jt = 0; jt < F::NJ; ++jt) {
            const int col = (wave * F::NJ + jt) * 16 + li;
#pragma unroll
            for (int kk = 0; kk < F::KC; ++kk) {
                f16x8 bv;
#pragma unroll
                for (int e = 0; e < 8; ++e) bv[e] = sm.v[32 * kk + 8 * lg + e][col];
#pragma unroll
                for (int rt = 0; rt < F::NR; ++rt)
                    if (32 * kk <= 16 * rt + 15)
                        U[rt][jt] = mma16(
                            *reinterpret_cast<const f16x8 *>(&sm.tb[16 * rt + li][32 * kk + 8 * lg]),
                            bv, U[rt][jt]);
            }
        }
#pragma unroll
        for (int iw = 0; iw < F::NIW; ++iw) {
            const int icol = (wave * F::NIW + iw) * 16 + li;
            f32x4 Wt[F::NR];
#pragma unroll
            for (int rt = 0; rt < F::NR; ++rt) Wt[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < F::KC; ++kk) {
                const f16x8 bk = *reinterpret_cast<const f16x8 *>(&sm.kt[icol][32 * kk + 8 * lg]);
#pragma unroll
                for (int rt = 0; rt < F::NR; ++rt)
                    if (32 * kk <= 16 * rt + 15)
                        Wt[rt] = mma16(
                            *reinterpret_cast<const f16x8 *>(&sm.tbg[16 * rt + li][32 * kk + 8 * lg]),
                            bk, Wt[rt]);
            }
#pragma unroll
            for (int rt = 0; rt < F::NR; ++rt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) sm.wn[16 * rt + 4 * lg + rr][icol] = f16(-Wt[rt][rr]);
        }
        __syncthreads();

        // ---- stage 4 (sequential part): Delta, O, next state
        // S as fp16 B operands over the key index: slot e < 4 -> tile 2kk row 4lg+e,
        // slot e >= 4 -> tile 2kk+1 row 4lg+e-4.  A operands read the matching k indices.
        f16x8 bS[F::KD][F::NJ];
#pragma unroll
        for (int kk = 0; kk < F::KD; ++kk)
#pragma unroll
            for (int jt = 0; jt < F::NJ; ++jt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bS[kk][jt][e] = f16(S[2 * kk][jt][e]);
                    bS[kk][jt][4 + e] = f16(S[2 * kk + 1][jt][e]);
                }
        // Delta = U + (-W) S   (accumulated onto U)
#pragma unroll
        for (int rt = 0; rt < F::NR; ++rt)
#pragma unroll
            for (int kk = 0; kk < F::KD; ++kk) {
                const f16 *wr = &sm.wn[16 * rt + li][32 * kk + 4 * lg];
                const f16x8 a = cat(*reinterpret_cast<const f16x4 *>(wr),
                                    *reinterpret_cast<const f16x4 *>(wr + 16));
#pragma unroll
                for (int jt = 0; jt < F::NJ; ++jt) U[rt][jt] = mma16(a, bS[kk][jt], U[rt][jt]);
            }
        // O = diag(exp(gamma)) Q S + P Delta
        f32x4 O[F::NR][F::NJ];
#pragma unroll
        for (int rt = 0; rt < F::NR; ++rt) {
#pragma unroll
            for (int jt = 0; jt < F::NJ; ++jt) O[rt][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < F::KD; ++kk) {
                const f16 *qr = &sm.q[16 * rt + li][32 * kk + 4 * lg];
                const f16x8 a = cat(*reinterpret_cast<const f16x4 *>(qr),
                                    *reinterpret_cast<const f16x4 *>(qr + 16));
#pragma unroll
                for (int jt = 0; jt < F::NJ; ++jt) O[rt][jt] = mma16(a, bS[kk][jt], O[rt][jt]);
            }
#pragma unroll
            for (int jt = 0; jt < F::NJ; ++jt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) O[rt][jt][rr] *= sm.Gam[16 * rt + 4 * lg + rr];
        }
        // Delta as fp16 B operands over the chunk index, plain and decayed to the chunk end
        f16x8 bD[F::KC][F::NJ], bDs[F::KC][F::NJ];
#pragma unroll
        for (int kk = 0; kk < F::KC; ++kk)
#pragma unroll
            for (int jt = 0; jt < F::NJ; ++jt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s0i = 32 * kk + 4 * lg + e, s1i = s0i + 16;
                    const float d0 = U[2 * kk][jt][e], d1 = U[2 * kk + 1][jt][e];
                    bD[kk][jt][e] = f16(d0);
                    bD[kk][jt][4 + e] = f16(d1);
                    bDs[kk][jt][e] = f16(d0 * sm.dec[s0i]);
                    bDs[kk][jt][4 + e] = f16(d1 * sm.dec[s1i]);
                }
#pragma unroll
        for (int rt = 0; rt < F::NR; ++rt)
#pragma unroll
            for (int kk = 0; kk < F::KC; ++kk)
                if (32 * kk <= 16 * rt + 15) {
                    const f16 *pr = &sm.p[16 * rt + li][32 * kk + 4 * lg];
                    const f16x8 a = cat(*reinterpret_cast<const f16x4 *>(pr),
                                        *reinterpret_cast<const f16x4 *>(pr + 16));
#pragma unroll
                    for (int jt = 0; jt < F::NJ; ++jt) O[rt][jt] = mma16(a, bD[kk][jt], O[rt][jt]);
                }
#pragma unroll
        for (int rt = 0; rt < F::NR; ++rt)
#pragma unroll
            for (int jt = 0; jt < F::NJ; ++jt) {
                const int col = (wave * F::NJ + jt) * 16 + li;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int r = 16 * rt + 4 * lg + rr;
                    if (r < Lc)
                        store_f32(o + ((static_cast<size_t>(b) * T + t0 + r) * Hv + hv) * DV + col,
                                  scale * O[rt][jt][rr]);
                }
            }
        // S = exp(gamma_last) S + K^T diag(exp(gamma_last - gamma)) Delta
        const float GC = sm.Gam[C - 1];
#pragma unroll
        for (int it = 0; it < F::NI; ++it) {
#pragma unroll
            for (int jt = 0; jt < F::NJ; ++jt) S[it][jt] *= GC;
#pragma unroll
            for (int kk = 0; kk < F::KC; ++kk) {
                const f16 *kr = &sm.kt[16 * it + li][32 * kk + 4 * lg];
                const f16x8 a = cat(*reinterpret_cast<const f16x4 *>(kr),
                                    *reinterpret_cast<const f16x4 *>(kr + 16));
#pragma unroll
                for (int jt = 0; jt < F::NJ; ++jt) S[it][jt] = mma16(a, bDs[kk][jt], S[it][jt]);
            }
        }
    }

    if (sT) {
#pragma unroll
        for (int it = 0; it < F::NI; ++it)
#pragma unroll
            for (int jt = 0; jt < F::NJ; ++jt) {
                const int col = (wave * F::NJ + jt) * 16 + li;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sT[sbase + static_cast<size_t>(16 * it + 4 * lg + r) * DV + col] = S[it][jt][r];
            }
    }
}

template <int DK, int DV, int C, typename TO> hipError_t launch_typed(const PrefillArgs &a) {
    auto kern = chunk_kernel<DK, DV, C, TO>;
    const size_t lds = sizeof(Smem<DK, DV, C>);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    const unsigned nblk = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hv);
    hipLaunchKernelGGL(kern, dim3(nblk), dim3(NT), lds, a.stream,
                       static_cast<const bf16_t *>(a.q), static_cast<const bf16_t *>(a.k),
                       static_cast<const bf16_t *>(a.v), static_cast<const bf16_t *>(a.beta),
                       static_cast<const bf16_t *>(a.g), a.s0, static_cast<TO *>(a.o), a.sT, a.T,
                       a.Hk, a.Hv, a.scale);
    return hipGetLastError();
}

template <int DK, int DV, int C> hipError_t launch_out(const PrefillArgs &a) {
    return a.out_dt == GDN_F32 ? launch_typed<DK, DV, C, float>(a)
                               : launch_typed<DK, DV, C, bf16_t>(a);
}

template <int DK, int DV> hipError_t launch_chunk(const PrefillArgs &a) {
    return a.chunk == 64 ? launch_out<DK, DV, 64>(a) : launch_out<DK, DV, 32>(a);
}

}  // namespace

bool chunk_mfma_supports(const PrefillArgs &a) {
    return a.in_dt == GDN_BF16 && (a.dk == 64 || a.dk == 128) && (a.dv == 64 || a.dv == 128) &&
           (a.chunk == 32 || a.chunk == 64);
}

size_t chunk_mfma_workspace(const PrefillArgs &) { return 0; }

hipError_t launch_chunk_mfma(const PrefillArgs &a) {
    if (!chunk_mfma_supports(a)) return hipErrorNotSupported;
    if (a.dk == 128)
        return a.dv == 128 ? launch_chunk<128, 128>(a) : launch_chunk<128, 64>(a);
    return a.dv == 128 ? launch_chunk<64, 128>(a) : launch_chunk<64, 64>(a);
}

}  // namespace gdn
