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

// ---------------------------------------------------------------------------------------
// Several tokens per call on the matrix cores: bf16 inputs, dk = dv = D in {64, 128}.
//
// The tokens are taken in chunks of up to 16 and each chunk is applied in the chunk form of
// Eq. (1) that the prefill uses (gamma = cumsum(g), D_rs = exp(gamma_r - gamma_s)):
//   A = strictly_lower(diag(beta) (K K^T o D)),  M = (I + A)^-1 diag(beta e^gamma),
//   Mu = (I + A)^-1 diag(beta),  W = M K,  U = Mu V,  Delta = U - W S,
//   O = scale (diag(e^gamma) Q S + (lower(Q K^T) o D) Delta),
//   S' = e^gamma_last S + K^T diag(e^(gamma_last - gamma)) Delta,
// so a chunk costs a handful of 16-row products against the state instead of a dk x dv
// rank-one update per token; the state is still read once and written once per call.  With
// L2 normalisation (K^ = diag(rk) K, Q^ = diag(rq) Q) the bf16 products K K^T and Q K^T use
// the inputs as given and take the norms as row and column factors; the fp16 operands are
// formed from the normalised rows.
//
// One workgroup of 4 wavefronts per (b, hv) state, two per CU.  The fp32 state stays in the
// token kernel's layout (a thread holds float4 column groups of consecutive rows: HBM is read
// and written in whole rows) and is updated there in fp32:
//   S' = e^gamma_last S + sum_t (e^(gamma_last - gamma_t) k_t) Delta_t^T,
// a rank-Tc update with no dependence between the tokens.  Only the products with the state
// go to the matrix cores: an fp16 copy of the scaled state, transposed through LDS, is the B
// operand of [W; e^gamma Q] S (16x16x32, k-step kk taking rows 32 kk + {4 lg .. 4 lg + 3,
// 16 + 4 lg .. 16 + 4 lg + 3}, the order in which W leaves its own 16x16x16 product), and
// Delta goes back through LDS to every thread.  (I + A)^-1 (16 x 16, fp32) is a forward
// substitution by one wavefront through LDS.  A chunk's inputs (k, q, v rows, the gates) are
// staged in LDS by one burst of coalesced loads, issued with the state's, so that no global
// load latency sits between the steps.
//
// Range: the fp16 copies of the value side (v, S, Delta) carry a power of two per column
// (pow2_scale of the column's largest |v| and |S|), taken back out of the fp32 results
// exactly, as in the prefill.  q and k are converted to fp16 as given (|q|, |k| < 65504).

typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 wmma32(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 wmma16(f16x4 a, f16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 wmma32_bf16(u16x8 a, u16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f16x4 to_h4(f32x4 x) {
    return f16x4{f16(x[0]), f16(x[1]), f16(x[2]), f16(x[3])};
}
__device__ __forceinline__ f16x8 cat8(f16x4 lo, f16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// sum over the four lanes l mod 16 + 16 r of a wavefront (see max_over_rows)
__device__ __forceinline__ float sum_over_rows(float x) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const unsigned w = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Tokens per chunk of the matrix-core decode, and the smallest T that takes it.
constexpr int kWyChunk = 16;
constexpr int kWyMinTokens = 5;  // measured crossover with the token kernel (B=256, 32 heads, d=128)

template <int D, typename TO>
__global__ void __launch_bounds__(256, 2)  // two states in flight per CU
decode_wy_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
                 const bf16_t *__restrict__ v, const bf16_t *__restrict__ beta,
                 const bf16_t *__restrict__ g, const float *state_in, float *state_out,
                 TO *__restrict__ o, int T, int Hk, int Hv, float scale, unsigned flags) {
    constexpr int C = kWyChunk;
    constexpr int KD = D / 32;   // 32-wide k-steps over dk
    constexpr int NJ = D / 64;   // 16-column tiles per wavefront in the products
    constexpr int CG = D / 4;    // float4 column groups of a state row
    constexpr int R = 256 / CG;  // row groups
    constexpr int RPT = D / R;   // consecutive state rows per thread
    constexpr int PT = D + 8;    // fp16 elements per row of the transposed state copy (padded)
    __shared__ float s_A[C][C + 1];   // strictly lower A
    __shared__ float s_P[C][C + 1];   // lower(Q^ K^^T o D)
    __shared__ float s_M[C][C + 1];   // (I + A)^-1 diag(beta e^gamma)
    __shared__ float s_Mu[C][C + 1];  // (I + A)^-1 diag(beta)
    // the chunk's inputs as given (rows past Tc zero), staged in one burst of loads
    __shared__ __attribute__((aligned(16))) bf16_t s_K[C][D], s_Q[C][D], s_V[C][D];
    __shared__ float s_bet[C], s_lga[C];  // beta and log alpha after the input prologue
    __shared__ __attribute__((aligned(16))) f16 s_ST[D][PT];   // sig S, transposed: [col][row]
    __shared__ __attribute__((aligned(16))) float s_D[C][D];   // sig Delta (first: column maxima)
    __shared__ float s_sig[D];  // the column scales sig
    __shared__ float s_kf[C];   // e^(gamma_last - gamma_t) rk_t per token

    const int head = blockIdx.x;  // b * Hv + hv
    const int b = head / Hv, hv = head - b * Hv;
    const int hq = hv / (Hv / Hk);
    const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cg = tid % CG, rg = tid / CG;  // state rows rg RPT .. + RPT - 1, columns 4 cg ..
    const size_t tok0 = static_cast<size_t>(b) * T;
    const bool norm = (flags & GDN_QK_L2NORM) != 0;

    // ---- the state, fp32, in whole rows (the token kernel's streaming pattern); every element
    //      is read before any is written, so state_out may be state_in
    f32x4 st[RPT];
    const size_t sbase = static_cast<size_t>(head) * D * D;
    if (state_in != nullptr) {  // one branch: every load in flight together
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            st[m] = *reinterpret_cast<const f32x4 *>(state_in + sbase + static_cast<size_t>(rg * RPT + m) * D + 4 * cg);
    } else {
#pragma unroll
        for (int m = 0; m < RPT; ++m) st[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int t0 = 0; t0 < T; t0 += C) {
        const int Tc = min(C, T - t0);
        if (t0 > 0) __syncthreads();  // the previous chunk's LDS contents have been read
        // ---- stage the chunk's k, q, v rows (16 bytes a thread) and gates in LDS
        for (int i = tid; i < C * (D / 8); i += 256) {
            const int t = i / (D / 8), off = 8 * (i - t * (D / 8));
            u16x8 xk = u16x8{0, 0, 0, 0, 0, 0, 0, 0}, xq = xk, xv = xk;
            if (t < Tc) {
                const size_t rq = (tok0 + t0 + t) * Hk + hq, rv = (tok0 + t0 + t) * Hv + hv;
                xk = *reinterpret_cast<const u16x8 *>(k + rq * D + off);
                xq = *reinterpret_cast<const u16x8 *>(q + rq * D + off);
                xv = *reinterpret_cast<const u16x8 *>(v + rv * D + off);
            }
            *reinterpret_cast<u16x8 *>(&s_K[t][off]) = xk;
            *reinterpret_cast<u16x8 *>(&s_Q[t][off]) = xq;
            *reinterpret_cast<u16x8 *>(&s_V[t][off]) = xv;
        }
        if (tid < C) {
            float bt = 0.f, la = 0.f;
            if (tid < Tc) {
                const size_t gi = (tok0 + t0 + tid) * Hv + hv;
                bt = beta_from_input(bf16_to_f32(beta[gi]), flags);
                la = log_alpha_from_input(bf16_to_f32(g[gi]), flags);
            }
            s_bet[tid] = bt;
            s_lga[tid] = la;
        }
        __syncthreads();  // the chunk's inputs are in LDS
        // ---- per-token scalars, lane li = token li (rows past Tc: beta = 0, log alpha = 0)
        const bool tv = li < Tc;
        const float bet = s_bet[li];
        float gam = s_lga[li];
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const float y = __shfl_up(gam, off, 16);
            if (li >= off) gam += y;
        }
        const float glast = __shfl(gam, 15);  // padded rows add 0: gamma of the last token
        // ---- k and q rows li (columns 32 kk + 8 lg ..), bf16 as given; zero past Tc
        u16x8 kf[KD], qf[KD];
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
            kf[kk] = *reinterpret_cast<const u16x8 *>(&s_K[li][32 * kk + 8 * lg]);
            qf[kk] = *reinterpret_cast<const u16x8 *>(&s_Q[li][32 * kk + 8 * lg]);
        }
        float rk = 1.f, rq = 1.f;  // 1 / row norms (GDN_QK_L2NORM), else 1
        if (norm) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int kk = 0; kk < KD; ++kk)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x1 = bf16_to_f32(kf[kk][e]), x2 = bf16_to_f32(qf[kk][e]);
                    sk += x1 * x1;
                    sq += x2 * x2;
                }
            rk = inv_norm_from_sumsq(sum_over_rows(sk));
            rq = inv_norm_from_sumsq(sum_over_rows(sq));
        }
        const float eg = expf(gam);  // e^gamma of token li (<= 1)
        // ---- one wavefront: A and P, (I + A)^-1 by forward substitution, M, Mu, k rows
        if (w == 0) {
            f32x4 G = {0.f, 0.f, 0.f, 0.f}, QK = G;
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) {
                G = wmma32_bf16(kf[kk], kf[kk], G);
                QK = wmma32_bf16(qf[kk], kf[kk], QK);
            }
            // lane (li, lg): G[4 lg + r][li]; row factors from the lanes of tokens 4 lg + r
            const float fa = bet * rk;  // A[r][c] = beta_r rk_r rk_c e^(gam_r - gam_c) G[r][c]
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * lg + r;
                const float rgam = __shfl(gam, row), rfa = __shfl(fa, row), rrq = __shfl(rq, row);
                const float dec = expf(fminf(rgam - gam, 0.f));
                s_A[row][li] = li < row ? rfa * rk * dec * G[r] : 0.f;
                s_P[row][li] = li <= row ? rrq * rk * dec * QK[r] : 0.f;
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // A visible to every lane
            // column li of (I + A)^-1: x_r = [r == c] - sum_{m < r} A[r][m] x_m
            float x[C];
#pragma unroll
            for (int r = 0; r < C; ++r) {
                float acc = r == li ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) acc -= s_A[r][m] * x[m];
                x[r] = acc;
            }
            if (lg == 0) {
                const float fm = bet * eg;
#pragma unroll
                for (int r = 0; r < C; ++r) {
                    s_M[r][li] = x[r] * fm;
                    s_Mu[r][li] = x[r] * bet;
                }
                s_kf[li] = expf(fminf(glast - gam, 0.f)) * rk;
            }
        }
        // ---- the column scales: the largest |S| and |v| of every column, over this thread's
        //      rows and tokens rg, rg + R, ..., then over the row groups
        float cmax[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float mx = 0.f;
#pragma unroll
            for (int m = 0; m < RPT; ++m) mx = fmaxf(mx, fabsf(st[m][c]));
            cmax[c] = mx;
        }
        for (int t = rg; t < Tc; t += R) {
#pragma unroll
            for (int c = 0; c < 4; ++c) cmax[c] = fmaxf(cmax[c], fabsf(bf16_to_f32(s_V[t][4 * cg + c])));
        }
        float *red = &s_D[0][0];  // [4 wavefronts][D]
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float mx = cmax[c];
            if constexpr (CG == 32) {
                mx = fmaxf(mx, __shfl_xor(mx, 32));
            } else {
                mx = max_over_rows(mx);  // CG == 16: lanes cg + 16 r
            }
            if (lane < CG) red[w * D + 4 * cg + c] = mx;
        }
        __syncthreads();  // the maxima, and wavefront 0's LDS operands, are written
        float sg[4], isg[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float mx = red[4 * cg + c];
#pragma unroll
            for (int ww = 1; ww < 4; ++ww) mx = fmaxf(mx, red[ww * D + 4 * cg + c]);
            pow2_scale(mx, sg[c], isg[c]);
        }
        // ---- sig S into LDS, transposed (the B operand reads 8 consecutive rows of a column)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (rg == 0) s_sig[4 * cg + c] = sg[c];
            if constexpr (RPT == 16) {
                f16x8 h0, h1;
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    h0[m] = f16(sg[c] * st[m][c]);
                    h1[m] = f16(sg[c] * st[8 + m][c]);
                }
                *reinterpret_cast<f16x8 *>(&s_ST[4 * cg + c][rg * RPT]) = h0;
                *reinterpret_cast<f16x8 *>(&s_ST[4 * cg + c][rg * RPT + 8]) = h1;
            } else {
                static_assert(RPT == 4, "state rows per thread");
                f16x4 h;
#pragma unroll
                for (int m = 0; m < 4; ++m) h[m] = f16(sg[c] * st[m][c]);
                *reinterpret_cast<f16x4 *>(&s_ST[4 * cg + c][rg * RPT]) = h;
            }
        }
        __syncthreads();  // sig S and the scales are in LDS
        // ---- products on the matrix cores, wavefront w: column tiles jt = NJ w + j.  k-step kk
        //      takes rows 32 kk + {4 lg .. 4 lg + 3, 16 + 4 lg .. 16 + 4 lg + 3} (the order in
        //      which W comes out of its own product); the Q operand is built in the same order
        auto bS = [&](int kk, int jt) {
            const f16 *col = &s_ST[16 * jt + li][32 * kk + 4 * lg];
            return cat8(*reinterpret_cast<const f16x4 *>(col),
                        *reinterpret_cast<const f16x4 *>(col + 16));
        };
        f32x4 Y1[NJ], Y0[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) Y1[j] = Y0[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            const float fq = tv ? eg * rq : 0.f;  // e^gamma rq Q, row li
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) {
                const u16x4 lo = *reinterpret_cast<const u16x4 *>(&s_Q[li][32 * kk + 4 * lg]);
                const u16x4 hi = *reinterpret_cast<const u16x4 *>(&s_Q[li][32 * kk + 16 + 4 * lg]);
                f16x8 a;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a[e] = f16(fq * bf16_to_f32(lo[e]));
                    a[4 + e] = f16(fq * bf16_to_f32(hi[e]));
                }
#pragma unroll
                for (int j = 0; j < NJ; ++j) Y1[j] = wmma32(a, bS(kk, NJ * w + j), Y1[j]);
            }
        }
        // W = M K^ (K^ = diag(rk) K, normalised before the fp16 conversion): W^T = K^^T M^T on
        // 16x16x16 products (k = tokens 4 lg .. 4 lg + 3); lane (li, lg) = W[li][16 nb + 4 lg + r]
        float kn[4];  // rk of tokens 4 lg + e
#pragma unroll
        for (int e = 0; e < 4; ++e) kn[e] = __shfl(rk, 4 * lg + e);
        f16x4 mB, muA, pA;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            mB[e] = f16(s_M[li][4 * lg + e]);
            muA[e] = f16(s_Mu[li][4 * lg + e]);
            pA[e] = f16(s_P[li][4 * lg + e]);
        }
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
            f32x4 wt[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f16x4 ka;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ka[e] = f16(kn[e] * bf16_to_f32(s_K[4 * lg + e][16 * (2 * kk + h) + li]));
                wt[h] = wmma16(ka, mB, f32x4{0.f, 0.f, 0.f, 0.f});
            }
            const f16x8 wa = cat8(to_h4(wt[0]), to_h4(wt[1]));
#pragma unroll
            for (int j = 0; j < NJ; ++j) Y0[j] = wmma32(wa, bS(kk, NJ * w + j), Y0[j]);
        }
        // ---- U = Mu (sig V), sig Delta = U - W (sig S), the outputs; sig Delta to LDS
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int col = 16 * (NJ * w + j) + li;
            const float sgj = s_sig[col], osc = scale / sgj;  // exact: a power of two
            f16x4 vb;
#pragma unroll
            for (int e = 0; e < 4; ++e) vb[e] = f16(sgj * bf16_to_f32(s_V[4 * lg + e][col]));
            const f32x4 dl = wmma16(muA, vb, f32x4{0.f, 0.f, 0.f, 0.f}) - Y0[j];
            const f32x4 O = wmma16(pA, to_h4(dl), Y1[j]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * lg + r;
                if (t < Tc) store_f32(o + ((tok0 + t0 + t) * Hv + hv) * D + col, osc * O[r]);
                s_D[t][col] = dl[r];
            }
        }
        __syncthreads();  // sig Delta is in LDS (and every thread is done with the maxima)
        // ---- S' = e^gamma_last S + K^T diag(e^(gamma_last - gamma) rk) Delta, in fp32 on this
        //      thread's rows and columns (Delta = (sig Delta) / sig: exact)
        const float gC = expf(glast);
#pragma unroll
        for (int m = 0; m < RPT; ++m) st[m] *= gC;
        for (int t = 0; t < Tc; ++t) {
            f32x4 dv = *reinterpret_cast<const f32x4 *>(&s_D[t][4 * cg]);
#pragma unroll
            for (int c = 0; c < 4; ++c) dv[c] *= isg[c];
            const float kt = s_kf[t];
            float kr[RPT];
            if constexpr (RPT == 16) {
                const u16x8 k0 = *reinterpret_cast<const u16x8 *>(&s_K[t][rg * RPT]);
                const u16x8 k1 = *reinterpret_cast<const u16x8 *>(&s_K[t][rg * RPT + 8]);
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    kr[m] = kt * bf16_to_f32(k0[m]);
                    kr[8 + m] = kt * bf16_to_f32(k1[m]);
                }
            } else {
                const u16x4 k0 = *reinterpret_cast<const u16x4 *>(&s_K[t][rg * RPT]);
#pragma unroll
                for (int m = 0; m < 4; ++m) kr[m] = kt * bf16_to_f32(k0[m]);
            }
#pragma unroll
            for (int m = 0; m < RPT; ++m) st[m] += kr[m] * dv;
        }
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        __builtin_nontemporal_store(st[m], reinterpret_cast<f32x4 *>(state_out + sbase + static_cast<size_t>(rg * RPT + m) * D + 4 * cg));
}

template <int D, typename TO> hipError_t launch_wy(const DecodeArgs &a) {
    const unsigned nblk = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hv);
    hipLaunchKernelGGL((decode_wy_kernel<D, TO>), dim3(nblk), dim3(256), 0, a.stream,
                       static_cast<const bf16_t *>(a.q), static_cast<const bf16_t *>(a.k),
                       static_cast<const bf16_t *>(a.v), static_cast<const bf16_t *>(a.beta),
                       static_cast<const bf16_t *>(a.g), a.state_in, a.state, static_cast<TO *>(a.o),
                       a.T, a.Hk, a.Hv, a.scale, a.flags);
    return hipGetLastError();
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
    // the matrix-core form reads q, k and v rows with 16-byte loads
    const bool qk16 = reinterpret_cast<uintptr_t>(a.q) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(a.k) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(a.v) % 16 == 0;
    if (a.in_dt == GDN_BF16 && a.T >= kWyMinTokens && a.dk == a.dv &&
        (a.dk == 64 || a.dk == 128) && qk16) {
        if (a.dk == 128)
            return a.out_dt == GDN_F32 ? launch_wy<128, float>(a) : launch_wy<128, bf16_t>(a);
        return a.out_dt == GDN_F32 ? launch_wy<64, float>(a) : launch_wy<64, bf16_t>(a);
    }
    switch (a.dk) {
    case 16: return launch_dk<16>(a);
    case 32: return launch_dk<32>(a);
    case 64: return launch_dk<64>(a);
    case 128: return launch_dk<128>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
