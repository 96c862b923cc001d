// chunk_split.hip -- two-kernel chunk-parallel prefill for shapes with few (b, hv) chains.
//
// Same exact rewriting of Eq. (1) of the explainer page "論文解説: Qwen3.8-Next の設計"
// (ta-paperlens.web.app, section "GDNの中身") as chunk_mfma.hip:
//
//   gamma = cumsum(g) within a chunk,  D_rs = exp(gamma_r - gamma_s) (s <= r)
//   A = strictly_lower(diag(beta) (K K^T o D)),   U = (I + A)^-1 diag(beta) V,
//   W = (I + A)^-1 diag(beta e^gamma) K,          Delta = U - W S,
//   O = scale (diag(e^gamma) Q S + (lower(Q K^T) o D) Delta),
//   S_next = e^gamma_last S + K^T diag(e^(gamma_last - gamma)) Delta.
//
// Everything that does not depend on the state S is computed by prep_kernel, fully in
// parallel over (chunk, chain), one wavefront each; scan_kernel then walks the chunks of one
// chain in order for one 16-column tile of the state, and forms the outputs as it goes.
// This trades extra HBM traffic (the per-chunk operands go through a workspace) for
// parallelism: a chain of T/C chunks no longer waits for the per-chunk triangular solve,
// which is what bounds a single-pass kernel when there are fewer chains than compute units.
//
// Range: U, the state S and Delta scale with v and S0, so their fp16 copies carry a power of
// two (pow2_scale), taken back out of the fp32 sums exactly.  Prep scales each chunk's U by one
// chosen from the chunk's largest |v|, and stores with e^gamma_last the inverse scale and three
// bounds: um = max|U|, wm = D max|W| (>= every row sum of |W|) and nb = C sqrt(D) max|k| um
// (>= every column 2-norm of K^T dec U).  The scan keeps its fp32 state pre-scaled by one power
// of two per 16-column tile, chosen from a bound nu on the columns' 2-norms that needs no
// reduction on the sequential path: for unit keys and beta in [0, 1] every token's map
// S -> alpha (I - beta k k^T) S has 2-norm at most alpha, so a chunk multiplies a column's
// 2-norm by at most e^gamma_last before adding at most nb:  nu' = e^gamma_last nu + nb, and
// |Delta| <= um + wm nu.  The scaled operands then stay below 2^9 in magnitude (no fp16
// overflow, whatever the magnitude of v and S0); a loose bound only lowers them, and values
// stay exact to fp16's normal precision down to 2^-14.
//
// The workspace holds, per (chain, chunk), the scan kernel's MFMA operands already in
// fragment order -- for every 16x16x32 A operand one 1 KiB block, lane-major, 16 bytes per
// lane -- so each operand reaches the scan kernel's registers with one coalesced 16-byte load
// per lane and no LDS.  The prep kernel produces them without any transpose through LDS:
// multiplying a row fragment by a 0/1 selection matrix on the matrix cores yields the tile in
// the accumulator (column) layout, and a product whose left factor is the transpose of an
// accumulator-layout tile takes that tile's registers as its A operand unchanged.
#include <algorithm>
#include <stdlib.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma_f16_k32(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_bf16_k32(u16x8 a, u16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f16_k16(f16x4 a, f16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x4 h4(f32x4 x) {
    return f16x4{f16(x[0]), f16(x[1]), f16(x[2]), f16(x[3])};
}
__device__ __forceinline__ f16x8 cat(f16x4 lo, f16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

constexpr int kProgStride = 32;  // unsigned long longs per chain's scan-progress word (256 B)
// floats at the end of every record: e^gamma_last, 1/usig, um, wm, nb (see below), unused
constexpr int kRecScalars = 8;

// Rows and record slots of one chain (sequence s, v head hv).  Every record belongs to a slot
// position of a unit: dense batches (cu == nullptr) give each chain (the unit) nrec =
// ceil(T / C) slots, chunk c in slot c.  Packed sequences give each head hv (the unit)
// nrec = floor(T / C) + num_seqs slots, and sequence s (starting at row a_s) takes the slots
// from floor(a_s / C) + s on.  Since ceil(len / C) <= floor((a_s mod C + len) / C) + 1,
// consecutive sequences never share a slot and the last one ends below nrec (for any offsets,
// as seq_range clamps them into [0, T]).
// The kernels run over a segment of slot positions [lo, lo + L) at a time, L fixed by the
// workspace: the record of slot position p of unit u sits at u L + p - lo, so the workspace
// holds L slots of every unit whatever the sequence length.
struct ChainSpan {
    size_t row0;    // first token row
    int len, nch;   // tokens; chunks
    int base;       // slot position of chunk 0
    int unit;       // the chain (dense) or the head (packed) whose slots it uses
};
template <int C>
__device__ __forceinline__ ChainSpan chain_span(const int32_t *cu, int T, int Hv, int chain) {
    const int s = chain / Hv, hv = chain - s * Hv;
    ChainSpan r;
    seq_range(cu, T, s, r.row0, r.len);
    r.nch = (r.len + C - 1) / C;
    r.base = cu == nullptr ? 0 : static_cast<int>(r.row0 / C) + s;
    r.unit = cu == nullptr ? chain : hv;
    return r;
}
// The chunks [cb, cb + n) of a chain that fall into the segment [lo, lo + L), and the address
// of the record of chunk cb.
struct SegSpan {
    int cb, n;
    size_t rec;  // record index of chunk cb in the workspace
};
__device__ __forceinline__ SegSpan seg_span(const ChainSpan &sp, int lo, int L) {
    SegSpan r;
    r.cb = max(0, lo - sp.base);
    r.n = max(0, min(sp.nch, lo + L - sp.base) - r.cb);
    r.rec = static_cast<size_t>(sp.unit) * L + (sp.base + r.cb - lo);
    return r;
}

template <int D, int C> struct SplitCfg {
    static constexpr int NR = C / 16;  // 16-row blocks of a chunk
    static constexpr int NI = D / 16;  // 16-wide tiles of a head dimension
    static constexpr int KD = D / 32;  // 32-wide k-steps over a head dimension
    static constexpr int KC = C / 32;  // 32-wide k-steps over the chunk
    // fragment-ordered workspace record of one (chain, chunk), in 16-byte units per lane
    static constexpr size_t FRAG = 64 * 16;            // one A-operand fragment: 1 KiB
    static constexpr size_t OFF_W = 0;                 // -W         [NR][KD]
    static constexpr size_t OFF_Q = OFF_W + NR * KD * FRAG;   // e^gamma Q  [NR][KD]
    static constexpr size_t OFF_K = OFF_Q + NR * KD * FRAG;   // K^T dec    [NI][KC]
    static constexpr size_t OFF_P = OFF_K + NI * KC * FRAG;   // P          [NR][KC]
    static constexpr size_t OFF_U = OFF_P + NR * KC * FRAG;   // U          [NI][NR] x 512 B
    static constexpr size_t OFF_S = OFF_U + NI * NR * 64 * 8;  // the chunk's scalars, one line
    static constexpr size_t REC = OFF_S + 128;                  // bytes per (chain, chunk)
    static_assert((D == 64 || D == 128) && (C == 32 || C == 64), "split kernel shape");
};

// ---------------------------------------------------------------------------------------
// prep_kernel: one wavefront per (chain, chunk) -- per record slot and head for packed
// sequences, where slots past a sequence's chunks have nothing to do.  NORM: q and k are
// L2-normalised per row here (then held as fp16 for the matrix cores, since the normalised
// values are not bf16); flags: the gate transforms of the input prologue.
template <int D, int C, bool NORM>
__global__ void __launch_bounds__(64)
prep_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
            const bf16_t *__restrict__ v, const bf16_t *__restrict__ beta,
            const bf16_t *__restrict__ g, unsigned char *__restrict__ ws,
            unsigned long long *__restrict__ prog,
            const int32_t *__restrict__ cu, int nseq, int T, int Hk, int Hv, int seg_lo,
            int seg_len, unsigned flags) {
    using F = SplitCfg<D, C>;
    constexpr int NR = F::NR, KD = F::KD;
    // products with a K or Q operand: bf16 inputs as stored, or fp16 once normalised
    auto mma_kq = [](u16x8 a, u16x8 b, f32x4 acc) {
        if constexpr (NORM)
            return mma_f16_k32(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc);
        else
            return mma_bf16_k32(a, b, acc);
    };
    // per-row gate values: gamma (chunk-local cumulative log gate), e^gamma,
    // e^(gamma_last - gamma), beta; rows past T have g = beta = 0
    __shared__ __attribute__((aligned(16))) float s_gam[64], s_Gam[64], s_dec[64], s_bet[64];
    __shared__ __attribute__((aligned(16))) float s_adT[NR][16][16];  // diagonal blocks of A, transposed
    __shared__ __attribute__((aligned(16))) f16 s_td[NR][16][20];     // their inverses (fp16)

    const int lane = threadIdx.x, li = lane & 15, lg = lane >> 4;
    // chunk-major grid: consecutive blocks are the chains of one chunk (the heads of one slot),
    // so with a multiple of 8 chains (heads) a chain's records are all written from the XCD
    // (block index mod 8) on which the scan kernel runs that chain
    const int nchains = nseq * Hv;
    // the scan kernel's progress words start at chunk 0 (it runs after this kernel completes)
    if (prog != nullptr && blockIdx.x == 0)
        for (int i = threadIdx.x; i < nchains; i += 64) prog[static_cast<size_t>(i) * kProgStride] = 0ull;
    // slot position seg_lo + pl of the segment; its record goes to unit * seg_len + pl
    int c, chain, pl;
    if (cu == nullptr) {
        pl = blockIdx.x / nchains;
        chain = blockIdx.x - pl * nchains;
        c = seg_lo + pl;
    } else {
        // the sequence whose slots start last at or before this slot (the slot starts
        // floor(a_s / C) + s increase with s)
        pl = blockIdx.x / Hv;
        const int slot = seg_lo + pl, h = blockIdx.x - pl * Hv;
        int s = -1;
        for (int i0 = 0; i0 < nseq; i0 += 64) {
            const int i = i0 + lane;
            const bool le = i < nseq && min(max(cu[i], 0), T) / C + i <= slot;
            const unsigned long long m = __ballot(le);
            if (m != 0ull) s = i0 + 63 - __clzll(static_cast<long long>(m));
        }
        if (s < 0) return;
        chain = s * Hv + h;
        c = slot - (min(max(cu[s], 0), T) / C + s);  // the chunk of sequence s in this slot
    }
    const ChainSpan sp = chain_span<C>(cu, T, Hv, chain);
    if (c >= sp.nch) return;  // a slot no chunk uses
    const int G = Hv / Hk;
    const int hv = chain % Hv, hq = hv / G;
    const int t0 = c * C, L = min(C, sp.len - t0);
    unsigned char *rec = ws + (static_cast<size_t>(sp.unit) * seg_len + pl) * F::REC;

    // ---- gate loads first: the vector-memory counter is in order, so their wait below
    //      does not include the K, Q, V loads issued after them
    // (index clamped into the chunk so that the loads need no branch; rows past L are zeroed
    // where the values are first used)
    const size_t gi = (sp.row0 + t0 + min(lane, L - 1)) * Hv + hv;
    const bf16_t g_raw = g[gi], b_raw = beta[gi];
    __builtin_amdgcn_sched_barrier(0);  // keep these two loads ahead of the ones below
    // ---- row fragments of K, Q, V (lane: row 16a + li, columns 32kk + 8lg .. +7), bf16
    //      Rows past the chunk's end load its last row (no branch, so the waits stay exact)
    //      and are zeroed by a mask.
    u16x8 Kf[NR][KD], Qf[NR][KD], Vf[NR][KD];
#pragma unroll
    for (int a = 0; a < NR; ++a) {
        const int r = 16 * a + li;
        const size_t row = sp.row0 + t0 + min(r, L - 1);
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
            const size_t oq = (row * Hk + hq) * D + 32 * kk + 8 * lg;
            Kf[a][kk] = *reinterpret_cast<const u16x8 *>(k + oq);
            Qf[a][kk] = *reinterpret_cast<const u16x8 *>(q + oq);
            Vf[a][kk] = *reinterpret_cast<const u16x8 *>(v + (row * Hv + hv) * D + 32 * kk + 8 * lg);
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // all loads are issued before anything waits
#pragma unroll
    for (int a = 0; a < NR; ++a) {
        const uint16_t m = (16 * a + li < L) ? 0xffff : 0;
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
            Kf[a][kk] &= m;
            Qf[a][kk] &= m;
            Vf[a][kk] &= m;
        }
    }
    float usig, uisig;  // U is stored as f16(usig * U); 1/usig goes next to e^gamma_last
    float kmax;         // max |k| over the chunk
    // ---- the chunk's largest |v| (bf16 magnitudes order as their bit patterns without the
    //      sign) sets usig
    {
        u16x8 vm = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int a = 0; a < NR; ++a)
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) vm = __builtin_elementwise_max(vm, Vf[a][kk] & (uint16_t)0x7fff);
        unsigned m = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = max(m, static_cast<unsigned>(vm[e]));
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) m = max(m, static_cast<unsigned>(__shfl_xor(static_cast<int>(m), off)));
        m = __builtin_amdgcn_readfirstlane(m);  // the same in every lane
        pow2_scale(__uint_as_float(m << 16), usig, uisig);
        if constexpr (NORM) {
            kmax = 1.f;  // normalised rows: |k_i| <= 1
        } else {
            u16x8 km8 = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int a = 0; a < NR; ++a)
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) km8 = __builtin_elementwise_max(km8, Kf[a][kk] & (uint16_t)0x7fff);
            unsigned mk = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) mk = max(mk, static_cast<unsigned>(km8[e]));
#pragma unroll
            for (int off = 1; off < 64; off <<= 1)
                mk = max(mk, static_cast<unsigned>(__shfl_xor(static_cast<int>(mk), off)));
            kmax = __uint_as_float(__builtin_amdgcn_readfirstlane(mk) << 16);
        }
        if (lane == 0) reinterpret_cast<float *>(rec + F::OFF_S)[1] = uisig;
    }
    if constexpr (NORM) {
        // row 16a + li is spread over the lanes li + 16 lg and the KD fragments of each
#pragma unroll
        for (int a = 0; a < NR; ++a) {
            float kss = 0.f, qss = 0.f;
#pragma unroll
            for (int kk = 0; kk < KD; ++kk)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = bf16_to_f32(Kf[a][kk][e]), y = bf16_to_f32(Qf[a][kk][e]);
                    kss += x * x;
                    qss += y * y;
                }
            kss += __shfl_xor(kss, 16);
            kss += __shfl_xor(kss, 32);
            qss += __shfl_xor(qss, 16);
            qss += __shfl_xor(qss, 32);
            const float kr = inv_norm_from_sumsq(kss), qr = inv_norm_from_sumsq(qss);
#pragma unroll
            for (int kk = 0; kk < KD; ++kk)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    Kf[a][kk][e] = __builtin_bit_cast(uint16_t, f16(kr * bf16_to_f32(Kf[a][kk][e])));
                    Qf[a][kk][e] = __builtin_bit_cast(uint16_t, f16(qr * bf16_to_f32(Qf[a][kk][e])));
                }
        }
    }
    // ---- gates: chunk-local inclusive cumulative sum of g (rows past L: g = beta = 0)
    {
        float gv = lane < L ? log_alpha_from_input(bf16_to_f32(g_raw), flags) : 0.f;
        const float bv = lane < L ? beta_from_input(bf16_to_f32(b_raw), flags) : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(gv, off);
            if (lane >= off) gv += y;
        }
        const float glast = __shfl(gv, C - 1);
        // every lane writes (no branch); entries past C are not read
        s_gam[lane] = gv;
        s_Gam[lane] = __expf(gv);
        s_dec[lane] = __expf(glast - gv);
        s_bet[lane] = bv;
        if (lane == 0) reinterpret_cast<float *>(rec + F::OFF_S)[0] = __expf(glast);
    }
    __syncthreads();
    // gate values in registers: accumulator-layout rows 16a + 4lg + rr (one 16-byte read
    // each) and row-layout rows 16a + li
    f32x4 gamA[NR], GamA[NR], decA[NR], betA[NR];
    float gamR[NR], GamR[NR], betR[NR];
#pragma unroll
    for (int a = 0; a < NR; ++a) {
        gamA[a] = *reinterpret_cast<const f32x4 *>(&s_gam[16 * a + 4 * lg]);
        GamA[a] = *reinterpret_cast<const f32x4 *>(&s_Gam[16 * a + 4 * lg]);
        decA[a] = *reinterpret_cast<const f32x4 *>(&s_dec[16 * a + 4 * lg]);
        betA[a] = *reinterpret_cast<const f32x4 *>(&s_bet[16 * a + 4 * lg]);
        gamR[a] = s_gam[16 * a + li];
        GamR[a] = s_Gam[16 * a + li];
        betR[a] = s_bet[16 * a + li];
    }

    // ---- KK^T: tile (m-block cb, n-block a) in accumulator layout holds
    //      KK^T[16a + li][16cb + 4lg + rr] (the product is symmetric), i.e. exactly the
    //      A-operand fragment of -A_{a,cb} for the substitution below.
    f16x4 anf[NR][NR];
#pragma unroll
    for (int a = 0; a < NR; ++a) {
        const int r = 16 * a + li;
#pragma unroll
        for (int cb = 0; cb <= a; ++cb) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) acc = mma_kq(Kf[cb][kk], Kf[a][kk], acc);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                    const int s = 16 * cb + 4 * lg + rr;
                const float av = (s < r) ? betR[a] * __expf(gamR[a] - gamA[cb][rr]) * acc[rr] : 0.f;
                if (cb == a)
                    s_adT[a][4 * lg + rr][li] = av;  // A[r][s] of the diagonal block, stored [s][r]
                else
                    anf[a][cb][rr] = f16(-av);
            }
        }
    }
    // ---- P = lower(Q K^T) o D, computed as K Q^T so that the accumulator layout is the
    //      scan kernel's A-operand fragment: lane holds P[16rt + li][16st + 4lg + rr]
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) {
        const int r = 16 * rt + li;
#pragma unroll
        for (int kc = 0; kc < F::KC; ++kc) {
            f16x4 half[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int st = 2 * kc + h;
                half[h] = f16x4{f16(0.f), f16(0.f), f16(0.f), f16(0.f)};
                if (st <= rt) {
                    f32x4 acc = zero4();
#pragma unroll
                    for (int kk = 0; kk < KD; ++kk) acc = mma_kq(Kf[st][kk], Qf[rt][kk], acc);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int s = 16 * st + 4 * lg + rr;
                        half[h][rr] = f16((s <= r) ? __expf(gamR[rt] - gamA[st][rr]) * acc[rr] : 0.f);
                    }
                }
            }
            *reinterpret_cast<f16x8 *>(rec + F::OFF_P + ((rt * F::KC + kc) * 64 + lane) * 16) =
                cat(half[0], half[1]);
        }
    }
    __syncthreads();

    // ---- inverses of the 16x16 diagonal blocks of I + A: lane (li, lg) solves column li of
    //      block lg by forward substitution in fp32; column s of the block is contiguous
    {
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == li) ? 1.f : 0.f;
        if (lg < NR) {
#pragma unroll
            for (int s = 0; s < 15; ++s) {
                float col[16];
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const f32x4 t = *reinterpret_cast<const f32x4 *>(&s_adT[lg][s][4 * r4]);
                    col[4 * r4] = t[0], col[4 * r4 + 1] = t[1], col[4 * r4 + 2] = t[2], col[4 * r4 + 3] = t[3];
                }
#pragma unroll
                for (int r = s + 1; r < 16; ++r) x[r] -= col[r] * x[s];
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) s_td[lg][r][li] = f16(x[r]);
        }
    }
    __syncthreads();
    f16x4 tf[NR];  // row li, columns 4lg..4lg+3 of each inverse block
#pragma unroll
    for (int a = 0; a < NR; ++a) tf[a] = *reinterpret_cast<const f16x4 *>(&s_td[a][li][4 * lg]);

    // ---- 0/1 selection fragment: B[k][n] = (k == 16h + n), and as an A operand
    //      A[m][k] = (k == 16h + m); both have the same register content
    //      (one = 1.0 in bf16 for V; in the K/Q operand type for K and Q)
    constexpr uint16_t kOneKQ = NORM ? 0x3c00 : 0x3f80;
    u16x8 sel[2], selkq[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool on = (8 * lg + e == 16 * h + li);
            sel[h][e] = on ? 0x3f80 : 0;
            selkq[h][e] = on ? kOneKQ : 0;
        }

    // largest |usig U| and |W| of this lane's fp16 operands, as stored (packed fp16 maxima)
    f16x4 umax4 = f16x4{f16(0.f), f16(0.f), f16(0.f), f16(0.f)}, wmax4 = umax4;
    // ---- panels: for every 16-column panel p = 2kk + h of the head dimension, the blocked
    //      forward substitution X_a = T_aa (R_a - sum_{cb<a} A_{a,cb} X_cb) for U (R =
    //      diag(beta) V) and W (R = diag(beta e^gamma) K), plus the scan kernel's Q and K^T
    //      operands
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
        f16x4 wq[NR][2], qq[NR][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int p = 2 * kk + h;
            f32x4 Ux[NR], Wx[NR];
            f16x4 kt[NR];
#pragma unroll
            for (int a = 0; a < NR; ++a) {
                const f32x4 Kt = mma_kq(Kf[a][kk], selkq[h], zero4());      // K[16a+4lg+rr][16p+li]
                const f32x4 Vt = mma_bf16_k32(Vf[a][kk], sel[h], zero4());  // V[16a+4lg+rr][16p+li]
                const f32x4 Qt = mma_kq(selkq[h], Qf[a][kk], zero4());      // Q[16a+li][16p+4lg+rr]
                f32x4 yu, yw;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    yu[rr] = usig * betA[a][rr] * Vt[rr];
                    yw[rr] = betA[a][rr] * GamA[a][rr] * Kt[rr];
                    kt[a][rr] = f16(decA[a][rr] * Kt[rr]);
                }
                const float gq = GamR[a];
                qq[a][h] = f16x4{f16(gq * Qt[0]), f16(gq * Qt[1]), f16(gq * Qt[2]), f16(gq * Qt[3])};
#pragma unroll
                for (int cb = 0; cb < a; ++cb) {
                    yu = mma_f16_k16(anf[a][cb], h4(Ux[cb]), yu);
                    yw = mma_f16_k16(anf[a][cb], h4(Wx[cb]), yw);
                }
                const f16x4 yu16 = h4(yu), yw16 = h4(yw);
                Ux[a] = mma_f16_k16(tf[a], yu16, zero4());
                Wx[a] = mma_f16_k16(tf[a], yw16, zero4());
                // (T_aa Y)^T = Y^T T_aa^T: lane holds W[16a + li][16p + 4lg + rr]
                const f32x4 WxT = mma_f16_k16(yw16, tf[a], zero4());
                wq[a][h] = f16x4{f16(-WxT[0]), f16(-WxT[1]), f16(-WxT[2]), f16(-WxT[3])};
                wmax4 = __builtin_elementwise_max(wmax4, __builtin_elementwise_abs(wq[a][h]));
                // U in accumulator layout: the scan kernel's initial Delta accumulator
                const f16x4 u16 = h4(Ux[a]);
                *reinterpret_cast<f16x4 *>(rec + F::OFF_U + ((p * NR + a) * 64 + lane) * 8) = u16;
                umax4 = __builtin_elementwise_max(umax4, __builtin_elementwise_abs(u16));
            }
            // K^T diag(dec) fragments of row tile p: slots e<4 -> block 2kc, e>=4 -> 2kc+1
#pragma unroll
            for (int kc = 0; kc < F::KC; ++kc)
                *reinterpret_cast<f16x8 *>(rec + F::OFF_K + ((p * F::KC + kc) * 64 + lane) * 16) =
                    cat(kt[2 * kc], kt[2 * kc + 1]);
        }
#pragma unroll
        for (int a = 0; a < NR; ++a) {
            *reinterpret_cast<f16x8 *>(rec + F::OFF_W + ((a * KD + kk) * 64 + lane) * 16) =
                cat(wq[a][0], wq[a][1]);
            *reinterpret_cast<f16x8 *>(rec + F::OFF_Q + ((a * KD + kk) * 64 + lane) * 16) =
                cat(qq[a][0], qq[a][1]);
        }
    }
    // ---- the chunk's bounds for the scan (K^T dec, stored in fp16, may round up by 2^-11:
    //      covered by the factor-of-128 margin between the scaled operands and fp16's range)
    float umax = fmaxf(fmaxf(float(umax4[0]), float(umax4[1])), fmaxf(float(umax4[2]), float(umax4[3])));
    float wmax = fmaxf(fmaxf(float(wmax4[0]), float(wmax4[1])), fmaxf(float(wmax4[2]), float(wmax4[3])));
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        umax = fmaxf(umax, __shfl_xor(umax, off));
        wmax = fmaxf(wmax, __shfl_xor(wmax, off));
    }
    if (lane == 0) {
        float *sc = reinterpret_cast<float *>(rec + F::OFF_S);
        sc[2] = umax * uisig;                  // max |U|
        sc[3] = static_cast<float>(D) * wmax;  // >= max_r sum_i |W[r][i]|
        // >= every column 2-norm of K^T dec U: ||K^T dec||_2 <= sqrt(C D) max|k|, ||U_j|| <=
        //    sqrt(C) max|U|
        sc[4] = static_cast<float>(C) * sqrtf(static_cast<float>(D)) * kmax * sc[2];
    }
}

// ---------------------------------------------------------------------------------------
// scan_kernel: one workgroup per (chain, 16-column tile of the state), chunks in order.
// NWV "state" wavefronts run only the state's own dependency chain:
//     Delta = U - W S ,    S <- e^gamma_last S + (K^T dec) Delta
// and NR "output" wavefronts (one per 16-row block of a chunk) form the outputs of the chunk
// the state wavefronts have just finished, from that chunk's starting state and Delta, which
// the state wavefronts leave in LDS:
//     O = scale ((e^gamma Q) S_c + P Delta)
// The output wavefronts stay one chunk behind and keep step with the two workgroup barriers
// of every chunk, so neither the starting states nor Delta ever go through HBM.
//
// The state wavefronts split the state's rows: wavefront w keeps rows 32w .. 32w+31 of the
// tile and needs only the matching slices of the chunk operands (columns 32w.. of -W, rows
// 32w.. of K^T dec: 8 KiB per chunk at D = 128, C = 64), which it streams straight into
// registers, several chunks ahead.  One wavefront alone streams at most about 48 GB/s on
// MI355X and one compute unit about 145 GB/s, so splitting the operand stream four ways is
// what shortens a chunk on the sequential path.  The partial products W[:, 32w..] S[32w.., :]
// are summed through LDS (each wavefront finishes some row blocks of Delta), and every
// wavefront then reads the whole of Delta back.

// Workgroup barrier that waits only for this wave's LDS traffic (not for global memory).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Tiles of one chain on one XCD (blocks i and i + 8 share an XCD), so that the chain's
// workspace records are fetched once and then served from that XCD's L2.
__device__ __forceinline__ void chain_tile_map(int blk, int nblk, int ntile, int &chain, int &tile) {
    if ((nblk / ntile) % 8 == 0) {
        chain = (blk & 7) + 8 * (blk / (8 * ntile));
        tile = (blk >> 3) % ntile;
    } else {
        chain = blk / ntile;
        tile = blk - chain * ntile;
    }
}

template <int D, int C> struct ScanCfg {
    using F = SplitCfg<D, C>;
    static constexpr int NWV = F::KD;                      // state wavefronts: 32 rows each
    static constexpr int NWO = F::NR;                      // output wavefronts: 16 rows each
    static constexpr int NRW = (F::NR + NWV - 1) / NWV;    // Delta row blocks finished per wave
    static constexpr int DEPTH = 4;                        // chunks of operands in flight
    static constexpr int NPF = 4;                          // prefetch workgroups per chain
    // chunks the prefetch runs ahead: as many as keep the prefetched records of the chains
    // sharing an XCD within ~2.27 MiB of its 4 MiB L2 (measured on the 262,144-token
    // workload, 2 chains per XCD: 16 chunks ahead -15% against 12, 18 or more thrash)
    static constexpr size_t kPrefetchBytesPerXcd = 2320 * 1024;
    static constexpr int kMaxPfd = 16;
    static_assert(DEPTH >= 2, "scan pipeline depth");
};

// Prefetch workgroups (launched with the scan, after its workgroups, on otherwise idle compute
// units of the chain's XCD): they touch one dword of every 128-byte line of the records the
// scan will read a few chunks later, so that the scan's own loads hit that XCD's L2 instead of
// waiting on HBM.  A compute unit keeps only so many misses in flight, so at HBM latency one
// scan workgroup streams far below its issue rate; the prefetch moves that latency to other
// compute units.  Pacing: the scan publishes the chunk it is on, in a 256-byte line of its own
// per chain (cleared by prep_kernel, which runs just before).
// The prefetch workgroup takes chunks in groups of one per wavefront: wavefront 0 polls, with
// a pause between polls, until the whole group is within pfd chunks of the scan, then every
// wavefront loads its chunk's share of the lines and waits for it.  It is only a hint: the
// scan never waits for it, and a prefetch workgroup gives up after a bounded number of polls.

template <int D, int C>
__device__ void prefetch_records(const unsigned char *__restrict__ ws,
                                 unsigned long long *__restrict__ prog,
                                 const int32_t *__restrict__ cu, int T, int Hv, int seg_lo,
                                 int seg_len, int nchains, int p, int w, int nwaves, int lane,
                                 int *s_done, int pfd) {
    using F = SplitCfg<D, C>;
    using SC = ScanCfg<D, C>;
    constexpr int LINES = static_cast<int>(F::REC / 128);
    constexpr int PER = (LINES + SC::NPF - 1) / SC::NPF;  // lines per prefetch workgroup
    constexpr int NLD = (PER + 63) / 64;                  // loads per wavefront and chunk
    constexpr int kMaxPolls = 1 << 16;
    int chain, part;
    if (nchains % 8 == 0) {  // same XCD as the chain's scan workgroups (block index mod 8)
        const int q = p >> 3;
        chain = (p & 7) + 8 * (q / SC::NPF);
        part = q % SC::NPF;
    } else {
        chain = p % nchains;
        part = p / nchains;
    }
    const SegSpan sg = seg_span(chain_span<C>(cu, T, Hv, chain), seg_lo, seg_len);
    const int nchunks = sg.n;
    const unsigned char *rec0 = ws + sg.rec * F::REC;
    unsigned long long *pw = prog + static_cast<size_t>(chain) * kProgStride;
    unsigned acc = 0;
    int polls = 0;
    for (int n0 = 0; n0 < nchunks; n0 += nwaves) {
        if (w == 0) {
            int done = 0;
            for (;;) {
                done = static_cast<int>(
                    __hip_atomic_load(pw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                if (n0 + nwaves - 1 < done + pfd) break;
                if (++polls > kMaxPolls) {
                    done = -1;
                    break;
                }
                __builtin_amdgcn_s_sleep(16);
            }
            if (lane == 0) *s_done = done;
        }
        __syncthreads();
        const int done = *s_done;
        if (done < 0) break;  // the same for every wavefront
        const int n = n0 + w;
        if (n < nchunks && n >= done) {
            const unsigned char *r = rec0 + static_cast<size_t>(n) * F::REC;
            unsigned v[NLD];
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int line = min(part * PER + 64 * i + lane, LINES - 1);
                v[i] = *reinterpret_cast<const unsigned *>(r + static_cast<size_t>(line) * 128);
            }
#pragma unroll
            for (int i = 0; i < NLD; ++i) acc ^= v[i];
        }
        __syncthreads();  // every wavefront has read *s_done (and its loads are back)
    }
    asm volatile("" ::"v"(acc));
}



template <int D, int C> struct ScanOps {  // one state wave's operands of one chunk
    f16x8 wf[SplitCfg<D, C>::NR];          // -W, rows 16a.., k-step w
    f16x8 kf[2][SplitCfg<D, C>::KC];       // K^T dec, row blocks 2w, 2w+1
    f16x4 uf[ScanCfg<D, C>::NRW];          // usig U of this tile, the row blocks this wave finishes
    float sc;                              // lane l: the chunk's scalar l mod kRecScalars
};

template <int D, int C> struct OutOps {   // one output wave's operands of one chunk
    f16x8 qf[SplitCfg<D, C>::KD];          // e^gamma Q, row block a
    f16x8 pf[SplitCfg<D, C>::KC];          // P, row block a
};

template <int D, int C, typename TO>
__global__ void __launch_bounds__(64 * (ScanCfg<D, C>::NWV + ScanCfg<D, C>::NWO))
scan_kernel(const unsigned char *__restrict__ ws, const float *s0, float *carry,
            float *__restrict__ nucarry, TO *__restrict__ o, const int32_t *__restrict__ cu,
            int T, int Hv, int seg_lo, int seg_len, float scale,
            unsigned long long *__restrict__ prog, int nscan, int pfd) {
    using F = SplitCfg<D, C>;
    using SC = ScanCfg<D, C>;
    constexpr int NR = F::NR, NI = F::NI, KD = F::KD, KC = F::KC;
    constexpr int NWV = SC::NWV, NRW = SC::NRW, DEPTH = SC::DEPTH;
    __shared__ f32x4 s_part[NWV][NR][64];  // partial Delta blocks (scaled as the state)
    __shared__ f16x4 s_dlt[NR][64];         // Delta, scaled as the next state, accumulator layout
    __shared__ f16x8 s_st[2][NWV][64];      // starting state of the chunk, B fragments (by parity)
    __shared__ float s_isg[2][64];          // 1 / the tile's state scale, chunk c in slot c & 1
    __shared__ float s_nu0[NWV][64];        // initial state: each wave's column sums of squares
    const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __builtin_assume(w >= 0 && w < NWV + SC::NWO);
    if (static_cast<int>(blockIdx.x) >= nscan) {
        prefetch_records<D, C>(ws, prog, cu, T, Hv, seg_lo, seg_len, nscan / NI,
                               blockIdx.x - nscan, w, NWV + SC::NWO, lane,
                               reinterpret_cast<int *>(&s_st[0][0][0]), pfd);
        return;
    }
    int chain, jt;
    chain_tile_map(blockIdx.x, nscan, NI, chain, jt);
    const int col = 16 * jt + li;
    const ChainSpan sp = chain_span<C>(cu, T, Hv, chain);
    const SegSpan sg = seg_span(sp, seg_lo, seg_len);
    // chunks cb .. cb + nchunks - 1 of the chain fall into this segment; none and not an empty
    // sequence on the first segment (which copies its initial state): nothing to do here
    const int cb = sg.cb, nchunks = sg.n;
    if (nchunks == 0 && !(sp.nch == 0 && seg_lo == 0)) return;  // the whole workgroup
    const unsigned char *rec0 = ws + sg.rec * F::REC;
    // the state enters from s0 at the chain's first chunk, else from the previous segment's
    // carry, and leaves through the carry (the final state after the last segment; may alias
    // s0: a chain writes it only after reading its own)
    const float *sin = cb == 0 ? s0 : carry;

    if (w >= NWV) {
        // ---- output wavefront: row block a of every chunk, one chunk behind the state
        lds_barrier();  // the state wavefronts' exchange of the initial state's maxima
        if (nchunks == 0) return;
        const int a = w - NWV;
        const int hv = chain % Hv;
        auto load = [&](OutOps<D, C> &op, int cc) {
            const unsigned char *r = rec0 + static_cast<size_t>(cc) * F::REC;
#pragma unroll
            for (int kk = 0; kk < KD; ++kk)
                op.qf[kk] = *reinterpret_cast<const f16x8 *>(r + F::OFF_Q + ((a * KD + kk) * 64 + lane) * 16);
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                op.pf[kc] = *reinterpret_cast<const f16x8 *>(r + F::OFF_P + ((a * KC + kc) * 64 + lane) * 16);
        };
        // chunk c - 1's starting state and Delta (scaled fp16) and their inverse scales
        f16x8 bS[KD], bD[KC];
        float bG, bI;
        auto emit = [&](const OutOps<D, C> &op, int c) {
            f32x4 O = zero4(), OD = zero4();
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) O = mma_f16_k32(op.qf[kk], bS[kk], O);
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                if (32 * kc <= 16 * a + 15) OD = mma_f16_k32(op.pf[kc], bD[kc], OD);
            O = bG * O + bI * OD;
            const int t0 = (cb + c) * C, L = min(C, sp.len - t0);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = 16 * a + 4 * lg + rr;
                if (r < L)
                    store_f32(o + ((sp.row0 + t0 + r) * Hv + hv) * D + col,
                              scale * O[rr]);
            }
        };
        // step c: barriers 1 (chunk c's starting state is in LDS) and 2 (its Delta is), then
        // both are read into registers -- before barrier 1 of chunk c + 1, after which Delta
        // is overwritten -- and chunk c - 1's outputs are formed meanwhile: in the state
        // wavefronts' longest phase, not in the short one between the two barriers
        const bool publish = prog != nullptr && a == 0 && jt == 0;
        auto step = [&](const OutOps<D, C> &prev, int c) {
            lds_barrier();
            // the scales between the barriers: slot c & 1 is written again (for chunk c + 2)
            // before barrier 1 of the next step, i.e. possibly before a read after barrier 2
            const float nG = s_isg[c & 1][lane], nI = s_isg[(c + 1) & 1][lane];
            lds_barrier();
            if (publish && lane == 0)  // the state wavefronts are on chunk c
                __hip_atomic_store(prog + static_cast<size_t>(chain) * kProgStride,
                                   static_cast<unsigned long long>(c), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            f16x8 nS[KD], nD[KC];
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) nS[kk] = s_st[c & 1][kk][lane];
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) nD[kc] = cat(s_dlt[2 * kc][lane], s_dlt[2 * kc + 1][lane]);
            if (c > 0) emit(prev, c - 1);
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) bS[kk] = nS[kk];
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) bD[kc] = nD[kc];
            bG = nG;
            bI = nI;
        };
        constexpr int RO = 3;  // ring of operand sets; slot (c mod RO) holds chunk c
        OutOps<D, C> ring[RO];
#pragma unroll
        for (int s = 0; s < RO; ++s) load(ring[s], min(s, nchunks - 1));
        // chunk c uses slot c mod RO in emit, one step later than its barriers
        int c0 = 0;
        for (; c0 + RO <= nchunks; c0 += RO) {
#pragma unroll
            for (int s = 0; s < RO; ++s) {
                const int c = c0 + s;
                step(ring[(s + RO - 1) % RO], c);            // emits chunk c - 1
                if (c > 0) load(ring[(s + RO - 1) % RO], min(c - 1 + RO, nchunks - 1));
            }
        }
#pragma unroll
        for (int s = 0; s < RO; ++s)
            if (c0 + s < nchunks) {
                const int c = c0 + s;
                step(ring[(s + RO - 1) % RO], c);
                if (c > 0) load(ring[(s + RO - 1) % RO], min(c - 1 + RO, nchunks - 1));
            }
        // the last chunk (constant ring indices only: a computed one would put the ring in
        // scratch memory)
#pragma unroll
        for (int s = 0; s < RO; ++s)
            if ((nchunks - 1) % RO == s) emit(ring[s], nchunks - 1);
        return;
    }

    // ---- state wavefront w: rows 32w + 16i + 4lg + rr of column col, held in fp32 scaled by
    //      sig (one power of two for the tile, isg = 1/sig)
    __builtin_assume(w < NWV);
    f32x4 S[2];
    const size_t sbase = static_cast<size_t>(chain) * D * D;
    if (sin != nullptr) {  // one branch, so that all loads are in flight together
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                S[i][rr] = sin[sbase + static_cast<size_t>(32 * w + 16 * i + 4 * lg + rr) * D + col];
    } else {
        S[0] = S[1] = zero4();
    }
    float sig, isg;
    float nu;  // bound on the 2-norm of every column of the tile at the start of the chunk
    // a later segment continues the chain with the bound and the scale it had: the same
    // operands, bit for bit, as one pass over all chunks (nucarry: [chain][tile] {nu, sig})
    float *nuc = nucarry != nullptr ? nucarry + 2 * (static_cast<size_t>(chain) * NI + jt) : nullptr;
    if (cb > 0) {
        nu = nuc[0];
        sig = nuc[1];
        isg = 1.f / sig;  // exact: a power of two
        S[0] *= sig;
        S[1] *= sig;
        s_isg[0][lane] = isg;
        lds_barrier();  // the output wavefronts' first barrier (the other branch's exchange)
    } else {
        float q = 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) q += S[i][rr] * S[i][rr];
        // the column's sum of squares over its four lanes and all state waves (through LDS),
        // then the tile's largest column 2-norm (rounded up a little for the fp32 sums)
        const unsigned qu = __float_as_uint(q);
        const auto a16 = __builtin_amdgcn_permlane16_swap(qu, qu, false, false);
        q = __uint_as_float(a16[0]) + __uint_as_float(a16[1]);
        const unsigned qv = __float_as_uint(q);
        const auto a32 = __builtin_amdgcn_permlane32_swap(qv, qv, false, false);
        s_nu0[w][lane] = __uint_as_float(a32[0]) + __uint_as_float(a32[1]);
        lds_barrier();
        float ss = 0.f;
#pragma unroll
        for (int v = 0; v < NWV; ++v) ss += s_nu0[v][lane];
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) ss = fmaxf(ss, __shfl_xor(ss, off));
        nu = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, ss)));
        nu = 1.0001f * sqrtf(nu);
        pow2_scale(nu, sig, isg);
        S[0] *= sig;
        S[1] *= sig;
        s_isg[0][lane] = isg;  // every state wave writes the same
    }
    auto load = [&](ScanOps<D, C> &op, int cc) {
        const unsigned char *r = rec0 + static_cast<size_t>(cc) * F::REC;
#pragma unroll
        for (int a = 0; a < NR; ++a)
            op.wf[a] = *reinterpret_cast<const f16x8 *>(r + F::OFF_W + ((a * KD + w) * 64 + lane) * 16);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                op.kf[i][kc] = *reinterpret_cast<const f16x8 *>(
                    r + F::OFF_K + (((2 * w + i) * KC + kc) * 64 + lane) * 16);
#pragma unroll
        for (int j = 0; j < NRW; ++j) {
            const int a = min(w + j * NWV, NR - 1);  // clamped: loaded but unused past NR
            op.uf[j] = *reinterpret_cast<const f16x4 *>(r + F::OFF_U + ((jt * NR + a) * 64 + lane) * 8);
        }
        // the chunk's scalars: lane l loads scalar l mod 8 of the record's last line (a vector
        // load -- a scalar load still in flight would hold up every LDS wait, which counts
        // scalar loads too), then every lane reads them from lanes 0..4
        op.sc = reinterpret_cast<const float *>(r + F::OFF_S)[lane & (kRecScalars - 1)];
    };
    auto step = [&](const ScanOps<D, C> &op, int c) {
        // k-step w of the B operand S (already scaled by sig)
        const f16x8 bS = cat(h4(S[0]), h4(S[1]));
        s_st[c & 1][w][lane] = bS;  // for the output wavefronts
        f32x4 pa[NR];
#pragma unroll
        for (int a = 0; a < NR; ++a) pa[a] = mma_f16_k32(op.wf[a], bS, zero4());
#pragma unroll
        for (int a = 0; a < NR; ++a) s_part[w][a][lane] = pa[a];
        // the independent products back to back, then their LDS writes
        __builtin_amdgcn_sched_group_barrier(0x008, NR, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, NR, 0);
        // while they run: e^gamma_last, 1/usig, um, wm, nb of the chunk (loaded DEPTH chunks
        // ago; the builtin moves 32-bit integers) and one scale sgn for Delta and the next state,
        //   |Delta| <= bd = um + wm nu,   column norms of S_next <= e^gamma_last nu + nb
        const int sci = __builtin_bit_cast(int, op.sc);
        const float gc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(sci, 0));
        const float ui = __builtin_bit_cast(float, __builtin_amdgcn_readlane(sci, 1));
        const float um = __builtin_bit_cast(float, __builtin_amdgcn_readlane(sci, 2));
        const float wm = __builtin_bit_cast(float, __builtin_amdgcn_readlane(sci, 3));
        const float nb = __builtin_bit_cast(float, __builtin_amdgcn_readlane(sci, 4));
        const float bd = um + wm * nu;
        nu = gc * nu + nb;
        float sgn, isgn;
        pow2_scale(fmaxf(nu, bd), sgn, isgn);
        const float fu = sgn * ui, fp = sgn * isg, f1 = gc * fp;  // exact: powers of two
        s_isg[(c + 1) & 1][lane] = isgn;  // for the output wavefronts (every state wave alike)
        lds_barrier();
#pragma unroll
        for (int j = 0; j < NRW; ++j) {
            const int a = w + j * NWV;
            if (a < NR) {
                f32x4 p[NWV];
#pragma unroll
                for (int v = 0; v < NWV; ++v) p[v] = s_part[v][a][lane];
                // issue all the partial reads before any of the sums that use them
                __builtin_amdgcn_sched_group_barrier(0x100, NWV, 0);
                f32x4 ps = p[0];
#pragma unroll
                for (int v = 1; v < NWV; ++v) ps += p[v];
                const f32x4 d = fu * f32x4{float(op.uf[j][0]), float(op.uf[j][1]),
                                           float(op.uf[j][2]), float(op.uf[j][3])} + fp * ps;
                s_dlt[a][lane] = h4(d);  // sgn Delta
            }
        }
        lds_barrier();
        // sgn S_next = sgn e^gamma_last S + K^T dec (sgn Delta): exact rescalings
        f16x8 bD[KC];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) bD[kc] = cat(s_dlt[2 * kc][lane], s_dlt[2 * kc + 1][lane]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            S[i] *= f1;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) S[i] = mma_f16_k32(op.kf[i][kc], bD[kc], S[i]);
        }
        sig = sgn;
        isg = isgn;
    };

    if (nchunks > 0) {
        // Ring of DEPTH chunks of operands in registers.  The main loop is branch-free, so the
        // compiler's vector-memory waits stay exact (each step waits only for its own chunk's
        // loads, issued DEPTH steps earlier); loads past the last chunk re-read the last chunk.
        ScanOps<D, C> ring[DEPTH];
#pragma unroll
        for (int s = 0; s < DEPTH; ++s) load(ring[s], min(s, nchunks - 1));
        int c0 = 0;
        for (; c0 + DEPTH <= nchunks; c0 += DEPTH) {
#pragma unroll
            for (int s = 0; s < DEPTH; ++s) {
                step(ring[s], c0 + s);
                load(ring[s], min(c0 + s + DEPTH, nchunks - 1));
            }
        }
#pragma unroll
        for (int s = 0; s < DEPTH; ++s)
            if (c0 + s < nchunks) step(ring[s], c0 + s);
    }
    if (carry) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                carry[sbase + static_cast<size_t>(32 * w + 16 * i + 4 * lg + rr) * D + col] = isg * S[i][rr];
    }
    if (nuc != nullptr && w == 0 && lane == 0) {
        nuc[0] = nu;
        nuc[1] = sig;
    }
}

// Record slots per unit: per chain (dense) or per head (packed sequences); units.
template <int C> int split_nrec(const PrefillArgs &a) {
    return a.cu == nullptr ? (a.T + C - 1) / C : a.T / C + a.B;
}
inline size_t split_units(const PrefillArgs &a) {
    return static_cast<size_t>(a.cu == nullptr ? a.B * a.Hv : a.Hv);
}
// The records the default workspace holds at most (2 GiB, or GDN_SPLIT_RECORD_BYTES when the
// environment sets it, e.g. to test several segments on short inputs); longer sequences run
// in segments.
inline size_t split_record_bytes() {
    const char *e = getenv("GDN_SPLIT_RECORD_BYTES");
    const long long v = e != nullptr ? atoll(e) : 0;
    return v > 0 ? static_cast<size_t>(v) : size_t(2) << 30;
}

// Workspace: records of L slot positions of every unit | per-chain scan progress (256 B each)
// | the state carried between segments (fp32, one per chain) | the scan's bound and scale
// carried with it (two floats per chain and 16-column tile, padded to 256 B).
template <int D, int C> size_t split_carry_scales_bytes(const PrefillArgs &a) {
    const size_t n = static_cast<size_t>(a.B) * a.Hv * (D / 16) * 2 * sizeof(float);
    return (n + 255) / 256 * 256;
}
template <int D, int C> size_t split_fixed_bytes(const PrefillArgs &a) {
    const size_t chains = static_cast<size_t>(a.B) * a.Hv;
    return chains * kProgStride * sizeof(unsigned long long) + chains * D * D * sizeof(float) +
           split_carry_scales_bytes<D, C>(a);
}
template <int D, int C> size_t split_ws_bytes(const PrefillArgs &a, bool smallest) {
    const size_t slot_row = split_units(a) * SplitCfg<D, C>::REC;
    const size_t nrec = static_cast<size_t>(split_nrec<C>(a));
    const size_t L = smallest ? 1 : std::min(nrec, std::max<size_t>(1, split_record_bytes() / slot_row));
    return L * slot_row + split_fixed_bytes<D, C>(a);
}

template <int D, int C, typename TO> hipError_t launch_split_typed(const PrefillArgs &a) {
    using SC = ScanCfg<D, C>;
    using F = SplitCfg<D, C>;
    const int nrec = split_nrec<C>(a);
    const size_t units = split_units(a), chains = static_cast<size_t>(a.B) * a.Hv;
    // slot positions per segment: as many as the workspace holds (at least one, checked by
    // the caller)
    const size_t fixed = split_fixed_bytes<D, C>(a), slot_row = units * F::REC;
    if (a.ws_bytes < fixed + slot_row) return hipErrorInvalidValue;
    const int L = static_cast<int>(std::min<size_t>(nrec, (a.ws_bytes - fixed) / slot_row));
    const int nseg = (nrec + L - 1) / L;
    unsigned char *ws = static_cast<unsigned char *>(a.ws);
    unsigned long long *prog = reinterpret_cast<unsigned long long *>(ws + static_cast<size_t>(L) * slot_row);
    float *carry_ws = reinterpret_cast<float *>(reinterpret_cast<unsigned char *>(prog) +
                                                chains * kProgStride * sizeof(unsigned long long));
    float *nucarry = nseg > 1 ? carry_ws + chains * D * D : nullptr;
    // the state between segments: the final-state buffer if there is one, else the workspace's
    float *carry = a.sT != nullptr ? a.sT : (nseg > 1 ? carry_ws : nullptr);
    // prefetch workgroups only where the scan leaves compute units idle (one workgroup of
    // either kind fills a compute unit's registers)
    const size_t nscan = chains * (D / 16);
    const size_t npf = chains * (D / 16 + SC::NPF) <= 256 ? chains * SC::NPF : 0;
    const size_t per_xcd = (chains + 7) / 8;  // chains whose records share one XCD's L2
    const int pfd = static_cast<int>(std::max<size_t>(
        2, std::min<size_t>(SC::kMaxPfd, SC::kPrefetchBytesPerXcd / (per_xcd * F::REC))));
    auto prep = (a.flags & GDN_QK_L2NORM) ? prep_kernel<D, C, true> : prep_kernel<D, C, false>;
    for (int sg = 0; sg < nseg; ++sg) {
        const int lo = sg * L, nslot = std::min(L, nrec - lo);
        hipLaunchKernelGGL(prep, dim3(static_cast<unsigned>(units * nslot)), dim3(64), 0, a.stream,
                           static_cast<const bf16_t *>(a.q), static_cast<const bf16_t *>(a.k),
                           static_cast<const bf16_t *>(a.v), static_cast<const bf16_t *>(a.beta),
                           static_cast<const bf16_t *>(a.g), ws, npf ? prog : nullptr, a.cu,
                           a.B, a.T, a.Hk, a.Hv, lo, L, a.flags);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((scan_kernel<D, C, TO>), dim3(static_cast<unsigned>(nscan + npf)),
                           dim3(64 * (SC::NWV + SC::NWO)), 0, a.stream, ws, a.s0, carry,
                           nucarry, static_cast<TO *>(a.o), a.cu, a.T, a.Hv, lo, L, a.scale,
                           npf ? prog : nullptr, static_cast<int>(nscan), pfd);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int D, int C> hipError_t launch_split_out(const PrefillArgs &a) {
    return a.out_dt == GDN_F32 ? launch_split_typed<D, C, float>(a)
                               : launch_split_typed<D, C, bf16_t>(a);
}

}  // namespace

bool chunk_split_supports(const PrefillArgs &a) {
    return a.in_dt == GDN_BF16 && a.dk == a.dv && (a.dk == 64 || a.dk == 128) &&
           (a.chunk == 32 || a.chunk == 64);
}

size_t chunk_split_workspace(const PrefillArgs &a, bool smallest) {
    if (!chunk_split_supports(a)) return 0;
    if (a.dk == 128)
        return a.chunk == 64 ? split_ws_bytes<128, 64>(a, smallest)
                             : split_ws_bytes<128, 32>(a, smallest);
    return a.chunk == 64 ? split_ws_bytes<64, 64>(a, smallest) : split_ws_bytes<64, 32>(a, smallest);
}

hipError_t launch_chunk_split(const PrefillArgs &a) {
    if (!chunk_split_supports(a)) return hipErrorNotSupported;
    if (a.dk == 128)
        return a.chunk == 64 ? launch_split_out<128, 64>(a) : launch_split_out<128, 32>(a);
    return a.chunk == 64 ? launch_split_out<64, 64>(a) : launch_split_out<64, 32>(a);
}

}  // namespace gdn
