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
//     then staged in LDS: q and k as fp16 (exact for unit rows), v as stored (bf16).
//   * KK^T and QK^T: v_mfma_f32_16x16x32_f16 on exact inputs, fp32 accumulation.
//   * (I + A)^-1 is never formed: the 16x16 diagonal blocks are inverted in fp32 by forward
//     substitution, and U, W come from a blocked forward substitution over 16-row blocks,
//     X_a = T_aa (R_a - sum_{c<a} A_ac X_c), on v_mfma_f32_16x16x16_f16 -- every wavefront
//     solves its own two 16-column panels (of diag(beta) V and diag(beta e^gamma) K), so the
//     solve needs no barrier.
//   * Derived fp32 operands (W, S, Delta, P, X) are rounded to fp16 for the MFMAs; every sum
//     accumulates in fp32 and the fp32 state itself is never rounded.  The value side (U,
//     Delta, S, O) is linear in (v, S0) and column-separable, so each wavefront scales its
//     columns' fp16 copies by a power of two chosen per chunk from the column's largest |S|
//     and |beta v| (pow2_scale) and takes the scale back out of the fp32 results exactly: no
//     magnitude of v or S0 overflows fp16 or sinks into its subnormals.
//   * The accumulator layout (lane l holds rows 4(l/16)..4(l/16)+3 of column l%16) is fed
//     straight back as a B operand, with the k index of the A operand permuted to match, so
//     the state and the solve panels never leave registers.
//   * O is staged in LDS and written with coalesced 16-byte stores at the top of the next
//     chunk, before the next prefetch is issued (the vector-memory counter is in-order).
//
// Segmented plan (few, long chains).  The chunk maps above are affine in the state, so a
// segment of chunks maps any entry state S_in to S_out = M S_in + N, with N its result from
// the zero state and M = prod over its chunks of (e^gamma_last I - K^T dec W).  Every chain is
// cut into nseg segments: the kernel in mode kTrans runs segments 0 .. nseg-2 in parallel and
// returns (M, N) for each (segment 0's N starts from the initial state), seg_combine_kernel
// chains them into every segment's entry state (fp32 matrix cores), and the kernel in mode
// kOut then runs all segments in parallel from their entry states.  At most 256 (chain,
// segment) units, one workgroup per compute unit: for 16 chains of 4,096 chunks, 16 segments
// of 256 chunks per chain instead of one workgroup walking 4,096 chunks.
//   Both passes need every chunk's Tm = (I + A)^-1.  With room for it in the workspace, the
// transition (mode kTransTm, then over all nseg segments) forms it once and stores it, and the
// output pass (kOutTm) reads it back.  Neither pass then forms U or W: since U - W S =
// Tm (diag(beta) V - diag(beta e^gamma) K S), the state products run on K (already in LDS)
// and Delta = Tm R is one dense product; the output pass also skips K K^T, the diagonal-block
// inverses and the substitution, and needs 2 barriers per chunk instead of 5 (both passes
// stage the next chunk's inputs in stage 4, so neither needs a barrier after stage 0).
#include <algorithm>
#include <stddef.h>
#include <stdlib.h>
#include <type_traits>

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
// Inclusive prefix sum over the 64 lanes of a wavefront with DPP: row shifts by 1, 2, 4, 8
// within each row of 16 lanes, then the totals of rows 0 and 2 broadcast into rows 1 and 3
// (row_bcast:15) and that of rows 0-1 into rows 2 and 3 (row_bcast:31).  Lanes with no source
// add 0 (bound_ctrl), masked rows keep theirs.  No LDS permutes.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or_zero(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, ROWS, 0xf, true));
}
__device__ __forceinline__ float wave_inclusive_sum(float x) {
    x += dpp_or_zero<0x111, 0xf>(x);  // row_shr:1
    x += dpp_or_zero<0x112, 0xf>(x);  // row_shr:2
    x += dpp_or_zero<0x114, 0xf>(x);  // row_shr:4
    x += dpp_or_zero<0x118, 0xf>(x);  // row_shr:8
    x += dpp_or_zero<0x142, 0xa>(x);  // row_bcast:15 into rows 1, 3
    x += dpp_or_zero<0x143, 0xc>(x);  // row_bcast:31 into rows 2, 3
    return x;
}
// v of lane N of each group of four lanes, in all four (DPP quad_perm [N, N, N, N])
template <int N> __device__ __forceinline__ float quad_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 N * 0x55, 0xf, 0xf, false));
}
template <int N, typename Fn, int I = 0> __device__ __forceinline__ void static_for(Fn &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, Fn, I + 1>(static_cast<Fn &&>(f));
    }
}
// x, as a value the compiler cannot see through (nothing derived from it moves above this)
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}
// x, in hand here: the wait for a load into x happens at this point.  The compiler otherwise
// keeps a load that only some wavefronts issue as outstanding in all of them and waits for it
// -- that is, for every global access issued so far -- wherever its register is reused.
__device__ __forceinline__ void settle(f32x4 &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void settle(bf16_t &x) {
    unsigned u = x;
    asm volatile("" : "+v"(u));
    x = static_cast<bf16_t>(u);
}

// Power-of-two exponents for the fp16 copies of a value column (pow2_scale's rule as an
// exponent: m 2^e in [2^8, 2^9), e = 0 for m = 0, Inf or NaN, |e| <= 100).  A column carried at
// 2^e keeps e while its largest magnitude m stays in [2^6, 2^9) at that scale: the upper end
// keeps the fp16 operands as far from overflow as a fresh choice would, the lower end lets m
// drift by 8x before the fp32 state has to be rescaled (fp16's relative precision is the same
// over its normal range).
__device__ __forceinline__ int pow2_exponent(float m) {
    const int eb = static_cast<int>((__float_as_uint(m) >> 23) & 0xffu);
    const int ok = static_cast<int>(static_cast<unsigned>(eb - 1) < 254u);
    return ok * min(max(135 - eb, -100), 100);
}
__device__ __forceinline__ int next_exponent(float m, int e) {
    const float ms = __builtin_amdgcn_ldexpf(m, e);
    return (ms >= 64.f && ms < 512.f) ? e : pow2_exponent(m);
}
__device__ __forceinline__ float exp2i(int e) {  // 2^e for |e| <= 126
    return __uint_as_float(static_cast<uint32_t>(127 + e) << 23);
}
// x 2^de for every lane; skipped when no lane of the wavefront changes its exponent
template <int N> __device__ __forceinline__ void rescale(f32x4 (&x)[N], int de) {
    if (__builtin_amdgcn_ballot_w64(de != 0) == 0) return;
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) x[i][r] = __builtin_amdgcn_ldexpf(x[i][r], de);
}

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
    static_assert((D == 64 || D == 128) && (C == 32 || C == 64), "chunk kernel shape");
    static constexpr int NO = C * D / 4 / NT;  // 16-byte pieces of o per thread
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
    bf16_t v[C][F::PV];       // V rows (bf16, as stored)
    f16 p[C][F::PT];          // lower(Q K^T) o D (columns permuted)
    f16 wn[C][F::PQ];         // -W (columns permuted)
    f16 an[C][F::PA];         // -A, off-diagonal 16x16 blocks (lower)
    f16 td[F::NR][16][24];    // inverses of the diagonal blocks of I + A, fp16
    float adT[F::NR][16][20]; // diagonal blocks of A, fp32, transposed: [block][col][row]
    // per-chunk gates, double-buffered by chunk parity (those of the next chunk are formed
    // while this one runs)
    float gam[2][C];          // gamma (chunk-local cumulative log-gate)
    float Gam[2][C];          // exp(gamma)
    float dec[2][C];          // exp(gamma_last - gamma)
    float bet[2][C];          // beta
    float bg[2][C];           // beta exp(gamma)
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

// MODE kOut: the prefill itself -- outputs o, and the final state.  MODE kTrans: the segment
// transition of the segmented plan -- no outputs; besides the state N (from zero, or from s0
// on segment 0) it carries M, started at the identity and advanced by the same chunk maps
// without their value part:  M <- e^gamma_last M - K^T dec W M.  After the segment,
// S_out = M S_in + N for any state S_in entering it (Eq. (1) is affine in the state).
// MODE kTransTm: kTrans that also stores every chunk's (I + A)^-1 (below), for every segment
// including the last; kOutTm: kOut that reads it back instead of forming it (no K K^T, no
// diagonal-block inverses, no substitution, no W): Delta = Tm (diag(beta) V - diag(beta
// e^gamma) K S), since U - W S = Tm diag(beta) V - Tm diag(beta e^gamma) K S.
enum { kOut = 0, kTrans = 1, kOutTm = 2, kTransTm = 3 };

// Tm = (I + A)^-1 of a chunk, kept between the two passes of the segmented plan: its NB lower
// 16x16 blocks (a, cb), cb <= a, in the order a (a + 1) / 2 + cb, each as the 64 lanes' A
// operands of v_mfma_f32_16x16x16_f16 (lane l: row 16a + l % 16, columns 16cb + 4 (l / 16)
// .. + 3, four fp16 values): NB * 512 bytes per chunk.  The chunk of sequence b whose first
// row is t0 (of all the token rows) takes slot t0 / C + b of head hv's tm_nslot slots
// (sequences start anywhere, but the slots of sequence b end before the first of b + 1, so
// slots never collide; tm_nslot = ceil(rows / C) + B).
template <int C> struct TmGeom {
    static constexpr int NR = C / 16, NB = NR * (NR + 1) / 2;
    static constexpr int HALVES = NB * 256;  // per chunk
};
__device__ __forceinline__ constexpr int tri_row(int bi) {  // a of block bi = a (a + 1) / 2 + cb
    return bi >= 6 ? 3 : bi >= 3 ? 2 : bi >= 1 ? 1 : 0;
}

// Units: blocks [p nchains, (p + 1) nchains) run segment p (chunks p L .. p L + L - 1 of every
// chain, L = seg_chunks; seg_chunks = 0: L = ceil(chunks / nseg) from each chain's own length,
// for packed sequences, whose lengths only the device knows; a segment past a chain's end is
// empty: its transition is the identity; one segment with L >= the chunk count is the whole
// sequence).  kOut reads
// its initial state at s0 + p s0_seg_stride + chain D^2 and writes the final state on the last
// segment only; kTrans writes M, N of (segment p, chain) to mn + (p nchains + chain) 2 D^2.
template <int D, int C, typename TO, int MODE>
__global__ void __launch_bounds__((Cfg<D, C>::NT))
chunk_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
             const bf16_t *__restrict__ v, const bf16_t *__restrict__ beta,
             const bf16_t *__restrict__ g, const float *__restrict__ s0, TO *__restrict__ o,
             float *__restrict__ sT, int T, const int32_t *__restrict__ cu, unsigned flags,
             int Hk, int Hv, float scale, int nchains, int seg_chunks, int nseg,
             size_t s0_seg_stride, float *__restrict__ mn, uint16_t *__restrict__ tm,
             int tm_nslot) {
    using F = Cfg<D, C>;
    constexpr int NT = F::NT, NR = F::NR;
    constexpr bool TRANS = MODE == kTrans || MODE == kTransTm;
    constexpr bool TMW = MODE == kTransTm, TMR = MODE == kOutTm;
    constexpr int NB = TmGeom<C>::NB, TMH = TmGeom<C>::HALVES;
    constexpr int NTP = (NB * 32 + NT - 1) / NT;  // 16-byte pieces of Tm per thread
    // The wavefront that loads the gate inputs and forms the gates: the last with 8 wavefronts
    // (kOutTm: it has the fewest P tiles in stage 1; else it inverts one diagonal block in
    // stage 2, the shortest job there), 1 with 4 (wavefront 0 inverts in stage 2)
    constexpr int GW = TMR || F::NW == 8 ? F::NW - 1 : 1;
    // kOutTm stage 1: the P tiles are dealt out in turn, so the first NB mod NW wavefronts have
    // one more; with NB = 10 tiles over 8 wavefronts (C = 64, D = 128: PAIRP) wavefronts 6
    // and 7 take two tiles of row 3 each on one Q operand instead.  K^T is built by the
    // wavefronts w in [KTW, KTE), those with one tile.
    constexpr bool PAIRP = NB == 10 && F::NW == 8;
    // kTransTm with C = 64 and 8 wavefronts: K^T and the gates in stage 1 (see there)
    constexpr bool KT1 = TMW && NR == 4 && F::NW == 8;
    constexpr int KTW = PAIRP ? 0 : NB % F::NW, KTE = PAIRP ? 6 : F::NW;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    Smem<D, C> &sm = *reinterpret_cast<Smem<D, C> *>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;
    const int G = Hv / Hk;
    const int seg = static_cast<int>(blockIdx.x) / nchains;
    const int chain = chain_of_block(static_cast<int>(blockIdx.x) - seg * nchains, nchains, G);
    const int b = chain / Hv, hv = chain - b * Hv, hq = hv / G;
    const int col = 16 * wave + li;  // the state column this lane holds
    size_t base;  // this segment's first row and length
    int len;
    {
        int len0;
        seq_range(cu, T, b, base, len0);
        const long nch0 = (static_cast<long>(len0) + C - 1) / C;
        const long L = seg_chunks > 0 ? seg_chunks : (nch0 + nseg - 1) / nseg;
        const long start = static_cast<long>(seg) * L * C;
        len = static_cast<int>(max(0L, min(static_cast<long>(len0) - start, L * C)));
        base += static_cast<size_t>(min(start, static_cast<long>(len0)));
    }

    // ---- the state: tile it holds rows 16it + 4lg + r of column `col`, carried as 2^es S (es
    //      per column, a power of two chosen as described at next_exponent; 0 at the start)
    f32x4 S[F::NI];
    int es = 0;
    const size_t sbase = static_cast<size_t>(chain) * D * D;
    const float *sin = s0 == nullptr ? nullptr
                       : TRANS       ? (seg == 0 ? s0 + sbase : nullptr)
                                     : s0 + seg * s0_seg_stride + sbase;
    if (sin != nullptr) {  // one branch, so that all loads are in flight together
#pragma unroll
        for (int it = 0; it < F::NI; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[it][r] = sin[static_cast<size_t>(16 * it + 4 * lg + r) * D + col];
        // in hand before the chunk loop, where a wait for them would wait for every global
        // access in flight (the prefetches, the output stores)
#pragma unroll
        for (int it = 0; it < F::NI; ++it) settle(S[it]);
    } else {
#pragma unroll
        for (int it = 0; it < F::NI; ++it) S[it] = zero4();
    }
    // kTrans: the transition M, tiles as S, from the identity, carried as 2^em M
    f32x4 M[TRANS ? F::NI : 1];
    int em = 0;
    if constexpr (TRANS) {
#pragma unroll
        for (int it = 0; it < F::NI; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r) M[it][r] = (16 * it + 4 * lg + r == col) ? 1.f : 0.f;
    }

    // ---- raw inputs of coming chunks, prefetched into registers (rows past the end read as 0):
    //      q one chunk ahead; k, v and the gate inputs two chunks ahead in kOut, kOutTm and
    //      kTransTm (staged in LDS a chunk earlier than q, see stage 4), one in kTrans (staged
    //      in stage 0: its two states leave no registers to stage them during stage 4)
    u16x8 pq[F::NQ], pk[F::NQ], pv[F::NQ];
    u16x8 ptm[TMR ? NTP : 1];  // kOutTm: the chunk's Tm, one chunk ahead (with q)
    bf16_t pg = 0, pb = 0;
    // where chunk cidx's Tm record starts (in halves) in the tm records
    auto tm_slot = [&](int cidx) {
        return (static_cast<size_t>(hv) * tm_nslot + (base + static_cast<size_t>(cidx) * C) / C +
                static_cast<size_t>(b)) * TMH;
    };
    auto prefetch_q = [&](int cidx) {
        if constexpr (!TRANS) {
            const int tt = cidx * C, L = min(C, len - tt);
#pragma unroll
            for (int n = 0; n < F::NQ; ++n) {
                const int idx = tid + n * NT, r = idx / (D / 8), cc = idx - r * (D / 8);
                pq[n] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
                if (r < L)
                    pq[n] = *reinterpret_cast<const u16x8 *>(
                        q + ((base + tt + r) * Hk + hq) * D + cc * 8);
            }
        }
        if constexpr (TMR) {
            const uint16_t *src = tm + tm_slot(cidx);
#pragma unroll
            for (int n = 0; n < NTP; ++n) {
                const int idx = tid + n * NT;
                ptm[n] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
                if (idx < NB * 32) ptm[n] = *reinterpret_cast<const u16x8 *>(src + idx * 8);
            }
        }
    };
    auto prefetch_kv = [&](int cidx) {
        const int tt = cidx * C, L = min(C, len - tt);
#pragma unroll
        for (int n = 0; n < F::NQ; ++n) {
            const int idx = tid + n * NT, r = idx / (D / 8), cc = idx - r * (D / 8);
            pk[n] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
            pv[n] = pk[n];
            if (r < L) {
                const size_t row = base + tt + r;
                pk[n] = *reinterpret_cast<const u16x8 *>(k + (row * Hk + hq) * D + cc * 8);
                pv[n] = *reinterpret_cast<const u16x8 *>(v + (row * Hv + hv) * D + cc * 8);
            }
        }
        pg = 0;
        pb = 0;
        if (wave == GW && lane < L) {  // the gates: wavefront GW forms them (gates(), below)
            const size_t gi = (base + tt + lane) * Hv + hv;
            pg = g[gi];
            pb = beta[gi];
        }
    };
    // One 8-column piece of a q or k row as fp16: scaled by 1 / the row's norm with
    // GDN_QK_L2NORM (the D/8 consecutive lanes holding the row reduce its sum of squares), else
    // converted as it is.  Two copies of each staging loop (l2n), so that the common case
    // carries no unit multiply.
    auto half_row = [&](const u16x8 &x, auto l2n) {
        f16x8 h;
        if constexpr (decltype(l2n)::value) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a = bf16_to_f32(x[e]);
                ss += a * a;
            }
#pragma unroll
            for (int off = 1; off < D / 8; off <<= 1) ss += __shfl_xor(ss, off);
            const float sc = inv_norm_from_sumsq(ss);
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = f16(sc * bf16_to_f32(x[e]));
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = f16(bf16_to_f32(x[e]));
        }
        return h;
    };
    // columns 8cc .. 8cc+7 of a q or k row are two runs of 4 in the permuted order
    auto put_row = [&](f16 (*dst)[F::PQ], int r, int cc, f16x8 h) {
        *reinterpret_cast<f16x4 *>(&dst[r][kperm(cc * 8)]) = f16x4{h[0], h[1], h[2], h[3]};
        *reinterpret_cast<f16x4 *>(&dst[r][kperm(cc * 8 + 4)]) = f16x4{h[4], h[5], h[6], h[7]};
    };
    auto put_q = [&](auto l2n) {
#pragma unroll
        for (int n = 0; n < F::NQ; ++n) {
            const int idx = tid + n * NT, r = idx / (D / 8), cc = idx - r * (D / 8);
            put_row(sm.q, r, cc, half_row(pq[n], l2n));
        }
    };
    auto put_kv = [&](auto l2n) {
#pragma unroll
        for (int n = 0; n < F::NQ; ++n) {
            const int idx = tid + n * NT, r = idx / (D / 8), cc = idx - r * (D / 8);
            put_row(sm.k, r, cc, half_row(pk[n], l2n));
            *reinterpret_cast<u16x8 *>(&sm.v[r][cc * 8]) = pv[n];
        }
    };
    auto with_norm = [&](auto &&f) {
        if (flags & GDN_QK_L2NORM)
            f(std::true_type{});
        else
            f(std::false_type{});
    };
    // wavefront GW: the gates of chunk cidx into buffer cidx & 1, from pg, pb (rows past the end:
    // g = beta = 0)
    auto gates = [&](int cidx) {
        const int L = min(C, len - cidx * C), gb = cidx & 1;
        float gv = lane < L ? log_alpha_from_input(bf16_to_f32(pg), flags) : 0.f;
        gv = wave_inclusive_sum(gv);  // inclusive prefix sum over the chunk
        const float glast = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gv), C - 1));
        if (lane < C) {
            const float eg = __expf(gv), bt = lane < L ? beta_from_input(bf16_to_f32(pb), flags) : 0.f;
            sm.gam[gb][lane] = gv;
            sm.Gam[gb][lane] = eg;
            sm.dec[gb][lane] = __expf(glast - gv);
            sm.bet[gb][lane] = bt;
            sm.bg[gb][lane] = bt * eg;
        }
    };

    // Tm in LDS.  kTransTm: as rows (row r, column s at tmrow[r][s]), written by the panel
    // solves of stage 3 into the output staging area that kTrans leaves unused, and stored as
    // A-operand fragments by store_tm after the next barrier.  kOutTm: the fragments as
    // stored, double-buffered by chunk parity in the -A and -W arrays that kOutTm leaves
    // unused (tmfb).
    using SmemT = Smem<D, C>;
    f16(*tmrow)[F::PA] = reinterpret_cast<f16(*)[F::PA]>(&sm.ost[0][0]);
    auto tmfb = [&](int buf) -> f16 * {  // kOutTm: two buffers, by chunk parity
        return buf ? &sm.wn[0][0] : &sm.an[0][0];
    };
    auto put_tm = [&](int buf) {
        f16 *dst = tmfb(buf);
#pragma unroll
        for (int n = 0; n < NTP; ++n) {
            const int idx = tid + n * NT;
            if (idx < NB * 32) *reinterpret_cast<u16x8 *>(dst + idx * 8) = ptm[n];
        }
    };
    static_assert(sizeof(sm.ost) >= sizeof(f16) * C * F::PA && sizeof(sm.an) >= 2 * TMH && sizeof(sm.wn) >= 2 * TMH &&
                      offsetof(SmemT, ost) % 16 == 0 && offsetof(SmemT, an) % 16 == 0 &&
                      offsetof(SmemT, wn) % 16 == 0,
                  "Tm staging");
    auto store_tm = [&](int cidx) {  // 16-byte pieces: the fragments of lanes 2p', 2p' + 1
        uint16_t *dst = tm + tm_slot(cidx);
        for (int idx = tid; idx < NB * 32; idx += NT) {
            const int bi = idx >> 5, l = 2 * (idx & 31), a = tri_row(bi), cb = bi - a * (a + 1) / 2;
            const f16 *src = &tmrow[16 * a + (l & 15)][16 * cb + 4 * (l >> 4)];
            *reinterpret_cast<f16x8 *>(dst + idx * 8) =
                cat(*reinterpret_cast<const f16x4 *>(src), *reinterpret_cast<const f16x4 *>(src + F::PA));
        }
    };

    const int nchunks = (len + C - 1) / C;
    if (nchunks > 0) {
        prefetch_q(0);
        prefetch_kv(0);
        if constexpr (!TRANS || TMW) with_norm(put_kv);  // chunk 0's k, v (LDS is not in use yet)
        if constexpr (TMR) {  // and q, Tm
            with_norm(put_q);
            put_tm(0);
        }
        if (wave == GW) gates(0);
        if constexpr (!TRANS || TMW) prefetch_kv(1);
        if constexpr (TMR)
            if (nchunks > 1) prefetch_q(1);
    }
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C, cb = c & 1;
        lds_barrier();  // the previous chunk is done with every LDS buffer
        if constexpr (TMW) {
            // ---- stage 0 of kTransTm: the previous chunk's Tm out of LDS (this chunk's k and v
            //      were staged in stage 4 of the previous one; stage 3 next writes Tm two barriers
            //      from here, so this stage needs none of its own)
            if (c > 0) store_tm(c - 1);
        } else if constexpr (TRANS) {
            // ---- stage 0 of the transition: this chunk's k and v in LDS, prefetch of the next
            with_norm(put_kv);
            if (c + 1 < nchunks) prefetch_kv(c + 1);
            lds_barrier();
        } else {
            // ---- stage 0: stage this chunk's q in LDS, store the previous chunk's output, prefetch
            //      the next q (this chunk's k and v were staged during the previous chunk; kOutTm:
            //      q and Tm too, so this stage only stores)
            if constexpr (!TMR) with_norm(put_q);  // (kOutTm: staged in stage 4 of the last chunk)
            if (c > 0) {
                const int tp = t0 - C;  // the previous chunk is always a full one
#pragma unroll
                for (int n = 0; n < F::NO; ++n) {
                    const int idx = tid + n * NT, r = idx / (D / 4), cc = idx - r * (D / 4);
                    const f32x4 x = *reinterpret_cast<const f32x4 *>(&sm.ost[r][cc * 4]);
                    store4<TO>(o + ((base + tp + r) * Hv + hv) * D + cc * 4, x);
                }
            }
            if constexpr (!TMR) {
                if (c + 1 < nchunks) prefetch_q(c + 1);
                lds_barrier();
            }
            // (kOutTm: no barrier -- the stores only read the output staging, which stage 4
            // writes one barrier on, after every wavefront's LDS reads here have completed)
        }

        if constexpr (TMR) {
            // ---- kOutTm stage 1: P = lower(Q K^T) o D (tiles shared out over the wavefronts),
            //      K^T (by the wavefronts w >= KTW), and per wavefront over its own columns:
            //      K S and Q S, and R = diag(beta) V - diag(beta e^gamma) K S, all carried
            //      scaled by sig
            settle(pg);  // the next chunk's gate inputs (loaded by wavefront GW only)
            settle(pb);
            if (wave == GW && c + 1 < nchunks) gates(c + 1);  // its inputs came with the prefetch
            // (lane offsets made opaque: the LDS addresses of this stage and stage 4 are formed
            // here, not kept in registers across the chunk loop)
            const int li = opaque(lane & 15), lg = opaque(lane >> 4);
            const int col = 16 * wave + li;
            f32x4 yv[NR];
            float vmax = 0.f;
#pragma unroll
            for (int a = 0; a < NR; ++a)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int r = 16 * a + 4 * lg + rr;
                    yv[a][rr] = sm.bet[cb][r] * bf16_to_f32(sm.v[r][col]);
                    vmax = fmaxf(vmax, fabsf(yv[a][rr]));
                }
            {
                float smax = 0.f;
#pragma unroll
                for (int it = 0; it < F::NI; ++it)
#pragma unroll
                    for (int r = 0; r < 4; ++r) smax = fmaxf(smax, fabsf(S[it][r]));
                vmax = max_over_rows(fmaxf(vmax, __builtin_amdgcn_ldexpf(smax, -es)));
                const int en = next_exponent(vmax, es);
                rescale(S, en - es);
                es = en;
            }
            const float sig = exp2i(es), isig = exp2i(-es);
            f16x8 bS[F::KD];
#pragma unroll
            for (int kk = 0; kk < F::KD; ++kk)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bS[kk][e] = f16(S[2 * kk][e]);
                    bS[kk][4 + e] = f16(S[2 * kk + 1][e]);
                }
            f32x4 R[NR], O[NR];
#pragma unroll
            for (int rt = 0; rt < NR; ++rt) {
                f32x4 ks = zero4();
                O[rt] = zero4();
#pragma unroll
                for (int kk = 0; kk < F::KD; ++kk) {
                    const f16x8 ak = *reinterpret_cast<const f16x8 *>(&sm.k[16 * rt + li][32 * kk + 8 * lg]);
                    const f16x8 aq = *reinterpret_cast<const f16x8 *>(&sm.q[16 * rt + li][32 * kk + 8 * lg]);
                    ks = mma_k32(ak, bS[kk], ks);
                    O[rt] = mma_k32(aq, bS[kk], O[rt]);
                }
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int r = 16 * rt + 4 * lg + rr;
                    O[rt][rr] *= sm.Gam[cb][r];
                    R[rt][rr] = sig * yv[rt][rr] - sm.bg[cb][r] * ks[rr];
                }
            }
            // P tile (rt, st), st <= rt: the decayed, masked fp16 values into LDS
            auto pput = [&](int rt, int st, const f32x4 &acc) {
                const int s = 16 * st + li;
                const float gs = sm.gam[cb][s];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int r = 16 * rt + 4 * lg + rr;
                    const float d = (s <= r) ? __expf(sm.gam[cb][r] - gs) : 0.f;
                    sm.p[r][kperm(s)] = f16(acc[rr] * d);
                    // the tile right of the diagonal is read by P Delta
                    if (st == rt && rt + 1 < NR) sm.p[r][kperm(s + 16)] = f16(0.f);
                }
            };
            if constexpr (PAIRP) {
                // wavefront w < 6 takes tile w (triangle order); wavefronts 6 and 7 the pairs
                // (3, 0..1) and (3, 2..3), one Q operand feeding both products
                if (wave < 6) {
                    const int rt = tri_row(wave), st = wave - rt * (rt + 1) / 2;
                    f32x4 acc = zero4();
#pragma unroll
                    for (int kk = 0; kk < F::KD; ++kk)
                        acc = mma_k32(*reinterpret_cast<const f16x8 *>(&sm.q[16 * rt + li][32 * kk + 8 * lg]),
                                      *reinterpret_cast<const f16x8 *>(&sm.k[16 * st + li][32 * kk + 8 * lg]),
                                      acc);
                    pput(rt, st, acc);
                } else {
                    const int st = 2 * (wave - 6);
                    f32x4 a0 = zero4(), a1 = zero4();
#pragma unroll
                    for (int kk = 0; kk < F::KD; ++kk) {
                        const f16x8 aq = *reinterpret_cast<const f16x8 *>(&sm.q[48 + li][32 * kk + 8 * lg]);
                        a0 = mma_k32(aq, *reinterpret_cast<const f16x8 *>(&sm.k[16 * st + li][32 * kk + 8 * lg]), a0);
                        a1 = mma_k32(aq, *reinterpret_cast<const f16x8 *>(&sm.k[16 * st + 16 + li][32 * kk + 8 * lg]), a1);
                    }
                    pput(3, st, a0);
                    pput(3, st + 1, a1);
                }
            } else {
                for (int j = wave; j < NB; j += F::NW) {
                    const int rt = tri_row(j), st = j - rt * (rt + 1) / 2;
                    f32x4 acc = zero4();
#pragma unroll
                    for (int kk = 0; kk < F::KD; ++kk)
                        acc = mma_k32(*reinterpret_cast<const f16x8 *>(&sm.q[16 * rt + li][32 * kk + 8 * lg]),
                                      *reinterpret_cast<const f16x8 *>(&sm.k[16 * st + li][32 * kk + 8 * lg]),
                                      acc);
                    pput(rt, st, acc);
                }
            }
            for (int idx = tid - 64 * KTW; idx >= 0 && idx < D * (C / 8) && wave < KTE;
                 idx += NT - 64 * KTW - 64 * (F::NW - KTE)) {
                const int i = idx % D, s8 = idx / D, ki = kperm(i);
                f16x8 x;  // stored positions 8 s8 .. 8 s8 + 7 of row i of K^T
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = sm.k[kunperm(s8 * 8 + e)][ki];
                *reinterpret_cast<f16x8 *>(&sm.kt[i][s8 * 8]) = x;
            }
            lds_barrier();

            // ---- kOutTm stage 4: the next chunk's k and v into LDS (nothing below reads them),
            //      the prefetch of the chunk after it; Delta = Tm R, O += P Delta, next state
            with_norm(put_kv);
            prefetch_kv(c + 2);
            with_norm(put_q);       // q and Tm of the next chunk: stage 1 was the last reader of
            put_tm((c + 1) & 1);    // this chunk's q; its Tm is in the other buffer
            if (c + 2 < nchunks) prefetch_q(c + 2);
            const f16 *tmf = tmfb(c & 1);
            f32x4 Dl[NR];
#pragma unroll
            for (int a = 0; a < NR; ++a) {
                Dl[a] = zero4();
#pragma unroll
                for (int cb2 = 0; cb2 <= a; ++cb2)
                    Dl[a] = mma_k16(*reinterpret_cast<const f16x4 *>(
                                        tmf + ((a * (a + 1) / 2 + cb2) * 64 + lane) * 4),
                                    to_f16x4(R[cb2]), Dl[a]);
            }
            f16x8 bD[F::KC], bDs[F::KC];
#pragma unroll
            for (int kk = 0; kk < F::KC; ++kk)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s0i = 32 * kk + 4 * lg + e, s1i = s0i + 16;
                    const float d0 = Dl[2 * kk][e], d1 = Dl[2 * kk + 1][e];
                    bD[kk][e] = f16(d0);
                    bD[kk][4 + e] = f16(d1);
                    bDs[kk][e] = f16(d0 * sm.dec[cb][s0i]);
                    bDs[kk][4 + e] = f16(d1 * sm.dec[cb][s1i]);
                }
            const float oscale = scale * isig;  // exact: isig is a power of two
#pragma unroll
            for (int rt = 0; rt < NR; ++rt) {
#pragma unroll
                for (int kk = 0; kk < F::KC; ++kk)
                    if (32 * kk <= 16 * rt + 15)
                        O[rt] = mma_k32(*reinterpret_cast<const f16x8 *>(&sm.p[16 * rt + li][32 * kk + 8 * lg]),
                                        bD[kk], O[rt]);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) sm.ost[16 * rt + 4 * lg + rr][col] = oscale * O[rt][rr];
            }
            const float GC = sm.Gam[cb][C - 1];
#pragma unroll
            for (int it = 0; it < F::NI; ++it) {
                S[it] *= GC;
#pragma unroll
                for (int kk = 0; kk < F::KC; ++kk)
                    S[it] = mma_k32(*reinterpret_cast<const f16x8 *>(&sm.kt[16 * it + li][32 * kk + 8 * lg]),
                                    bDs[kk], S[it]);
            }
            continue;
        }

        // ---- stage 1: KK^T -> A, QK^T -> P (lower-triangular 16x16 tiles), and K^T
        {
        const int li_ = li, lg_ = lg;
        // Jobs: wavefront w < NR takes row tile w of K K^T; wavefront w >= NR row tile
        // 2 NR - 1 - w of Q K^T (kTrans, which needs only K K^T: the same row tiles of K K^T, the
        // columns of odd parity).  Wavefronts w and w + 4 share a SIMD, so each SIMD gets row
        // tiles r and NR - 1 - r: (r + 1) + (NR - r) lower 16x16 tiles, the same for every SIMD
        // (one SIMD holding both longest row tiles took twice as long).
        // (kTrans: the lane's row and column offsets are made opaque here, so that the compiler
        // forms this stage's LDS addresses in the loop instead of keeping them in registers
        // across it -- the transition's second state leaves no registers for that)
        const int li = TRANS ? opaque(li_) : li_, lg = TRANS ? opaque(lg_) : lg_;
        for (int job = wave; job < 2 * NR; job += F::NW) {
            const bool isq = !TRANS && job >= NR;
            const int rt = job >= NR ? 2 * NR - 1 - job : job;
            const int par = job >= NR ? 1 : 0;
            const f16 *arow = isq ? &sm.q[16 * rt + li][0] : &sm.k[16 * rt + li][0];
            f16x8 af[F::KD];
#pragma unroll
            for (int kk = 0; kk < F::KD; ++kk)
                af[kk] = *reinterpret_cast<const f16x8 *>(arow + 32 * kk + 8 * lg);
            float gr[4], br[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                gr[rr] = sm.gam[cb][16 * rt + 4 * lg + rr];
                br[rr] = sm.bet[cb][16 * rt + 4 * lg + rr];
            }
            // the decayed, scaled tile (rt, st) into LDS: P (isq), else -A off the diagonal and
            // A on it (fp32, transposed)
            auto put_tile = [&](int st, const f32x4 &acc) {
                const int s = 16 * st + li;
                const float gs = sm.gam[cb][s];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int r = 16 * rt + 4 * lg + rr;
                    const float d = (s <= r) ? __expf(gr[rr] - gs) : 0.f;
                    if (isq) {
                        sm.p[r][kperm(s)] = f16(acc[rr] * d);
                    } else {
                        const float av = (s < r) ? br[rr] * d * acc[rr] : 0.f;
                        if (st == rt)
                            sm.adT[rt][li][4 * lg + rr] = av;
                        else
                            sm.an[r][s] = f16(-av);
                    }
                }
            };
            if constexpr (TRANS) {
                // the job's tiles st = par and par + 2 (those <= rt), both products issued before
                // either tile is stored (a tile past rt is computed on row NR - 1 and dropped)
                const int st0 = par, st1 = par + 2;
                const int k0 = min(st0, NR - 1), k1 = min(st1, NR - 1);
                f32x4 a0 = zero4(), a1 = zero4();
#pragma unroll
                for (int kk = 0; kk < F::KD; ++kk) {
                    a0 = mma_k32(af[kk], *reinterpret_cast<const f16x8 *>(&sm.k[16 * k0 + li][32 * kk + 8 * lg]), a0);
                    a1 = mma_k32(af[kk], *reinterpret_cast<const f16x8 *>(&sm.k[16 * k1 + li][32 * kk + 8 * lg]), a1);
                }
                if (st0 <= rt) put_tile(st0, a0);
                if (st1 <= rt) put_tile(st1, a1);
                continue;
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
                put_tile(st, acc);
            }
            if (isq && rt + 1 < NR) {  // the tile right of the diagonal is read by P Delta
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    sm.p[16 * rt + 4 * lg + rr][kperm(16 * (rt + 1) + li)] = f16(0.f);
            }
        }
        if constexpr (KT1) {
            // kTransTm, C = 64, 8 wavefronts: the wavefronts with at most one K K^T tile here
            // (0, 1, 5, 6 and 7) build K^T, and 7 forms the next chunk's gates, so that stage 2
            // holds only the diagonal-block inverses
            settle(pg);
            settle(pb);
            if (wave == GW && c + 1 < nchunks) gates(c + 1);  // its inputs came with the prefetch
            const int kw = wave < 2 ? wave : wave - 3;  // 0, 1, 2, 3, 4 for waves 0, 1, 5, 6, 7
            if (wave < 2 || wave >= 5) {
                for (int idx = 64 * kw + lane; idx < D * (C / 8); idx += 320) {
                    const int i = idx % D, s8 = idx / D, ki = kperm(i);
                    f16x8 x;  // stored positions 8 s8 .. 8 s8 + 7 of row i of K^T
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = sm.k[kunperm(s8 * 8 + e)][ki];
                    *reinterpret_cast<f16x8 *>(&sm.kt[i][s8 * 8]) = x;
                }
            }
        }
        }
        lds_barrier();

        // ---- stage 2: the inverses of the 16x16 diagonal blocks of I + A (fp32 forward
        //      substitution by columns: step s updates every later row with x_s, a dependent
        //      chain of 15 steps), and K^T for the state update and the W panels.  With 8
        //      wavefronts, wavefronts 4 .. 4 + NR - 1 take one block each, four lanes a column;
        //      with 4, wavefront 0 takes them all, one lane a column, while the others build
        //      K^T
        settle(pg);  // the next chunk's gate inputs (loaded by wavefront GW only)
        settle(pb);
        if constexpr (F::NW == 8) {
            // wavefront 4 + b inverts block b: lane l holds rows 4q .. 4q + 3 (q = l mod 4) of
            // column j = l / 4, so a column is a DPP quad.  Step s: x_s from lane s / 4 of the
            // quad, then x_r -= A[r][s] x_s for the lane's four rows (A[r][s] = 0 for r <= s,
            // so no lane needs a mask): 15 steps of one broadcast and four FMAs.  The other
            // wavefronts build K^T meanwhile
            if (wave >= 4 && wave < 4 + NR) {
                const int bb = wave - 4, j = lane >> 2, q = lane & 3;
                float x[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = (4 * q + i == j) ? 1.f : 0.f;
                f32x4 a[15];  // A[4q + i][s], every s, loaded before the chain starts
#pragma unroll
                for (int st = 0; st < 15; ++st)
                    a[st] = *reinterpret_cast<const f32x4 *>(&sm.adT[bb][st][4 * q]);
                static_for<15>([&](auto stc) {
                    constexpr int st = decltype(stc)::value;
                    const float xs = quad_bcast<st / 4>(x[st % 4]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] -= a[st][i] * xs;
                });
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.td[bb][4 * q + i][j] = f16(x[i]);
            }
            if (!KT1 && wave == GW && c + 1 < nchunks) gates(c + 1);  // its inputs came with the prefetch
            // K^T by the wavefronts that invert nothing (0 .. 3 and 4 + NR ..; KT1: in stage 1)
            const int kb = wave < 4 ? tid : tid - 64 * NR;
            for (int idx = kb; !KT1 && (wave < 4 || wave >= 4 + NR) && idx < D * (C / 8);
                 idx += NT - 64 * NR) {
                const int i = idx % D, s8 = idx / D, ki = kperm(i);
                f16x8 x;  // stored positions 8 s8 .. 8 s8 + 7 of row i of K^T
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = sm.k[kunperm(s8 * 8 + e)][ki];
                *reinterpret_cast<f16x8 *>(&sm.kt[i][s8 * 8]) = x;
            }
        } else {
            if (wave == 0) {
                float x[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] = (r == li) ? 1.f : 0.f;
                if (lg < NR) {
#pragma unroll
                    for (int st = 0; st < 15; ++st) {
                        float colv[16];
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4) {
                            const f32x4 t = *reinterpret_cast<const f32x4 *>(&sm.adT[lg][st][4 * r4]);
                            colv[4 * r4] = t[0], colv[4 * r4 + 1] = t[1], colv[4 * r4 + 2] = t[2], colv[4 * r4 + 3] = t[3];
                        }
#pragma unroll
                        for (int r = st + 1; r < 16; ++r) x[r] -= colv[r] * x[st];
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) sm.td[lg][r][li] = f16(x[r]);
                }
            } else {
                if (wave == GW && c + 1 < nchunks) gates(c + 1);  // its inputs came with the prefetch
                for (int idx = tid - 64; idx < D * (C / 8); idx += NT - 64) {
                    const int i = idx % D, s8 = idx / D, ki = kperm(i);
                    f16x8 x;  // stored positions 8 s8 .. 8 s8 + 7 of row i of K^T
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = sm.k[kunperm(s8 * 8 + e)][ki];
                    *reinterpret_cast<f16x8 *>(&sm.kt[i][s8 * 8]) = x;
                }
            }
        }
        lds_barrier();

        if constexpr (TMW) {
            // ---- kTransTm stage 3, per wavefront over its own columns: the scales of N and M
            //      for this chunk (as in stage 3 of the other modes), then R_N = diag(beta) V -
            //      diag(beta e^gamma) K N and R_M = -diag(beta e^gamma) K M (fp16, as the
            //      operands of stage 4 take them); then wavefront j < NR solves column panel j
            //      of Tm = (I + A)^-1 by blocked substitution, X_a = T_aa (delta_aj I -
            //      sum_{cb < a} A_{a,cb} X_cb) (X_a = 0 for a < j), into tmrow: read back in
            //      stage 4 and stored after the next barrier
            f16x4 RN[NR], RM[NR];
            // (lane offsets made opaque, so that the compiler forms these stages' LDS addresses
            // here instead of keeping them in registers across the chunk loop)
            const int li = opaque(lane & 15), lg = opaque(lane >> 4);
            auto rprod = [&]() {
                f32x4 yv[NR];
                float vmax = 0.f;
#pragma unroll
                for (int a = 0; a < NR; ++a)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int r = 16 * a + 4 * lg + rr;
                        yv[a][rr] = sm.bet[cb][r] * bf16_to_f32(sm.v[r][col]);
                        vmax = fmaxf(vmax, fabsf(yv[a][rr]));
                    }
                float smax = 0.f, mmax = 0.f;
#pragma unroll
                for (int it = 0; it < F::NI; ++it)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        smax = fmaxf(smax, fabsf(S[it][r]));
                        mmax = fmaxf(mmax, fabsf(M[it][r]));
                    }
                vmax = max_over_rows(fmaxf(vmax, __builtin_amdgcn_ldexpf(smax, -es)));
                const int en = next_exponent(vmax, es);
                rescale(S, en - es);
                es = en;
                const float mm = max_over_rows(__builtin_amdgcn_ldexpf(mmax, -em));
                const int enm = next_exponent(mm, em);
                rescale(M, enm - em);
                em = enm;
                // k-steps outermost, so that one k-step of the B operands is live at a time
                f32x4 kn[NR], km[NR];
#pragma unroll
                for (int rt = 0; rt < NR; ++rt) {
                    kn[rt] = zero4();
                    km[rt] = zero4();
                }
#pragma unroll
                for (int kk = 0; kk < F::KD; ++kk) {
                    f16x8 bS, bM;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bS[e] = f16(S[2 * kk][e]);
                        bS[4 + e] = f16(S[2 * kk + 1][e]);
                        bM[e] = f16(M[2 * kk][e]);
                        bM[4 + e] = f16(M[2 * kk + 1][e]);
                    }
#pragma unroll
                    for (int rt = 0; rt < NR; ++rt) {
                        const f16x8 ak = *reinterpret_cast<const f16x8 *>(&sm.k[16 * rt + li][32 * kk + 8 * lg]);
                        kn[rt] = mma_k32(ak, bS, kn[rt]);
                        km[rt] = mma_k32(ak, bM, km[rt]);
                    }
                }
                const float sig = exp2i(es);
#pragma unroll
                for (int rt = 0; rt < NR; ++rt) {
                    f32x4 rn, rm;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const float bgr = sm.bg[cb][16 * rt + 4 * lg + rr];
                        rn[rr] = sig * yv[rt][rr] - bgr * kn[rt][rr];
                        rm[rr] = -bgr * km[rt][rr];
                    }
                    RN[rt] = to_f16x4(rn);
                    RM[rt] = to_f16x4(rm);
                }
            };
            rprod();
            if (wave < NR) {
                // the blocks' A operands, loaded before the chain starts
                f16x4 anb[NB], tdb[NR];
#pragma unroll
                for (int a = 0; a < NR; ++a) {
                    tdb[a] = *reinterpret_cast<const f16x4 *>(&sm.td[a][li][4 * lg]);
#pragma unroll
                    for (int cb2 = 0; cb2 < a; ++cb2)
                        anb[a * (a - 1) / 2 + cb2] =
                            *reinterpret_cast<const f16x4 *>(&sm.an[16 * a + li][16 * cb2 + 4 * lg]);
                }
                f16x4 X[NR];  // as the fp16 operands (and the stored values) they become
#pragma unroll
                for (int a = 0; a < NR; ++a) {
                    f32x4 yx;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) yx[rr] = (a == wave && 4 * lg + rr == li) ? 1.f : 0.f;
#pragma unroll
                    for (int cb2 = 0; cb2 < a; ++cb2) yx = mma_k16(anb[a * (a - 1) / 2 + cb2], X[cb2], yx);
                    X[a] = to_f16x4(mma_k16(tdb[a], to_f16x4(yx), zero4()));
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) tmrow[16 * a + 4 * lg + rr][16 * wave + li] = X[a][rr];
                }
            }
            lds_barrier();

            // ---- kTransTm stage 4: the next chunk's k and v into LDS (nothing here reads them)
            //      and the prefetch of the chunk after it; Delta_N = Tm R_N, Delta_M = Tm R_M,
            //      then N and M through K^T diag(e^(gamma_last - gamma)) as in the other
            //      transition
            with_norm(put_kv);
            prefetch_kv(c + 2);
            f32x4 DN[NR], DM[NR];
#pragma unroll
            for (int a = 0; a < NR; ++a) {
                DN[a] = zero4();
                DM[a] = zero4();
#pragma unroll
                for (int cb2 = 0; cb2 <= a; ++cb2) {
                    const f16x4 at = *reinterpret_cast<const f16x4 *>(&tmrow[16 * a + li][16 * cb2 + 4 * lg]);
                    DN[a] = mma_k16(at, RN[cb2], DN[a]);
                    DM[a] = mma_k16(at, RM[cb2], DM[a]);
                }
            }
            f16x8 bDs[F::KC], bDm[F::KC];
#pragma unroll
            for (int kk = 0; kk < F::KC; ++kk)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s0i = 32 * kk + 4 * lg + e, s1i = s0i + 16;
                    bDs[kk][e] = f16(DN[2 * kk][e] * sm.dec[cb][s0i]);
                    bDs[kk][4 + e] = f16(DN[2 * kk + 1][e] * sm.dec[cb][s1i]);
                    bDm[kk][e] = f16(DM[2 * kk][e] * sm.dec[cb][s0i]);
                    bDm[kk][4 + e] = f16(DM[2 * kk + 1][e] * sm.dec[cb][s1i]);
                }
            const float GC = sm.Gam[cb][C - 1];
#pragma unroll
            for (int it = 0; it < F::NI; ++it) {
                S[it] *= GC;
                M[it] *= GC;
#pragma unroll
                for (int kk = 0; kk < F::KC; ++kk) {
                    const f16x8 ak = *reinterpret_cast<const f16x8 *>(&sm.kt[16 * it + li][32 * kk + 8 * lg]);
                    S[it] = mma_k32(ak, bDs[kk], S[it]);
                    M[it] = mma_k32(ak, bDm[kk], M[it]);
                }
            }
            continue;
        }

        // ---- stage 3: blocked forward substitution for this wave's panels,
        //      U[:, 16w..] = (I+A)^-1 diag(beta) V[:, 16w..]  (kept in registers)
        //      W[:, 16w..] = (I+A)^-1 diag(beta e^gamma) K[:, 16w..]  (-W to LDS)
        //      The value side of this column (U, Delta, S, O) is carried scaled by sig = 2^es, from
        //      the column's largest |beta v| in the chunk and |S| at its start (next_exponent).
        f32x4 yv[NR];
        float vmax = 0.f;
#pragma unroll
        for (int a = 0; a < NR; ++a)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = 16 * a + 4 * lg + rr;
                yv[a][rr] = sm.bet[cb][r] * bf16_to_f32(sm.v[r][col]);
                vmax = fmaxf(vmax, fabsf(yv[a][rr]));
            }
        {
            float smax = 0.f;
#pragma unroll
            for (int it = 0; it < F::NI; ++it)
#pragma unroll
                for (int r = 0; r < 4; ++r) smax = fmaxf(smax, fabsf(S[it][r]));
            // the column's four lanes; |S| = 2^-es |carried S|
            vmax = max_over_rows(fmaxf(vmax, __builtin_amdgcn_ldexpf(smax, -es)));
            const int en = next_exponent(vmax, es);
            rescale(S, en - es);
            es = en;
        }
        const float sig = exp2i(es), isig = exp2i(-es);
        if constexpr (TRANS) {  // the same for the columns of M
            float mmax = 0.f;
#pragma unroll
            for (int it = 0; it < F::NI; ++it)
#pragma unroll
                for (int r = 0; r < 4; ++r) mmax = fmaxf(mmax, fabsf(M[it][r]));
            const float m = max_over_rows(__builtin_amdgcn_ldexpf(mmax, -em));
            const int en = next_exponent(m, em);
            rescale(M, en - em);
            em = en;
        }
        f32x4 U[NR], Wp[NR];
#pragma unroll
        for (int a = 0; a < NR; ++a) {
            const f16x4 kv4 = *reinterpret_cast<const f16x4 *>(&sm.kt[col][kperm(16 * a + 4 * lg)]);
            f32x4 yu, yw;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = 16 * a + 4 * lg + rr;
                yu[rr] = sig * yv[a][rr];
                yw[rr] = sm.bg[cb][r] * float(kv4[rr]);
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

        // ---- kOut: the next chunk's k and v into LDS (stage 3 was the last reader of this chunk's;
        //      stage 4 reads neither), then the prefetch of the chunk after it -- all of it
        //      independent of stage 4's products, free to interleave with them.  Past the last
        //      chunk the rows are zero and nothing reads them.
        if constexpr (!TRANS) {
            with_norm(put_kv);
            prefetch_kv(c + 2);
        }

        if constexpr (TRANS) {
            // ---- stage 4 of the transition: N as the state (U - W N), M with no value part
            //      (-W M); both updated through K^T diag(e^(gamma_last - gamma)), each column
            //      scaled by its own power of two
            // k-steps outermost, so that only one k-step of the B operands is live at a time
            f32x4 DM[NR];
#pragma unroll
            for (int rt = 0; rt < NR; ++rt) DM[rt] = zero4();
#pragma unroll
            for (int kk = 0; kk < F::KD; ++kk) {
                f16x8 bS, bM;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bS[e] = f16(S[2 * kk][e]);
                    bS[4 + e] = f16(S[2 * kk + 1][e]);
                    bM[e] = f16(M[2 * kk][e]);
                    bM[4 + e] = f16(M[2 * kk + 1][e]);
                }
#pragma unroll
                for (int rt = 0; rt < NR; ++rt) {
                    const f16x8 aw = *reinterpret_cast<const f16x8 *>(&sm.wn[16 * rt + li][32 * kk + 8 * lg]);
                    U[rt] = mma_k32(aw, bS, U[rt]);
                    DM[rt] = mma_k32(aw, bM, DM[rt]);
                }
            }
            f16x8 bDs[F::KC], bDm[F::KC];
#pragma unroll
            for (int kk = 0; kk < F::KC; ++kk)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s0i = 32 * kk + 4 * lg + e, s1i = s0i + 16;
                    bDs[kk][e] = f16(U[2 * kk][e] * sm.dec[cb][s0i]);
                    bDs[kk][4 + e] = f16(U[2 * kk + 1][e] * sm.dec[cb][s1i]);
                    bDm[kk][e] = f16(DM[2 * kk][e] * sm.dec[cb][s0i]);
                    bDm[kk][4 + e] = f16(DM[2 * kk + 1][e] * sm.dec[cb][s1i]);
                }
            const float GC = sm.Gam[cb][C - 1];
#pragma unroll
            for (int it = 0; it < F::NI; ++it) {
                S[it] *= GC;
                M[it] *= GC;
#pragma unroll
                for (int kk = 0; kk < F::KC; ++kk) {
                    const f16x8 ak = *reinterpret_cast<const f16x8 *>(&sm.kt[16 * it + li][32 * kk + 8 * lg]);
                    S[it] = mma_k32(ak, bDs[kk], S[it]);
                    M[it] = mma_k32(ak, bDm[kk], M[it]);
                }
            }
            continue;
        }

        // ---- stage 4 (sequential part): Delta, O, next state -- U, Delta, O, S scaled by sig
        // sig S as fp16 B operands over the key index: slot e < 4 -> tile 2kk row 4lg+e,
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
            for (int rr = 0; rr < 4; ++rr) O[rt][rr] *= sm.Gam[cb][16 * rt + 4 * lg + rr];
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
                bDs[kk][e] = f16(d0 * sm.dec[cb][s0i]);
                bDs[kk][4 + e] = f16(d1 * sm.dec[cb][s1i]);
            }
        // O += P Delta, staged in LDS for the coalesced store at the top of the next chunk
        // (stored from the accumulators, 4-byte pieces of 4 rows per instruction, the call took
        // 11% longer; stored in the next chunk from registers, 19%)
        const float oscale = scale * isig;  // exact: isig is a power of two
#pragma unroll
        for (int rt = 0; rt < NR; ++rt) {
#pragma unroll
            for (int kk = 0; kk < F::KC; ++kk)
                if (32 * kk <= 16 * rt + 15)
                    O[rt] = mma_k32(*reinterpret_cast<const f16x8 *>(&sm.p[16 * rt + li][32 * kk + 8 * lg]),
                                    bD[kk], O[rt]);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sm.ost[16 * rt + 4 * lg + rr][col] = oscale * O[rt][rr];
        }
        // S = e^gamma_last S + K^T diag(e^(gamma_last - gamma)) Delta, all carried scaled by
        // sig: sig S_next = e^gamma_last (sig S) + K^T diag(..) (sig Delta)
        const float GC = sm.Gam[cb][C - 1];
#pragma unroll
        for (int it = 0; it < F::NI; ++it) {
            S[it] *= GC;
#pragma unroll
            for (int kk = 0; kk < F::KC; ++kk)
                S[it] = mma_k32(*reinterpret_cast<const f16x8 *>(&sm.kt[16 * it + li][32 * kk + 8 * lg]),
                                bDs[kk], S[it]);
        }
    }

    if constexpr (TRANS) {  // M and N of the segment (addresses formed only here)
        if constexpr (TMW) {  // the last chunk's Tm; the last segment's map is not needed
            lds_barrier();
            if (nchunks > 0) store_tm(nchunks - 1);
            if (seg == nseg - 1) return;
        }
        float *pm = mn + (static_cast<size_t>(seg) * nchains + chain) * 2 * D * D;
        const int lgo = opaque(lg), colo = opaque(col);
#pragma unroll
        for (int it = 0; it < F::NI; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const size_t e = static_cast<size_t>(16 * it + 4 * lgo + r) * D + colo;
                pm[e] = __builtin_amdgcn_ldexpf(M[it][r], -em);
                pm[D * D + e] = __builtin_amdgcn_ldexpf(S[it][r], -es);
            }
        return;
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
    if (sT && seg == nseg - 1) {
#pragma unroll
        for (int it = 0; it < F::NI; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sT[sbase + static_cast<size_t>(16 * it + 4 * lg + r) * D + col] =
                    __builtin_amdgcn_ldexpf(S[it][r], -es);
    }
}

// ---- segmented plan: the entry state of every segment from the transitions of the ones
//      before it, in fp32.  entry[0] = S0 (or 0); segment 0's N already started from S0, so
//      entry[1] = N_0; entry[p] = M_{p-1} entry[p-1] + N_{p-1}.  One workgroup of 4 wavefronts
//      per (chain, 16-column tile); the products run on the fp32 matrix cores
//      (v_mfma_f32_16x16x4_f32), wavefront w forming row tiles w TPW .. of the new state.  The
//      state tile is kept in LDS in the accumulator layout, and k-step (t, r) of a product
//      sums over rows 16 t + 4 j + r (j = 0..3): register r of accumulator tile t is then that
//      k-step's B operand as it stands, and the matching A operand (columns 16 t + 4 j + r of
//      M) is one 16-byte LDS read for r = 0..3.  M_{p+1} and N_{p+1} are loaded into registers
//      while step p runs.
template <int D> struct CombineSmem {
    float m[D][D + 8];     // M_p, row-major; pitch 8 mod 32 dwords for the 16-byte A reads
    f32x4 st[D / 16][64];  // the state tile: [row tile][lane], accumulator layout
};

__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int D>
__global__ void __launch_bounds__(256)
seg_combine_kernel(const float *s0, const float *__restrict__ mn, float *__restrict__ entry,
                   int nchains, int nseg) {
    constexpr int NT = D / 16, TPW = NT / 4;  // row tiles; per wavefront
    constexpr int NM = D * D / 4 / 256;        // 16-byte pieces of M per thread
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    CombineSmem<D> &sm = *reinterpret_cast<CombineSmem<D> *>(smem_raw);
    const int chain = blockIdx.x / NT, jt = blockIdx.x - chain * NT;
    const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int w = tid >> 6, col = 16 * jt + li;
    const size_t DD = static_cast<size_t>(D) * D, cs = static_cast<size_t>(nchains) * DD;
    const size_t sb = static_cast<size_t>(chain) * DD;
    auto mp = [&](int p) { return mn + (static_cast<size_t>(p) * nchains + chain) * 2 * DD; };
    auto at = [&](int t, int r) { return static_cast<size_t>(16 * t + 4 * lg + r) * D + col; };
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int t = w * TPW + i;
        f32x4 x;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            entry[sb + at(t, r)] = s0 != nullptr ? s0[sb + at(t, r)] : 0.f;
            x[r] = mp(0)[DD + at(t, r)];  // N_0
            entry[cs + sb + at(t, r)] = x[r];
        }
        sm.st[t][lane] = x;
    }
    if (nseg <= 2) return;
    f32x4 mr[NM], nx[TPW];
    auto load_mn = [&](int p) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(mp(p));
#pragma unroll
        for (int n = 0; n < NM; ++n) mr[n] = src[tid + 256 * n];
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) nx[i][r] = mp(p)[DD + at(w * TPW + i, r)];
    };
    auto stage_m = [&]() {
#pragma unroll
        for (int n = 0; n < NM; ++n) {
            const int idx = tid + 256 * n, r = idx / (D / 4), c4 = idx - r * (D / 4);
            *reinterpret_cast<f32x4 *>(&sm.m[r][4 * c4]) = mr[n];
        }
    };
    load_mn(1);
    stage_m();
    for (int p = 1; p + 1 < nseg; ++p) {
        __syncthreads();  // M_p and the state tile are in LDS
        f32x4 acc[TPW][2];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            acc[i][0] = nx[i];
            acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (p + 2 < nseg) load_mn(p + 1);  // consumed after this step's products
        f32x4 bS[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) bS[t] = sm.st[t][lane];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const f32x4 a4 = *reinterpret_cast<const f32x4 *>(
                    &sm.m[16 * (w * TPW + i) + li][16 * t + 4 * lg]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][t & 1] = mma_f32(a4[r], bS[t][r], acc[i][t & 1]);
            }
        __syncthreads();  // every wavefront is done reading M_p and the state tile
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int t = w * TPW + i;
            const f32x4 x = acc[i][0] + acc[i][1];
            sm.st[t][lane] = x;
#pragma unroll
            for (int r = 0; r < 4; ++r) entry[(p + 1) * cs + sb + at(t, r)] = x[r];
        }
        if (p + 2 < nseg) stage_m();
    }
}

// Workspace of the segmented plan: the maps M, N of segments 0 .. nseg-2 and every segment's
// entry state (fp32), then -- optional: the plan runs without them, forming Tm twice -- the
// Tm records (uint16 halves), tm_nslot slots per value head.
size_t seg_map_bytes(const PrefillArgs &a, const SegGeom &sg) {
    const size_t DD = static_cast<size_t>(a.dk) * a.dv, chains = static_cast<size_t>(a.B) * a.Hv;
    return (static_cast<size_t>(sg.nseg - 1) * 2 + sg.nseg) * chains * DD * sizeof(float);
}
int seg_tm_slots(const PrefillArgs &a) {
    const long rows = a.cu != nullptr ? a.T : static_cast<long>(a.B) * a.T;
    return static_cast<int>((rows + a.chunk - 1) / a.chunk + a.B);
}
// At most this many bytes of records (the split plan's bound on its own): longer inputs form
// Tm in both passes, so the workspace stays bounded for any T.
constexpr size_t kSegTmMaxBytes = size_t(2) << 30;
size_t seg_tm_bytes(const PrefillArgs &a) {
    const char *env = getenv("GDN_SEG_NO_TM");  // A/B switch: form Tm in both passes
    if (env != nullptr && atoi(env) != 0) return 0;
    const size_t nr = a.chunk / 16;
    const size_t bytes = static_cast<size_t>(a.Hv) * seg_tm_slots(a) * (nr * (nr + 1) / 2) * 512;
    return bytes <= kSegTmMaxBytes ? bytes : 0;
}

template <int D, int C, typename TO, int MODE>
hipError_t launch_mode(const PrefillArgs &a, unsigned nblk, int nchains, int seg_chunks,
                       int nseg, const float *s0, size_t s0_seg_stride, float *mn,
                       uint16_t *tm = nullptr, int tm_nslot = 0) {
    auto kern = chunk_kernel<D, C, TO, MODE>;
    const size_t lds = sizeof(Smem<D, C>);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(nblk), dim3(Cfg<D, C>::NT), lds, a.stream,
                       static_cast<const bf16_t *>(a.q), static_cast<const bf16_t *>(a.k),
                       static_cast<const bf16_t *>(a.v), static_cast<const bf16_t *>(a.beta),
                       static_cast<const bf16_t *>(a.g), s0, static_cast<TO *>(a.o), a.sT, a.T,
                       a.cu, a.flags, a.Hk, a.Hv, a.scale, nchains, seg_chunks, nseg,
                       s0_seg_stride, mn, tm, tm_nslot);
    return hipGetLastError();
}

template <int D, int C, typename TO> hipError_t launch_typed(const PrefillArgs &a) {
    const int nchains = a.B * a.Hv;
    const SegGeom sg = seg_geometry(a);
    if (sg.nseg <= 1)
        return launch_mode<D, C, TO, kOut>(a, static_cast<unsigned>(nchains), nchains, 1 << 30,
                                           1, a.s0, 0, nullptr);
    // segmented: transitions of segments 0 .. nseg-2, their entry states, then every segment.
    // With room for the Tm records (seg_tm_bytes), the transition pass also runs the last
    // segment and stores every chunk's Tm for the output pass.
    const size_t DD = static_cast<size_t>(D) * D;
    float *mn = static_cast<float *>(a.ws);
    float *entry = mn + static_cast<size_t>(sg.nseg - 1) * nchains * 2 * DD;
    const size_t maps = seg_map_bytes(a, sg), tmb = seg_tm_bytes(a);
    const bool use_tm = tmb > 0 && a.ws_bytes >= maps + tmb;
    uint16_t *tm = use_tm ? reinterpret_cast<uint16_t *>(static_cast<unsigned char *>(a.ws) + maps)
                          : nullptr;
    const int tm_nslot = seg_tm_slots(a);
    hipError_t e =
        use_tm ? launch_mode<D, C, float, kTransTm>(a, static_cast<unsigned>(sg.nseg * nchains),
                                                    nchains, sg.seg_chunks, sg.nseg, a.s0, 0, mn,
                                                    tm, tm_nslot)
               : launch_mode<D, C, float, kTrans>(
                     a, static_cast<unsigned>((sg.nseg - 1) * nchains), nchains, sg.seg_chunks,
                     sg.nseg, a.s0, 0, mn);
    if (e != hipSuccess) return e;
    const size_t clds = sizeof(CombineSmem<D>);
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(seg_combine_kernel<D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(clds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(seg_combine_kernel<D>, dim3(static_cast<unsigned>(nchains * (D / 16))),
                       dim3(256), clds, a.stream, a.s0, mn, entry, nchains, sg.nseg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (use_tm)
        return launch_mode<D, C, TO, kOutTm>(a, static_cast<unsigned>(sg.nseg * nchains), nchains,
                                             sg.seg_chunks, sg.nseg, entry,
                                             static_cast<size_t>(nchains) * DD, nullptr, tm,
                                             tm_nslot);
    return launch_mode<D, C, TO, kOut>(a, static_cast<unsigned>(sg.nseg * nchains), nchains,
                                       sg.seg_chunks, sg.nseg, entry,
                                       static_cast<size_t>(nchains) * DD, nullptr);
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

SegGeom seg_geometry(const PrefillArgs &a) {
    SegGeom g{1, 1 << 30};
    if (!a.seg || a.B <= 0 || a.T <= 0) return g;
    const long nch = (static_cast<long>(a.T) + a.chunk - 1) / a.chunk;
    const long chains = static_cast<long>(a.B) * a.Hv;
    if (a.cu != nullptr) {  // packed: every chain in the same number of segments, each chain's
        g.nseg = static_cast<int>(std::max(1L, kSegTargetUnits / chains));  // own length
        g.seg_chunks = 0;                                                  // on the device
        return g;
    }
    long len = 0;  // chunks per segment
    const char *env = getenv("GDN_SEG_CHUNKS");
    if (env != nullptr && atol(env) > 0) {
        len = atol(env);  // a segment length pinned for tests and measurements
    } else {
        const long want = std::max(1L, kSegTargetUnits / chains);  // segments per chain
        len = (nch + want - 1) / want;
    }
    len = std::min(len, nch);
    g.nseg = static_cast<int>((nch + len - 1) / len);
    g.seg_chunks = static_cast<int>(len);
    return g;
}

size_t chunk_mfma_workspace(const PrefillArgs &a, bool least) {
    const SegGeom sg = seg_geometry(a);
    if (sg.nseg <= 1) return 0;
    return seg_map_bytes(a, sg) + (least ? 0 : seg_tm_bytes(a));
}

hipError_t launch_chunk_mfma(const PrefillArgs &a) {
    if (!chunk_mfma_supports(a)) return hipErrorNotSupported;
    return a.dk == 128 ? launch_chunk<128>(a) : launch_chunk<64>(a);
}

}  // namespace gdn
