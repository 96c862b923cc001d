// qsa.hip -- the QSA compressed indexer: which key blocks each query attends to.
//
// Explainer page "論文解説: Qwen3.8-Next の設計" (ta-paperlens.web.app), section "部品②: QSA":
// the keys (one shared key head, the indexer being multi-query attention with four query
// heads) are cut into blocks of r tokens and mean-pooled before the position encoding, each
// block gets one position (its first token), rotary encoding covers part of the head
// dimension, and a token budget of K tokens (K / r blocks) keeps the most important blocks.
//
// Readings of what the page leaves open (the oracle and include/gdn.h state the same):
//   - block j holds tokens j*r .. min((j+1)r, T) - 1 and is eligible for the query at t when
//     its last token is at or before t;
//   - rotate-half pairing (i, i + R/2) for i < R/2, angle pos * base^(-2i/R);
//   - the importance of block j for query t is the sum over the four heads of the softmax
//     over eligible blocks of scale * q_{t,h} . kbar_j;
//   - the nsel most important eligible blocks are kept (ties: lower index), ascending.
//
// Four kernels:
//   rope_q_kernel   rotated queries -> fp16 with a power-of-two scale per (token, head) row
//   pool_k_kernel   block means, rotated at the block's first position -> fp32, plus one
//                   partial max |kbar| per 64 blocks
//   pack_k_kernel   fp32 -> fp16 with one power-of-two scale per batch (from the partial
//                   maxima), stored in MFMA-fragment order
//   select_kernel   one wavefront per 16 queries: the scores on the matrix cores (fp16 in,
//                   fp32 accumulate) in sweeps over the eligible blocks -- one for the softmax
//                   statistics, up to four for an exact 8-bit radix select of the nsel-th
//                   largest importance, one that writes the kept block indices in order.
// Recomputing the scores in every sweep costs less than storing them: a score row costs 4 B
// of HBM traffic per block against 1024 multiply-adds on the matrix cores, and the sweeps are
// bound by the exponentials on the vector units either way.
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kHq = 4;             // query heads per token: the four rows of an MFMA group
constexpr int kTok = 16;           // queries per wavefront
constexpr int kPoolBlocks = 64;    // blocks per workgroup of the key kernels (one partial max)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mma(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// sin and cos of pos * base^(-2m/R): the angle is formed and reduced to [-pi, pi] in fp64
// (positions reach 2^20 and more, where an fp32 angle would be off by a large fraction of a
// radian), then evaluated in fp32.
__device__ __forceinline__ void rope_angle(double pos, int m, int R, double log2base, float &c,
                                           float &s) {
    const double inv_freq = exp2(-(2.0 * m / R) * log2base);
    const double th = pos * inv_freq;
    const double n = rint(th * 0.15915494309189535);       // 1 / (2 pi)
    double red = fma(-n, 6.283185307179586, th);           // 2 pi, high part
    red = fma(-n, 2.4492935982947064e-16, red);            // 2 pi, low part
    sincosf(static_cast<float>(red), &s, &c);
}

// Rotated value of element i of a row whose elements are x(i): rotate-half over the first R.
template <typename F>
__device__ __forceinline__ float rope_elem(F x, int i, int R, double pos, double log2base) {
    const int h = R / 2;
    if (i >= R) return x(i);
    float c, s;
    if (i < h) {
        rope_angle(pos, i, R, log2base, c, s);
        return x(i) * c - x(i + h) * s;
    }
    rope_angle(pos, i - h, R, log2base, c, s);
    return x(i - h) * s + x(i) * c;
}

// 2^(14 - e) where max = f 2^e, f in [0.5, 1): scales the largest magnitude into [2^13, 2^14),
// well inside fp16 (and exact: a power of two).
__device__ __forceinline__ int scale_exp(float maxabs) {
    int e;
    frexpf(maxabs, &e);
    return 14 - e;
}

__device__ __forceinline__ float wave_max(float x) {
    for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

// ---------------------------------------------------------------------------------------
// rope_q_kernel: one wavefront per (token, head) row; block = the four heads of one token.
// Writes the fp16 row, 1/scale, and an upper bound of the fp16 row's L2 norm.
template <int D, typename TI>
__global__ void __launch_bounds__(256)
rope_q_kernel(const TI *__restrict__ q, f16 *__restrict__ q16, float *__restrict__ qinv,
              float *__restrict__ qnorm, int T, int R, double log2base) {
    const int lane = threadIdx.x & 63, h = threadIdx.x >> 6;
    const size_t tok = blockIdx.x;  // b * T + t
    const double pos = static_cast<double>(tok % static_cast<size_t>(T));
    const TI *row = q + (tok * kHq + h) * D;
    auto x = [&](int i) { return load_f32(row + i); };
    float out[D / 64];
    float mx = 0.f;
#pragma unroll
    for (int u = 0; u < D / 64; ++u) {
        out[u] = rope_elem(x, lane + 64 * u, R, pos, log2base);
        mx = fmaxf(mx, fabsf(out[u]));
    }
    const int e = scale_exp(wave_max(mx));
    f16 *dst = q16 + (tok * kHq + h) * D;
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < D / 64; ++u) {
        const f16 v = static_cast<f16>(ldexpf(out[u], e));
        dst[lane + 64 * u] = v;
        ss += static_cast<float>(v) * static_cast<float>(v);
    }
    for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off);
    if (lane == 0) {
        qinv[tok * kHq + h] = ldexpf(1.f, -e);
        qnorm[tok * kHq + h] = sqrtf(ss) * (1.f + 0x1p-20f);
    }
}

// ---------------------------------------------------------------------------------------
// pool_k_kernel: workgroup p of batch b pools blocks 64p .. 64p+63 (16 per wavefront) and
// writes the largest element magnitude and the largest row norm it produced to part[b][p].
template <int D, typename TI>
__global__ void __launch_bounds__(256)
pool_k_kernel(const TI *__restrict__ k, float *__restrict__ kf, float2 *__restrict__ part, int T,
              int r, int nb, int nparts, int R, double log2base) {
    __shared__ float s_max[4], s_nrm[4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int b = blockIdx.x / nparts, p = blockIdx.x % nparts;
    const TI *kb = k + static_cast<size_t>(b) * T * D;
    float mx = 0.f, nx = 0.f;
    for (int jj = 0; jj < kPoolBlocks / 4; ++jj) {
        const int j = p * kPoolBlocks + w * (kPoolBlocks / 4) + jj;
        if (j >= nb) break;
        const int t0 = j * r, t1 = min(t0 + r, T);
        const float inv = 1.f / static_cast<float>(t1 - t0);
        auto mean = [&](int i) {
            float s = 0.f;
            for (int t = t0; t < t1; ++t) s += load_f32(kb + static_cast<size_t>(t) * D + i);
            return s * inv;
        };
        float *dst = kf + (static_cast<size_t>(b) * nb + j) * D;
        float ss = 0.f;
#pragma unroll
        for (int u = 0; u < D / 64; ++u) {
            const float y = rope_elem(mean, lane + 64 * u, R, static_cast<double>(t0), log2base);
            dst[lane + 64 * u] = y;
            mx = fmaxf(mx, fabsf(y));
            ss += y * y;
        }
        for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off);
        nx = fmaxf(nx, ss);
    }
    mx = wave_max(mx);
    if (lane == 0) { s_max[w] = mx; s_nrm[w] = nx; }
    __syncthreads();
    if (threadIdx.x == 0)
        part[static_cast<size_t>(b) * nparts + p] =
            make_float2(fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3])),
                        sqrtf(fmaxf(fmaxf(s_nrm[0], s_nrm[1]), fmaxf(s_nrm[2], s_nrm[3]))));
}

// ---------------------------------------------------------------------------------------
// pack_k_kernel: every workgroup of batch b reduces the batch's partial maxima (the same value
// in each) and converts its 64 blocks to fp16 with the batch's power-of-two scale; the first one
// also stores {inverse scale, upper bound of the fp16 rows' L2 norms}.
//
// The fp16 keys are stored in MFMA-fragment order: for every tile of 16 blocks and every 32-wide
// k-step, the 64 lanes' 16-byte B-operand pieces (lane l: block 16 tile + l%16, dimensions
// 32 s + 8 (l/16) .. +7) lie contiguously in 1 KiB, so the select kernel reads each operand
// with one fully coalesced load.  Blocks past the end of the last tile are zero.
template <int D>
__global__ void __launch_bounds__(256)
pack_k_kernel(const float *__restrict__ kf, const float2 *__restrict__ part,
              f16 *__restrict__ k16, float2 *__restrict__ kstat, int nb, int nparts) {
    constexpr int KD = D / 32;
    __shared__ float s_max[4], s_nrm[4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int b = blockIdx.x / nparts, p = blockIdx.x % nparts;
    float mx = 0.f, nx = 0.f;
    for (int i = threadIdx.x; i < nparts; i += 256) {
        const float2 v = part[static_cast<size_t>(b) * nparts + i];
        mx = fmaxf(mx, v.x);
        nx = fmaxf(nx, v.y);
    }
    mx = wave_max(mx);
    nx = wave_max(nx);
    if (lane == 0) { s_max[w] = mx; s_nrm[w] = nx; }
    __syncthreads();
    const int e = scale_exp(fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3])));
    if (p == 0 && threadIdx.x == 0) {
        // fp16 rounding grows a row by at most a factor (1 + 2^-11), plus the absolute
        // rounding of subnormal elements
        const float n = fmaxf(fmaxf(s_nrm[0], s_nrm[1]), fmaxf(s_nrm[2], s_nrm[3]));
        kstat[b] = make_float2(ldexpf(1.f, -e), ldexpf(n, e) * (1.f + 0x1p-9f) + 0x1p-14f);
    }
    const int ntk = (nb + 15) / 16;
    const int tile0 = p * (kPoolBlocks / 16), ntl = min(kPoolBlocks / 16, ntk - tile0);
    const size_t obase = (static_cast<size_t>(b) * ntk + tile0) * KD * 512;  // in fp16 elements
    for (int i = threadIdx.x; i < ntl * KD * 64; i += 256) {
        const int ln = i & 63, s = (i >> 6) % KD, tl = (i >> 6) / KD;
        const int j = (tile0 + tl) * 16 + (ln & 15), d0 = 32 * s + 8 * (ln >> 4);
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (j < nb) {
            const float *src = kf + (static_cast<size_t>(b) * nb + j) * D + d0;
            const float4 lo = *reinterpret_cast<const float4 *>(src);
            const float4 hi = *reinterpret_cast<const float4 *>(src + 4);
            v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
            v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
        }
        f16x8 h;
#pragma unroll
        for (int u = 0; u < 8; ++u) h[u] = static_cast<f16>(ldexpf(v[u], e));
        *reinterpret_cast<f16x8 *>(k16 + obase + (static_cast<size_t>(tl) * KD + s) * 512 +
                                   8 * ln) = h;
    }
}

// ---------------------------------------------------------------------------------------
// select_kernel: one wavefront per 16 consecutive queries of one batch.
//
// MFMA layout (16x16x32): the A operand row m = lane & 15 is query 4a + m/4, head m % 4 of row
// tile a (a = 0..3); the B operand column n = lane & 15 is block 16 jt + n.  The accumulator
// of lane l then holds, for row tile a, the four head scores of query 4a + l/16 against block
// 16 jt + l%16 -- a query's four heads sit in one lane, so the head sum needs no exchange.
//
// Every sweep over the blocks is software-pipelined: the matrix-core products of tile jt + 1
// are issued between the vector instructions that consume tile jt, and the key fragments of a
// tile are loaded a whole tile ahead.  The loop bodies have no branches (masked histogram
// updates go to a per-lane dummy counter, masked stores through a buffer resource whose range
// check drops them), so the loads stay in flight across iterations.
//
// The importance of an element is formed by one function in every sweep, so its fp32 bits are
// identical wherever it is compared.
__device__ __forceinline__ float head_sum(f32x4 acc, const float *cf, const float *ls) {
    float i = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[0], cf[0], -ls[0]));
    i += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[1], cf[1], -ls[1]));
    i += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[2], cf[2], -ls[2]));
    i += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[3], cf[3], -ls[3]));
    return i;
}

__device__ __forceinline__ int group_popc(unsigned long long m, int g) {
    return __builtin_popcount(static_cast<unsigned>(m >> (16 * g)) & 0xffffu);
}
__device__ __forceinline__ int group_below(unsigned long long m, int g, int c) {
    return __builtin_popcount(static_cast<unsigned>(m >> (16 * g)) & ((1u << c) - 1u));
}

// One MFMA, then nv vector instructions, n times: keeps the matrix core busy while the
// wavefront works through the previous tile.
#define QSA_INTERLEAVE(n, nv)                                                                  \
    _Pragma("unroll") for (int _i = 0; _i < (n); ++_i) {                                       \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                     \
        __builtin_amdgcn_sched_group_barrier(0x002, (nv), 0);                                  \
    }

template <int N> struct Nv { static constexpr int value = N; };
typedef Nv<3> NV3;
typedef Nv<4> NV4;

constexpr int kHistWords = kTok * 256 + 64;  // 16 histograms of 256 bins, 64 dummy counters
constexpr unsigned kOob = 0x7ffffff0u;       // a buffer offset past any range: store dropped
constexpr int kCand = 64;                    // most keys a query may gather in the last sweep
constexpr int kPer = 8;                      // kept blocks per lane the merge holds in registers

template <int D, bool IMP>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2)))
select_kernel(const f16 *__restrict__ q16, const float *__restrict__ qinv,
              const float *__restrict__ qnorm, const f16 *__restrict__ k16,
              const float2 *__restrict__ kstat, int32_t *__restrict__ sel,
              float *__restrict__ imp, int B, int T, int r, int nb, int nsel, float scale_log2e) {
    constexpr int KD = D / 32;
    __shared__ unsigned s_hist[kHistWords];
    __shared__ unsigned s_lo[kTok], s_hi[kTok];
    __shared__ int s_shift[kTok], s_krem[kTok], s_kt[kTok], s_act[kTok], s_coll[kTok],
        s_ncand[kTok];

    const int lane = threadIdx.x, g = lane >> 4, c = lane & 15;
    const int ntt = (T + kTok - 1) / kTok;
    const int b = blockIdx.x % B;
    const int tile = ntt - 1 - blockIdx.x / B;  // the longest rows first
    const int t0 = tile * kTok;
    auto nelig = [&](int t) { return t >= T ? 0 : (t == T - 1 ? nb : (t + 1) / r); };
    const int ntj = (nelig(min(t0 + kTok - 1, T - 1)) + 15) / 16;

    // operands and per-element constants
    f16x8 qa[4][KD];
    float cf[4][4], ls[4][4];
    int ne[4];
    const float2 ks = kstat[b];
    const float ksc = ks.x * scale_log2e;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int tq = min(t0 + 4 * a + (c >> 2), T - 1);
        const f16 *row = q16 + ((static_cast<size_t>(b) * T + tq) * kHq + (c & 3)) * D + 8 * g;
#pragma unroll
        for (int s = 0; s < KD; ++s) qa[a][s] = *reinterpret_cast<const f16x8 *>(row + 32 * s);
        const int t = t0 + 4 * a + g;
        ne[a] = nelig(t);
        const size_t qr = (static_cast<size_t>(b) * T + min(t, T - 1)) * kHq;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            cf[a][h] = qinv[qr + h] * ksc;
            // |score * cf| <= |cf| ||q16|| ||k16||: an upper bound of every exponent of the row
            ls[a][h] = fabsf(cf[a][h]) * qnorm[qr + h] * ks.y * (1.f + 0x1p-10f);
        }
    }
    // fragment-ordered keys (pack_k_kernel): one coalesced 1 KiB load per operand
    const int ntk = (nb + 15) / 16;
    const f16 *kbase = k16 + static_cast<size_t>(b) * ntk * KD * 512 + 8 * lane;
    auto load_b = [&](int jt, f16x8 (&kb)[KD]) {
        const size_t o = static_cast<size_t>(min(jt, ntk - 1)) * KD * 512;
#pragma unroll
        for (int s = 0; s < KD; ++s)
            kb[s] = *reinterpret_cast<const f16x8 *>(kbase + o + s * 512);
    };
    auto scores = [&](const f16x8 (&kb)[KD], f32x4 (&acc)[4]) {
#pragma unroll
        for (int s = 0; s < KD; ++s)
#pragma unroll
            for (int a = 0; a < 4; ++a)
                acc[a] = mma(qa[a][s], kb[s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[a]);
    };
    // the pipelined sweep: body(jt, acc) consumes tile jt; NV = its vector instructions per
    // matrix-core product, for the interleave
    auto sweep = [&](auto &&body, auto nv_tag) {
        constexpr int NV = decltype(nv_tag)::value;
        if (ntj == 0) return;
        f16x8 K0[KD], K1[KD];
        f32x4 A0[4], A1[4];
        load_b(0, K0);
        load_b(min(1, ntj - 1), K1);
        scores(K0, A0);
        int jt = 0;
        for (; jt + 2 <= ntj; jt += 2) {
            load_b(min(jt + 2, ntj - 1), K0);
            __builtin_amdgcn_sched_barrier(0);
            scores(K1, A1);
            body(jt, A0);
            QSA_INTERLEAVE(4 * KD, NV)
            __builtin_amdgcn_sched_barrier(0);
            load_b(min(jt + 3, ntj - 1), K1);
            __builtin_amdgcn_sched_barrier(0);
            scores(K0, A0);
            body(jt + 1, A1);
            QSA_INTERLEAVE(4 * KD, NV)
            __builtin_amdgcn_sched_barrier(0);
        }
        if (jt < ntj) body(jt, A0);
    };

    // ---- sweep 1: per (query, head) sum of 2^(x - bound) over the eligible blocks, x the
    //      score in log2 units; lse = bound + log2(sum).  If a sum comes out below 2^-100 (the
    //      bound far above every score: huge norms), the wavefront redoes the sweep with a
    //      running maximum instead.
    {
        float sm[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int h = 0; h < 4; ++h) sm[a][h] = 0.f;
        sweep([&](int jt, f32x4 (&acc)[4]) {
            const int j = 16 * jt + c;
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float e = __builtin_amdgcn_exp2f(
                        __builtin_fmaf(acc[a][h], cf[a][h], -ls[a][h]));
                    sm[a][h] += j < ne[a] ? e : 0.f;
                }
        }, NV3{});
        bool low = false;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                float l = sm[a][h];
                for (int off = 1; off < 16; off <<= 1) l += __shfl_xor(l, off);
                l = __shfl(l, lane & 48);  // every lane of the group: lane 16g's bits
                low |= ne[a] > 0 && !(l >= 0x1p-100f);
                ls[a][h] = l > 0.f ? ls[a][h] + __log2f(l) : INFINITY;
            }
        if (__ballot(low) != 0ull) {
            float mx[4][4];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int h = 0; h < 4; ++h) { mx[a][h] = -3.402823466e38f; sm[a][h] = 0.f; }
            sweep([&](int jt, f32x4 (&acc)[4]) {
                const int j = 16 * jt + c;
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const float x = j < ne[a] ? acc[a][h] * cf[a][h] : -INFINITY;
                        const float d = x - mx[a][h];
                        const float e = __builtin_amdgcn_exp2f(-fabsf(d));
                        const bool gt = x > mx[a][h];
                        sm[a][h] = gt ? __builtin_fmaf(sm[a][h], e, 1.f) : sm[a][h] + e;
                        mx[a][h] = gt ? x : mx[a][h];
                    }
            }, NV4{});
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    float m = mx[a][h], l = sm[a][h];
                    for (int off = 1; off < 16; off <<= 1) {
                        const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
                        const float mn = fmaxf(m, m2);
                        l = l * __builtin_amdgcn_exp2f(m - mn) +
                            l2 * __builtin_amdgcn_exp2f(m2 - mn);
                        m = mn;
                    }
                    const float lse = l > 0.f ? m + __log2f(l) : INFINITY;
                    ls[a][h] = __shfl(lse, lane & 48);
                }
        }
    }

    // ---- exact selection of the nsel largest keys per query (key = the fp32 bits of the
    //      importance: positive floats order as their bits).  Each pass histograms the keys of
    //      a query that lie in its current range [lo, hi) into 256 bins and narrows the range
    //      to the bin holding the krem-th largest of them.  A query is done when a whole bin is
    //      kept (count == krem) or the range is one value (keep its first krem copies in index
    //      order).  In the end a block is kept if key >= hi, or lo <= key < hi among the first
    //      kt such blocks; a query with at most nsel eligible blocks keeps all (lo = hi = 0).
    //      A query whose range holds at most kCand keys stops early ("gathers"): the last sweep
    //      writes its blocks with key >= hi and collects the in-range (key, block) pairs in
    //      LDS, and a merge afterwards ranks them and inserts the krem best in index order.
    //
    //      The first pass bins by 1/16 of a binade over the 16 binades below 4.004 / nsel: the
    //      importances of a query sum to 4 (four distributions), so the nsel-th largest cannot
    //      exceed 4 / nsel, and the bins fall where the keys spread instead of on the few
    //      exponent values they share.  The two end bins hold everything below and above.
    const unsigned wtop = __float_as_uint(4.f * (1.f + 0x1p-10f) / static_cast<float>(nsel)) >> 19;
    const unsigned wbase = wtop - 254u;
    if (lane < kTok) {
        s_lo[lane] = 0u;
        s_hi[lane] = 0u;
        s_shift[lane] = 0;
        s_kt[lane] = 0x7fffffff;
        s_krem[lane] = nsel;
        s_act[lane] = nelig(t0 + lane) > nsel;
        s_coll[lane] = 0;
        s_ncand[lane] = 0;
    }
    for (int pass = 0; pass < 5; ++pass) {
        __syncthreads();
        int any = 0;
#pragma unroll
        for (int tk = 0; tk < kTok; ++tk) any |= s_act[tk];
        if (!any) break;
        for (int i = lane; i < kHistWords; i += 64) s_hist[i] = 0u;
        unsigned lo[4], wd[4];
        int sh[4];
        bool act[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int tk = 4 * a + g;
            lo[a] = s_lo[tk];
            wd[a] = s_hi[tk] - s_lo[tk];
            sh[a] = s_shift[tk];
            act[a] = s_act[tk];
        }
        __syncthreads();
        if (pass == 0) {
            sweep([&](int jt, f32x4 (&acc)[4]) {
                const int j = 16 * jt + c;
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    unsigned key = __float_as_uint(head_sum(acc[a], cf[a], ls[a]));
                    asm volatile("" : "+v"(key));  // computed by every lane: no branch around it
                    const int d = min(max(static_cast<int>((key >> 19) - wbase), 0), 255);
                    const unsigned idx = (act[a] & (j < ne[a])) ? (4 * a + g) * 256 + d
                                                               : kTok * 256 + lane;
                    atomicAdd(&s_hist[idx], 1u);
                }
            }, NV4{});
        } else {
            sweep([&](int jt, f32x4 (&acc)[4]) {
                const int j = 16 * jt + c;
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    unsigned key = __float_as_uint(head_sum(acc[a], cf[a], ls[a]));
                    asm volatile("" : "+v"(key));
                    const unsigned off = key - lo[a];
                    const unsigned idx = (act[a] & (j < ne[a]) & (off < wd[a]))
                                             ? (4 * a + g) * 256 + (off >> sh[a])
                                             : kTok * 256 + lane;
                    atomicAdd(&s_hist[idx], 1u);
                }
            }, NV4{});
        }
        __syncthreads();
        // per active query: the bin holding the krem-th largest key of the range
        for (int tk = 0; tk < kTok; ++tk) {
            if (!s_act[tk]) continue;
            const int krem = s_krem[tk];
            const uint4 h4 = *reinterpret_cast<const uint4 *>(&s_hist[tk * 256 + 4 * lane]);
            const int own = static_cast<int>(h4.x + h4.y + h4.z + h4.w);
            int suf = own;  // sum over lanes >= lane
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_down(suf, off);
                if (lane + off < 64) suf += y;
            }
            const int above = suf - own;
            const bool here = above < krem && krem <= suf;
            int digit = 0, abv = above, cnt = 0;
            if (here) {
                const unsigned hb[4] = {h4.x, h4.y, h4.z, h4.w};
                int run = above;
#pragma unroll
                for (int q = 3; q >= 0; --q) {
                    if (run + static_cast<int>(hb[q]) >= krem) {
                        digit = 4 * lane + q;
                        abv = run;
                        cnt = static_cast<int>(hb[q]);
                        break;
                    }
                    run += static_cast<int>(hb[q]);
                }
            }
            const int src = __ffsll(static_cast<long long>(__ballot(here))) - 1;
            digit = __shfl(digit, src);
            abv = __shfl(abv, src);
            cnt = __shfl(cnt, src);
            if (lane == 0) {
                const unsigned d = static_cast<unsigned>(digit);
                unsigned nlo, nhi;
                if (pass == 0) {
                    nlo = d == 0 ? 0u : (wbase + d) << 19;
                    nhi = d == 255 ? 0x80000000u : (wbase + d + 1) << 19;
                } else {
                    const unsigned l0 = s_lo[tk];
                    const int shf = s_shift[tk];
                    nlo = l0 + (d << shf);
                    nhi = min(s_hi[tk], nlo + (1u << shf));
                }
                const int left = krem - abv;  // to keep from the new range
                s_lo[tk] = nlo;
                s_hi[tk] = nhi;
                s_krem[tk] = left;
                const unsigned w = nhi - nlo;
                s_shift[tk] = w <= 256u ? 0 : 32 - __clz(w - 1u) - 8;
                if (cnt == left) {
                    s_act[tk] = 0;          // the whole range is kept
                } else if (w == 1u || pass == 4) {
                    s_kt[tk] = left;        // one key value: its first `left` copies
                    s_act[tk] = 0;
                } else if (cnt <= kCand) {
                    s_coll[tk] = 1;         // few keys left in the range: gather and rank them
                    s_ncand[tk] = cnt;
                    s_kt[tk] = 0;
                    s_act[tk] = 0;
                }
            }
        }
    }
    __syncthreads();

    // ---- last sweep: write the kept blocks in ascending order (and the importance)
    unsigned lo[4], wd[4], hi[4];
    int kt[4], cnt[4], ties[4];
    bool coll[4];
    int anytie = 0;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int tk = 4 * a + g;
        lo[a] = s_lo[tk];
        hi[a] = s_hi[tk];
        wd[a] = hi[a] - lo[a];
        kt[a] = s_kt[tk];
        coll[a] = s_coll[tk] != 0;
        cnt[a] = 0;
        ties[a] = 0;
    }
    // gathered pairs of query tl: keys at s_hist[tl * kCand + i], blocks kTok * kCand further
    unsigned *const s_ck = s_hist;
    int *const s_cj = reinterpret_cast<int *>(s_hist + kTok * kCand);
#pragma unroll
    for (int tk = 0; tk < kTok; ++tk) anytie |= s_kt[tk] != 0x7fffffff;
    const int rows = min(kTok, T - t0);
    const size_t row0 = static_cast<size_t>(b) * T + t0;
    const __amdgpu_buffer_rsrc_t sel_rs = __builtin_amdgcn_make_buffer_rsrc(
        sel + row0 * nsel, 0, rows * nsel * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t imp_rs = __builtin_amdgcn_make_buffer_rsrc(
        IMP ? static_cast<void *>(imp + row0 * nb) : static_cast<void *>(sel), 0,
        IMP ? rows * nb * 4 : 0, 0x00020000);
    auto out_body = [&](int jt, f32x4 (&acc)[4], auto tie_tag) {
        constexpr bool TIES = decltype(tie_tag)::value != 0;
        const int j = 16 * jt + c;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            float iv = head_sum(acc[a], cf[a], ls[a]);
            asm volatile("" : "+v"(iv));  // computed by every lane: no branch around it
            const unsigned key = __float_as_uint(iv);
            const bool el = j < ne[a];
            bool take = el && key >= hi[a];
            unsigned long long meq = 0ull;
            if (TIES) {
                const bool inr = el && key - lo[a] < wd[a];
                meq = __ballot(inr);
                const int tpos = ties[a] + group_below(meq, g, c);
                take = take || (inr && tpos < kt[a]);
                if (coll[a] && inr) {  // at most kCand in-range keys: tpos < kCand
                    s_ck[(4 * a + g) * kCand + tpos] = key;
                    s_cj[(4 * a + g) * kCand + tpos] = j;
                }
            } else {
                take = take || (el && key - lo[a] < wd[a]);
            }
            const unsigned long long mt = __ballot(take);
            const int pos = cnt[a] + group_below(mt, g, c);
            const int tl = 4 * a + g;  // query within the tile
            const unsigned so = take && pos < nsel ? static_cast<unsigned>(tl * nsel + pos) * 4u
                                                   : kOob;
            __builtin_amdgcn_raw_buffer_store_b32(j, sel_rs, static_cast<int>(so), 0, 0);
            if (IMP) {
                const unsigned io = j < nb ? static_cast<unsigned>(tl * nb + j) * 4u : kOob;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(el ? iv : 0.f), imp_rs,
                                                      static_cast<int>(io), 0, 0);
            }
            cnt[a] += group_popc(mt, g);
            if (TIES) ties[a] += group_popc(meq, g);
        }
    };
    if (anytie)
        sweep([&](int jt, f32x4 (&acc)[4]) { out_body(jt, acc, Nv<1>{}); }, NV4{});
    else
        sweep([&](int jt, f32x4 (&acc)[4]) { out_body(jt, acc, Nv<0>{}); }, NV4{});
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int t = t0 + 4 * a + g;
        if (t >= T) continue;
        const size_t rowo = static_cast<size_t>(b) * T + t;
        if (!coll[a])  // a gathering query fills all nsel slots in the merge
            for (int p = cnt[a] + c; p < nsel; p += 16) sel[rowo * nsel + p] = -1;
        if (IMP)
            for (int j = 16 * ntj + c; j < nb; j += 16) imp[rowo * nb + j] = 0.f;
    }

    // ---- merge of the gathering queries, one row per step with the whole wavefront: the
    //      row holds its nd = nsel - krem blocks with key >= hi in ascending order; of its nc
    //      gathered pairs (ascending block order, lane i holds pair i) the krem of smallest
    //      rank (larger key first, then lower block) are chosen, and the two sorted lists are
    //      interleaved in place.  Up to 64 * kPer kept blocks are read into registers at once;
    //      a longer row goes in 64-entry chunks from its end (the kept blocks only move right,
    //      so no chunk lands on one still unread).  The chosen pairs are stored last.
    __syncthreads();
    __threadfence_block();  // the row's own stores above are visible to every lane
    for (int tl = 0; tl < kTok; ++tl) {
        if (!s_coll[tl]) continue;  // only set for rows t0 + tl < T with > nsel eligible blocks
        int32_t *const row = sel + (static_cast<size_t>(b) * T + t0 + tl) * nsel;
        const int left = s_krem[tl], nd = nsel - left, nc = s_ncand[tl];
        const unsigned myk = lane < nc ? s_ck[tl * kCand + lane] : 0u;
        const int myj = lane < nc ? s_cj[tl * kCand + lane] : 0;
        int rank = 0;
        for (int m = 0; m < nc; ++m) {
            const unsigned km = __builtin_amdgcn_readlane(myk, m);
            rank += km > myk || (km == myk && m < lane);
        }
        const unsigned long long chosen = __ballot(lane < nc && rank < left);
        int below = 0;  // for a chosen lane: kept blocks with a lower index than its own
        // one batch of kept blocks: add[s] = chosen blocks below jd[s]; below += kept blocks
        // of the batch under each chosen block
        auto count = [&](const int *jd, int *add, int n) {
            for (unsigned long long mk = chosen; mk != 0ull; mk &= mk - 1ull) {
                const int m = __ffsll(static_cast<long long>(mk)) - 1;
                const int jc = __builtin_amdgcn_readlane(myj, m);
                int lt = 0;
                for (int s = 0; s < n; ++s) {
                    add[s] += jc < jd[s];
                    lt += __popcll(__ballot(jd[s] < jc));
                }
                below += lane == m ? lt : 0;
            }
        };
        if (nd <= 64 * kPer) {
            int jd[kPer], add[kPer];
#pragma unroll
            for (int s = 0; s < kPer; ++s) {
                const int p = lane + 64 * s;
                jd[s] = p < nd ? row[p] : 0x7fffffff;
                add[s] = 0;
            }
            count(jd, add, kPer);
#pragma unroll
            for (int s = 0; s < kPer; ++s) {
                const int p = lane + 64 * s;
                if (p < nd) row[p + add[s]] = jd[s];
            }
        } else {
            for (int p0 = (nd - 1) & ~63; p0 >= 0; p0 -= 64) {
                const int p = p0 + lane;
                int jd[1] = {p < nd ? row[p] : 0x7fffffff}, add[1] = {0};
                count(jd, add, 1);
                if (p < nd) row[p + add[0]] = jd[0];
            }
        }
        if ((chosen >> lane) & 1ull)
            row[__popcll(chosen & ((1ull << lane) - 1ull)) + below] = myj;
    }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct QsaLayout {
    size_t q16, qinv, qnorm, kf, k16, part, kstat, total;
    int nb, nparts;
};

QsaLayout qsa_layout(int B, int T, int d, int r) {
    QsaLayout L;
    L.nb = (T + r - 1) / r;
    L.nparts = (L.nb + kPoolBlocks - 1) / kPoolBlocks;
    const size_t BT = static_cast<size_t>(B) * T, Bn = static_cast<size_t>(B) * L.nb;
    size_t o = 0;
    L.q16 = o;   o = align256(o + BT * kHq * d * 2);
    L.qinv = o;  o = align256(o + BT * kHq * 4);
    L.qnorm = o; o = align256(o + BT * kHq * 4);
    L.kf = o;    o = align256(o + Bn * d * 4);
    L.k16 = o;   o = align256(o + static_cast<size_t>(B) * ((L.nb + 15) / 16) * 16 * d * 2);
    L.part = o;  o = align256(o + static_cast<size_t>(B) * L.nparts * 8);
    L.kstat = o; o = align256(o + static_cast<size_t>(B) * 8);
    L.total = o;
    return L;
}

template <int D, typename TI>
hipError_t launch_qsa_t(const QsaArgs &a) {
    const QsaLayout L = qsa_layout(a.B, a.T, D, a.r);
    char *ws = static_cast<char *>(a.ws);
    f16 *q16 = reinterpret_cast<f16 *>(ws + L.q16);
    float *qinv = reinterpret_cast<float *>(ws + L.qinv);
    float *qnorm = reinterpret_cast<float *>(ws + L.qnorm);
    float *kf = reinterpret_cast<float *>(ws + L.kf);
    f16 *k16 = reinterpret_cast<f16 *>(ws + L.k16);
    float2 *part = reinterpret_cast<float2 *>(ws + L.part);
    float2 *kstat = reinterpret_cast<float2 *>(ws + L.kstat);
    const double log2base = a.rope_dims > 0 ? log2(static_cast<double>(a.rope_base)) : 0.0;
    const size_t BT = static_cast<size_t>(a.B) * a.T;
    hipLaunchKernelGGL((rope_q_kernel<D, TI>), dim3(static_cast<unsigned>(BT)), dim3(256), 0,
                       a.stream, static_cast<const TI *>(a.q), q16, qinv, qnorm, a.T,
                       a.rope_dims, log2base);
    hipLaunchKernelGGL((pool_k_kernel<D, TI>), dim3(a.B * L.nparts), dim3(256), 0, a.stream,
                       static_cast<const TI *>(a.k), kf, part, a.T, a.r, L.nb, L.nparts,
                       a.rope_dims, log2base);
    hipLaunchKernelGGL((pack_k_kernel<D>), dim3(a.B * L.nparts), dim3(256), 0, a.stream, kf, part,
                       k16, kstat, L.nb, L.nparts);
    const int ntt = (a.T + kTok - 1) / kTok;
    if (a.imp != nullptr)
        hipLaunchKernelGGL((select_kernel<D, true>), dim3(a.B * ntt), dim3(64), 0, a.stream, q16,
                           qinv, qnorm, k16, kstat, a.sel, a.imp, a.B, a.T, a.r, L.nb, a.nsel,
                           a.scale * kLog2e);
    else
        hipLaunchKernelGGL((select_kernel<D, false>), dim3(a.B * ntt), dim3(64), 0, a.stream,
                           q16, qinv, qnorm, k16, kstat, a.sel, a.imp, a.B, a.T, a.r, L.nb,
                           a.nsel, a.scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

size_t qsa_workspace(int B, int T, int d, int r) { return qsa_layout(B, T, d, r).total; }

hipError_t launch_qsa(const QsaArgs &a) {
    const bool bf = a.in_dt == GDN_BF16;
    if (a.d == 128) return bf ? launch_qsa_t<128, bf16_t>(a) : launch_qsa_t<128, float>(a);
    return bf ? launch_qsa_t<64, bf16_t>(a) : launch_qsa_t<64, float>(a);
}

}  // namespace gdn
