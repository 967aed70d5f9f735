// Block selection: per-block gradient masses (one HBM streaming pass over
// dO), then per (batch, head) the budget threshold tau, the Philox draw, the
// 1/p weights and the compacted kept-block list, then the D row term of the
// kept blocks only (the backward reads no other row's D).
//
// Method: the LazyFlash journal entry on gyom.fr ("LazyFlash allège la
// rétropropagation de l'attention, 5,72 fois"), section "Un budget sur la masse
// de gradient, et un tirage qui garde le gradient non biaisé": blocks are ranked
// by the norm of their output gradient, a budget delta bounds the discarded
// share of gradient mass per head and per step, blocks are kept with a
// probability proportional to their gradient and reweighted to stay unbiased.
//
// Every floating-point operation that decides the kept set is done in IEEE
// double with one rounding per operation in a fixed order (this file is
// compiled with -ffp-contract=off), so the kept set is reproducible bit for
// bit by any implementation of the same rule.
#include "lf_common.h"
#include "lf_internal.h"

namespace lf {

// ---------------------------------------------------------------------------
// Kernel A: one workgroup of 256 threads per query block (b, h, i): its mass.
// The block is the run of L = block*d elements at row i*block of head (b, h);
// when N is not a multiple of block the last block's missing rows read as
// zeros (they add exact zeros to the mass).
// Thread t owns elements e + 8t + 2048s (e < 8, s < L/2048), loaded as one
// 16-byte vector per s (coalesced), which lets the fp64 halving tree run as:
// in-thread levels over s, then 8 cross-thread levels (t + 128, t + 64, ...,
// t + 1), then 3 in-vector levels over e.
// ---------------------------------------------------------------------------
// Eight consecutive elements as floats from a raw buffer (16-byte loads; past
// the buffer's end they read as zeros).  The loads carry the non-temporal
// hint: each byte is read once, and streaming it through the last-level
// cache would evict what the kernels before left there (the backward's dirty
// outputs among it, whose write-back then competes with these reads).
constexpr int kStreamLoad = 2;  // cache policy bits of a buffer load: nt
template <typename T>
__device__ __forceinline__ void load8_buf(__amdgpu_buffer_rsrc_t rs, int voff, int soff,
                                          float (&x)[8]) {
    if constexpr (sizeof(T) == 2) {
        const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kStreamLoad);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float(r[j] << 16);
            x[2 * j + 1] = __uint_as_float(r[j] & 0xffff0000u);
        }
    } else {
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kStreamLoad);
        const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16, soff, kStreamLoad);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = __uint_as_float(a[j]);
            x[4 + j] = __uint_as_float(b[j]);
        }
    }
}

template <typename T, int L, int HD>
__global__ __launch_bounds__(256) void mass_kernel(const T* __restrict__ dout,
                                                   double* __restrict__ mass, int N, int nqb) {
    constexpr int S = L / 2048;
    constexpr int ROWS = L / HD;  // = block
    const size_t blk = blockIdx.x;
    const size_t bh = blk / (size_t)nqb;
    const int row0 = (int)(blk % (size_t)nqb) * ROWS;
    const int t = threadIdx.x;
    // buffer loads over the head: rows past N read as zeros, with no branch
    const uint32_t head_bytes = (uint32_t)((size_t)N * HD * sizeof(T));
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(dout + bh * (size_t)N * HD, head_bytes);
    const int off0 = row0 * HD * (int)sizeof(T);  // the block's first row in the head

    float x[S][8];
#pragma unroll
    for (int s = 0; s < S; ++s) load8_buf<T>(rg, (8 * t + 2048 * s) * (int)sizeof(T), off0, x[s]);

    // squares are exact in fp64; only the additions round
    double v[S][8];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const double a = (double)x[s][e];
            v[s][e] = __dmul_rn(a, a);
        }
#pragma unroll
    for (int half = S / 2; half >= 1; half >>= 1)
#pragma unroll
        for (int s = 0; s < half; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) v[s][e] = __dadd_rn(v[s][e], v[s + half][e]);

    __shared__ double red[8][256];
#pragma unroll
    for (int e = 0; e < 8; ++e) red[e][t] = v[0][e];
    __syncthreads();
    if (t < 128) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[e][t] = __dadd_rn(red[e][t], red[e][t + 128]);
    }
    __syncthreads();
    if (t < 64) {
        double w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = __dadd_rn(red[e][t], red[e][t + 64]);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = __dadd_rn(w[e], __shfl_down(w[e], off));
        if (t == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = __dadd_rn(w[e], w[e + 4]);
#pragma unroll
            for (int e = 0; e < 2; ++e) w[e] = __dadd_rn(w[e], w[e + 2]);
            mass[blk] = __dadd_rn(w[0], w[1]);
        }
    }
}

// ---------------------------------------------------------------------------
// Kernel C: D = rowsum(dO * O) for the rows of kept blocks, one workgroup per
// query block (the same thread mapping as kernel A: each (t, s) covers 8
// columns of row (8t + 2048s) / HD); a skipped block's rows get D = 0, which
// the backward never reads (it loads nothing of a skipped block).
// ---------------------------------------------------------------------------
template <typename T, int L, int HD>
__global__ __launch_bounds__(256) void d_kept_kernel(const T* __restrict__ o,
                                                     const T* __restrict__ dout,
                                                     const float* __restrict__ block_w,
                                                     float* __restrict__ D, int N, int nqb) {
    constexpr int S = L / 2048;
    constexpr int LANES_PER_ROW = HD / 8;
    constexpr int ROWS = L / HD;
    const size_t blk = blockIdx.x;
    const size_t bh = blk / (size_t)nqb;
    const int row0 = (int)(blk % (size_t)nqb) * ROWS;
    const int nrows = min(ROWS, N - row0);  // rows of this block that exist
    const int t = threadIdx.x;
    float* Dr = D + bh * (size_t)N + row0;
    if (block_w[blk] == 0.f) {
        for (int r = t; r < nrows; r += 256) Dr[r] = 0.f;
        return;
    }
    const uint32_t head_bytes = (uint32_t)((size_t)N * HD * sizeof(T));
    const size_t head = bh * (size_t)N * HD;
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(dout + head, head_bytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(o + head, head_bytes);
    const int off0 = row0 * HD * (int)sizeof(T);
    float x[S][8], y[S][8];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int vo = (8 * t + 2048 * s) * (int)sizeof(T);
        load8_buf<T>(rg, vo, off0, x[s]);
        load8_buf<T>(ro, vo, off0, y[s]);
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) part += x[s][e] * y[s][e];
#pragma unroll
        for (int off = LANES_PER_ROW / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off);
        const int r = (8 * t + 2048 * s) / HD;
        if ((t % LANES_PER_ROW) == 0 && r < nrows) Dr[r] = part;
    }
}

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): the round multiplies
// words 0 and 2 by the two round constants and mixes the high halves with
// words 1, 3 and the key; the key gains the two Weyl constants before every
// round but the first.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t philox_first_word(uint64_t c0, uint64_t c1, uint64_t c2,
                                                      uint64_t c3, uint64_t k0, uint64_t k1) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += W0; k1 += W1; }
        const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
        const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
        const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    }
    return c0;
}

// ---------------------------------------------------------------------------
// Kernel B: one workgroup of 1024 threads per (b, h).
// LDS: sorted masses, running sums A and Q (3 * P doubles, P = pow2 >= nqb).
//
// The rule that turns masses into a keep set (section "Le choix des blocs pèse
// plus que la quantité sautée" compares the budget with two others):
//   kRuleBudget   tau from the budget delta on the discarded mass (above);
//   kRuleFraction the same draw with tau set so that the expected number of
//                 kept blocks is f times the number of positive-mass blocks n:
//                 on [m_(k), m_(k+1)] the expected count is (n - k) + A_k / tau,
//                 so the first interval whose right end already gives <= f n
//                 holds tau = A_k / (f n - (n - k));
//   kRuleTopk     the ceil(f n) largest masses, ties to the lower index, weight
//                 1, no draw; tau reports the smallest kept mass.
// All floating-point steps are explicit roundings in a fixed order, so the
// keep set is bit-reproducible.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kRuleBudget = 0, kRuleFraction = 1, kRuleTopk = 2;

// Running sums dst[k] = fl(dst[k - 1] + src[k]) for k < n, in ascending order
// (one rounding per addition), by one thread; the loads run one batch ahead
// of the dependent additions.  src and dst may be the same array.
__device__ __forceinline__ void running_sum(const double* src, double* dst, int n) {
    constexpr int NB = 16;
    double acc = 0.0, cur[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) cur[u] = src[min(u, n - 1)];
    int k0 = 0;
    for (; k0 + NB <= n; k0 += NB) {  // whole batches: no branch among the additions
        double nxt[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) nxt[u] = src[min(k0 + NB + u, n - 1)];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            acc = __dadd_rn(acc, cur[u]);
            dst[k0 + u] = acc;
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) cur[u] = nxt[u];
    }
    for (int u = 0; k0 + u < n; ++u) {  // the last, partial batch
        acc = __dadd_rn(acc, src[k0 + u]);
        dst[k0 + u] = acc;
    }
}

__global__ __launch_bounds__(kSelThreads) void tau_select_kernel(
    const double* __restrict__ mass, int rule, double param, uint64_t seed, int b0, int Hq,
    int nqb, int P, double* __restrict__ tau_out, float* __restrict__ block_w,
    int32_t* __restrict__ kept_idx, int32_t* __restrict__ kept_count) {
    extern __shared__ double smem[];
    double* srt = smem;       // [P]
    double* accA = smem + P;  // [P]
    double* accQ = smem + 2 * P;
    __shared__ int s_nonfinite, s_npos, s_kstar, s_wave[kSelThreads / 64], s_base;
    __shared__ int s_gt, s_eqw[kSelThreads / 64], s_eqbase;
    __shared__ double s_tau;

    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int b = bh / Hq, h = bh % Hq;
    const double* m = mass + (size_t)bh * nqb;
    if (tid == 0) { s_nonfinite = 0; s_npos = 0; s_kstar = 0x7fffffff; s_base = 0; s_gt = 0; s_eqbase = 0; }
    __syncthreads();

    int my_pos = 0, my_bad = 0;
    for (int i = tid; i < P; i += kSelThreads) {
        double v = __builtin_inf();
        if (i < nqb) {
            const double mi = m[i];
            if (!__builtin_isfinite(mi)) my_bad = 1;
            if (mi > 0.0) { v = mi; ++my_pos; }
        }
        srt[i] = v;
    }
    if (my_bad) atomicOr(&s_nonfinite, 1);
    if (my_pos) atomicAdd(&s_npos, my_pos);
    __syncthreads();
    const bool nonfinite = s_nonfinite != 0;
    const int n = s_npos;
    // fraction and top-k: the target count f n (one rounding)
    const double cnt = __dmul_rn(param, (double)n);
    const bool need_sort = !nonfinite && n > 0 &&
                           ((rule == kRuleBudget && param != 0.0) ||
                            (rule == kRuleFraction && cnt < (double)n) || rule == kRuleTopk);
    // top-k keeps the k largest: k = ceil(f n) (at least 1 for f > 0, n > 0)
    const int topk = min(n, (int)ceil(cnt));

    if (need_sort && P <= kSelThreads) {
        // bitonic sort, ascending (positives first, +inf padding last), one
        // element per thread: exchanges within a wave (j < 64) by shuffles,
        // the others through LDS.  The values are finite or +inf, so the pair
        // (min, max) is the same whichever way a tie is ordered.
        double x = tid < P ? srt[tid] : 0.0;
        for (int k = 2; k <= P; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                double y;
                if (j >= 64) {
                    __syncthreads();
                    if (tid < P) srt[tid] = x;
                    __syncthreads();
                    y = tid < P ? srt[tid ^ j] : 0.0;
                } else {
                    y = __shfl_xor(x, j);
                }
                const bool low = (tid & j) == 0, up = (tid & k) == 0;
                x = (low == up) ? fmin(x, y) : fmax(x, y);
            }
        }
        __syncthreads();
        if (tid < P) srt[tid] = x;
        __syncthreads();
    } else if (need_sort) {
        // bitonic sort, ascending (positives first, +inf padding last)
        for (int k = 2; k <= P; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int i = tid; i < P; i += kSelThreads) {
                    const int ixj = i ^ j;
                    if (ixj > i) {
                        const double a = srt[i], c = srt[ixj];
                        const bool up = (i & k) == 0;
                        if ((a > c) == up) { srt[i] = c; srt[ixj] = a; }
                    }
                }
                __syncthreads();
            }
        }
    }
    if (need_sort && rule == kRuleTopk) {
        if (tid == 0) s_tau = srt[n - topk];  // the k-th largest positive mass
    } else if (need_sort) {
        // running sums in ascending order, each addition rounded in turn:
        // A over the masses (wave 0) and Q over their squares (wave 1, the
        // squares formed first by all threads) run side by side
        for (int k = tid; k < n; k += kSelThreads) accQ[k] = __dmul_rn(srt[k], srt[k]);
        __syncthreads();
        if (tid == 0) running_sum(srt, accA, n);
        else if (tid == 64) running_sum(accQ, accQ, n);
        __syncthreads();
        if (rule == kRuleBudget) {
            const double target = __dmul_rn(param, accA[n - 1]);
            // first interval [m_(k), m_(k+1)] whose right end meets the budget
            for (int k = tid; k < n; k += kSelThreads) {
                const double hi = (k + 1 < n) ? srt[k + 1] : __builtin_inf();
                const double f_hi = __dsub_rn(accA[k], __ddiv_rn(accQ[k], hi));
                if (f_hi >= target) atomicMin(&s_kstar, k);
            }
            __syncthreads();
            if (tid == 0) {
                const int k = s_kstar;
                s_tau = __ddiv_rn(accQ[k], __dsub_rn(accA[k], target));
            }
        } else {
            // first interval whose right end already brings the expected count to cnt
            for (int k = tid; k < n; k += kSelThreads) {
                const double hi = (k + 1 < n) ? srt[k + 1] : __builtin_inf();
                const double sat = (double)(n - k - 1);
                if (__dadd_rn(sat, __ddiv_rn(accA[k], hi)) <= cnt) atomicMin(&s_kstar, k);
            }
            __syncthreads();
            if (tid == 0) {
                const int k = s_kstar;
                s_tau = __ddiv_rn(accA[k], __dsub_rn(cnt, (double)(n - k - 1)));
            }
        }
    } else if (tid == 0) {
        if (nonfinite) {
            s_tau = __builtin_nan("");
        } else if (n == 0) {
            s_tau = __builtin_inf();
        } else {  // every positive block kept: tau = smallest positive mass
            double mn = __builtin_inf();
            for (int i = 0; i < nqb; ++i) {
                const double mi = m[i];
                if (mi > 0.0 && mi < mn) mn = mi;
            }
            s_tau = mn;
        }
    }
    __syncthreads();
    const double tau = s_tau;
    const bool topk_rule = rule == kRuleTopk && !nonfinite;
    if (topk_rule && n > 0) {  // blocks strictly above the threshold are all kept
        int my_gt = 0;
        for (int i = tid; i < nqb; i += kSelThreads) my_gt += m[i] > tau;
        if (my_gt) atomicAdd(&s_gt, my_gt);
        __syncthreads();
    }
    const int ties_kept = topk_rule && n > 0 ? topk - s_gt : 0;  // of the blocks equal to tau

    // draw (or top-k test), weights and ascending compaction, 1024 blocks per round
    const int lane = tid & 63, wave = tid >> 6;
    float* wout = block_w + (size_t)bh * nqb;
    int32_t* kout = kept_idx + (size_t)bh * nqb;
    for (int base = 0; base < nqb; base += kSelThreads) {
        const int i = base + tid;
        bool keep = false, tie = false;
        double p = 0.0;
        if (i < nqb) {
            const double mi = m[i];
            if (nonfinite) {
                p = 1.0;
            } else if (topk_rule) {
                keep = n > 0 && mi > tau;
                tie = n > 0 && mi == tau;
            } else if (mi != 0.0) {
                p = fmin(1.0, __ddiv_rn(mi, tau));
            }
            if (!topk_rule) {
                const uint64_t x0 = philox_first_word((uint64_t)i, (uint64_t)h, (uint64_t)(b0 + b), 0ull,
                                                      seed, 0ull);
                const double u = (double)(x0 >> 11) * 0x1p-53;
                keep = u < p;
            }
        }
        if (topk_rule) {  // ties to the lower index: rank among this round's ties
            const uint64_t tb = __ballot(tie);
            const int trank = __popcll(tb & ((1ull << lane) - 1ull));
            if (lane == 0) s_eqw[wave] = __popcll(tb);
            __syncthreads();
            int toff = s_eqbase;
            for (int w = 0; w < wave; ++w) toff += s_eqw[w];
            if (tie && toff + trank < ties_kept) keep = true;
            __syncthreads();
            if (tid == 0) {
                int tot = 0;
                for (int w = 0; w < kSelThreads / 64; ++w) tot += s_eqw[w];
                s_eqbase += tot;
            }
        }
        if (i < nqb) wout[i] = keep ? (topk_rule ? 1.0f : (float)__ddiv_rn(1.0, p)) : 0.0f;
        const uint64_t ballot = __ballot(keep);
        const int before = __popcll(ballot & ((1ull << lane) - 1ull));
        if (lane == 0) s_wave[wave] = __popcll(ballot);
        __syncthreads();
        int off = s_base;
        for (int w = 0; w < wave; ++w) off += s_wave[w];
        if (keep) kout[off + before] = i;
        __syncthreads();
        if (tid == 0) {
            int tot = 0;
            for (int w = 0; w < kSelThreads / 64; ++w) tot += s_wave[w];
            s_base += tot;
        }
        __syncthreads();
    }
    const int count = s_base;
    for (int i = count + tid; i < nqb; i += kSelThreads) kout[i] = -1;
    if (tid == 0) {
        kept_count[bh] = count;
        tau_out[bh] = tau;
    }
}

// ---------------------------------------------------------------------------
template <typename T>
static hipError_t launch_mass(const Problem& pb, const void* dout, double* mass, hipStream_t st) {
    const unsigned nblk = (unsigned)((size_t)pb.B * pb.Hq * pb.nqb);
    const int L = pb.block * pb.d;
    const T* pd = static_cast<const T*>(dout);
#define LF_MASS(LL, DD)                                                                     \
    if (L == LL && pb.d == DD) {                                                            \
        hipLaunchKernelGGL((mass_kernel<T, LL, DD>), dim3(nblk), dim3(256), 0, st, pd, mass, \
                           pb.N, pb.nqb);                                                   \
        return hipGetLastError();                                                           \
    }
    LF_MASS(4096, 64)
    LF_MASS(8192, 64)
    LF_MASS(8192, 128)
    LF_MASS(16384, 128)
#undef LF_MASS
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_d_kept(const Problem& pb, const void* o, const void* dout,
                               const float* block_w, float* D, hipStream_t st) {
    const unsigned nblk = (unsigned)((size_t)pb.B * pb.Hq * pb.nqb);
    const int L = pb.block * pb.d;
    const T* po = static_cast<const T*>(o);
    const T* pd = static_cast<const T*>(dout);
#define LF_DK(LL, DD)                                                                        \
    if (L == LL && pb.d == DD) {                                                             \
        hipLaunchKernelGGL((d_kept_kernel<T, LL, DD>), dim3(nblk), dim3(256), 0, st, po, pd,  \
                           block_w, D, pb.N, pb.nqb);                                        \
        return hipGetLastError();                                                            \
    }
    LF_DK(4096, 64)
    LF_DK(8192, 64)
    LF_DK(8192, 128)
    LF_DK(16384, 128)
#undef LF_DK
    return hipErrorInvalidValue;
}

__global__ void empty_heads_kernel(double* __restrict__ tau, int32_t* __restrict__ kept_count,
                                   int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        tau[i] = __builtin_inf();
        kept_count[i] = 0;
    }
}

hipError_t launch_empty_heads(double* tau, int32_t* kept_count, int n, hipStream_t st) {
    hipLaunchKernelGGL(empty_heads_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       tau, kept_count, n);
    return hipGetLastError();
}

hipError_t launch_select(const Problem& pb, const void* o, const void* dout, int rule,
                         double param, uint64_t seed, float* D, double* mass, double* tau,
                         float* block_w, int32_t* kept_idx, int32_t* kept_count, hipStream_t st) {
    hipError_t e = pb.bf16 ? launch_mass<bf16>(pb, dout, mass, st)
                           : launch_mass<float>(pb, dout, mass, st);
    if (e != hipSuccess) return e;
    int P = 1;
    while (P < pb.nqb) P <<= 1;
    const size_t lds = 3 * (size_t)P * sizeof(double);
    if (lds > 65536) {
        e = hipFuncSetAttribute((const void*)tau_select_kernel,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(tau_select_kernel, dim3((unsigned)(pb.B * pb.Hq)), dim3(kSelThreads), lds,
                       st, mass, rule, param, seed, pb.b0, pb.Hq, pb.nqb, P, tau, block_w,
                       kept_idx, kept_count);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return pb.bf16 ? launch_d_kept<bf16>(pb, o, dout, block_w, D, st)
                   : launch_d_kept<float>(pb, o, dout, block_w, D, st);
}

}  // namespace lf
