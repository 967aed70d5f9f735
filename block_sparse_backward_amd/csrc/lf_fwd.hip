// Dense attention forward, FlashAttention tiling (exact softmax), saving O and
// the natural-log logsumexp of every score row.
//
// The method leaves the forward untouched (LazyFlash journal entry on gyom.fr,
// section "Le passage arrière fait deux fois le travail du passage avant");
// FlashAttention reorders the computation over query/key tiles to cut HBM
// traffic and stays exact (FlashAttention course page on voce.life, section
// "Le mécanisme").
//
// bf16 kernel (gfx950): one workgroup = 4 waves = 128 query rows of one head,
// two workgroups per CU.  Each wave owns 32 rows and walks 64-key tiles of K
// and V, double-buffered in LDS (swizzled; loaded straight from HBM with
// buffer loads to LDS, the next tile's loads issued among the current tile's
// score MFMAs), one barrier per tile.  The two waves that share a SIMD belong
// to different workgroups, so one's softmax runs while the other's MFMAs do.
// On 32x32x16 bf16 MFMAs, per tile and wave:
//   * S^T = K Q^T (A: K rows from LDS, B: Q^T in registers), so each lane holds
//     one query column: the row max is an in-lane max3 chain plus one
//     lane-half swap;
//   * P^T = exp2(S^T scale log2 e - m) in the accumulator layout is directly
//     the B operand of O^T += V^T P^T (the key order inside a 16-key step is
//     permuted the same way on both operands); V^T fragments come from
//     transposing LDS reads.
// The running max m is raised only when a tile's max exceeds it by more than
// 8 (log2 units), so P stays below 2^8 and the rescale of O and l (a rare
// branch) is skipped on almost every tile; O / l and m + log2 l are exact
// whatever m is.
// A negative softmax scale is applied by negating Q (exact in bf16), so the
// max of the raw scores is the max of the scaled ones.
// The float32 kernel is a plain per-row loop (small problems, exactness).
#include "lf_common.h"
#include "lf_internal.h"
#include "lf_tile.h"

namespace lf {

constexpr int kFwdBM = 128;  // query rows per workgroup (4 waves x 32)
constexpr int kFwdBN = 64;   // keys per tile
constexpr float kMaxSlack = 8.f;  // log2 units the running max may trail a tile's max

__device__ __forceinline__ void map_fwd_block(int bid, int B, int Hq, int Hkv, int nqt, bool causal,
                                              int& b, int& h, int& t) {
    const int G = Hq / Hkv;
    const int nG = B * Hkv;
    int tr;
    if (nG % kNumXcd == 0) {
        const int xcd = bid % kNumXcd, r = bid / kNumXcd;
        const int nhx = (nG / kNumXcd) * G;
        const int hi = r % nhx;
        tr = r / nhx;
        const int gid = xcd + kNumXcd * (hi / G);
        b = gid / Hkv;
        h = (gid % Hkv) * G + hi % G;
    } else {
        const int hi = bid % (B * Hq);
        tr = bid / (B * Hq);
        b = hi / Hq;
        h = hi % Hq;
    }
    t = causal ? nqt - 1 - tr : tr;  // longest causal rows first
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// S^T (+)= K Q^T step with the score accumulator in VGPRs (the softmax reads
// it).  The caller waits out the result latency (mfma_result_wait) before any
// VALU read of the scores.
__device__ __forceinline__ void mfma_kq(f32x16& s, bf16x8 kf, bf16x8 qf, bool first) {
    if (first)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(s) : "v"(kf), "v"(qf));
    else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(kf), "v"(qf));
}
__device__ __forceinline__ void mfma_result_wait(f32x16& s) {
    asm volatile("s_nop 7\n\ts_nop 4" : "+v"(s));
}

template <int HD, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(const bf16* __restrict__ q,
                                                          const bf16* __restrict__ k,
                                                          const bf16* __restrict__ v,
                                                          bf16* __restrict__ o,
                                                          float* __restrict__ lse, int B, int Hq,
                                                          int Hkv, int N, float cl2, int neg) {
    constexpr int KS = HD / 16;  // k-steps over the head dim
    constexpr int DT = HD / 32;  // 32-wide d tiles of O^T
    constexpr int TILE = kFwdBN * HD;
    constexpr int NLOAD = 2 * TILE / (64 * 8 * 4);  // buffer loads per wave per tile
    __shared__ __attribute__((aligned(16))) bf16 sK0[TILE];
    __shared__ __attribute__((aligned(16))) bf16 sV0[TILE];
    __shared__ __attribute__((aligned(16))) bf16 sK1[TILE];
    __shared__ __attribute__((aligned(16))) bf16 sV1[TILE];

    const int nqt = (N + kFwdBM - 1) / kFwdBM;
    int b, h, t;
    map_fwd_block(blockIdx.x, B, Hq, Hkv, nqt, CAUSAL, b, h, t);
    const int g = h / (Hq / Hkv);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
    const int l32 = lane & 31, hf = lane >> 5;
    const int q0 = t * kFwdBM;
    const int qw0 = q0 + 32 * wave;  // first row of this wave
    const int qrow = qw0 + l32;      // query column held by this lane
    const int lim = CAUSAL ? qrow : N - 1;  // keys past lim are hidden

    const size_t qoff = ((size_t)b * Hq + h) * (size_t)N * HD;
    const size_t kvoff = ((size_t)b * Hkv + g) * (size_t)N * HD;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + kvoff, (uint32_t)N * HD * sizeof(bf16));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + kvoff, (uint32_t)N * HD * sizeof(bf16));

    // Q^T fragments (B operands): column = query, k = head dim; rows past N are 0
    bf16x8 qf[KS];
    {
        const bool ok = qrow < N;
        const bf16* qp = q + qoff + (size_t)(ok ? qrow : 0) * HD + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
            if (!ok) x = u32x4{};
            if (neg) x ^= 0x80008000u;
            qf[ks] = __builtin_bit_cast(bf16x8, x);
        }
    }

    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
    float m_use = -__builtin_inf(), l_run = 0.f;

    const int last_row = min(q0 + kFwdBM, N) - 1;
    const int nkt = CAUSAL ? last_row / kFwdBN + 1 : (N + kFwdBN - 1) / kFwdBN;
    // tiles whose keys every row of the workgroup sees (a partial last tile,
    // past N, is masked)
    const int nfull = CAUSAL ? min(q0 / kFwdBN, nkt) : N / kFwdBN;
    const TileOffsets<HD> off(lane);

    auto fetch = [&](int kt, bf16* dk, bf16* dv) __attribute__((always_inline)) {
        const int soff = kt * kFwdBN * HD * (int)sizeof(bf16);
        load_tile_to_lds<HD, kFwdBN, 4>(rk, soff, dk, wave, lane);
        load_tile_to_lds<HD, kFwdBN, 4>(rv, soff, dv, wave, lane);
    };

    // Softmax of one 32-key half of a tile (s: the half's S^T accumulator,
    // register r holding key kh + 8 (r >> 2) + 4 hf + (r & 3)), cut into the
    // NSL slices that the tile spreads over the MFMAs of another product:
    //   slices 0-1 the in-lane max (masked keys excluded), slice 2 the lane-pair
    //   max, the running max and the rescale factor, slices 3.. the 16
    //   exponentials, their bf16 pairs (the MFMA operand) and the row sum.
    // The running max is raised only when the half's max exceeds it by more
    // than kMaxSlack, so the rescale is rare.
    struct HalfSoftmax {
        float mx, alpha;
        float p[16];
    };
    constexpr int NSL = 8;
    auto sm_slice = [&](auto MASKC, HalfSoftmax& st, f32x16& sh, bf16x8 (&pb)[2], int kh, int i)
        __attribute__((always_inline)) {
        constexpr bool MASK = decltype(MASKC)::value;
        const int lk = lim - kh - 4 * hf;  // register r is hidden iff 8 (r >> 2) + (r & 3) > lk
        if (i == 0) {
            if constexpr (MASK) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (8 * (r >> 2) + (r & 3) > lk) sh[r] = -__builtin_inf();
            }
            st.mx = __builtin_fmaxf(sh[0], sh[1]);
#pragma unroll
            for (int r = 2; r < 8; r += 2)
                st.mx = __builtin_fmaxf(__builtin_fmaxf(st.mx, sh[r]), sh[r + 1]);
        } else if (i == 1) {
#pragma unroll
            for (int r = 8; r < 16; r += 2)
                st.mx = __builtin_fmaxf(__builtin_fmaxf(st.mx, sh[r]), sh[r + 1]);
        } else if (i == 2) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.mx),
                                                             __float_as_uint(st.mx), false, false);
            const float m =
                __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * cl2;
            const float m_new = m > m_use + kMaxSlack ? m : m_use;
            st.alpha = m_new == m_use ? 1.f : fast_exp2(m_use - m_new);
            m_use = m_new;
            l_run *= st.alpha;
        } else {
            // elements [e0, e1) of the 16, in pairs
            const int e0 = (i - 3) * 16 / (NSL - 3) & ~1, e1 = (i - 2) * 16 / (NSL - 3) & ~1;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                if (e < e0 || e >= (i == NSL - 1 ? 16 : e1)) continue;
                float x = fast_exp2(__builtin_fmaf(sh[e], cl2, -m_use));
                if constexpr (MASK)
                    if (8 * (e >> 2) + (e & 3) > lk) x = 0.f;
                st.p[e] = x;
                if (e & 1) {
                    pb[e >> 3][(e & 7) - 1] = to_bf16(st.p[e - 1]);
                    pb[e >> 3][e & 7] = to_bf16(x);
                    l_run += st.p[e - 1] + x;
                    // keep the sum here: the compiler would otherwise sink the
                    // chain (and every P it reads) to the end of the loop body
                    asm volatile("" : "+v"(l_run));
                }
            }
        }
    };
    auto rescale = [&](float alpha) __attribute__((always_inline)) {
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
            // the factor passes through the asm so that the products cannot be
            // hoisted out of the branch (they are the identity when no lane needs them)
            float a = alpha;
            asm volatile("" : "+v"(a));
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] *= a;
        }
    };

    // One 64-key tile as two 32-key halves A and B: issue the next tile's loads
    // into the other buffer (past the end: the last tile again), then
    //   S_A | S_B with the softmax of A | PV_A with the softmax of B | PV_B,
    // each "|" a scheduling barrier and each "with" a hand interleave of one
    // MFMA and one slice of softmax work.  MASK: some keys of the tile are
    // hidden from some rows of the wave.
    auto tile = [&](auto MASKC, int kt, const bf16* sk, const bf16* sv, int kn, bf16* nk,
                    bf16* nv) __attribute__((always_inline)) {
        const int k0 = kt * kFwdBN;
        f32x16 sA, sB;
        bf16x8 pA[2], pB[2];
        HalfSoftmax stA, stB;
        bf16x8 kf[2][KS];
        fetch(kn, nk, nv);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kf[mt][ks] = frag_at<HD>(sk, 32 * mt, off.frag[ks]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) mfma_kq(sA, kf[0][ks], qf[ks], ks == 0);
        mfma_result_wait(sA);
        __builtin_amdgcn_sched_barrier(0);
        // S_B with the softmax of A; the V_A fragments are read meanwhile
        bf16x8 vA[2][DT], vB[2][DT];
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            mfma_kq(sB, kf[1][i], qf[i], i == 0);
            sm_slice(MASKC, stA, sA, pA, k0, i * NSL / KS);
            if (i * NSL / KS != (i + 1) * NSL / KS - 1)
                for (int j = i * NSL / KS + 1; j < (i + 1) * NSL / KS; ++j)
                    sm_slice(MASKC, stA, sA, pA, k0, j);
            if (i >= KS - 2) {
                const int kk = i - (KS - 2);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) vA[kk][dt] = tr_at<HD>(sv, 16 * kk, off.tr[dt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        mfma_result_wait(sB);
        rescale(stA.alpha);
        __builtin_amdgcn_sched_barrier(0);
        // PV_A with the softmax of B; the V_B fragments are read meanwhile
#pragma unroll
        for (int i = 0; i < 2 * DT; ++i) {
            const int kk = i / DT, dt = i % DT;
            acc[dt] = mfma32(vA[kk][dt], pA[kk], acc[dt]);
            sm_slice(MASKC, stB, sB, pB, k0 + 32, i * NSL / (2 * DT));
            if (i * NSL / (2 * DT) != (i + 1) * NSL / (2 * DT) - 1)
                for (int j = i * NSL / (2 * DT) + 1; j < (i + 1) * NSL / (2 * DT); ++j)
                    sm_slice(MASKC, stB, sB, pB, k0 + 32, j);
            if (i >= 2 * DT - 2) {
                const int kb = i - (2 * DT - 2);
#pragma unroll
                for (int dt2 = 0; dt2 < DT; ++dt2)
                    vB[kb][dt2] = tr_at<HD>(sv, 32 + 16 * kb, off.tr[dt2]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        rescale(stB.alpha);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma32(vB[kk][dt], pB[kk], acc[dt]);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto sync = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    fetch(0, sK0, sV0);
    sync();
    int kt = 0;
    for (; kt + 2 <= nfull; kt += 2) {
        tile(IntC<0>{}, kt, sK0, sV0, kt + 1, sK1, sV1);
        sync();
        tile(IntC<0>{}, kt + 1, sK1, sV1, min(kt + 2, nkt - 1), sK0, sV0);
        sync();
    }
    // the rest (the diagonal tiles of a causal walk among them) masked; a wave
    // that sees none of a tile's keys only issues its share of the next loads.
    // kt is even here, so the buffers alternate 0, 1 as in the loop above.
    auto tail = [&](int kt, const bf16* sk, const bf16* sv, bf16* nk, bf16* nv)
        __attribute__((always_inline)) {
        const int kn = min(kt + 1, nkt - 1);
        if (!CAUSAL || kt * kFwdBN <= qw0 + 31) tile(IntC<1>{}, kt, sk, sv, kn, nk, nv);
        else fetch(kn, nk, nv);
        sync();
    };
    for (; kt < nkt; kt += 2) {
        tail(kt, sK0, sV0, sK1, sV1);
        if (kt + 1 < nkt) tail(kt + 1, sK1, sV1, sK0, sV0);
    }

    // epilogue: O = O^T / l, LSE = (m + log2 l) ln 2 (l summed over the lane pair)
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run),
                                                     false, false);
    const float l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (qrow < N) {
        const float inv = 1.f / l;
        bf16* orow = o + qoff + (size_t)qrow * HD;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                bf16x4 w;
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) w[bb] = to_bf16(acc[dt][4 * a + bb] * inv);
                *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * a + 4 * hf) = w;
            }
        if (hf == 0) lse[((size_t)b * Hq + h) * N + qrow] = (m_use + __log2f(l)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// float32: one thread per query row, online softmax over all keys.
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ q,
                                                     const float* __restrict__ k,
                                                     const float* __restrict__ v,
                                                     float* __restrict__ o,
                                                     float* __restrict__ lse, int Hq, int Hkv,
                                                     int N, float scale, int causal) {
    const int bh = blockIdx.y;
    const int b = bh / Hq, h = bh % Hq, g = h / (Hq / Hkv);
    const int row = blockIdx.x * 64 + threadIdx.x;
    if (row >= N) return;
    const float* qr = q + ((size_t)bh * N + row) * HD;
    const float* kg = k + ((size_t)b * Hkv + g) * (size_t)N * HD;
    const float* vg = v + ((size_t)b * Hkv + g) * (size_t)N * HD;
    float qv[HD], acc[HD];
#pragma unroll
    for (int c = 0; c < HD; ++c) { qv[c] = qr[c]; acc[c] = 0.f; }
    float m = -__builtin_inf(), l = 0.f;
    const int nk = causal ? row + 1 : N;
    for (int j = 0; j < nk; ++j) {
        const float* kr = kg + (size_t)j * HD;
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < HD; ++c) s += qv[c] * kr[c];
        s *= scale;
        const float mn = fmaxf(m, s);
        const float alpha = expf(m - mn);
        const float p = expf(s - mn);
        l = l * alpha + p;
        const float* vr = vg + (size_t)j * HD;
#pragma unroll
        for (int c = 0; c < HD; ++c) acc[c] = acc[c] * alpha + p * vr[c];
        m = mn;
    }
    float* orow = o + ((size_t)bh * N + row) * HD;
#pragma unroll
    for (int c = 0; c < HD; ++c) orow[c] = acc[c] / l;
    lse[(size_t)bh * N + row] = m + logf(l);
}

// ---------------------------------------------------------------------------
hipError_t launch_fwd(const Problem& pb, const void* q, const void* k, const void* v, void* o,
                      float* lse, hipStream_t st) {
    if (!pb.bf16) {
        dim3 grid((unsigned)((pb.N + 63) / 64), (unsigned)(pb.B * pb.Hq));
#define LF_F32FWD(DD)                                                                          \
    if (pb.d == DD) {                                                                          \
        hipLaunchKernelGGL(fwd_f32_kernel<DD>, grid, dim3(64), 0, st, (const float*)q,         \
                           (const float*)k, (const float*)v, (float*)o, lse, pb.Hq, pb.Hkv,    \
                           pb.N, pb.scale, pb.causal);                                         \
        return hipGetLastError();                                                              \
    }
        LF_F32FWD(64)
        LF_F32FWD(128)
#undef LF_F32FWD
        return hipErrorInvalidValue;
    }
    const int nqt = (pb.N + kFwdBM - 1) / kFwdBM;
    dim3 grid((unsigned)(nqt * pb.B * pb.Hq));
    const float sl2 = __builtin_fabsf(pb.scale) * kLog2e;
    const int neg = pb.scale < 0.f;
#define LF_FWD(DD, CC)                                                                         \
    if (pb.d == DD && (pb.causal != 0) == CC) {                                                \
        hipLaunchKernelGGL((fwd_bf16_kernel<DD, CC>), grid, dim3(256), 0, st, (const bf16*)q,  \
                           (const bf16*)k, (const bf16*)v, (bf16*)o, lse, pb.B, pb.Hq, pb.Hkv, \
                           pb.N, sl2, neg);                                                    \
        return hipGetLastError();                                                              \
    }
    LF_FWD(64, true)
    LF_FWD(64, false)
    LF_FWD(128, true)
    LF_FWD(128, false)
#undef LF_FWD
    return hipErrorInvalidValue;
}

}  // namespace lf
