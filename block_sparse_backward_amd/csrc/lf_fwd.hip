// Dense attention forward, FlashAttention tiling (exact softmax), saving O and
// the natural-log logsumexp of every score row.
//
// The method leaves the forward untouched (LazyFlash journal entry on gyom.fr,
// section "Le passage arrière fait deux fois le travail du passage avant");
// FlashAttention reorders the computation over query/key tiles to cut HBM
// traffic and stays exact (FlashAttention course page on voce.life, section
// "Le mécanisme").
//
// bf16 kernel (gfx950): one workgroup = 4 waves = 128 query rows of one head;
// each wave owns 32 rows and walks 64-key tiles staged in LDS.  Scores are
// computed transposed, S^T = K Q^T, on 32x32x16 bf16 MFMAs, so that:
//   * each lane holds one query column: the row max and row sum of the online
//     softmax are in-lane reductions plus one exchange with lane l ^ 32;
//   * P^T in the accumulator layout is directly the B operand of
//     O^T += V^T P^T (the key order inside a 16-key step is permuted the same
//     way on both operands);
//   * V^T fragments come from the row-major V tile by transposing LDS reads.
// The float32 kernel is a plain per-row loop (small problems, exactness).
#include "lf_common.h"
#include "lf_internal.h"

namespace lf {

constexpr int kFwdBM = 128;  // query rows per workgroup
constexpr int kFwdBN = 64;   // keys per tile
constexpr int kPad = 8;      // bf16 elements of padding per LDS row

template <int HD>
struct FwdTile {
    static constexpr int LD = HD + kPad;            // LDS row stride (elements)
    static constexpr int CHUNKS = kFwdBN * HD / 8;  // 16-byte chunks per tile
    static constexpr int PER_THREAD = CHUNKS / 256;
};

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

template <int HD, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_bf16_kernel(const bf16* __restrict__ q,
                                                       const bf16* __restrict__ k,
                                                       const bf16* __restrict__ v,
                                                       bf16* __restrict__ o,
                                                       float* __restrict__ lse, int B, int Hq,
                                                       int Hkv, int N, float scale_log2) {
    using TL = FwdTile<HD>;
    constexpr int KS = HD / 16;  // k-steps over the head dim
    constexpr int DT = HD / 32;  // 32-wide d tiles of O^T
    __shared__ __attribute__((aligned(16))) bf16 sK[kFwdBN * TL::LD];
    __shared__ __attribute__((aligned(16))) bf16 sV[kFwdBN * TL::LD];

    const int nqt = (N + kFwdBM - 1) / kFwdBM;
    int b, h, t;
    map_fwd_block(blockIdx.x, B, Hq, Hkv, nqt, CAUSAL, b, h, t);
    const int g = h / (Hq / Hkv);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int q0 = t * kFwdBM;
    const int qw0 = q0 + 32 * wave;      // first row of this wave
    const int qrow = qw0 + l32;          // query column held by this lane
    const bool row_ok = qrow < N;

    const size_t qoff = ((size_t)b * Hq + h) * (size_t)N * HD;
    const size_t kvoff = ((size_t)b * Hkv + g) * (size_t)N * HD;
    const bf16* kg = k + kvoff;
    const bf16* vg = v + kvoff;

    // Q^T fragments (B operand): column = query, k = head dim.
    bf16x8 qf[KS];
    {
        const bf16* qr = q + qoff + (size_t)(row_ok ? qrow : 0) * HD;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qf[ks] = *reinterpret_cast<const bf16x8*>(qr + 16 * ks + 8 * hf);
            if (!row_ok) qf[ks] = bf16x8{};
        }
    }

    f32x16 acc_o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc_o[dt] = f32x16{};
    float m_run = -__builtin_inf(), l_run = 0.f;

    const int last_row = min(q0 + kFwdBM, N) - 1;
    const int nkt_all = (N + kFwdBN - 1) / kFwdBN;
    const int nkt = CAUSAL ? min(nkt_all, last_row / kFwdBN + 1) : nkt_all;

    // register prefetch of one K and one V tile
    u32x4 pk[TL::PER_THREAD], pv[TL::PER_THREAD];
    auto fetch = [&](int kt) {
#pragma unroll
        for (int c = 0; c < TL::PER_THREAD; ++c) {
            const int chunk = tid + 256 * c;
            const int row = chunk / (HD / 8), col = (chunk % (HD / 8)) * 8;
            const int key = kt * kFwdBN + row;
            if (key < N) {
                pk[c] = *reinterpret_cast<const u32x4*>(kg + (size_t)key * HD + col);
                pv[c] = *reinterpret_cast<const u32x4*>(vg + (size_t)key * HD + col);
            } else {
                pk[c] = u32x4{};
                pv[c] = u32x4{};
            }
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int c = 0; c < TL::PER_THREAD; ++c) {
            const int chunk = tid + 256 * c;
            const int row = chunk / (HD / 8), col = (chunk % (HD / 8)) * 8;
            *reinterpret_cast<u32x4*>(&sK[row * TL::LD + col]) = pk[c];
            *reinterpret_cast<u32x4*>(&sV[row * TL::LD + col]) = pv[c];
        }
    };

    fetch(0);
    for (int kt = 0; kt < nkt; ++kt) {
        stage();
        __syncthreads();
        if (kt + 1 < nkt) fetch(kt + 1);
        const int k0 = kt * kFwdBN;
        const bool wave_active = !CAUSAL || k0 <= qw0 + 31;
        if (wave_active) {
            // S^T = K Q^T : two 32-key tiles
            f32x16 s[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                s[mt] = f32x16{};
                const bf16* arow = &sK[(32 * mt + l32) * TL::LD + 8 * hf];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    s[mt] = mfma32(*reinterpret_cast<const bf16x8*>(arow + 16 * ks), qf[ks], s[mt]);
            }
            const bool need_mask = (CAUSAL && k0 + kFwdBN - 1 > qw0) || (k0 + kFwdBN > N);
            float mx = -__builtin_inf();
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = s[mt][r] * scale_log2;
                    if (need_mask) {
                        const int key = k0 + 32 * mt + 8 * (r >> 2) + 4 * hf + (r & 3);
                        if (key >= N || (CAUSAL && key > qrow)) x = -__builtin_inf();
                    }
                    s[mt][r] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -__builtin_inf()) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            float ls = 0.f;
            bf16x8 pb[4];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                float p[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    p[r] = fast_exp2(s[mt][r] - m_use);
                    ls += p[r];
                }
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    bf16x8 f;
#pragma unroll
                    for (int j = 0; j < 8; ++j) f[j] = to_bf16(p[8 * half + j]);
                    pb[2 * mt + half] = f;
                }
            }
            ls += __shfl_xor(ls, 32);
            l_run = l_run * alpha + ls;
            m_run = m_new;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc_o[dt] *= alpha;
            // O^T += V^T P^T : A = V^T via transposing reads of the row-major V tile.
            const int G16 = lane >> 4, j16 = lane & 15;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int rbase = 16 * ks + 4 * (G16 >> 1) + (j16 >> 2);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int col = 32 * dt + 16 * (G16 & 1) + 4 * (j16 & 3);
                    const bf16x4 lo = lds_read_tr(&sV[rbase * TL::LD + col]);
                    const bf16x4 hi = lds_read_tr(&sV[(rbase + 8) * TL::LD + col]);
                    acc_o[dt] = mfma32(cat(lo, hi), pb[ks], acc_o[dt]);
                }
            }
        }
        __syncthreads();
    }

    // epilogue: O = O^T / l, LSE = (m + log2 l) * ln 2
    if (row_ok) {
        const float inv = 1.f / l_run;
        bf16* orow = o + qoff + (size_t)qrow * HD;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                bf16x4 w;
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) w[bb] = to_bf16(acc_o[dt][4 * a + bb] * inv);
                *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * a + 4 * hf) = w;
            }
        if (hf == 0) lse[((size_t)b * Hq + h) * N + qrow] = (m_run + __log2f(l_run)) * kLn2;
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
    const float sl2 = pb.scale * kLog2e;
#define LF_FWD(DD, CC)                                                                         \
    if (pb.d == DD && (pb.causal != 0) == CC) {                                                \
        hipLaunchKernelGGL((fwd_bf16_kernel<DD, CC>), grid, dim3(256), 0, st, (const bf16*)q,  \
                           (const bf16*)k, (const bf16*)v, (bf16*)o, lse, pb.B, pb.Hq, pb.Hkv, \
                           pb.N, sl2);                                                         \
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
