// Block-sparse attention backward over the kept query blocks only.
//
// Method: LazyFlash journal entry on gyom.fr ("LazyFlash allège la
// rétropropagation de l'attention, 5,72 fois"): section "Un budget sur la masse
// de gradient, et un tirage qui garde le gradient non biaisé" (skipped query
// blocks are never loaded nor computed; kept blocks carry a 1/p weight) and
// section "Trois tailles de modèle, 19 découpages sur 21" (the FlashAttention
// backward consumes the per-block weights directly).
//
// The gradient computed is the dense attention gradient of dO' = keep*w*dO:
//   P  = exp(scale Q K^T - LSE) (causal mask),   D = rowsum(dO * O),
//   dP = dO V^T,   dS = P * (dP - D),
//   dV = sum_i w_i P_i^T dO_i,   dK = scale sum_i w_i dS_i^T Q_i,
//   dQ_i = w_i scale dS_i K            (rows of skipped blocks: 0).
// The weight is folded into the exponent: exp2(s - (LSE log2 e - log2 w)) =
// w P, so dS and the dV/dK/dQ products carry it for free.
//
// bf16 kernel (gfx950): one workgroup of 4 waves per (batch, kv head, 128-key
// tile); wave w owns keys 32w..32w+31 and keeps its K/V fragments and its
// dK/dV accumulators in registers for the whole walk.  The workgroup walks the
// kept blocks of the Hq/Hkv query heads of its group in 64-row sub-tiles
// (Q, dO, LSE', D staged in LDS) and per sub-tile does, on 32x32x16 MFMAs:
//   S = Q K_w^T and dP = dO V_w^T (A from LDS rows, B in registers),
//   dV_w += P^T dO and dK_w += dS^T Q (A = P / dS straight from the score
//   accumulators, B from transposing LDS reads of the row-major tiles),
//   dQ_tile = dS K (dS^T through LDS, K^T fragments in registers), added with
//   float atomics into an fp32 workspace; a last pass scales and converts it.
// Skipped blocks never enter the loop, so their tiles are never read.
#include "lf_common.h"
#include "lf_internal.h"

namespace lf {

constexpr int kBN = 128;  // keys per workgroup
constexpr int kBM = 64;   // query rows per sub-tile
constexpr int kBPad = 8;

__device__ __forceinline__ void map_bwd_block(int bid, int B, int Hkv, int nkt, int& b, int& g,
                                              int& j) {
    const int nG = B * Hkv;
    int gid;
    if (nG % kNumXcd == 0) {
        const int xcd = bid % kNumXcd, r = bid / kNumXcd;
        const int ngx = nG / kNumXcd;
        gid = xcd + kNumXcd * (r % ngx);
        j = r / ngx;
    } else {
        gid = bid % nG;
        j = bid / nG;
    }
    b = gid / Hkv;
    g = gid % Hkv;
    (void)nkt;
}

// first position in the ascending list with value >= x
__device__ __forceinline__ int lower_bound_i32(const int32_t* list, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (list[mid] < x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

template <int HD, int BLK, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ lse, const bf16* __restrict__ dout, const float* __restrict__ Drow,
    const int32_t* __restrict__ kept_idx, const int32_t* __restrict__ kept_count,
    const float* __restrict__ block_w, bf16* __restrict__ dk, bf16* __restrict__ dv,
    float* __restrict__ dq_acc, int B, int Hq, int Hkv, int N, int nqb, float scale,
    float scale_log2) {
    constexpr int KS = HD / 16;        // k-steps over the head dim
    constexpr int DT = HD / 32;        // 32-wide head-dim tiles
    constexpr int LD = HD + kBPad;     // row stride of sQ / sdO / sK
    constexpr int LDT = kBM + kBPad;   // row stride of sdsT (q contiguous)
    constexpr int CH = kBM * HD / 8;   // 16-byte chunks per staged tile
    constexpr int CPT = CH / 256;

    __shared__ __attribute__((aligned(16))) bf16 sQ[kBM * LD];
    __shared__ __attribute__((aligned(16))) bf16 sdO[kBM * LD];
    __shared__ __attribute__((aligned(16))) bf16 sdsT[kBN * LDT];
    __shared__ __attribute__((aligned(16))) float sLse[kBM];
    __shared__ __attribute__((aligned(16))) float sD[kBM];

    const int nkt = (N + kBN - 1) / kBN;
    int b, g, j;
    map_bwd_block(blockIdx.x, B, Hkv, nkt, b, g, j);
    const int G = Hq / Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5, G16 = lane >> 4, j16 = lane & 15;
    const int k0 = j * kBN;
    const int key = k0 + 32 * wave + l32;  // key column held by this lane
    const bool key_ok = key < N;

    const size_t kvoff = ((size_t)b * Hkv + g) * (size_t)N * HD;

    // K and V fragments (B operands of S = Q K^T, dP = dO V^T)
    bf16x8 kf[KS], vf[KS];
    {
        const size_t r = kvoff + (size_t)(key_ok ? key : 0) * HD;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kf[ks] = *reinterpret_cast<const bf16x8*>(k + r + 16 * ks + 8 * hf);
            vf[ks] = *reinterpret_cast<const bf16x8*>(v + r + 16 * ks + 8 * hf);
            if (!key_ok) { kf[ks] = bf16x8{}; vf[ks] = bf16x8{}; }
        }
    }
    // K^T fragments for dQ = dS K: B[k = key, n = d], this wave's d tile.
    // Staged once through LDS (sQ/sdO hold the 128 x HD K tile here).
    constexpr int QT_DQ = (HD == 128) ? 2 : 1;   // q tiles per wave in dQ
    const int dq_d0 = (HD == 128) ? 32 * wave : 32 * (wave & 1);
    const int dq_qt0 = (HD == 128) ? 0 : (wave >> 1);
    bf16x8 ktf[kBN / 16];
    {
        // rows 0..63 of the K tile go to sQ, rows 64..127 to sdO
        for (int c = tid; c < kBN * HD / 8; c += 256) {
            const int row = c / (HD / 8), col = (c % (HD / 8)) * 8;
            const int kk = k0 + row;
            u32x4 val = u32x4{};
            if (kk < N) val = *reinterpret_cast<const u32x4*>(k + kvoff + (size_t)kk * HD + col);
            bf16* dst = (row < kBM) ? &sQ[row * LD + col] : &sdO[(row - kBM) * LD + col];
            *reinterpret_cast<u32x4*>(dst) = val;
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kBN / 16; ++ks) {
            const int r0 = 16 * ks + 8 * hf + (j16 >> 2);
            const int col = dq_d0 + 16 * (G16 & 1) + 4 * (j16 & 3);
            const bf16* p0 = (r0 < kBM) ? &sQ[r0 * LD + col] : &sdO[(r0 - kBM) * LD + col];
            const int r1 = r0 + 4;
            const bf16* p1 = (r1 < kBM) ? &sQ[r1 * LD + col] : &sdO[(r1 - kBM) * LD + col];
            ktf[ks] = cat(lds_read_tr(p0), lds_read_tr(p1));
        }
        __syncthreads();
    }

    f32x16 acc_dk[DT], acc_dv[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) { acc_dk[dt] = f32x16{}; acc_dv[dt] = f32x16{}; }

    for (int hg = 0; hg < G; ++hg) {
        const int h = g * G + hg;
        const int bh = b * Hq + h;
        const int cnt = min(max(kept_count[bh], 0), nqb);
        const int32_t* list = kept_idx + (size_t)bh * nqb;
        const int start = CAUSAL ? lower_bound_i32(list, cnt, k0 / BLK) : 0;
        const size_t qoff = (size_t)bh * (size_t)N * HD;
        for (int pos = start; pos < cnt; ++pos) {
            const int i = list[pos];
            if ((unsigned)i >= (unsigned)nqb) continue;  // malformed list: skip
            const float lw = __log2f(block_w[(size_t)bh * nqb + i]);
#pragma unroll 1
            for (int st = 0; st < BLK / kBM; ++st) {
                const int qs0 = i * BLK + st * kBM;
                if (CAUSAL && qs0 + kBM - 1 < k0) continue;
                // ---- stage Q, dO rows, LSE' and D
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    const int chunk = tid + 256 * c;
                    const int row = chunk / (HD / 8), col = (chunk % (HD / 8)) * 8;
                    const size_t src = qoff + (size_t)(qs0 + row) * HD + col;
                    *reinterpret_cast<u32x4*>(&sQ[row * LD + col]) =
                        *reinterpret_cast<const u32x4*>(q + src);
                    *reinterpret_cast<u32x4*>(&sdO[row * LD + col]) =
                        *reinterpret_cast<const u32x4*>(dout + src);
                }
                if (tid < kBM) {
                    sLse[tid] = lse[(size_t)bh * N + qs0 + tid] * kLog2e - lw;
                } else if (tid < 2 * kBM) {
                    sD[tid - kBM] = Drow[(size_t)bh * N + qs0 + tid - kBM];
                }
                __syncthreads();

                // ---- S = Q K_w^T, dP = dO V_w^T   (rows = q, cols = keys)
                f32x16 s[2], dp[2];
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    s[qt] = f32x16{};
                    dp[qt] = f32x16{};
                    const bf16* qa = &sQ[(32 * qt + l32) * LD + 8 * hf];
                    const bf16* oa = &sdO[(32 * qt + l32) * LD + 8 * hf];
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        s[qt] = mfma32(*reinterpret_cast<const bf16x8*>(qa + 16 * ks), kf[ks], s[qt]);
                        dp[qt] = mfma32(*reinterpret_cast<const bf16x8*>(oa + 16 * ks), vf[ks], dp[qt]);
                    }
                }
                // ---- P' = w P and dS' = w dS, in the accumulator layout
                const bool need_mask = (CAUSAL && k0 + kBN - 1 > qs0) || (k0 + kBN > N);
                bf16x8 pa[4], da[4];
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    float pv[16], dv_[16];
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const int ql = 32 * qt + 8 * a + 4 * hf;
                        const f32x4 L4 = *reinterpret_cast<const f32x4*>(&sLse[ql]);
                        const f32x4 D4 = *reinterpret_cast<const f32x4*>(&sD[ql]);
#pragma unroll
                        for (int bb = 0; bb < 4; ++bb) {
                            const int r = 4 * a + bb;
                            float p = fast_exp2(s[qt][r] * scale_log2 - L4[bb]);
                            if (need_mask) {
                                const int qg = qs0 + ql + bb;
                                if (!key_ok || (CAUSAL && key > qg)) p = 0.f;
                            }
                            pv[r] = p;
                            dv_[r] = p * (dp[qt][r] - D4[bb]);
                        }
                    }
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        bf16x8 fp, fd;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            fp[e] = to_bf16(pv[8 * half + e]);
                            fd[e] = to_bf16(dv_[8 * half + e]);
                        }
                        pa[2 * qt + half] = fp;
                        da[2 * qt + half] = fd;
                    }
                    // dS^T to LDS: key row (32w + l32), 4 consecutive q per store
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        bf16x4 w4;
#pragma unroll
                        for (int bb = 0; bb < 4; ++bb) w4[bb] = to_bf16(dv_[4 * a + bb]);
                        *reinterpret_cast<bf16x4*>(
                            &sdsT[(32 * wave + l32) * LDT + 32 * qt + 8 * a + 4 * hf]) = w4;
                    }
                }
                // ---- dV_w += P'^T dO, dK_w += dS'^T Q   (B via transposing reads)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int rb = 16 * ks + 4 * hf + (j16 >> 2);
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const int col = 32 * dt + 16 * (G16 & 1) + 4 * (j16 & 3);
                        const bf16x8 bo = cat(lds_read_tr(&sdO[rb * LD + col]),
                                              lds_read_tr(&sdO[(rb + 8) * LD + col]));
                        acc_dv[dt] = mfma32(pa[ks], bo, acc_dv[dt]);
                        const bf16x8 bq = cat(lds_read_tr(&sQ[rb * LD + col]),
                                              lds_read_tr(&sQ[(rb + 8) * LD + col]));
                        acc_dk[dt] = mfma32(da[ks], bq, acc_dk[dt]);
                    }
                }
                __syncthreads();
                // ---- dQ tile = dS' K : A = dS' via transposing reads of dS^T
#pragma unroll
                for (int qq = 0; qq < QT_DQ; ++qq) {
                    const int qt = dq_qt0 + qq;
                    f32x16 acc = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < kBN / 16; ++ks) {
                        const int r0 = 16 * ks + 8 * hf + (j16 >> 2);
                        const int col = 32 * qt + 16 * (G16 & 1) + 4 * (j16 & 3);
                        const bf16x8 a = cat(lds_read_tr(&sdsT[r0 * LDT + col]),
                                             lds_read_tr(&sdsT[(r0 + 4) * LDT + col]));
                        acc = mfma32(a, ktf[ks], acc);
                    }
                    float* dst = dq_acc + qoff + (size_t)qs0 * HD + dq_d0 + l32;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int ql = 32 * qt + 8 * (r >> 2) + 4 * hf + (r & 3);
                        atomicAdd(dst + (size_t)ql * HD, acc[r]);
                    }
                }
                __syncthreads();
            }
        }
    }

    // ---- epilogue: dK = scale * acc, dV = acc, bf16
    const size_t out = kvoff;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kr = k0 + 32 * wave + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (kr < N) {
                const size_t o = out + (size_t)kr * HD + 32 * dt + l32;
                dk[o] = to_bf16(acc_dk[dt][r] * scale);
                dv[o] = to_bf16(acc_dv[dt][r]);
            }
        }
}

// Zero the fp32 dQ accumulator rows of kept blocks (one workgroup per block).
template <int HD, int BLK>
__global__ __launch_bounds__(256) void dq_zero_kernel(const float* __restrict__ block_w,
                                                      float* __restrict__ dq_acc) {
    const size_t blk = blockIdx.x;
    if (block_w[blk] == 0.f) return;
    f32x4* dst = reinterpret_cast<f32x4*>(dq_acc + blk * (size_t)(BLK * HD));
    for (int c = threadIdx.x; c < BLK * HD / 4; c += 256) dst[c] = f32x4{};
}

// dQ = scale * accumulator for kept blocks, exact zeros for skipped blocks.
template <int HD, int BLK>
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ block_w,
                                                         const float* __restrict__ dq_acc,
                                                         bf16* __restrict__ dq, float scale) {
    const size_t blk = blockIdx.x;
    const bool kept = block_w[blk] != 0.f;
    const f32x4* src = reinterpret_cast<const f32x4*>(dq_acc + blk * (size_t)(BLK * HD));
    bf16x4* dst = reinterpret_cast<bf16x4*>(dq + blk * (size_t)(BLK * HD));
    for (int c = threadIdx.x; c < BLK * HD / 4; c += 256) {
        bf16x4 o4 = bf16x4{};
        if (kept) {
            const f32x4 x = src[c];
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = to_bf16(x[e] * scale);
        }
        dst[c] = o4;
    }
}

// ---------------------------------------------------------------------------
// float32 path: plain loops, no workspace.
// dK/dV: one thread per key row; dQ: one thread per query row.
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(64) void bwd_f32_dkdv_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ lse, const float* __restrict__ dout, const float* __restrict__ Drow,
    const int32_t* __restrict__ kept_idx, const int32_t* __restrict__ kept_count,
    const float* __restrict__ block_w, float* __restrict__ dk, float* __restrict__ dv, int Hq,
    int Hkv, int N, int nqb, int blk, float scale, int causal) {
    const int bg = blockIdx.y;
    const int b = bg / Hkv, g = bg % Hkv, G = Hq / Hkv;
    const int jrow = blockIdx.x * 64 + threadIdx.x;
    if (jrow >= N) return;
    const float* kr = k + ((size_t)bg * N + jrow) * HD;
    const float* vr = v + ((size_t)bg * N + jrow) * HD;
    float kv[HD], vv[HD], ak[HD], av[HD];
#pragma unroll
    for (int c = 0; c < HD; ++c) { kv[c] = kr[c]; vv[c] = vr[c]; ak[c] = 0.f; av[c] = 0.f; }
    for (int hg = 0; hg < G; ++hg) {
        const int bh = b * Hq + g * G + hg;
        const int cnt = min(max(kept_count[bh], 0), nqb);
        for (int pos = 0; pos < cnt; ++pos) {
            const int i = kept_idx[(size_t)bh * nqb + pos];
            if ((unsigned)i >= (unsigned)nqb) continue;  // malformed list: skip
            const float w = block_w[(size_t)bh * nqb + i];
            for (int r = i * blk; r < (i + 1) * blk; ++r) {
                if (causal && r < jrow) continue;
                const float* qr = q + ((size_t)bh * N + r) * HD;
                const float* dr = dout + ((size_t)bh * N + r) * HD;
                float s = 0.f, dp = 0.f;
#pragma unroll
                for (int c = 0; c < HD; ++c) { s += qr[c] * kv[c]; dp += dr[c] * vv[c]; }
                const float p = w * expf(s * scale - lse[(size_t)bh * N + r]);
                const float ds = p * (dp - Drow[(size_t)bh * N + r]);
#pragma unroll
                for (int c = 0; c < HD; ++c) { av[c] += p * dr[c]; ak[c] += ds * qr[c]; }
            }
        }
    }
    float* okr = dk + ((size_t)bg * N + jrow) * HD;
    float* ovr = dv + ((size_t)bg * N + jrow) * HD;
#pragma unroll
    for (int c = 0; c < HD; ++c) { okr[c] = ak[c] * scale; ovr[c] = av[c]; }
}

template <int HD>
__global__ __launch_bounds__(64) void bwd_f32_dq_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ lse, const float* __restrict__ dout, const float* __restrict__ Drow,
    const float* __restrict__ block_w, float* __restrict__ dq, int Hq, int Hkv, int N, int nqb,
    int blk, float scale, int causal) {
    const int bh = blockIdx.y;
    const int b = bh / Hq, h = bh % Hq, g = h / (Hq / Hkv);
    const int row = blockIdx.x * 64 + threadIdx.x;
    if (row >= N) return;
    float* out = dq + ((size_t)bh * N + row) * HD;
    const float w = block_w[(size_t)bh * nqb + row / blk];
    if (w == 0.f) {
#pragma unroll
        for (int c = 0; c < HD; ++c) out[c] = 0.f;
        return;
    }
    const float* qr = q + ((size_t)bh * N + row) * HD;
    const float* dr = dout + ((size_t)bh * N + row) * HD;
    const float* kg = k + ((size_t)b * Hkv + g) * (size_t)N * HD;
    const float* vg = v + ((size_t)b * Hkv + g) * (size_t)N * HD;
    float qv[HD], dov[HD], acc[HD];
#pragma unroll
    for (int c = 0; c < HD; ++c) { qv[c] = qr[c]; dov[c] = dr[c]; acc[c] = 0.f; }
    const float L = lse[(size_t)bh * N + row], Dr = Drow[(size_t)bh * N + row];
    const int nk = causal ? row + 1 : N;
    for (int jj = 0; jj < nk; ++jj) {
        const float* kr = kg + (size_t)jj * HD;
        const float* vr = vg + (size_t)jj * HD;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < HD; ++c) { s += qv[c] * kr[c]; dp += dov[c] * vr[c]; }
        const float ds = w * expf(s * scale - L) * (dp - Dr);
#pragma unroll
        for (int c = 0; c < HD; ++c) acc[c] += ds * kr[c];
    }
#pragma unroll
    for (int c = 0; c < HD; ++c) out[c] = acc[c] * scale;
}

// ---------------------------------------------------------------------------
hipError_t launch_bwd(const Problem& pb, const void* q, const void* k, const void* v,
                      const float* lse, const void* dout, const float* D,
                      const int32_t* kept_idx, const int32_t* kept_count, const float* block_w,
                      void* dq, void* dk, void* dv, float* dq_acc, unsigned phases,
                      hipStream_t st) {
    const bool prep = phases & 1u, main = phases & 2u, fin = phases & 4u;
    if (!pb.bf16) {
        if (!main) return hipSuccess;
        dim3 gkv((unsigned)((pb.N + 63) / 64), (unsigned)(pb.B * pb.Hkv));
        dim3 gq((unsigned)((pb.N + 63) / 64), (unsigned)(pb.B * pb.Hq));
#define LF_F32BWD(DD)                                                                          \
    if (pb.d == DD) {                                                                          \
        hipLaunchKernelGGL(bwd_f32_dkdv_kernel<DD>, gkv, dim3(64), 0, st, (const float*)q,     \
                           (const float*)k, (const float*)v, lse, (const float*)dout, D,       \
                           kept_idx, kept_count, block_w, (float*)dk, (float*)dv, pb.Hq,       \
                           pb.Hkv, pb.N, pb.nqb, pb.block, pb.scale, pb.causal);               \
        hipLaunchKernelGGL(bwd_f32_dq_kernel<DD>, gq, dim3(64), 0, st, (const float*)q,        \
                           (const float*)k, (const float*)v, lse, (const float*)dout, D,       \
                           block_w, (float*)dq, pb.Hq, pb.Hkv, pb.N, pb.nqb, pb.block,         \
                           pb.scale, pb.causal);                                               \
        return hipGetLastError();                                                              \
    }
        LF_F32BWD(64)
        LF_F32BWD(128)
#undef LF_F32BWD
        return hipErrorInvalidValue;
    }
    const unsigned nblocks = (unsigned)((size_t)pb.B * pb.Hq * pb.nqb);
    const int nkt = (pb.N + kBN - 1) / kBN;
    const unsigned nwg = (unsigned)(pb.B * pb.Hkv * nkt);
    const float sl2 = pb.scale * kLog2e;
#define LF_BWD(DD, BB, CC)                                                                      \
    if (pb.d == DD && pb.block == BB && (pb.causal != 0) == CC) {                               \
        if (prep)                                                                               \
            hipLaunchKernelGGL((dq_zero_kernel<DD, BB>), dim3(nblocks), dim3(256), 0, st,       \
                               block_w, dq_acc);                                                \
        if (main)                                                                               \
            hipLaunchKernelGGL((bwd_bf16_kernel<DD, BB, CC>), dim3(nwg), dim3(256), 0, st,      \
                               (const bf16*)q, (const bf16*)k, (const bf16*)v, lse,             \
                               (const bf16*)dout, D, kept_idx, kept_count, block_w, (bf16*)dk,  \
                               (bf16*)dv, dq_acc, pb.B, pb.Hq, pb.Hkv, pb.N, pb.nqb, pb.scale,  \
                               sl2);                                                            \
        if (fin)                                                                                \
            hipLaunchKernelGGL((dq_convert_kernel<DD, BB>), dim3(nblocks), dim3(256), 0, st,    \
                               block_w, dq_acc, (bf16*)dq, pb.scale);                           \
        return hipGetLastError();                                                               \
    }
    LF_BWD(64, 64, true)
    LF_BWD(64, 64, false)
    LF_BWD(64, 128, true)
    LF_BWD(64, 128, false)
    LF_BWD(128, 64, true)
    LF_BWD(128, 64, false)
    LF_BWD(128, 128, true)
    LF_BWD(128, 128, false)
#undef LF_BWD
    return hipErrorInvalidValue;
}

}  // namespace lf
