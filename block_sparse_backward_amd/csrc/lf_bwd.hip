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
// w P, so dS and every product carry it for free.
//
// Two walks, both deterministic (no floating-point atomics; every sum is
// taken in a fixed order):
//
// dkdv_bf16_kernel -- one workgroup of 8 waves (two per SIMD) per (batch, kv
//   head, 128-key tile).  Waves w and w + 4 own keys 32 (w & 3) .. + 31 and keep
//   their K/V fragments in registers for the whole walk; wave w accumulates
//   dV of those keys, wave w + 4 dK.  The workgroup walks the kept blocks of
//   the Hq/Hkv query heads of its group in 64-row sub-tiles; of each, the dV
//   wave computes S = Q K_w^T and dP = dO V_w^T for rows 0..31, the dK wave for
//   rows 32..63 (32x32x16 bf16 MFMAs, A: LDS rows, B: registers; the dP
//   products start from -D).  Each turns its scores into P' and dS', keeps
//   the operand of its own accumulator and sends the other to its partner
//   through LDS, so dV_w += P'^T dO and dK_w += dS'^T Q each run over all 64
//   rows (A: P'/dS' in the score layout, B: transposing LDS reads).  One
//   barrier per sub-tile; the dV/dK products of sub-tile t-1 run alongside
//   the softmax of t, and the two waves of a SIMD fill each other's stalls.
//
// dQ: dq_plan_kernel -> dq_bf16_kernel -> dq_finalize_kernel.  The plan lists
//   the kept blocks longest first (causal blocks see more keys the later they
//   sit) and, when few blocks are kept, cuts long blocks into chunks of key
//   steps so the persistent walk is not bound by its longest item; zero-fill
//   items for the rows of skipped blocks follow.  Each workgroup of the walk
//   takes items from a queue; its waves own 32 query rows each and keep Q and
//   dO fragments, the LSE'/D row terms and the dQ accumulator in registers,
//   while two wave streams take the even and odd 64-key steps staged in
//   double-buffered LDS.  Scores are computed transposed, S^T = K Q^T and
//   dP^T = V dO^T, so dS^T in the accumulator layout is directly the A operand
//   of dQ += dS K; K^T comes from transposing LDS reads.  A one-chunk block
//   writes its dq rows; chunks write fp32 partials that the finalize pass adds
//   in chunk order.  The queue position is the only atomic.
#include <mutex>

#include "lf_common.h"
#include "lf_internal.h"
#include "lf_tile.h"

namespace lf {

constexpr int kBN = 128;  // keys per dK/dV workgroup
constexpr int kBM = 64;   // query rows per dK/dV sub-tile
constexpr int kQN = 64;   // keys per dQ step

// Workgroup -> (batch, kv group, key tile), key tiles in ascending order (the
// longest causal walks first).  Workgroups are dispatched round-robin over the
// 8 XCDs; a kv group stays on one XCD for kRotate consecutive key tiles (its
// kept Q/dO rows are then shared in that XCD's L2) and then moves on to the
// next XCD, so each XCD gets a share of every group: the groups' kept work
// differs, and a group pinned to one XCD would leave the others idle.
constexpr int kRotate = 8;
__device__ __forceinline__ void map_bwd_block(int bid, int B, int Hkv, int& b, int& g, int& j) {
    const int nG = B * Hkv;
    int gid;
    if (nG % kNumXcd == 0) {
        const int xcd = bid % kNumXcd, r = bid / kNumXcd;
        const int ngx = nG / kNumXcd;
        j = r / ngx;
        gid = (xcd + j / kRotate) % kNumXcd + kNumXcd * (r % ngx);
    } else {
        gid = bid % nG;
        j = bid / nG;
    }
    b = gid / Hkv;
    g = gid % Hkv;
}

// Walk over the work of one workgroup: the heads of its group, their kept
// blocks in ascending order, and the 64-row sub-tiles of each block that reach
// the workgroup's keys under the causal mask.  The walk position is uniform
// (scalar registers); the kept list is read 64 entries at a time into one
// vector register per wave (entry pos - cbase in lane pos - cbase) and looked
// up with v_readlane, so moving to the next sub-tile costs no memory round
// trip.  A head's count and first entries are requested together (one round
// trip); the block weights are not part of the walk (each sub-tile's weight is
// loaded with its rows).
template <int BLK, bool CAUSAL>
struct Walk {
    static_assert(kBN % BLK == 0 && BLK % kBM == 0, "key tiles start on block boundaries");
    const int32_t* kept_idx;
    const int32_t* kept_count;
    int Hq, nqb, G, b, g, k0, lane;
    int hg, cnt, pos, st, i, bh, cbase;
    int vidx;    // kept_idx[bh][cbase + lane]  (or a large sentinel past cnt)

    // entries c .. c + 63 of the current head's list (unmasked; clamped reads)
    __device__ __forceinline__ int chunk_raw(int c) const {
        return kept_idx[(size_t)bh * nqb + min(c + lane, nqb - 1)];
    }
    __device__ __forceinline__ void set_chunk(int c, int raw) {
        cbase = __builtin_amdgcn_readfirstlane(c);
        vidx = c + lane < cnt ? raw : 0x7fffffff;
    }
    __device__ __forceinline__ void load_chunk(int c) { set_chunk(c, chunk_raw(c)); }
    // makes head h of the group current (its list is then requested with
    // chunk_raw(0) and taken up by load_head)
    __device__ __forceinline__ void begin_head(int h) {
        hg = h;
        bh = b * Hq + g * G + hg;
    }
    // `raw` = chunk_raw(0) of the current head, requested before its count is
    // read, so the two round trips overlap; leaves pos at the first kept block
    // whose rows reach key k0 (all of them when not causal)
    __device__ __forceinline__ void load_head(int raw) {
        cnt = __builtin_amdgcn_readfirstlane(min(max(kept_count[bh], 0), nqb));
        st = 0;
        pos = cnt;
        const int first_block = CAUSAL ? k0 / BLK : 0;
        for (int c = 0; c < cnt; c += 64) {
            set_chunk(c, c == 0 ? raw : chunk_raw(c));
            const uint64_t m = __builtin_amdgcn_ballot_w64(vidx >= first_block);
            if (m) {
                pos = __builtin_amdgcn_readfirstlane(c + (int)__builtin_ctzll(m));
                break;
            }
        }
    }
    // advance until (hg, pos, st) names a valid sub-tile; false when none is left
    __device__ __forceinline__ bool settle() {
        while (true) {
            if (pos >= cnt) {
                if (hg + 1 >= G) return false;
                begin_head(hg + 1);
                load_head(chunk_raw(0));
                continue;
            }
            if (pos - cbase >= 64) load_chunk(pos & ~63);
            i = __builtin_amdgcn_readlane(vidx, pos - cbase);
            if ((unsigned)i >= (unsigned)nqb || st >= BLK / kBM) {  // malformed entry or block done
                ++pos;
                st = 0;
                continue;
            }
            if (CAUSAL && i * BLK + st * kBM + kBM - 1 < k0) {  // rows all before the keys
                ++st;
                continue;
            }
            return true;
        }
    }
    // the caller made head 0 current (begin_head(0)) and passes its
    // chunk_raw(0), requested ahead of other loads
    __device__ __forceinline__ bool first(int raw0) {
        load_head(raw0);
        return settle();
    }
    // Fast paths first: the next sub-tile of the same block, then the next
    // kept block of the register chunk.  Neither needs the causal test: the
    // key tile starts at a multiple of the block size, so every sub-tile of a
    // block at or after the first one reaching the keys reaches them too.
    __device__ __forceinline__ bool next() {
        if (++st < BLK / kBM) return true;
        const int np = pos + 1 - cbase;
        if (pos + 1 < cnt && np < 64) {
            const int ni = __builtin_amdgcn_readlane(vidx, np);
            if ((unsigned)ni < (unsigned)nqb) {
                pos += 1;
                st = 0;
                i = ni;
                return true;
            }
        }
        return settle();  // chunk, head or list end, or a malformed entry
    }
    __device__ __forceinline__ int q0() const { return i * BLK + st * kBM; }
};

// ---------------------------------------------------------------------------
// dQ phase (bf16): plan -> persistent walk -> finalize.
//
// The work of a kept block is its key steps (64 keys each) that the causal mask
// lets it see, so block lengths differ by up to nqb x.  With few kept blocks
// the longest block would set the run time, so when fewer than 2 * kDqGrid
// blocks are kept the plan cuts blocks into chunks of about equal length and
// the chunks' fp32 partials are added in a fixed order by the finalize pass
// (deterministic).  The persistent kernel takes items from a queue, longest
// blocks first.
// ---------------------------------------------------------------------------
constexpr int kDqGrid = 256;                 // persistent workgroups (one per CU)
constexpr int kDqChunkItems = 4 * kDqGrid;   // chunking aims at about this many chunks
constexpr int kDqMaxSlots = kDqChunkItems + 2 * kDqGrid;  // fp32 partial tiles, see dq_plan_kernel
constexpr int kDqMinChunk = 16;              // key steps per chunk, at least
constexpr int kDqChunkBelow = 2 * kDqGrid;   // chunk blocks when fewer are kept
constexpr int kDqZeroPer = 8;                // skipped blocks per zero-fill item
constexpr int kDqFinSplit = 4;               // finalize workgroups per chunked block

struct DqWorkspace {  // carved out of the caller's workspace
    int* ctrl;        // [0] items, [1] queue position, [2] chunked blocks
    int4* items;      // compute: {bh, block, first step | end step << 16, partial slot or -1}
                      // zero fill: {-1, first skipped-list entry, entries, 0}
    int2* blk;        // per (bh, block): {first slot or -1, chunks}
    int* skip;        // skipped blocks, (bh, block) in memory order
    int* chunked;     // blocks cut into chunks
    float* part;      // [kDqMaxSlots][BLK * HD]
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// compute items: one per kept block, or (chunking) at most 2 T / CL <= kDqMaxSlots
// chunks plus one per block; zero-fill items: one per kDqZeroPer skipped blocks
__host__ __device__ inline size_t dq_max_items(size_t nblocks) {
    return nblocks + (size_t)kDqMaxSlots + nblocks / kDqZeroPer + 1;
}

__host__ __device__ inline size_t dq_workspace_bytes(size_t nblocks, int blk, int hd) {
    return align256(64 * sizeof(int)) + align256(dq_max_items(nblocks) * sizeof(int4)) +
           align256(nblocks * sizeof(int2)) + align256(nblocks * sizeof(int)) +
           align256(kDqChunkBelow * sizeof(int)) + (size_t)kDqMaxSlots * blk * hd * sizeof(float);
}

__host__ __device__ inline DqWorkspace dq_workspace(void* base, size_t nblocks, int blk, int hd) {
    char* p = static_cast<char*>(base);
    DqWorkspace w;
    w.ctrl = reinterpret_cast<int*>(p);
    p += align256(64 * sizeof(int));
    w.items = reinterpret_cast<int4*>(p);
    p += align256(dq_max_items(nblocks) * sizeof(int4));
    w.blk = reinterpret_cast<int2*>(p);
    p += align256(nblocks * sizeof(int2));
    w.skip = reinterpret_cast<int*>(p);
    p += align256(nblocks * sizeof(int));
    w.chunked = reinterpret_cast<int*>(p);
    p += align256(kDqChunkBelow * sizeof(int));
    w.part = reinterpret_cast<float*>(p);
    (void)blk;
    (void)hd;
    return w;
}

// Block-wide exclusive scans of M ints per thread (NT threads) at once:
// x[m] becomes its exclusive prefix and total[m] the sum.  `sh` holds
// (NT / 64 + 1) M ints.
template <int NT, int M>
__device__ __forceinline__ void block_scan(int (&x)[M], int* sh, int (&total)[M]) {
    constexpr int NW = NT / 64, SP = NW + 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int inc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) inc[m] = x[m];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int y = __shfl_up(inc[m], off);
            if (lane >= off) inc[m] += y;
        }
    if (lane == 63)
#pragma unroll
        for (int m = 0; m < M; ++m) sh[SP * m + wave] = inc[m];
    __syncthreads();
    if (threadIdx.x < M) {
        int* q = sh + SP * threadIdx.x;
        int run = 0;
        for (int w = 0; w < NW; ++w) {
            const int t = q[w];
            q[w] = run;
            run += t;
        }
        q[NW] = run;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M; ++m) {
        total[m] = sh[SP * m + NW];
        x[m] = sh[SP * m + wave] + inc[m] - x[m];
    }
    __syncthreads();
}

// One workgroup of 1024 threads.  Entries e = 0 .. E-1 run over (block i
// descending, head bh ascending); an entry is kept when its block weight is
// non-zero.  Emits the items in that order and the per-block slot table.
// Chunk lengths never exceed this many key steps: chunking happens with fewer
// than kDqChunkBelow kept blocks of at most 8192 steps, cut into T / kDqChunkItems
// step pieces or longer.
constexpr int kDqMaxChunk = ((kDqChunkBelow - 1) * 8192 + kDqChunkItems - 1) / kDqChunkItems;

constexpr int kDqPlanLds = 16384;  // block weights the plan stages in LDS (64 KiB)
constexpr int kDqBucketInts = kDqMaxChunk + 1;
// The plan, run by one workgroup of NT threads.  LDS: `sw` (swcap floats; the
// weights are staged there when they fit), `bucket` (kDqBucketInts ints: chunk
// count, then next queue position, per length) and `sh` (3 (NT / 64 + 1) ints).
template <int BLK, int NT>
__device__ __forceinline__ void dq_plan_body(const float* __restrict__ block_w, int BHq, int nqb,
                                             int N, int causal, DqWorkspace ws, float* sw,
                                             int swcap, int* bucket, int* sh) {
    const int E = BHq * nqb;
    const int tid = threadIdx.x;
    // the passes below visit the weights in a strided order, four times: read
    // them once, coalesced, into LDS when they fit
    const bool staged = E <= swcap;
    if (staged) {
        for (int x = 4 * tid; x < E; x += 4 * NT) {
            if (x + 4 <= E && (E & 3) == 0) {
                *reinterpret_cast<f32x4*>(&sw[x]) = *reinterpret_cast<const f32x4*>(&block_w[x]);
            } else {
                for (int y = x; y < min(E, x + 4); ++y) sw[y] = block_w[y];
            }
        }
        __syncthreads();
    }
    // one copy of the plan per source of the weights, so each reads its own
    // address space (a choice between the two would read through flat loads)
    auto plan = [&](auto weight) __attribute__((always_inline)) {
        const int per = (E + NT - 1) / NT;
        const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
        const int nks = (N + kQN - 1) / kQN;  // key steps of a head (the last may be partial)
        auto steps = [&](int i) { return causal ? min((i * BLK + BLK - 1) / kQN + 1, nks) : nks; };
        auto entry = [&](int e, int& bh, int& i) {
            i = nqb - 1 - e / BHq;
            bh = e % BHq;
        };
        // pass 1: kept blocks K and their total key steps T
        int kc = 0, ts = 0;
        for (int e = e0; e < e1; ++e) {
            int bh, i;
            entry(e, bh, i);
            if (weight(bh * nqb + i) != 0.f) {
                ++kc;
                ts += steps(i);
            }
        }
        int kt2[2] = {kc, ts}, tot2[2];
        block_scan<NT>(kt2, sh, tot2);
        const int kpre = kt2[0], K = tot2[0], T = tot2[1];
        const bool chunking = K < kDqChunkBelow;
        const int CL = chunking ? max(kDqMinChunk, (T + kDqChunkItems - 1) / kDqChunkItems) : (1 << 30);
        // pass 2: compute items, partial slots and chunked blocks per thread
        int ni = 0, nsl = 0, nck = 0;
        for (int e = e0; e < e1; ++e) {
            int bh, i;
            entry(e, bh, i);
            if (weight(bh * nqb + i) != 0.f) {
                const int nch = (steps(i) + CL - 1) / CL;
                ni += nch;
                nsl += nch > 1 ? nch : 0;
                nck += nch > 1;
            }
        }
        int isc[3] = {ni, nsl, nck}, itot[3];
        block_scan<NT>(isc, sh, itot);
        int it = isc[0], sl = isc[1], ck = isc[2];
        const int n_items = itot[0], n_chunked = itot[2];
        if (chunking) {
            // Queue order longest first over all chunks (not block by block): a
            // counting sort by chunk length, so short remainders end the queue.
            for (int c = tid; c <= CL; c += NT) bucket[c] = 0;
            __syncthreads();
            for (int e = e0; e < e1; ++e) {
                int bh, i;
                entry(e, bh, i);
                if (weight(bh * nqb + i) != 0.f) {
                    const int L = steps(i);
                    const int nch = (L + CL - 1) / CL;
                    for (int c = 0; c < nch; ++c)
                        atomicAdd(&bucket[((c + 1) * L) / nch - (c * L) / nch], 1);
                }
            }
            __syncthreads();
            // exclusive prefix over lengths, longest first: bucket[len] = first
            // queue position of its chunks
            constexpr int PER = (kDqBucketInts + NT - 1) / NT;
            int cnt[PER], tot = 0;
    #pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int len = CL - (tid * PER + u);
                cnt[u] = len >= 1 ? bucket[len] : 0;
                tot += cnt[u];
            }
            int run1[1] = {tot}, all[1];
            block_scan<NT>(run1, sh, all);
            int run = run1[0];
    #pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int len = CL - (tid * PER + u);
                if (len >= 1) bucket[len] = run;
                run += cnt[u];
            }
            __syncthreads();
        }
        int sk = e0 - kpre;  // skipped blocks before this thread's entries
        for (int e = e0; e < e1; ++e) {
            int bh, i;
            entry(e, bh, i);
            const int blk = bh * nqb + i;
            int2 info = make_int2(-1, 0);
            if (weight(blk) != 0.f) {
                const int L = steps(i);
                const int nch = (L + CL - 1) / CL;
                info = make_int2(nch > 1 ? sl : -1, nch);
                for (int c = 0; c < nch; ++c) {
                    // equal chunks (lengths differ by at most one step)
                    const int s0 = (c * L) / nch, s1 = ((c + 1) * L) / nch;
                    const int at = chunking ? atomicAdd(&bucket[s1 - s0], 1) : it++;
                    ws.items[at] = make_int4(bh, i, s0 | (s1 << 16), nch > 1 ? sl + c : -1);
                }
                if (nch > 1) {
                    sl += nch;
                    ws.chunked[ck++] = blk;
                }
            } else {
                ws.skip[sk++] = blk;
            }
            ws.blk[blk] = info;
        }
        // zero-fill items go last: they take up the walk's tail
        const int n_skip = E - K;
        const int n_zero = (n_skip + kDqZeroPer - 1) / kDqZeroPer;
        for (int z = tid; z < n_zero; z += NT)
            ws.items[n_items + z] =
                make_int4(-1, z * kDqZeroPer, min(kDqZeroPer, n_skip - z * kDqZeroPer), 0);
        if (tid == 0) {
            ws.ctrl[0] = n_items + n_zero;
            ws.ctrl[1] = 0;
            ws.ctrl[2] = n_chunked;
        }
    };
    if (staged) plan([&](int blk) { return sw[blk]; });
    else plan([&](int blk) { return block_w[blk]; });
}

template <int BLK>
__global__ __launch_bounds__(1024) void dq_plan_kernel(const float* __restrict__ block_w, int BHq,
                                                       int nqb, int N, int causal, DqWorkspace ws) {
    __shared__ int sh[3 * 17];
    __shared__ int bucket[kDqBucketInts];
    __shared__ float sw[kDqPlanLds];
    dq_plan_body<BLK, 1024>(block_w, BHq, nqb, N, causal, ws, sw, kDqPlanLds, bucket, sh);
}

// Persistent dQ walk.  Each item is one kept block's key steps [s0, s1).  A
// workgroup has 4 waves of 32 query rows: for 128-row blocks one stream of 4
// waves takes every step (two workgroups per CU); for 64-row blocks two
// streams of 2 waves split the steps, even to stream 0 and odd to stream 1,
// and add their partials in LDS at the end.  The result goes to the dq rows
// (single-chunk block) or to the item's fp32 partial slot.  Each stream
// double-buffers its K/V tiles in two LDS arrays of its own, and the code of
// each stream and buffer names its arrays at compile time: loads to LDS into
// one array then never hold back the LDS reads of another (the compiler waits
// for a load to LDS before reading the same array).  The next step's loads go
// out among the current step's score MFMAs.  Steps run without branches: keys
// the causal mask hides, and a stream's missing last step, add exact zeros.
// dK/dV walk with two waves per SIMD: 8 waves per (batch, kv head, 128-key
// tile).  Waves w and w + 4 share keys 32 (w & 3) .. + 31 (their K/V
// fragments in registers); wave w < 4 accumulates dV of those keys and
// computes S, dP for rows 0..31 of each 64-row sub-tile, wave w + 4
// accumulates dK and computes rows 32..63.  Each sends its partner the
// operand the partner lacks (the dV wave its dS', the dK wave its P') through
// LDS, so each accumulator sees all 64 rows.  Per sub-tile t, between two
// barriers: S, dP(t) for the wave's rows; then dV or dK of t-1 (own operand
// for its rows, the partner's for the others; B: transposing reads of t-1's
// dO or Q) interleaved with the softmax of t; then the exchange.  Q and dO
// tiles arrive by loads straight to LDS into three named buffers (t-1, t,
// t+1), the loop unrolled by three so the compiler sees which array each
// load writes.  With PLAN, workgroup 0 instead runs the dQ plan (on this
// kernel's LDS) while the others walk, so the plan costs the walk one CU for
// its run time rather than a launch of its own.
template <int HD, int BLK, bool CAUSAL, bool PLAN>
__global__ __launch_bounds__(512, 1) void dkdv_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ lse, const bf16* __restrict__ dout, const float* __restrict__ Drow,
    const int32_t* __restrict__ kept_idx, const int32_t* __restrict__ kept_count,
    const float* __restrict__ block_w, bf16* __restrict__ dk, bf16* __restrict__ dv, int B, int Hq,
    int Hkv, int N, int nqb, float scale, float scale_log2, DqWorkspace ws) {
    constexpr int KS = HD / 16;     // k-steps over the head dim
    constexpr int DT = HD / 32;     // 32-wide head-dim tiles
    constexpr int TILE = kBM * HD;  // one staged Q or dO tile (swizzled)
    constexpr int NW = 8;
    __shared__ __attribute__((aligned(16))) bf16 sQ0[TILE];
    __shared__ __attribute__((aligned(16))) bf16 sO0[TILE];
    __shared__ __attribute__((aligned(16))) bf16 sQ1[TILE];
    __shared__ __attribute__((aligned(16))) bf16 sO1[TILE];
    __shared__ __attribute__((aligned(16))) bf16 sQ2[TILE];
    __shared__ __attribute__((aligned(16))) bf16 sO2[TILE];
    __shared__ __attribute__((aligned(16))) float sL[3][kBM];  // LSE' per buffer
    __shared__ __attribute__((aligned(16))) float sN[3][kBM];  // -D per buffer
    __shared__ __attribute__((aligned(16))) u32x4 sX[2][NW][2][64];  // [parity][sender][half][lane]

    if constexpr (PLAN) {
        static_assert(sizeof(sQ0) >= kDqBucketInts * sizeof(int), "plan buckets fit one tile");
        static_assert(sizeof(sL) >= 3 * (NW + 1) * sizeof(int), "plan scan space");
        if (blockIdx.x == 0) {
            dq_plan_body<BLK, NW * 64>(block_w, B * Hq, nqb, N, CAUSAL, ws,
                                       reinterpret_cast<float*>(&sX[0][0][0][0]),
                                       (int)(sizeof(sX) / sizeof(float)),
                                       reinterpret_cast<int*>(sQ0), &reinterpret_cast<int*>(sL)[0]);
            return;
        }
    }
    int b, g, j;
    map_bwd_block(blockIdx.x - (PLAN ? 1 : 0), B, Hkv, b, g, j);
    const int G = Hq / Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave & 3;
    const int l32 = lane & 31, hf = lane >> 5;
    const int k0 = j * kBN;
    const int key = k0 + 32 * kg + l32;  // key column held by this lane
    const bool key_ok = key < N;
    const size_t kvoff = ((size_t)b * Hkv + g) * (size_t)N * HD;
    const f32x16 zero16 = {};
    const TileOffsets<HD> off(lane);

    Walk<BLK, CAUSAL> W;
    W.kept_idx = kept_idx;
    W.kept_count = kept_count;
    W.lane = lane;
    W.Hq = Hq;
    W.nqb = nqb;
    W.G = G;
    W.b = b;
    W.g = g;
    W.k0 = k0;
    W.begin_head(0);
    // the walk's first request (count and first kept entries of the group's
    // first head) goes out before the K/V rows, so that waiting for it does
    // not wait for them; keys past N read as zeros (buffer bounds)
    const int raw0 = W.chunk_raw(0);
    bf16x8 kf[KS], vf[KS];
    {
        const uint32_t kv_bytes = (uint32_t)N * HD * sizeof(bf16);
        const auto rk = make_rsrc(k + kvoff, kv_bytes), rv = make_rsrc(v + kvoff, kv_bytes);
        const int r = key * HD * (int)sizeof(bf16);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int o = r + (16 * ks + 8 * hf) * (int)sizeof(bf16);
            kf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0));
            vf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, o, 0, 0));
        }
    }
    const bool has_work = W.first(raw0);

    float pld = 0.f, pw = 1.f;
    bool pld_ok = true;
    const uint32_t head_bytes = (uint32_t)N * HD * sizeof(bf16);
    // a sub-tile's Q and dO rows go straight to LDS; its LSE and D values to
    // one register (threads 0..63 LSE, the others D, each wave a copy)
    auto fetch = [&](int bh, int qs0, bf16* tq, bf16* to) __attribute__((always_inline)) {
        bh = __builtin_amdgcn_readfirstlane(bh);
        qs0 = __builtin_amdgcn_readfirstlane(qs0);
        const size_t hoff = (size_t)bh * N * HD;
        const int soff = qs0 * HD * (int)sizeof(bf16);
        load_tile_to_lds<HD, kBM, NW>(make_rsrc(q + hoff, head_bytes), soff, tq, wave, lane);
        load_tile_to_lds<HD, kBM, NW>(make_rsrc(dout + hoff, head_bytes), soff, to, wave, lane);
        const int row = qs0 + (tid & (kBM - 1));
        pld_ok = row < N;
        pld = (tid < kBM ? lse : Drow)[(size_t)bh * N + (pld_ok ? row : N - 1)];
        pw = block_w[(size_t)bh * nqb + qs0 / BLK];
    };
    // LSE' = LSE log2 e - log2 w and -D (the start of the dP products); rows
    // past N get LSE' = +inf (P = 0) and D = 0
    auto stage_rows = [&](float* sl, float* sn) __attribute__((always_inline)) {
        if (tid < kBM) sl[tid] = pld_ok ? pld * kLog2e - __log2f(pw) : __builtin_inf();
        else if (tid < 2 * kBM) sn[tid - kBM] = pld_ok ? -pld : 0.f;
    };
    // Zero packed P', dS' of the wave's rows (32 R + 8 (r >> 2) + 4 hf + (r & 3))
    // where the mask hides the pair: kept iff 32 R + 8 (r >> 2) + (r & 3) >= thr
    auto mask_pairs = [&](int R, int thr, bf16x8 (&pa)[2], bf16x8 (&da)[2])
                          __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            u32x4 wp = __builtin_bit_cast(u32x4, pa[h]), wd = __builtin_bit_cast(u32x4, da[h]);
            asm volatile("" : "+v"(wp), "+v"(wd));  // keeps the work behind the branch
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int r = 8 * h + 2 * w, row = 32 * R + 8 * (r >> 2) + (r & 3);
                const uint32_t keep = (row >= thr ? 0xffffu : 0u) | (row + 1 >= thr ? 0xffff0000u : 0u);
                wp[w] &= keep;
                wd[w] &= keep;
            }
            pa[h] = __builtin_bit_cast(bf16x8, wp);
            da[h] = __builtin_bit_cast(bf16x8, wd);
        }
    };

    // The walk of one role (R = 0: dV, rows 0..31; R = 1: dK, rows 32..63).
    auto walk = [&](auto RC) __attribute__((always_inline)) {
        constexpr int R = decltype(RC)::value;
        f32x16 acc[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16;
        if (has_work) {
            int cur_bh = W.bh, cur_q0 = W.q0();
            fetch(cur_bh, cur_q0, sQ0, sO0);
            {   // the "previous" sub-tile of the first one: zero rows, zero
                // exchanged operands, so its dV/dK products add exact zeros
                u32x4* zq = reinterpret_cast<u32x4*>(sQ2);
                u32x4* zo = reinterpret_cast<u32x4*>(sO2);
                for (int c = tid; c < TILE / 8; c += NW * 64) { zq[c] = u32x4{}; zo[c] = u32x4{}; }
                u32x4* zx = &sX[1][0][0][0];
                for (int c = tid; c < NW * 2 * 64; c += NW * 64) zx[c] = u32x4{};
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            stage_rows(sL[0], sN[0]);
            __syncthreads();

            constexpr int NMF = 4 * DT;                 // dV or dK MFMAs per sub-tile
            constexpr int EPC = (16 + NMF - 1) / NMF;   // softmax elements per chunk
            constexpr int kAhead = 3;
            bf16x8 own[2] = {};  // this wave's operand of the previous sub-tile
            int par = 0;         // exchange buffer written by this sub-tile
            auto iter = [&](const bf16* cq, const bf16* co, const float* cl, const float* cn,
                            const bf16* pq, const bf16* po, bf16* nq, bf16* no, float* nl,
                            float* nn) __attribute__((always_inline)) -> bool {
                const bool more = W.next();
                // the next sub-tile (this one again after the last: a harmless
                // reload keeps the iteration free of branches)
                const int nx_bh = more ? W.bh : cur_bh;
                const int nx_q0 = more ? W.q0() : cur_q0;
                const int thr = !key_ok ? (1 << 30) : (CAUSAL ? key - cur_q0 - 4 * hf : -(1 << 30));
                const bool wave_masked = __builtin_amdgcn_readfirstlane(
                    (int)(k0 + 32 * kg + 31 >= N || (CAUSAL && cur_q0 + 32 * R < k0 + 32 * kg + 31)));
                fetch(nx_bh, nx_q0, nq, no);

                // S = Q K_w^T and dP - D for this wave's 32 rows of sub-tile t
                f32x16 s, dp;
                {
                    bf16x8 aq[KS], ao[KS];
                    f32x16 nd;
#pragma unroll
                    for (int a2 = 0; a2 < 4; ++a2) {
                        const f32x4 x = *reinterpret_cast<const f32x4*>(cn + 32 * R + 8 * a2 + 4 * hf);
#pragma unroll
                        for (int e = 0; e < 4; ++e) nd[4 * a2 + e] = x[e];
                    }
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        aq[ks] = frag_at<HD>(cq, 32 * R, off.frag[ks]);
                        ao[ks] = frag_at<HD>(co, 32 * R, off.frag[ks]);
                    }
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        s = mfma32(aq[ks], kf[ks], ks ? s : zero16);
                        dp = mfma32(ao[ks], vf[ks], ks ? dp : nd);
                    }
                    pipeline_schedule<2 * KS + 4, 2 * KS, 1, 12>();
                    __builtin_amdgcn_sched_barrier(0);
                }

                // dV (R = 0: P'^T dO) or dK (R = 1: dS'^T Q) of sub-tile t-1 over
                // its 64 rows, with the softmax of t: MFMA m covers row tile qm
                // (own rows first), 16-row half hm, head-dim tile dm
                const bf16* tb = R ? pq : po;
                bf16x8 prt[2];  // the partner's operand, read shortly before its MFMAs
                auto bfrag = [&](int m) __attribute__((always_inline)) {
                    const int qm = m < 2 * DT ? R : 1 - R, hm = (m / DT) & 1, dm = m % DT;
                    return tr_at<HD>(tb, 32 * qm + 16 * hm, off.tr[dm]);
                };
                bf16x8 bfr[NMF];
                f32x4 L4[4];
                float pv[16], dsv[16];
                bf16x8 pa[2], da[2];
#pragma unroll
                for (int a2 = 0; a2 < 2; ++a2)
                    L4[a2] = *reinterpret_cast<const f32x4*>(cl + 32 * R + 8 * a2 + 4 * hf);
#pragma unroll
                for (int m = 0; m < kAhead; ++m) bfr[m] = bfrag(m);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int m = 0; m < NMF; ++m) {
                    if (m + kAhead < NMF) bfr[m + kAhead] = bfrag(m + kAhead);
                    if (m == 2 * DT - 2) {
#pragma unroll
                        for (int h = 0; h < 2; ++h)
                            prt[h] = __builtin_bit_cast(bf16x8, sX[par ^ 1][wave ^ 4][h][lane]);
                    }
                    if ((m * EPC) % 4 == 0 && (m * EPC) / 4 + 2 < 4) {
                        const int a2 = (m * EPC) / 4 + 2;
                        L4[a2] = *reinterpret_cast<const f32x4*>(cl + 32 * R + 8 * a2 + 4 * hf);
                    }
                    const int hm = (m / DT) & 1, dm = m % DT;
                    acc[dm] = mfma32(m < 2 * DT ? own[hm] : prt[hm], bfr[m], acc[dm]);
#pragma unroll
                    for (int e = 0; e < EPC; ++e) {
                        const int r = m * EPC + e;
                        if (r < 16) {
                            const int a2 = r >> 2, bb = r & 3;
                            const float p = fast_exp2(s[r] * scale_log2 - L4[a2][bb]);
                            pv[r] = p;
                            dsv[r] = p * dp[r];
                            if (r & 1) {
                                pa[r >> 3][(r & 7) - 1] = to_bf16(pv[r - 1]);
                                pa[r >> 3][r & 7] = to_bf16(pv[r]);
                                da[r >> 3][(r & 7) - 1] = to_bf16(dsv[r - 1]);
                                da[r >> 3][r & 7] = to_bf16(dsv[r]);
                            }
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                asm volatile("" : "+v"(pa[0]), "+v"(pa[1]), "+v"(da[0]), "+v"(da[1]));
                if (wave_masked) mask_pairs(R, thr, pa, da);
                // the partner gets the operand it lacks, this wave keeps its own
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    sX[par][wave][h][lane] = __builtin_bit_cast(u32x4, R ? pa[h] : da[h]);
                    own[h] = R ? da[h] : pa[h];
                }
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                stage_rows(nl, nn);
                __syncthreads();
                par ^= 1;
                cur_bh = nx_bh;
                cur_q0 = nx_q0;
                return more;
            };
            int last;
            while (true) {
                if (!iter(sQ0, sO0, sL[0], sN[0], sQ2, sO2, sQ1, sO1, sL[1], sN[1])) { last = 0; break; }
                if (!iter(sQ1, sO1, sL[1], sN[1], sQ0, sO0, sQ2, sO2, sL[2], sN[2])) { last = 1; break; }
                if (!iter(sQ2, sO2, sL[2], sN[2], sQ1, sO1, sQ0, sO0, sL[0], sN[0])) { last = 2; break; }
            }
            // dV or dK of the last sub-tile
            {
                const bf16* lq = last == 0 ? sQ0 : last == 1 ? sQ1 : sQ2;
                const bf16* lo = last == 0 ? sO0 : last == 1 ? sO1 : sO2;
                const bf16* tb = R ? lq : lo;
                bf16x8 prt[2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    prt[h] = __builtin_bit_cast(bf16x8, sX[par ^ 1][wave ^ 4][h][lane]);
#pragma unroll
                for (int m = 0; m < NMF; ++m) {
                    const int qm = m < 2 * DT ? R : 1 - R, hm = (m / DT) & 1, dm = m % DT;
                    acc[dm] = mfma32(m < 2 * DT ? own[hm] : prt[hm],
                                     tr_at<HD>(tb, 32 * qm + 16 * hm, off.tr[dm]), acc[dm]);
                }
            }
        }
        // The accumulators leave through LDS, so that each lane stores 16
        // contiguous bytes: the role's 128 keys x HD go to two staging tiles
        // (dV: sQ0, sO0; dK: sQ1, sO1; keys 64 t .. 64 t + 63 in tile t), in the
        // swizzled layout of the walk's tiles, once every wave is done with them.
        __syncthreads();
        {
            bf16* stg = R ? (kg < 2 ? sQ1 : sO1) : (kg < 2 ? sQ0 : sO0);
            const float sc = R ? scale : 1.f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * (kg & 1) + 8 * (r >> 2) + 4 * hf + (r & 3);
                    const int col = 32 * dt + l32;
                    stg[row * HD + (((col >> 3) ^ swz<HD>(row)) << 3) + (col & 7)] =
                        to_bf16(acc[dt][r] * sc);
                }
        }
        __syncthreads();
        {
            constexpr int CPR = HD / 8;                   // 16-byte chunks per row
            constexpr int NCH = 2 * kBM * CPR / 256;      // chunks per thread of the role
            const bf16* t0 = R ? sQ1 : sQ0;
            const bf16* t1 = R ? sO1 : sO0;
            bf16* out = R ? dk : dv;
            const int rt = tid & 255;
#pragma unroll
            for (int m = 0; m < NCH; ++m) {
                const int c = rt + 256 * m;
                const int t = c / (kBM * CPR), row = (c / CPR) % kBM, cc = c % CPR;
                const bf16* tile = t ? t1 : t0;
                const u32x4 x = *reinterpret_cast<const u32x4*>(
                    tile + row * HD + ((cc ^ swz<HD>(row)) << 3));
                const int kr = k0 + kBM * t + row;
                if (kr < N)
                    *reinterpret_cast<u32x4*>(out + kvoff + (size_t)kr * HD + 8 * cc) = x;
            }
        }
    };
    if (wave >= 4) walk(IntC<1>{});
    else walk(IntC<0>{});
}

template <int BLK>
struct DqShape {
    static constexpr int NS = BLK >= 128 ? 1 : 2;  // streams per workgroup
    static constexpr int NW = BLK / 32;            // waves per stream
    static constexpr int NT = NS * NW * 64;        // threads per workgroup
    static constexpr int PER_CU = NS == 1 ? 2 : 1; // workgroups per CU
};

template <int HD, int BLK, bool CAUSAL>
__global__ __launch_bounds__(DqShape<BLK>::NT, 2) void dq_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ lse, const bf16* __restrict__ dout, const float* __restrict__ Drow,
    const float* __restrict__ block_w, bf16* __restrict__ dq, DqWorkspace ws, int B, int Hq,
    int Hkv, int N, int nqb, float scale, float scale_log2) {
    constexpr int NS = DqShape<BLK>::NS, NW = DqShape<BLK>::NW, NT = DqShape<BLK>::NT;
    static_assert(NT == 256, "four waves per workgroup");
    constexpr int KS = HD / 16;
    constexpr int DT = HD / 32;
    constexpr int TILE = kQN * HD;  // one staged K or V tile (swizzled)
    // a stream's fp32 partial (NW waves x 32 rows x HD) fits in its two buffers
    static_assert(NW * 32 * HD * sizeof(float) <= 2 * 2 * TILE * sizeof(bf16), "epilogue space");
    __shared__ __attribute__((aligned(16))) bf16 sA0[2 * TILE];  // stream 0: K | V, buffer 0
    __shared__ __attribute__((aligned(16))) bf16 sA1[2 * TILE];  // stream 0, buffer 1
    __shared__ __attribute__((aligned(16))) bf16 sB0[NS == 2 ? 2 * TILE : 8];  // stream 1, buffer 0
    __shared__ __attribute__((aligned(16))) bf16 sB1[NS == 2 ? 2 * TILE : 8];  // stream 1, buffer 1
    __shared__ int s_item;

    const int tid = threadIdx.x, lane = tid & 63, wave_all = tid >> 6;
    const int stream = wave_all / NW, wave = wave_all % NW;
    const int l32 = lane & 31, hf = lane >> 5;
    const f32x16 zero16 = {};
    const TileOffsets<HD> off(lane);
    const int n_items = __builtin_amdgcn_readfirstlane(ws.ctrl[0]);
    const int G = Hq / Hkv;

    while (true) {
        if (tid == 0) s_item = atomicAdd(&ws.ctrl[1], 1);
        __syncthreads();
        const int t_item = __builtin_amdgcn_readfirstlane(s_item);
        __syncthreads();
        if (t_item >= n_items) break;
        // the item is wave-uniform: keep it in scalar registers
        const int4 item = ws.items[t_item];
        if (__builtin_amdgcn_readfirstlane(item.x) < 0) {  // zero-fill skipped blocks
            const int z0 = __builtin_amdgcn_readfirstlane(item.y);
            const int zn = __builtin_amdgcn_readfirstlane(item.z);
            for (int zz = 0; zz < zn; ++zz) {
                const int blk = __builtin_amdgcn_readfirstlane(ws.skip[z0 + zz]);
                const int zbh = blk / nqb, zr0 = (blk % nqb) * BLK;
                u32x4* dst = reinterpret_cast<u32x4*>(dq + ((size_t)zbh * N + zr0) * HD);
                if (zr0 + BLK <= N) {
#pragma unroll
                    for (int c = 0; c < BLK * HD / 8 / NT; ++c) dst[c * NT + tid] = u32x4{};
                } else {  // a partial last block: rows past N stay untouched
                    for (int c = tid; c < (N - zr0) * HD / 8; c += NT) dst[c] = u32x4{};
                }
            }
            continue;
        }
        const int bh = __builtin_amdgcn_readfirstlane(item.x);
        const int i = __builtin_amdgcn_readfirstlane(item.y);
        const int st0 = __builtin_amdgcn_readfirstlane(item.z & 0xffff);
        const int st1 = __builtin_amdgcn_readfirstlane(item.z >> 16);
        const int slot = __builtin_amdgcn_readfirstlane(item.w);
        const int b = bh / Hq, g = (bh % Hq) / G;
        const size_t qoff = (size_t)bh * N * HD;
        const float lw = __log2f(block_w[(size_t)bh * nqb + i]);
        const int qrow = i * BLK + 32 * wave + l32;  // query column held by this lane
        // a row past N (the last block may be partial) reads row N - 1 and then
        // gets zero fragments, LSE' = +inf (P = 0) and D = 0: it adds nothing
        const bool row_ok = qrow < N;
        const int qr = row_ok ? qrow : N - 1;

        // Q^T and dO^T fragments (B operands): column = query, k = head dim
        bf16x8 qf[KS], of[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qf[ks] = *reinterpret_cast<const bf16x8*>(q + qoff + (size_t)qr * HD + 16 * ks + 8 * hf);
            of[ks] = *reinterpret_cast<const bf16x8*>(dout + qoff + (size_t)qr * HD + 16 * ks + 8 * hf);
            if (!row_ok) { qf[ks] = bf16x8{}; of[ks] = bf16x8{}; }
        }
        const float lse_l = row_ok ? lse[(size_t)bh * N + qr] * kLog2e - lw : __builtin_inf();
        const float d_l = row_ok ? Drow[(size_t)bh * N + qr] : 0.f;

        f32x16 acc[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16;

        const size_t kvoff = ((size_t)b * Hkv + g) * (size_t)N * HD;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + kvoff, (uint32_t)N * HD * sizeof(bf16));
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + kvoff, (uint32_t)N * HD * sizeof(bf16));
        const int nkt = st1 - st0;
        const int nit = (nkt + NS - 1) / NS;  // iterations: step NS t + stream

        auto walk = [&](auto SC, bf16* buf0, bf16* buf1) {
            constexpr int S = decltype(SC)::value;
            // the K and V tiles of iteration t (a step past the end reloads the last)
            auto fetch = [&](int t, bf16* dst) {
                const int kt = min(NS * t + S, nkt - 1);
                const int soff = (st0 + kt) * kQN * HD * (int)sizeof(bf16);
                load_tile_to_lds<HD, kQN, NW>(rk, soff, dst, wave, lane);
                load_tile_to_lds<HD, kQN, NW>(rv, soff, dst + TILE, wave, lane);
            };
            auto step = [&](int t, const bf16* sk, bf16* nxt) {
                const int kt = NS * t + S;
                const int k0 = (st0 + kt) * kQN;
                // key kk of this lane's query is kept iff kk <= lim; only a step
                // on the causal diagonal (or a stream's missing last step) hides
                // pairs of this wave, and only then are they zeroed
                const int lim = kt < nkt ? (CAUSAL ? qrow : 0x7fffffff) : -1;
                const bool step_masked = __builtin_amdgcn_readfirstlane(
                    (int)(kt >= nkt || (CAUSAL && k0 + kQN - 1 > i * BLK + 32 * wave)));
                const bf16* sv = sk + TILE;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {  // 32-key halves of the step
                    f32x16 s, dp;
                    {
                        if (mt == 0) fetch(t + 1, nxt);  // issued among the MFMAs below
                        bf16x8 ak[KS], av[KS];
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) {
                            ak[ks] = frag_at<HD>(sk, 32 * mt, off.frag[ks]);
                            av[ks] = frag_at<HD>(sv, 32 * mt, off.frag[ks]);
                        }
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) {
                            s = mfma32(ak[ks], qf[ks], ks ? s : zero16);
                            dp = mfma32(av[ks], of[ks], ks ? dp : zero16);
                        }
                        if (mt == 0) pipeline_schedule_vmem<2 * KS, 2 * KS, 1, 6, 2 * TILE / (64 * 8 * NW)>();
                        else pipeline_schedule<2 * KS, 2 * KS, 1, 6>();
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    // dS'^T = P' (dP - D) in the accumulator layout (row = key, col = query)
                    bf16x8 da[2];
                    {
                        float dsv[16];
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float p = fast_exp2(s[r] * scale_log2 - lse_l);
                            dsv[r] = p * (dp[r] - d_l);
                        }
#pragma unroll
                        for (int half = 0; half < 2; ++half) {
                            bf16x8 fd;
#pragma unroll
                            for (int e = 0; e < 8; ++e) fd[e] = to_bf16(dsv[8 * half + e]);
                            da[half] = fd;
                        }
                        if (step_masked) {  // zero the packed dS' of hidden pairs
#pragma unroll
                            for (int half = 0; half < 2; ++half) {
                                u32x4 w = __builtin_bit_cast(u32x4, da[half]);
                                asm volatile("" : "+v"(w));  // keeps the work behind the branch
#pragma unroll
                                for (int c = 0; c < 4; ++c) {
                                    const int r = 8 * half + 2 * c;
                                    const int kk = k0 + 32 * mt + 8 * (r >> 2) + 4 * hf + (r & 3);
                                    w[c] &= (kk <= lim ? 0xffffu : 0u) | (kk + 1 <= lim ? 0xffff0000u : 0u);
                                }
                                da[half] = __builtin_bit_cast(bf16x8, w);
                            }
                        }
                    }
                    // dQ += dS' K over these 32 keys; K^T fragments by transposing reads
                    {
                        bf16x8 kb[2][DT];
#pragma unroll
                        for (int half = 0; half < 2; ++half)
#pragma unroll
                            for (int dt = 0; dt < DT; ++dt)
                                kb[half][dt] = tr_at<HD>(sk, 32 * mt + 16 * half, off.tr[dt]);
#pragma unroll
                        for (int half = 0; half < 2; ++half)
#pragma unroll
                            for (int dt = 0; dt < DT; ++dt)
                                acc[dt] = mfma32(da[half], kb[half][dt], acc[dt]);
                        pipeline_schedule<4 * DT, 2 * DT, 2, 4>();
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
            };
            fetch(0, buf0);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            for (int t = 0; t < nit; t += 2) {
                step(t, buf0, buf1);
                if (t + 1 < nit) step(t + 1, buf1, buf0);
            }
        };
        if constexpr (NS == 1) {
            walk(IntC<0>{}, sA0, sA1);
        } else {
            if (stream == 0) walk(IntC<0>{}, sA0, sA1);
            else walk(IntC<1>{}, sB0, sB1);
        }

        constexpr int WREG = 32 * HD;                     // floats per wave region
        constexpr int WPB = (2 * TILE * 2) / (WREG * 4);  // wave regions per buffer
        if constexpr (NS == 2) {
            // stream 1 hands its partial to stream 0 through its own two buffers
            // (lane-major, 16 floats per C tile, one region per wave)
            float* xr = reinterpret_cast<float*>(wave / WPB ? sB1 : sB0) + (wave % WPB) * WREG;
            if (stream == 1) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) xr[(dt * 16 + r) * 64 + lane] = acc[dt][r];
            }
            __syncthreads();
            if (stream == 0) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[dt][r] += xr[(dt * 16 + r) * 64 + lane];
            }
        }
        // stream 0 scales and stages the result row-major in its buffers for
        // 16-byte writes by every thread
        const int row0 = 4 * hf;  // plus 8 (r >> 2) + (r & 3) within the wave's 32 rows
        if (stream == 0) {
            if (slot < 0) {  // bf16 rows: all NW waves' rows fit in sA0
                bf16* ob = sA0 + (32 * wave + row0) * HD + l32;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        ob[(8 * (r >> 2) + (r & 3)) * HD + 32 * dt] = to_bf16(acc[dt][r] * scale);
            } else {  // fp32 rows: WPB waves per buffer
                float* of32 = reinterpret_cast<float*>(wave / WPB ? sA1 : sA0) +
                              ((wave % WPB) * 32 + row0) * HD + l32;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        of32[(8 * (r >> 2) + (r & 3)) * HD + 32 * dt] = acc[dt][r] * scale;
            }
        }
        __syncthreads();
        if (slot < 0) {
            bf16* dq_rows = dq + qoff + (size_t)i * BLK * HD;
            const int nrow = min(BLK, N - i * BLK);  // rows of the block that exist
            if (nrow == BLK) {
#pragma unroll
                for (int c = 0; c < BLK * HD / 8 / NT; ++c)
                    reinterpret_cast<u32x4*>(dq_rows)[c * NT + tid] =
                        reinterpret_cast<const u32x4*>(sA0)[c * NT + tid];
            } else {
                for (int c = tid; c < nrow * HD / 8; c += NT)
                    reinterpret_cast<u32x4*>(dq_rows)[c] = reinterpret_cast<const u32x4*>(sA0)[c];
            }
        } else {
            float* part = ws.part + (size_t)slot * BLK * HD;
            constexpr int PB = WPB * WREG / 4;  // 16-byte pieces per buffer
            for (int c = tid; c < BLK * HD / 4; c += NT)
                reinterpret_cast<f32x4*>(part)[c] =
                    reinterpret_cast<const f32x4*>(c < PB ? sA0 : sA1)[c < PB ? c : c - PB];
        }
        __syncthreads();  // the staging buffers are reused by the next item
    }
}

// dq rows of the blocks cut into chunks: the in-order sum of their chunk
// partials (every other block's rows were written by the walk).  Workgroup
// kDqFinSplit c + h does part h of the rows of chunked block c; the grid covers
// the most chunked blocks the plan can list.
template <int HD, int BLK>
__global__ __launch_bounds__(256) void dq_finalize_kernel(DqWorkspace ws, bf16* __restrict__ dq,
                                                          int N, int nqb) {
    const int c = blockIdx.x / kDqFinSplit, h = blockIdx.x % kDqFinSplit;
    if (c >= ws.ctrl[2]) return;
    const int e = ws.chunked[c];
    const int2 info = ws.blk[e];
    constexpr int NV = BLK * HD / 8 / kDqFinSplit;  // 8-element pieces of this workgroup
    const int r0 = (e % nqb) * BLK;
    // pieces of rows past N (a partial last block) are not written
    const int nv = min(NV, max(0, (min(BLK, N - r0) * HD / 8) - h * NV));
    bf16x8* out = reinterpret_cast<bf16x8*>(dq + ((size_t)(e / nqb) * N + r0) * HD) + h * NV;
    const f32x4* p0 = reinterpret_cast<const f32x4*>(ws.part + (size_t)info.x * BLK * HD) + 2 * h * NV;
    constexpr size_t PS = (size_t)BLK * HD / 4;  // f32x4 per partial
    for (int v = threadIdx.x; v < nv; v += 256) {
        f32x4 s0 = p0[2 * v], s1 = p0[2 * v + 1];
        for (int j = 1; j < info.y; ++j) {
            s0 += p0[j * PS + 2 * v];
            s1 += p0[j * PS + 2 * v + 1];
        }
        bf16x8 o;
#pragma unroll
        for (int z = 0; z < 4; ++z) {
            o[z] = to_bf16(s0[z]);
            o[4 + z] = to_bf16(s1[z]);
        }
        out[v] = o;
    }
}

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
            for (int r = i * blk; r < min((i + 1) * blk, N); ++r) {
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
// Static scratch, for callers that cannot allocate: the dQ phase's workspace
// in a file-scope device array of fixed size.  Every GPU the library runs on
// holds its own copy at its own address until the process ends.  On the host
// the array's name is only a stand-in for the symbol: its device address is
// looked up once per device, with that device current, and only that address
// is ever passed to kernels.  The workspace needs no clearing (the dQ plan
// writes every word the walk and the finalize read), and every call on one
// GPU shares its array, so calls that overlap on one GPU race.
constexpr size_t kStaticScratchBytes = size_t(128) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's scratch address, looked up on first use.
hipError_t static_scratch(int device, void** ptr) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != device) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        g_scratch_ptr[device] = p;
    }
    *ptr = g_scratch_ptr[device];
    return hipSuccess;
}
}  // namespace

size_t static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t launch_bwd_static(const Problem& pb, const void* q, const void* k, const void* v,
                             const float* lse, const void* dout, const float* D,
                             const int32_t* kept_idx, const int32_t* kept_count,
                             const float* block_w, void* dq, void* dk, void* dv, hipStream_t st) {
    int device = 0;
    hipError_t e = hipStreamGetDevice(st, &device);  // the stream's GPU (NULL: the current one)
    if (e != hipSuccess) return e;
    void* ws = nullptr;
    if ((e = static_scratch(device, &ws)) != hipSuccess) return e;
    return launch_bwd(pb, q, k, v, lse, dout, D, kept_idx, kept_count, block_w, dq, dk, dv, ws,
                      1u | 2u, st);
}

size_t bwd_workspace_bytes(const Problem& pb) {
    if (!pb.bf16) return 0;
    return dq_workspace_bytes((size_t)pb.B * pb.Hq * pb.nqb, pb.block, pb.d);
}

hipError_t launch_bwd(const Problem& pb, const void* q, const void* k, const void* v,
                      const float* lse, const void* dout, const float* D,
                      const int32_t* kept_idx, const int32_t* kept_count, const float* block_w,
                      void* dq, void* dk, void* dv, void* workspace, unsigned phases,
                      hipStream_t st) {
    const bool do_kv = phases & 1u, do_q = phases & 2u;
    if (!pb.bf16) {
        dim3 gkv((unsigned)((pb.N + 63) / 64), (unsigned)(pb.B * pb.Hkv));
        dim3 gq((unsigned)((pb.N + 63) / 64), (unsigned)(pb.B * pb.Hq));
#define LF_F32BWD(DD)                                                                          \
    if (pb.d == DD) {                                                                          \
        if (do_kv)                                                                             \
            hipLaunchKernelGGL(bwd_f32_dkdv_kernel<DD>, gkv, dim3(64), 0, st, (const float*)q, \
                               (const float*)k, (const float*)v, lse, (const float*)dout, D,   \
                               kept_idx, kept_count, block_w, (float*)dk, (float*)dv, pb.Hq,   \
                               pb.Hkv, pb.N, pb.nqb, pb.block, pb.scale, pb.causal);           \
        if (do_q)                                                                              \
            hipLaunchKernelGGL(bwd_f32_dq_kernel<DD>, gq, dim3(64), 0, st, (const float*)q,    \
                               (const float*)k, (const float*)v, lse, (const float*)dout, D,   \
                               block_w, (float*)dq, pb.Hq, pb.Hkv, pb.N, pb.nqb, pb.block,     \
                               pb.scale, pb.causal);                                           \
        return hipGetLastError();                                                              \
    }
        LF_F32BWD(64)
        LF_F32BWD(128)
#undef LF_F32BWD
        return hipErrorInvalidValue;
    }
    const int nkt = (pb.N + kBN - 1) / kBN;
    const unsigned nwg_kv = (unsigned)(pb.B * pb.Hkv * nkt);
    const size_t nblocks = (size_t)pb.B * pb.Hq * pb.nqb;
    const float sl2 = pb.scale * kLog2e;
    // the workspace may be NULL when only the dK/dV half runs: no pointer
    // arithmetic on it then (the kernels get an all-NULL view they never use)
    const DqWorkspace ws = workspace ? dq_workspace(workspace, nblocks, pb.block, pb.d)
                                     : DqWorkspace{};
#define LF_BWD(DD, BB, CC)                                                                      \
    if (pb.d == DD && pb.block == BB && (pb.causal != 0) == CC) {                               \
        /* with both phases, the plan rides along in the dK/dV launch where it fits */          \
        constexpr bool fuse_ok = kBM * DD * sizeof(bf16) >= kDqBucketInts * sizeof(int);        \
        const bool fused = fuse_ok && do_kv && do_q;                                            \
        if (do_kv && fused)                                                                     \
            hipLaunchKernelGGL((dkdv_bf16_kernel<DD, BB, CC, fuse_ok>), dim3(nwg_kv + 1),        \
                               dim3(512), 0, st, (const bf16*)q, (const bf16*)k, (const bf16*)v, \
                               lse, (const bf16*)dout, D, kept_idx, kept_count, block_w,        \
                               (bf16*)dk, (bf16*)dv, pb.B, pb.Hq, pb.Hkv, pb.N, pb.nqb,         \
                               pb.scale, sl2, ws);                                              \
        else if (do_kv)                                                                         \
            hipLaunchKernelGGL((dkdv_bf16_kernel<DD, BB, CC, false>), dim3(nwg_kv), dim3(512),  \
                               0, st, (const bf16*)q, (const bf16*)k, (const bf16*)v, lse,      \
                               (const bf16*)dout, D, kept_idx, kept_count, block_w, (bf16*)dk,  \
                               (bf16*)dv, pb.B, pb.Hq, pb.Hkv, pb.N, pb.nqb, pb.scale, sl2, ws); \
        if (do_q) {                                                                             \
            if (!fused)                                                                         \
                hipLaunchKernelGGL((dq_plan_kernel<BB>), dim3(1), dim3(1024), 0, st, block_w,   \
                                   pb.B * pb.Hq, pb.nqb, pb.N, pb.causal, ws);                  \
            hipLaunchKernelGGL((dq_bf16_kernel<DD, BB, CC>),                                     \
                               dim3(kDqGrid * DqShape<BB>::PER_CU), dim3(DqShape<BB>::NT), 0, st, \
                               (const bf16*)q, (const bf16*)k, (const bf16*)v, lse,             \
                               (const bf16*)dout, D, block_w, (bf16*)dq, ws, pb.B, pb.Hq,       \
                               pb.Hkv, pb.N, pb.nqb, pb.scale, sl2);                            \
            hipLaunchKernelGGL((dq_finalize_kernel<DD, BB>), dim3(kDqFinSplit * kDqChunkBelow),   \
                               dim3(256), 0, st,                                                \
                               ws, (bf16*)dq, pb.N, pb.nqb);                                    \
        }                                                                                       \
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
