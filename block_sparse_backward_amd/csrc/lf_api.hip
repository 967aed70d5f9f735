// C ABI of liblazyflash.so (declared in include/lazyflash.h): host-side
// argument validation, then kernel launches on the caller's stream.
// Validation touches no GPU state, so every error path runs without a device.
#include <cmath>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <vector>

#include "lazyflash.h"
#include "lf_internal.h"

namespace {

thread_local char g_err[256] = "";

lf_status fail(lf_status st, const char* msg) {
    std::snprintf(g_err, sizeof(g_err), "%s", msg);
    return st;
}

lf_status hip_status(hipError_t e) {
    if (e == hipSuccess) {
        g_err[0] = '\0';
        return LF_OK;
    }
    std::snprintf(g_err, sizeof(g_err), "HIP error %d: %s", (int)e, hipGetErrorString(e));
    return LF_EHIP;
}

constexpr int kMaxBlocksPerHead = 4096;

// Checks the shape; on success fills `pb` and sets `empty` for B == 0 or N == 0.
lf_status check_shape(const lf_shape* s, lf::Problem& pb, bool& empty) {
    if (!s) return fail(LF_EINVAL, "shape is NULL");
    if (s->batch < 0 || s->seqlen < 0) return fail(LF_EINVAL, "batch and seqlen must be >= 0");
    if (s->heads_q < 1 || s->heads_kv < 1) return fail(LF_EINVAL, "heads_q and heads_kv must be >= 1");
    if (s->heads_q % s->heads_kv != 0) return fail(LF_EINVAL, "heads_q must be a multiple of heads_kv");
    if (s->dtype != LF_BF16 && s->dtype != LF_F32) return fail(LF_EINVAL, "unknown dtype");
    if (s->head_dim < 1 || s->block < 1) return fail(LF_EINVAL, "head_dim and block must be >= 1");
    if (!std::isfinite(s->scale)) return fail(LF_EINVAL, "scale must be finite");
    if (s->head_dim != 64 && s->head_dim != 128) return fail(LF_EUNSUPPORTED, "head_dim must be 64 or 128");
    if (s->block != 64 && s->block != 128) return fail(LF_EUNSUPPORTED, "block must be 64 or 128");
    // in 64 bits: seqlen + block - 1 overflows int32 for the longest lengths
    const int64_t nqb = ((int64_t)s->seqlen + s->block - 1) / s->block;
    if (nqb > kMaxBlocksPerHead) return fail(LF_EUNSUPPORTED, "ceil(seqlen / block) must be <= 4096");
    const double elems = (double)s->batch * s->heads_q * s->seqlen * s->head_dim;
    if (elems > 9.0e15) return fail(LF_EINVAL, "tensor too large");
    pb.B = s->batch;
    pb.Hq = s->heads_q;
    pb.Hkv = s->heads_kv;
    pb.N = s->seqlen;
    pb.d = s->head_dim;
    pb.block = s->block;
    pb.nqb = (int)nqb;  // the last block may be partial
    pb.causal = s->causal != 0;
    pb.scale = s->scale;
    pb.bf16 = s->dtype == LF_BF16;
    empty = s->batch == 0 || s->seqlen == 0;
    return LF_OK;
}

bool any_null(std::initializer_list<const void*> ptrs) {
    for (const void* p : ptrs)
        if (!p) return true;
    return false;
}

// true when a non-NULL pointer of the list is not a multiple of `a` bytes
bool misaligned(std::initializer_list<const void*> ptrs, uintptr_t a) {
    for (const void* p : ptrs)
        if (reinterpret_cast<uintptr_t>(p) % a != 0) return true;
    return false;
}
constexpr const char* kAlignMsg =
    "misaligned pointer (element tensors and workspace: 16 bytes; other arrays: their element "
    "size)";

// A variable-length batch: shape->batch sequences, sequence b of
// cu[b + 1] - cu[b] tokens (shape->seqlen is not used).  Checks every
// sequence before anything is launched; fills one Problem per sequence.
lf_status check_varlen(const lf_shape* s, const int32_t* cu, std::vector<lf::Problem>& seqs) {
    if (!s) return fail(LF_EINVAL, "shape is NULL");
    if (s->batch < 0) return fail(LF_EINVAL, "batch must be >= 0");
    if (s->batch > 0 && !cu) return fail(LF_EINVAL, "cu_seqlens is NULL");
    if (s->batch > 0 && cu[0] != 0) return fail(LF_EINVAL, "cu_seqlens[0] must be 0");
    seqs.clear();
    for (int b = 0; b < s->batch; ++b) {
        if (cu[b + 1] < cu[b]) return fail(LF_EINVAL, "cu_seqlens must be nondecreasing");
        lf_shape one = *s;
        one.batch = 1;
        one.seqlen = cu[b + 1] - cu[b];
        lf::Problem pb;
        bool empty;
        const lf_status st = check_shape(&one, pb, empty);
        if (st != LF_OK) return st;
        pb.b0 = b;
        seqs.push_back(pb);
    }
    if (s->batch == 0) {  // the shape's other fields are still checked
        lf_shape one = *s;
        one.batch = 0;
        one.seqlen = 0;
        lf::Problem pb;
        bool empty;
        return check_shape(&one, pb, empty);
    }
    return LF_OK;
}

// byte offset helpers for the packed layouts of a variable-length batch
inline const void* at(const void* p, size_t bytes) { return static_cast<const char*>(p) + bytes; }
inline void* at(void* p, size_t bytes) { return static_cast<char*>(p) + bytes; }
template <typename T>
inline T* at(T* p, size_t elems) { return p + elems; }

}  // namespace

extern "C" {

const char* lf_status_str(lf_status st) {
    switch (st) {
        case LF_OK: return "LF_OK";
        case LF_EINVAL: return "LF_EINVAL";
        case LF_EUNSUPPORTED: return "LF_EUNSUPPORTED";
        case LF_EHIP: return "LF_EHIP";
        default: break;
    }
    return "unknown lf_status";
}

const char* lf_last_error(void) { return g_err; }

int32_t lf_abi_version(void) { return LF_ABI_VERSION; }

lf_status lf_attn_fwd(const lf_shape* s, const void* q, const void* k, const void* v, void* o,
                      float* lse, void* stream) {
    lf::Problem pb;
    bool empty;
    lf_status st = check_shape(s, pb, empty);
    if (st != LF_OK) return st;
    if (empty) return hip_status(hipSuccess);
    if (any_null({q, k, v, o, lse})) return fail(LF_EINVAL, "NULL tensor pointer");
    if (misaligned({q, k, v, o}, 16) || misaligned({lse}, 4)) return fail(LF_EINVAL, kAlignMsg);
    return hip_status(lf::launch_fwd(pb, q, k, v, o, lse, (hipStream_t)stream));
}

lf_status lf_block_select_rule(const lf_shape* s, const void* o, const void* dout,
                               int32_t rule, double param, uint64_t seed, float* D, double* mass,
                               double* tau, float* block_w, int32_t* kept_idx,
                               int32_t* kept_count, void* stream) {
    lf::Problem pb;
    bool empty;
    lf_status st = check_shape(s, pb, empty);
    if (st != LF_OK) return st;
    if (rule == LF_SELECT_BUDGET) {
        if (!(param >= 0.0 && param < 1.0)) return fail(LF_EINVAL, "delta must be in [0, 1)");
    } else if (rule == LF_SELECT_FRACTION || rule == LF_SELECT_TOPK) {
        if (!(param > 0.0 && param <= 1.0)) return fail(LF_EINVAL, "fraction must be in (0, 1]");
    } else {
        return fail(LF_EINVAL, "unknown selection rule");
    }
    if (empty) return hip_status(hipSuccess);
    if (any_null({o, dout, D, mass, tau, block_w, kept_idx, kept_count}))
        return fail(LF_EINVAL, "NULL tensor pointer");
    if (misaligned({o, dout}, 16) || misaligned({D, block_w, kept_idx, kept_count}, 4) ||
        misaligned({mass, tau}, 8))
        return fail(LF_EINVAL, kAlignMsg);
    return hip_status(lf::launch_select(pb, o, dout, rule, param, seed, D, mass, tau, block_w,
                                        kept_idx, kept_count, (hipStream_t)stream));
}

lf_status lf_block_select(const lf_shape* s, const void* o, const void* dout, double delta,
                          uint64_t seed, float* D, double* mass, double* tau, float* block_w,
                          int32_t* kept_idx, int32_t* kept_count, void* stream) {
    return lf_block_select_rule(s, o, dout, LF_SELECT_BUDGET, delta, seed, D, mass, tau, block_w,
                                kept_idx, kept_count, stream);
}

lf_status lf_bwd_workspace_size(const lf_shape* s, size_t* bytes) {
    lf::Problem pb;
    bool empty;
    lf_status st = check_shape(s, pb, empty);
    if (st != LF_OK) return st;
    if (!bytes) return fail(LF_EINVAL, "bytes is NULL");
    *bytes = empty ? 0 : lf::bwd_workspace_bytes(pb);
    return hip_status(hipSuccess);
}

lf_status lf_attn_bwd_phases(const lf_shape* s, const void* q, const void* k, const void* v,
                             const float* lse, const void* dout, const float* D,
                             const int32_t* kept_idx, const int32_t* kept_count,
                             const float* block_w, void* dq, void* dk, void* dv, void* workspace,
                             size_t workspace_bytes, uint32_t phases, void* stream) {
    lf::Problem pb;
    bool empty;
    lf_status st = check_shape(s, pb, empty);
    if (st != LF_OK) return st;
    if (phases == 0 || (phases & ~LF_BWD_ALL) != 0) return fail(LF_EINVAL, "bad phase mask");
    if (empty) return hip_status(hipSuccess);
    if (any_null({q, k, v, lse, dout, D, kept_idx, kept_count, block_w}) ||
        ((phases & LF_BWD_DQ) && !dq) || ((phases & LF_BWD_DKDV) && (!dk || !dv)))
        return fail(LF_EINVAL, "NULL tensor pointer");
    if (misaligned({q, k, v, dout, dq, dk, dv, workspace}, 16) ||
        misaligned({lse, D, kept_idx, kept_count, block_w}, 4))
        return fail(LF_EINVAL, kAlignMsg);
    if (phases & LF_BWD_DQ) {
        const size_t need = lf::bwd_workspace_bytes(pb);
        if (need > 0 && !workspace) return fail(LF_EINVAL, "workspace is NULL");
        if (workspace_bytes < need) return fail(LF_EINVAL, "workspace too small (see lf_bwd_workspace_size)");
    }
    return hip_status(lf::launch_bwd(pb, q, k, v, lse, dout, D, kept_idx, kept_count, block_w, dq,
                                     dk, dv, workspace, phases, (hipStream_t)stream));
}

lf_status lf_attn_bwd(const lf_shape* s, const void* q, const void* k, const void* v,
                      const float* lse, const void* dout, const float* D,
                      const int32_t* kept_idx, const int32_t* kept_count, const float* block_w,
                      void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      void* stream) {
    return lf_attn_bwd_phases(s, q, k, v, lse, dout, D, kept_idx, kept_count, block_w, dq, dk, dv,
                              workspace, workspace_bytes, LF_BWD_ALL, stream);
}

lf_status lf_attn_bwd_noalloc(const lf_shape* s, const void* q, const void* k, const void* v,
                              const float* lse, const void* dout, const float* D,
                              const int32_t* kept_idx, const int32_t* kept_count,
                              const float* block_w, void* dq, void* dk, void* dv, void* stream) {
    lf::Problem pb;
    bool empty;
    lf_status st = check_shape(s, pb, empty);
    if (st != LF_OK) return st;
    if (empty) return hip_status(hipSuccess);
    if (any_null({q, k, v, lse, dout, D, kept_idx, kept_count, block_w, dq, dk, dv}))
        return fail(LF_EINVAL, "NULL tensor pointer");
    if (misaligned({q, k, v, dout, dq, dk, dv}, 16) ||
        misaligned({lse, D, kept_idx, kept_count, block_w}, 4))
        return fail(LF_EINVAL, kAlignMsg);
    const size_t need = lf::bwd_workspace_bytes(pb), have = lf::static_scratch_bytes();
    if (need > have) {
        std::snprintf(g_err, sizeof(g_err),
                      "the problem needs %zu bytes of scratch, more than the %zu bytes of the "
                      "static scratch (use lf_attn_bwd with a workspace)", need, have);
        return LF_EUNSUPPORTED;
    }
    return hip_status(lf::launch_bwd_static(pb, q, k, v, lse, dout, D, kept_idx, kept_count,
                                            block_w, dq, dk, dv, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// Variable-length batches (layouts in lazyflash.h): one launch sequence per
// sequence on the caller's stream, each sequence a fixed-length problem of
// batch 1 on its slice of the packed tensors.
// ---------------------------------------------------------------------------
lf_status lf_attn_fwd_varlen(const lf_shape* s, const int32_t* cu, const void* q, const void* k,
                             const void* v, void* o, float* lse, void* stream) {
    std::vector<lf::Problem> seqs;
    lf_status st = check_varlen(s, cu, seqs);
    if (st != LF_OK) return st;
    if (cu && s->batch > 0 && cu[s->batch] > 0 && any_null({q, k, v, o, lse}))
        return fail(LF_EINVAL, "NULL tensor pointer");
    if (misaligned({q, k, v, o}, 16) || misaligned({lse}, 4)) return fail(LF_EINVAL, kAlignMsg);
    const size_t elt = s->dtype == LF_BF16 ? 2 : 4, d = (size_t)s->head_dim;
    for (const lf::Problem& pb : seqs) {
        if (pb.N == 0) continue;
        const size_t t0 = (size_t)cu[pb.b0];
        const hipError_t e = lf::launch_fwd(
            pb, at(q, pb.Hq * t0 * d * elt), at(k, pb.Hkv * t0 * d * elt),
            at(v, pb.Hkv * t0 * d * elt), at(o, pb.Hq * t0 * d * elt), at(lse, pb.Hq * t0),
            (hipStream_t)stream);
        if (e != hipSuccess) return hip_status(e);
    }
    return hip_status(hipSuccess);
}

lf_status lf_block_select_varlen(const lf_shape* s, const int32_t* cu, const void* o,
                                 const void* dout, int32_t rule, double param, uint64_t seed,
                                 float* D, double* mass, double* tau, float* block_w,
                                 int32_t* kept_idx, int32_t* kept_count, void* stream) {
    std::vector<lf::Problem> seqs;
    lf_status st = check_varlen(s, cu, seqs);
    if (st != LF_OK) return st;
    if (rule == LF_SELECT_BUDGET) {
        if (!(param >= 0.0 && param < 1.0)) return fail(LF_EINVAL, "delta must be in [0, 1)");
    } else if (rule == LF_SELECT_FRACTION || rule == LF_SELECT_TOPK) {
        if (!(param > 0.0 && param <= 1.0)) return fail(LF_EINVAL, "fraction must be in (0, 1]");
    } else {
        return fail(LF_EINVAL, "unknown selection rule");
    }
    if (s->batch > 0 && any_null({o, dout, D, mass, tau, block_w, kept_idx, kept_count}))
        return fail(LF_EINVAL, "NULL tensor pointer");
    if (misaligned({o, dout}, 16) || misaligned({D, block_w, kept_idx, kept_count}, 4) ||
        misaligned({mass, tau}, 8))
        return fail(LF_EINVAL, kAlignMsg);
    const size_t elt = s->dtype == LF_BF16 ? 2 : 4, d = (size_t)s->head_dim;
    size_t cb = 0;  // blocks of the sequences before this one
    for (const lf::Problem& pb : seqs) {
        const size_t t0 = (size_t)cu[pb.b0], hq = (size_t)pb.Hq;
        if (pb.N == 0) {  // no blocks: nothing kept, tau = +inf
            const hipError_t e = lf::launch_empty_heads(at(tau, hq * pb.b0),
                                                        at(kept_count, hq * pb.b0), pb.Hq,
                                                        (hipStream_t)stream);
            if (e != hipSuccess) return hip_status(e);
            continue;
        }
        const hipError_t e = lf::launch_select(
            pb, at(o, hq * t0 * d * elt), at(dout, hq * t0 * d * elt), rule, param, seed,
            at(D, hq * t0), at(mass, hq * cb), at(tau, hq * pb.b0), at(block_w, hq * cb),
            at(kept_idx, hq * cb), at(kept_count, hq * pb.b0), (hipStream_t)stream);
        if (e != hipSuccess) return hip_status(e);
        cb += (size_t)pb.nqb;
    }
    return hip_status(hipSuccess);
}

lf_status lf_bwd_workspace_size_varlen(const lf_shape* s, const int32_t* cu, size_t* bytes) {
    std::vector<lf::Problem> seqs;
    lf_status st = check_varlen(s, cu, seqs);
    if (st != LF_OK) return st;
    if (!bytes) return fail(LF_EINVAL, "bytes is NULL");
    size_t need = 0;
    for (const lf::Problem& pb : seqs)
        if (pb.N > 0) need = std::max(need, lf::bwd_workspace_bytes(pb));
    *bytes = need;
    return hip_status(hipSuccess);
}

lf_status lf_attn_bwd_varlen(const lf_shape* s, const int32_t* cu, const void* q, const void* k,
                             const void* v, const float* lse, const void* dout, const float* D,
                             const int32_t* kept_idx, const int32_t* kept_count,
                             const float* block_w, void* dq, void* dk, void* dv, void* workspace,
                             size_t workspace_bytes, void* stream) {
    std::vector<lf::Problem> seqs;
    lf_status st = check_varlen(s, cu, seqs);
    if (st != LF_OK) return st;
    if (s->batch > 0 &&
        any_null({q, k, v, lse, dout, D, kept_idx, kept_count, block_w, dq, dk, dv}))
        return fail(LF_EINVAL, "NULL tensor pointer");
    if (misaligned({q, k, v, dout, dq, dk, dv, workspace}, 16) ||
        misaligned({lse, D, kept_idx, kept_count, block_w}, 4))
        return fail(LF_EINVAL, kAlignMsg);
    size_t need = 0;
    for (const lf::Problem& pb : seqs)
        if (pb.N > 0) need = std::max(need, lf::bwd_workspace_bytes(pb));
    if (need > 0 && !workspace) return fail(LF_EINVAL, "workspace is NULL");
    if (workspace_bytes < need) return fail(LF_EINVAL, "workspace too small (see lf_bwd_workspace_size_varlen)");
    const size_t elt = s->dtype == LF_BF16 ? 2 : 4, d = (size_t)s->head_dim;
    size_t cb = 0;
    for (const lf::Problem& pb : seqs) {
        if (pb.N == 0) continue;
        const size_t t0 = (size_t)cu[pb.b0], hq = (size_t)pb.Hq, hk = (size_t)pb.Hkv;
        // the sequences run one after the other on the stream and share the workspace
        const hipError_t e = lf::launch_bwd(
            pb, at(q, hq * t0 * d * elt), at(k, hk * t0 * d * elt), at(v, hk * t0 * d * elt),
            at(lse, hq * t0), at(dout, hq * t0 * d * elt), at(D, hq * t0), at(kept_idx, hq * cb),
            at(kept_count, hq * pb.b0), at(block_w, hq * cb), at(dq, hq * t0 * d * elt),
            at(dk, hk * t0 * d * elt), at(dv, hk * t0 * d * elt), workspace, LF_BWD_ALL,
            (hipStream_t)stream);
        if (e != hipSuccess) return hip_status(e);
        cb += (size_t)pb.nqb;
    }
    return hip_status(hipSuccess);
}

}  // extern "C"
