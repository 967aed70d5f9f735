// C ABI of liblazyflash.so (declared in include/lazyflash.h): host-side
// argument validation, then kernel launches on the caller's stream.
// Validation touches no GPU state, so every error path runs without a device.
#include <cmath>
#include <cstdio>
#include <cstring>

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
    if ((s->seqlen + s->block - 1) / s->block > kMaxBlocksPerHead)
        return fail(LF_EUNSUPPORTED, "ceil(seqlen / block) must be <= 4096");
    const double elems = (double)s->batch * s->heads_q * s->seqlen * s->head_dim;
    if (elems > 9.0e15) return fail(LF_EINVAL, "tensor too large");
    pb.B = s->batch;
    pb.Hq = s->heads_q;
    pb.Hkv = s->heads_kv;
    pb.N = s->seqlen;
    pb.d = s->head_dim;
    pb.block = s->block;
    pb.nqb = (s->seqlen + s->block - 1) / s->block;  // the last block may be partial
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

}  // namespace

extern "C" {

const char* lf_status_str(lf_status st) {
    switch (st) {
        case LF_OK: return "LF_OK";
        case LF_EINVAL: return "LF_EINVAL";
        case LF_EUNSUPPORTED: return "LF_EUNSUPPORTED";
        case LF_EHIP: return "LF_EHIP";
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

}  // extern "C"
