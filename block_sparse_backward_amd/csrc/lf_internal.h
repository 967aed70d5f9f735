// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lf {

// A validated problem shape (see lazyflash.h for the meaning of each field).
struct Problem {
    int B, Hq, Hkv, N, d, block, nqb, causal;
    float scale;
    bool bf16;
    int b0 = 0;  // batch index of the first batch entry in the draw's counter
};

hipError_t launch_fwd(const Problem& pb, const void* q, const void* k, const void* v, void* o,
                      float* lse, hipStream_t st);

// rule: 0 budget (param = delta), 1 fixed fraction, 2 top-k (param = f)
hipError_t launch_select(const Problem& pb, const void* o, const void* dout, int rule,
                         double param, uint64_t seed, float* D, double* mass, double* tau,
                         float* block_w, int32_t* kept_idx, int32_t* kept_count, hipStream_t st);

// tau = +inf and kept_count = 0 for the n heads of an empty sequence
hipError_t launch_empty_heads(double* tau, int32_t* kept_count, int n, hipStream_t st);

hipError_t launch_bwd(const Problem& pb, const void* q, const void* k, const void* v,
                      const float* lse, const void* dout, const float* D,
                      const int32_t* kept_idx, const int32_t* kept_count, const float* block_w,
                      void* dq, void* dk, void* dv, void* workspace, unsigned phases,
                      hipStream_t st);

// Device workspace bytes of launch_bwd for a validated problem (0 for fp32).
size_t bwd_workspace_bytes(const Problem& pb);

// launch_bwd (both phases) with the workspace in the library's static device
// scratch of the stream's GPU (no allocation); the problem's workspace must fit
// static_scratch_bytes().
size_t static_scratch_bytes();
hipError_t launch_bwd_static(const Problem& pb, const void* q, const void* k, const void* v,
                             const float* lse, const void* dout, const float* D,
                             const int32_t* kept_idx, const int32_t* kept_count,
                             const float* block_w, void* dq, void* dk, void* dv, hipStream_t st);

// Workgroup -> work-item maps that keep every workgroup of one key/value head
// group on one XCD (workgroups are dispatched round-robin over the 8 XCDs, each
// with its own L2), so the K/V, Q and dO tiles a group shares stay in one L2.
constexpr int kNumXcd = 8;

}  // namespace lf
