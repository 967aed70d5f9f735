// LDS tile layout, staging and MFMA helpers shared by the attention kernels
// (gfx950: 64-lane waves, 32x32x16 bf16 MFMA, 64 LDS banks of 4 bytes).
#pragma once

#include "lf_common.h"

namespace lf {

// LDS tiles are row-major [ROWS][HD] bf16 with no padding; the 16-byte chunk c
// of row r is stored at chunk position c ^ swz(r).  With this map both reads
// the kernels make are free of bank conflicts (64 banks of 4 bytes): a
// 32x32x16 operand fragment (16 lanes reading one chunk of 16 consecutive
// rows) and a transposing read (32 lanes reading 4 consecutive chunks of 4
// consecutive rows, rows starting at a multiple of 4).
template <int HD>
__device__ __forceinline__ constexpr int swz(int r) {
    return HD == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Loads a swizzled [ROWS][HD] bf16 tile straight from HBM into LDS with 16-byte
// buffer loads: lane l of a wave-instruction writes LDS bytes [16 l, 16 l + 16)
// after the instruction's base, so slot S = 64 m + l is chunk position S % CPR
// of row S / CPR, and the lane fetches the logical chunk that belongs there.
// `soff` is the byte offset of the tile's first row inside the buffer `rs`.
template <int HD, int ROWS, int NWAVES>
__device__ __forceinline__ void load_tile_to_lds(__amdgpu_buffer_rsrc_t rs, int soff, bf16* lds,
                                                 int wave, int lane) {
    constexpr int CPR = HD / 8;
    constexpr int NINST = ROWS * CPR / 64;
    static_assert(ROWS * CPR % 64 == 0, "slot layout");
    static_assert(NINST % NWAVES == 0, "whole rounds");
    // rows advance by RS per round; the swizzle repeats every 16 rows, so when
    // RS is a multiple of 16 one lane offset serves every round and the round
    // moves the scalar offset
    constexpr int RS = 64 * NWAVES / CPR;
    constexpr bool kPeriodic = RS % 16 == 0;
    const int S0 = 64 * wave + lane;
    const int voff0 =
        ((S0 / CPR) * HD + ((S0 % CPR) ^ swz<HD>(S0 / CPR)) * 8) * (int)sizeof(bf16);
#pragma unroll
    for (int mm = 0; mm < NINST / NWAVES; ++mm) {
        const int m = wave + NWAVES * mm;
        if constexpr (kPeriodic) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + 512 * m), 16, voff0,
                                                     soff + mm * RS * HD * (int)sizeof(bf16), 0, 0);
        } else {
            const int S = 64 * m + lane;
            const int row = S / CPR, c = (S % CPR) ^ swz<HD>(S / CPR);
            const int voff = (row * HD + c * 8) * (int)sizeof(bf16);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + 512 * m), 16, voff, soff,
                                                     0, 0);
        }
    }
}

// Per-lane byte offsets into a swizzled tile, fixed for the kernel's life:
//   frag[ks]    32x32x16 operand fragment of row (R + l32), head-dim chunk
//               2 ks + hf, for any R that is a multiple of 16;
//   tr[dt][s]   transposing read of rows R + 4 hf + (j16 >> 2) + 8 s, columns
//               32 dt + 16 (G16 & 1) + 4 (j16 & 3) .. +3, R a multiple of 16.
// R * HD * 2 is then an immediate offset of the LDS instruction.
template <int HD>
struct TileOffsets {
    int frag[HD / 16];
    int tr[HD / 32][2];
    __device__ __forceinline__ TileOffsets(int lane) {
        const int l32 = lane & 31, hf = lane >> 5, G16 = lane >> 4, j16 = lane & 15;
        constexpr int rowB = HD * 2;
#pragma unroll
        for (int ks = 0; ks < HD / 16; ++ks)
            frag[ks] = l32 * rowB + 16 * ((2 * ks + hf) ^ swz<HD>(l32));
#pragma unroll
        for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int r = 4 * hf + (j16 >> 2) + 8 * s;
                const int c = 4 * dt + 2 * (G16 & 1) + ((j16 >> 1) & 1);
                tr[dt][s] = r * rowB + 16 * (c ^ swz<HD>(r)) + 8 * (j16 & 1);
            }
    }
};

template <int HD>
__device__ __forceinline__ bf16x8 frag_at(const bf16* tile, int R, int off) {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) + R * HD * 2 + off);
}
template <int HD>
__device__ __forceinline__ bf16x8 tr_at(const bf16* tile, int R, const int (&off)[2]) {
    const char* t = reinterpret_cast<const char*>(tile) + R * HD * 2;
    return cat(lds_read_tr(reinterpret_cast<const bf16*>(t + off[0])),
               lds_read_tr(reinterpret_cast<const bf16*>(t + off[1])));
}

// Scheduling hint for a block of NR LDS reads feeding NM MFMAs: issue AHEAD
// reads first, then alternate one MFMA with PER reads, then the last MFMAs.
// (Only orders instructions already in the scheduling region.)
template <int NR, int NM, int PER, int AHEAD>
__device__ __forceinline__ void pipeline_schedule() {
    constexpr int kDsRead = 0x100, kMfma = 0x008;
    __builtin_amdgcn_sched_group_barrier(kDsRead, AHEAD, 0);
    constexpr int rest = NR - AHEAD;
    constexpr int steps = rest / PER;
#pragma unroll
    for (int i = 0; i < steps; ++i) {
        __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kDsRead, PER, 0);
    }
    if (rest % PER) __builtin_amdgcn_sched_group_barrier(kDsRead, rest % PER, 0);
    __builtin_amdgcn_sched_group_barrier(kMfma, NM - steps, 0);
}

// As pipeline_schedule, with NV buffer loads of other work issued one per MFMA
// from the first MFMA on.
template <int NR, int NM, int PER, int AHEAD, int NV>
__device__ __forceinline__ void pipeline_schedule_vmem() {
    constexpr int kDsRead = 0x100, kMfma = 0x008, kVmemRead = 0x020;
    __builtin_amdgcn_sched_group_barrier(kDsRead, AHEAD, 0);
    constexpr int rest = NR - AHEAD;
    constexpr int steps = rest / PER;
#pragma unroll
    for (int i = 0; i < steps; ++i) {
        __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kDsRead, PER, 0);
        if (i < NV) __builtin_amdgcn_sched_group_barrier(kVmemRead, 1, 0);
    }
    if (rest % PER) __builtin_amdgcn_sched_group_barrier(kDsRead, rest % PER, 0);
    __builtin_amdgcn_sched_group_barrier(kMfma, NM - steps, 0);
}

template <int V>
struct IntC {
    static constexpr int value = V;
};

}  // namespace lf
