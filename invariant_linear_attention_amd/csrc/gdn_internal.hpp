// gdn_internal.hpp -- host-side plumbing shared by the C-ABI front end (gdn_api.hip)
// and the per-head-dim kernel translation units (gdn_dk*.hip).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// Largest batch whose sequences the prefill kernel orders longest first.
constexpr int kMaxRankedSeqs = 128;

// Kernel arguments of the varlen prefill (passed by value as the kernarg segment).
struct PrefillParams {
    const void *q, *k, *v;
    const float *g, *beta, *h0;
    const int32_t *cu_seqlens;
    void *out;
    float *hT;
    int64_t total_tokens;
    int32_t n_seqs, hk, hv, dv;
    int32_t rank_by_length;  // workgroups take sequences longest first (n_seqs <= kMaxRankedSeqs)
    int32_t tiles;           // row tiles per value head (set by the launcher)
};

// Kernel arguments of one decode step.
struct DecodeParams {
    const void *q, *k, *v;
    const float *g, *beta;
    float *pool;
    const int32_t *state_idx;
    void *out;
    int32_t batch, hk, hv, dv, pool_size;
};

// A launch shape: `lanes` lanes hold one state row, each lane holds `rows` rows,
// and a workgroup has `waves` waves; it owns waves * (64 / lanes) * rows
// consecutive rows of one value head.
struct Plan {
    int lanes;
    int rows;
    int waves;
};

// Per-head-dim entry points, defined in gdn_dk{16,32,64,128}.hip.
#define GDN_DECLARE_DK(DK)                                                                     \
    bool plan_available_dk##DK(bool decode, int io_dtype, Plan plan);                                     \
    hipError_t launch_prefill_dk##DK(const PrefillParams &p, int io_dtype, Plan plan, hipStream_t s); \
    hipError_t launch_decode_dk##DK(const DecodeParams &p, int io_dtype, Plan plan, hipStream_t s);
GDN_DECLARE_DK(16)
GDN_DECLARE_DK(32)
GDN_DECLARE_DK(64)
GDN_DECLARE_DK(128)
#undef GDN_DECLARE_DK

}  // namespace gdn
