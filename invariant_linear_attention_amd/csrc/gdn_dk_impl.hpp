// gdn_dk_impl.hpp -- instantiates the kernels for one key dim GDN_DK and exposes the
// per-dim launchers declared in gdn_internal.hpp.  Included once by each gdn_dk*.hip.
#pragma once
#ifndef GDN_DK
#error "define GDN_DK before including gdn_dk_impl.hpp"
#endif

#include "gdn_kernels.hpp"

#define GDN_PASTE2(a, b) a##b
#define GDN_PASTE(a, b) GDN_PASTE2(a, b)
#define GDN_FN(name) GDN_PASTE(name, GDN_PASTE(_dk, GDN_DK))

namespace gdn {
namespace {

// Prefill launch shapes compiled for this dk: (lanes, rows per lane, waves).
// Lanes above 4 need whole leaves per lane: 8 lanes for dk >= 64, 16 for dk = 128.
constexpr bool prefill_compiled(int lanes, int rows, int waves) {
    if (waves == 8) return GDN_DK == 128 && ((lanes == 8 && rows == 1) || (lanes == 16 && rows == 2));
    if (waves != 1 && waves != 2 && waves != 4) return false;
    if (lanes == 4) return rows == 1 || rows == 2 || (GDN_DK == 128 && rows == 4 && waves <= 2);
    if (lanes == 8) return GDN_DK >= 64 && (rows == 1 || rows == 2);
    // (16, 1, 1) would own 4 rows per workgroup, less than one 16-byte bf16 vector.
    if (lanes == 16) return GDN_DK == 128 && (rows == 2 || rows == 4 || (rows == 1 && waves >= 2));
    return false;
}

constexpr bool decode_compiled(int lanes, int rows, int waves) {
    if (lanes != 4 || (waves != 1 && waves != 2 && waves != 4)) return false;
    return rows == 1 || rows == 2 || (GDN_DK == 128 && rows == 4 && waves <= 2);
}

template <class IO>
hipError_t prefill_io(const PrefillParams &p, Plan plan, hipStream_t s) {
#define GDN_CASE(L_, R_, NW_)                                                  \
    if (plan.lanes == L_ && plan.rows == R_ && plan.waves == NW_)              \
        return launch_prefill_t<GDN_DK, IO, L_, R_, NW_>(p, s);
    GDN_CASE(4, 1, 1) GDN_CASE(4, 1, 2) GDN_CASE(4, 1, 4)
    GDN_CASE(4, 2, 1) GDN_CASE(4, 2, 2) GDN_CASE(4, 2, 4)
#if GDN_DK == 128
    GDN_CASE(4, 4, 1) GDN_CASE(4, 4, 2)
#endif
#if GDN_DK >= 64
    GDN_CASE(8, 1, 1) GDN_CASE(8, 1, 2) GDN_CASE(8, 1, 4)
    GDN_CASE(8, 2, 1) GDN_CASE(8, 2, 2) GDN_CASE(8, 2, 4)
#endif
#if GDN_DK == 128
    GDN_CASE(16, 1, 2) GDN_CASE(16, 1, 4)
    GDN_CASE(16, 2, 1) GDN_CASE(16, 2, 2) GDN_CASE(16, 2, 4) GDN_CASE(16, 2, 8)
    GDN_CASE(16, 4, 1) GDN_CASE(16, 4, 2) GDN_CASE(16, 4, 4)
    GDN_CASE(8, 1, 8)
#endif
#undef GDN_CASE
    return hipErrorInvalidValue;
}

template <class IO>
hipError_t decode_io(const DecodeParams &p, Plan plan, hipStream_t s) {
#define GDN_CASE(R_, NW_) \
    if (plan.lanes == 4 && plan.rows == R_ && plan.waves == NW_) return launch_decode_t<GDN_DK, IO, R_, NW_>(p, s);
    GDN_CASE(1, 1) GDN_CASE(1, 2) GDN_CASE(1, 4)
    GDN_CASE(2, 1) GDN_CASE(2, 2) GDN_CASE(2, 4)
#if GDN_DK == 128
    GDN_CASE(4, 1) GDN_CASE(4, 2)
#endif
#undef GDN_CASE
    return hipErrorInvalidValue;
}

}  // namespace

bool GDN_FN(plan_available)(bool decode, int io_dtype, Plan plan) {
    if (io_dtype != GDN_F32 && io_dtype != GDN_BF16) return false;
    return decode ? decode_compiled(plan.lanes, plan.rows, plan.waves)
                  : prefill_compiled(plan.lanes, plan.rows, plan.waves);
}

hipError_t GDN_FN(launch_prefill)(const PrefillParams &p, int io_dtype, Plan plan, hipStream_t s) {
    return io_dtype == GDN_BF16 ? prefill_io<IoBf16>(p, plan, s) : prefill_io<IoF32>(p, plan, s);
}

hipError_t GDN_FN(launch_decode)(const DecodeParams &p, int io_dtype, Plan plan, hipStream_t s) {
    return io_dtype == GDN_BF16 ? decode_io<IoBf16>(p, plan, s) : decode_io<IoF32>(p, plan, s);
}

}  // namespace gdn
