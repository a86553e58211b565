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

// Launch shapes compiled for this dk.  (rows per quad, waves per workgroup)
constexpr bool shape_compiled(int rows, int waves) {
    if (waves != 1 && waves != 2 && waves != 4) return false;
    if (rows == 1 || rows == 2) return true;
    return GDN_DK == 128 && rows == 4 && waves <= 2;
}

template <class IO>
hipError_t prefill_io(const PrefillParams &p, Plan plan, hipStream_t s) {
#define GDN_CASE(R_, NW_) \
    if (plan.rows == R_ && plan.waves == NW_) return launch_prefill_t<GDN_DK, IO, R_, NW_>(p, s);
    GDN_CASE(1, 1) GDN_CASE(1, 2) GDN_CASE(1, 4)
    GDN_CASE(2, 1) GDN_CASE(2, 2) GDN_CASE(2, 4)
#if GDN_DK == 128
    GDN_CASE(4, 1) GDN_CASE(4, 2)
#endif
#undef GDN_CASE
    return hipErrorInvalidValue;
}

template <class IO>
hipError_t decode_io(const DecodeParams &p, Plan plan, hipStream_t s) {
#define GDN_CASE(R_, NW_) \
    if (plan.rows == R_ && plan.waves == NW_) return launch_decode_t<GDN_DK, IO, R_, NW_>(p, s);
    GDN_CASE(1, 1) GDN_CASE(1, 2) GDN_CASE(1, 4)
    GDN_CASE(2, 1) GDN_CASE(2, 2) GDN_CASE(2, 4)
#if GDN_DK == 128
    GDN_CASE(4, 1) GDN_CASE(4, 2)
#endif
#undef GDN_CASE
    return hipErrorInvalidValue;
}

}  // namespace

bool GDN_FN(plan_available)(int io_dtype, Plan plan) {
    return (io_dtype == GDN_F32 || io_dtype == GDN_BF16) && shape_compiled(plan.rows, plan.waves);
}

hipError_t GDN_FN(launch_prefill)(const PrefillParams &p, int io_dtype, Plan plan, hipStream_t s) {
    return io_dtype == GDN_BF16 ? prefill_io<IoBf16>(p, plan, s) : prefill_io<IoF32>(p, plan, s);
}

hipError_t GDN_FN(launch_decode)(const DecodeParams &p, int io_dtype, Plan plan, hipStream_t s) {
    return io_dtype == GDN_BF16 ? decode_io<IoBf16>(p, plan, s) : decode_io<IoF32>(p, plan, s);
}

}  // namespace gdn
