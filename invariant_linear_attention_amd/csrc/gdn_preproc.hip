// gdn_preproc.hip -- the fused preprocessing as a pass of its own (gdn_preprocess)
// and its gradients (gdn_preprocess_backward).
//
// The gated delta rule layer (Yang, Kautz, Hatamizadeh, ICLR 2025) L2-normalises
// queries and keys and forms the decay and the write strength from logits,
// g = -exp(A_log) softplus(a + dt_bias) and beta = sigmoid(b), right before the
// recurrence.  The recurrent kernels do this on the fly (gdn_dims.pre); a trainer
// that differentiates through it needs the preprocessed values as tensors and the
// map of their gradients back to the raw inputs.  The forward pass here evaluates
// every quantity by the same fp32 operations, in the same order, as the fused
// kernels (gdn_kernels.hpp), so the recurrence on its outputs gives the fused
// forward's bits.  The backward:
//     x^ = x r, r = rsq(sum x^2 + eps):   dx = (dy - x^ (x^ . dy)) r
//     da = dg (-exp(A_log) sigmoid(a + dt_bias)),   db = dbeta beta (1 - beta)
//     dA_log[h] = sum_t dg g,   ddt_bias[h] = sum_t da     (all tokens, fixed order)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"
#include "gdn_internal.hpp"
#include "gdn_kernels.hpp"

#pragma clang fp contract(off)

namespace gdn {
namespace {

constexpr int kPreThreads = 256;

// Four consecutive elements of a q or k row (a leaf of the norm's sum).
template <class IO>
__device__ __forceinline__ float4 load_leaf(const void *base, size_t idx) {
    return IO::load4(base, idx);
}

// q and k rows: DK / 4 lanes per row, each holding one leaf of 4 consecutive
// columns.  The sum of squares is the fused kernels' tree: leaves (x0 x0, then fma
// with x1, x2, x3), added pairwise across the row's lanes in column order.
template <int DK, class IO, bool BWD>
__global__ __launch_bounds__(kPreThreads) void gdn_pre_rows_kernel(PreParams p) {
    constexpr int NL = DK / 4, RPB = kPreThreads / NL;
    const int64_t rows = p.total_tokens * p.hk;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / NL;
    const int leaf = threadIdx.x % NL;
    if (row >= rows) return;  // (a whole row group: the cross-lane sums stay inside it)
    const bool norm = p.flags & GDN_PRE_QK_L2NORM;
    const size_t off = (size_t)row * DK + 4 * leaf;
#pragma unroll
    for (int side = 0; side < 2; ++side) {
        const float4 x4 = load_leaf<IO>(side ? p.k : p.q, off);
        const float x[4] = {x4.x, x4.y, x4.z, x4.w};
        float r = 1.f;
        if (norm) r = norm_scale(group_sum<NL>(sumsq4(x[0], x[1], x[2], x[3])), p.eps);
        if constexpr (!BWD) {
            float *dst = side ? p.kn : p.qn;
            *reinterpret_cast<float4 *>(dst + off) =
                norm ? make_float4(x[0] * r, x[1] * r, x[2] * r, x[3] * r) : x4;
        } else {
            const float4 dy4 = *reinterpret_cast<const float4 *>((side ? p.dkn : p.dqn) + off);
            float *dst = side ? p.dk : p.dq;
            if (!norm) {
                *reinterpret_cast<float4 *>(dst + off) = dy4;
                continue;
            }
            const float dy[4] = {dy4.x, dy4.y, dy4.z, dy4.w};
            float xh[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) xh[i] = x[i] * r;
            // x^ . dy over the row: the same leaves and tree as the sum of squares
            float t = xh[0] * dy[0];
            t = __builtin_fmaf(xh[1], dy[1], t);
            t = __builtin_fmaf(xh[2], dy[2], t);
            t = __builtin_fmaf(xh[3], dy[3], t);
            t = group_sum<NL>(t);
            float dx[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) dx[i] = __builtin_fmaf(-xh[i], t, dy[i]) * r;
            *reinterpret_cast<float4 *>(dst + off) = make_float4(dx[0], dx[1], dx[2], dx[3]);
        }
    }
}

// g and beta (forward) or their logits' gradients (backward), one element per thread.
template <bool BWD>
__global__ __launch_bounds__(kPreThreads) void gdn_pre_gate_kernel(PreParams p) {
    const int64_t i = (int64_t)blockIdx.x * kPreThreads + threadIdx.x;
    if (i >= p.total_tokens * p.hv) return;
    const int h = (int)(i % p.hv);
    const bool gated = p.flags & GDN_PRE_GATE_LOGITS;
    if constexpr (!BWD) {
        if (gated) {
            const float amp = gate_amplitude(p.A_log[h]);
            const float dtb = p.dt_bias ? p.dt_bias[h] : 0.f;
            p.g[i] = gate_from_logit(amp, dtb, p.a[i]);
            p.beta[i] = sigmoid_f32(p.b[i]);
        } else {
            p.g[i] = p.a[i];
            p.beta[i] = p.b[i];
        }
    } else {
        if (gated) {
            const float amp = gate_amplitude(p.A_log[h]);
            const float dtb = p.dt_bias ? p.dt_bias[h] : 0.f;
            p.da[i] = p.dg[i] * (-amp * sigmoid_f32(p.a[i] + dtb));
            const float bt = sigmoid_f32(p.b[i]);
            p.db[i] = (p.dbeta[i] * bt) * (1.f - bt);
        } else {
            p.da[i] = p.dg[i];
            p.db[i] = p.dbeta[i];
        }
    }
}

// dA_log[h] = sum_t dg g and ddt_bias[h] = sum_t da, in two launches.  First, per
// block of kParamTok tokens: lane h of each of four waves adds its head's terms of
// every fourth token in token order (the lanes read consecutive heads of a token
// row), and the waves' sums meet as (w0 + w1) + (w2 + w3); the block sums go to the
// da and db buffers, head-major, before the gate kernel writes those.  Then one
// workgroup per head adds its blocks: thread i takes blocks i, i + 256, ... in
// order, and the threads' sums meet in a fixed halving tree.
constexpr int kParamTok = 64;

__global__ __launch_bounds__(256) void gdn_pre_param_part_kernel(PreParams p) {
    __shared__ float ps[2][4][64];
    const int64_t blk = blockIdx.x, nblk = gridDim.x;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int h = blockIdx.y * 64 + lane;
    float a_acc = 0.f, d_acc = 0.f;
    if (h < p.hv) {
        const float amp = gate_amplitude(p.A_log[h]);
        const float dtb = p.dt_bias ? p.dt_bias[h] : 0.f;
        const int64_t t0 = blk * kParamTok;
        const int64_t t1 = t0 + kParamTok < p.total_tokens ? t0 + kParamTok : p.total_tokens;
#pragma unroll 4
        for (int64_t t = t0 + wv; t < t1; t += 4) {
            const size_t i = (size_t)t * p.hv + h;
            const float dg = p.dg[i], a = p.a[i];
            const float g = gate_from_logit(amp, dtb, a);
            const float da = dg * (-amp * sigmoid_f32(a + dtb));
            a_acc = a_acc + dg * g;
            d_acc = d_acc + da;
        }
    }
    ps[0][wv][lane] = a_acc;
    ps[1][wv][lane] = d_acc;
    __syncthreads();
    if (wv != 0 || h >= p.hv) return;
    p.da[(size_t)h * nblk + blk] = (ps[0][0][lane] + ps[0][1][lane]) + (ps[0][2][lane] + ps[0][3][lane]);
    p.db[(size_t)h * nblk + blk] = (ps[1][0][lane] + ps[1][1][lane]) + (ps[1][2][lane] + ps[1][3][lane]);
}

__global__ __launch_bounds__(kPreThreads) void gdn_pre_param_sum_kernel(PreParams p, int64_t nblk) {
    __shared__ float sa[kPreThreads], sd[kPreThreads];
    const int h = blockIdx.x, tid = threadIdx.x;
    float a_acc = 0.f, d_acc = 0.f;
    for (int64_t b = tid; b < nblk; b += kPreThreads) {
        a_acc = a_acc + p.da[(size_t)h * nblk + b];
        d_acc = d_acc + p.db[(size_t)h * nblk + b];
    }
    sa[tid] = a_acc;
    sd[tid] = d_acc;
    for (int w = kPreThreads / 2; w >= 1; w /= 2) {
        __syncthreads();
        if (tid < w) {
            sa[tid] = sa[tid] + sa[tid + w];
            sd[tid] = sd[tid] + sd[tid + w];
        }
    }
    if (tid == 0) {
        if (p.dA_log) p.dA_log[h] = sa[0];
        if (p.ddt_bias) p.ddt_bias[h] = sd[0];
    }
}

template <int DK, class IO, bool BWD>
hipError_t rows_launch(const PreParams &p, hipStream_t s) {
    constexpr int RPB = kPreThreads / (DK / 4);
    const int64_t rows = p.total_tokens * p.hk;
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL((gdn_pre_rows_kernel<DK, IO, BWD>), dim3((unsigned)((rows + RPB - 1) / RPB)),
                       dim3(kPreThreads), 0, s, p);
    return hipGetLastError();
}

template <class IO, bool BWD>
hipError_t rows_io(const PreParams &p, int dk, hipStream_t s) {
    switch (dk) {
        case 16: return rows_launch<16, IO, BWD>(p, s);
        case 32: return rows_launch<32, IO, BWD>(p, s);
        case 64: return rows_launch<64, IO, BWD>(p, s);
        case 128: return rows_launch<128, IO, BWD>(p, s);
        default: return hipErrorInvalidValue;
    }
}

template <bool BWD>
hipError_t pre_launch(const PreParams &p, int dk, int io_dtype, hipStream_t s) {
    hipError_t e = io_dtype == GDN_BF16 ? rows_io<IoBf16, BWD>(p, dk, s) : rows_io<IoF32, BWD>(p, dk, s);
    if (e != hipSuccess) return e;
    // the parameter gradients first: their partial sums use da and db as scratch
    if (BWD && (p.flags & GDN_PRE_GATE_LOGITS) && (p.dA_log || p.ddt_bias)) {
        const int64_t nblk = (p.total_tokens + kParamTok - 1) / kParamTok;
        if (nblk > 0) {
            hipLaunchKernelGGL(gdn_pre_param_part_kernel, dim3((unsigned)nblk, (unsigned)((p.hv + 63) / 64)), dim3(256),
                               0, s, p);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(gdn_pre_param_sum_kernel, dim3((unsigned)p.hv), dim3(kPreThreads), 0, s, p, nblk);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t n = p.total_tokens * p.hv;
    if (n > 0) {
        hipLaunchKernelGGL((gdn_pre_gate_kernel<BWD>), dim3((unsigned)((n + kPreThreads - 1) / kPreThreads)),
                           dim3(kPreThreads), 0, s, p);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

hipError_t launch_preprocess(const PreParams &p, int dk, int io_dtype, bool backward, hipStream_t s) {
    return backward ? pre_launch<true>(p, dk, io_dtype, s) : pre_launch<false>(p, dk, io_dtype, s);
}

}  // namespace gdn
