// gdn_conv.hip -- the short causal convolution with a carried state (gdn_short_conv).
//
// Per sequence n, channel c and token t, with K taps (fixed fp32 order, the same
// for every call shape, so a decode step -- one token per sequence -- and a cut
// prefill give the bits of one long prefill):
//     z = bias[c];  z = fma(w[c][j], x(t - (K-1) + j, c), z) for j = 0 .. K-1;
//     y = z * sigmoid(z)  (with SiLU), rounded to the io dtype.
// x(s, c) before the sequence's first token comes from the state slot.  Two
// launches on the caller's stream: the outputs (reading the old state), then the
// new states; the stream orders them, so a slot may be updated in place.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"
#include "gdn_internal.hpp"
#include "gdn_kernels.hpp"

namespace gdn {
namespace {

constexpr int kConvThreads = 256;  // consecutive channels of one token group

__device__ __forceinline__ int64_t clamp_cu(const ConvParams &p, int i) {
    int64_t v = p.cu_seqlens[i];
    return v < 0 ? 0 : (v > p.total_tokens ? p.total_tokens : v);
}

__device__ __forceinline__ int64_t slot_of(const int32_t *idx, int n, int pool_size) {
    const int64_t s = idx ? (int64_t)idx[n] : (int64_t)n;
    return (s >= 0 && s < pool_size) ? s : -1;
}

// Sequence holding token t: the last n with cu[n] <= t (uniform: t is the same
// for the whole workgroup), clamped into [0, N-1].  The proportional guess
// t * N / T is exact for equal lengths (decode: one token per sequence); otherwise
// a binary search.
__device__ int seq_of(const ConvParams &p, int64_t t) {
    const int g = (int)(t * p.n_seqs / (p.total_tokens > 0 ? p.total_tokens : 1));
    if (g < p.n_seqs && clamp_cu(p, g) <= t && clamp_cu(p, g + 1) > t) return g;
    int lo = 0, hi = p.n_seqs;  // answer in [lo, hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (clamp_cu(p, mid) <= t) lo = mid; else hi = mid;
    }
    return lo;
}

// One thread: VEC consecutive channels (16 bytes) of TOK consecutive tokens, a
// fully unrolled sliding window over 16-byte input rows (coalesced across the
// workgroup's channels), each row read once.  A token group inside one sequence
// loads all its rows up front; a group that meets a sequence start goes token by
// token, refilling the window from the new sequence's state.  TOK = 1 serves
// calls whose sequences are a token or two long (decode).
template <class IO, int K, int TOK>
__global__ __launch_bounds__(kConvThreads) void gdn_conv_kernel(ConvParams p) {
    constexpr int M = K - 1, V = IO::VEC;
    constexpr int kConvTokens = TOK;
    const int64_t cv = p.channels / V;  // 16-byte vectors per token row
    const int64_t vblocks = (cv + kConvThreads - 1) / kConvThreads;
    const int64_t t0 = (int64_t)(blockIdx.x / vblocks) * kConvTokens;
    const int64_t vec = (int64_t)(blockIdx.x % vblocks) * kConvThreads + threadIdx.x;
    if (vec >= cv || t0 >= p.total_tokens) return;
    const int64_t c0 = vec * V;

    auto row = [&](int64_t s, float (&f)[V]) {  // inputs of token s (zero outside [0, T))
        uint4 r = make_uint4(0, 0, 0, 0);
        if (s >= 0 && s < p.total_tokens)
            r = *reinterpret_cast<const uint4 *>(static_cast<const char *>(p.x) + ((size_t)s * p.channels + c0) * IO::ESZ);
        IO::unpack(r, f);
    };
    float wc[V][K], bc[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
#pragma unroll
        for (int j = 0; j < K; ++j) wc[e][j] = p.w[(c0 + e) * K + j];
        bc[e] = p.bias ? p.bias[c0 + e] : 0.f;
    }

    int n = seq_of(p, t0);
    int64_t tb = clamp_cu(p, n), te = clamp_cu(p, n + 1);
    auto emit = [&](int64_t t, const float (&wv)[K][V]) {
        float yv[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
            float z = bc[e];
#pragma unroll
            for (int j = 0; j < K; ++j) z = __builtin_fmaf(wc[e][j], wv[j][e], z);
            yv[e] = p.silu ? z * sigmoid_f32(z) : z;
        }
        IO::store_vec(p.y, (size_t)t * p.channels + c0, yv);
    };
    if (TOK > 1 && t0 - M >= tb && t0 + TOK <= te) {  // inside one sequence: straight-line
        uint4 raw[TOK + M];
#pragma unroll
        for (int r = 0; r < TOK + M; ++r)
            raw[r] = *reinterpret_cast<const uint4 *>(static_cast<const char *>(p.x) +
                                                      ((size_t)(t0 - M + r) * p.channels + c0) * IO::ESZ);
        float wv[K][V];
#pragma unroll
        for (int j = 0; j < M; ++j) IO::unpack(raw[j], wv[j]);
#pragma unroll
        for (int i = 0; i < TOK; ++i) {
            IO::unpack(raw[i + M], wv[M]);
            emit(t0 + i, wv);
#pragma unroll
            for (int j = 0; j < M; ++j) {
#pragma unroll
                for (int e = 0; e < V; ++e) wv[j][e] = wv[j + 1][e];
            }
        }
        return;
    }
    // win[j] = inputs of token t - M + j: x rows inside the sequence, state before it.
    float win[K][V];
    auto state_window = [&]() {  // the window before the first token of sequence n
        const int64_t src = slot_of(p.src_idx, n, p.pool_size);
        // this thread's V channels hold M values each, contiguous: M 16-byte words
        float stv[M * V];
#pragma unroll
        for (int q = 0; q < M; ++q) {
            uint4 r = make_uint4(0, 0, 0, 0);
            if (src >= 0)
                r = *reinterpret_cast<const uint4 *>(static_cast<const char *>(p.state) +
                                                      (((size_t)src * p.channels + c0) * M + (size_t)q * V) * IO::ESZ);
            float f[V];
            IO::unpack(r, f);
#pragma unroll
            for (int e = 0; e < V; ++e) stv[q * V + e] = f[e];
        }
#pragma unroll
        for (int j = 0; j < M; ++j) {
#pragma unroll
            for (int e = 0; e < V; ++e) win[j][e] = stv[e * M + j];
        }
    };
    if (t0 == tb) {
        state_window();
    } else {
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const int64_t s = t0 - M + j;
            if (s >= tb) {
                row(s, win[j]);
            } else {  // the group starts fewer than M tokens into the sequence
                const int64_t src = slot_of(p.src_idx, n, p.pool_size);
#pragma unroll
                for (int e = 0; e < V; ++e)
                    win[j][e] = src >= 0 ? IO::load1(p.state, ((size_t)src * p.channels + c0 + e) * M + (s - tb + M)) : 0.f;
            }
        }
    }
    const int nt = (int)((p.total_tokens - t0) < kConvTokens ? (p.total_tokens - t0) : kConvTokens);
#pragma unroll
    for (int i = 0; i < kConvTokens; ++i) {
        if (i >= nt) continue;  // uniform; keeps every register index static
        const int64_t t = t0 + i;
        if (t >= te) {  // a sequence starts at t (empty ones skipped): its state fills the window
            while (n + 1 < p.n_seqs && clamp_cu(p, n + 1) <= t) ++n;
            tb = clamp_cu(p, n);
            te = clamp_cu(p, n + 1);
            state_window();
        }
        row(t, win[M]);
        emit(t, win);
#pragma unroll
        for (int j = 0; j < M; ++j) {
#pragma unroll
            for (int e = 0; e < V; ++e) win[j][e] = win[j + 1][e];
        }
    }
}

// New state of (sequence blockIdx.y, VEC channels per thread): its last K-1 inputs.
// The VEC channels' states are M * VEC contiguous values (channel-major), moved as
// M 16-byte words.
template <class IO, int K>
__global__ __launch_bounds__(kConvThreads) void gdn_conv_state_kernel(ConvParams p) {
    constexpr int M = K - 1, V = IO::VEC;
    const int64_t vec = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
    const int n = blockIdx.y;
    if (vec >= p.channels / V) return;
    const int64_t c0 = vec * V;
    const int64_t dst = slot_of(p.dst_idx, n, p.pool_size);
    if (dst < 0) return;
    const int64_t src = slot_of(p.src_idx, n, p.pool_size);
    const int64_t tb = clamp_cu(p, n);
    int64_t te = clamp_cu(p, n + 1);
    te = te < tb ? tb : te;
    const int64_t len = te - tb;
    float v[M][V];  // v[m][e]: new state entry m of channel c0 + e (read all first: dst may be src)
    float old[M * V];  // the old state block, needed when the sequence is shorter than M
    if (len < M) {
#pragma unroll
        for (int q = 0; q < M; ++q) {
            uint4 r = make_uint4(0, 0, 0, 0);
            if (src >= 0)
                r = *reinterpret_cast<const uint4 *>(static_cast<const char *>(p.state) +
                                                      (((size_t)src * p.channels + c0) * M + (size_t)q * V) * IO::ESZ);
            float f[V];
            IO::unpack(r, f);
#pragma unroll
            for (int e = 0; e < V; ++e) old[q * V + e] = f[e];
        }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int64_t s = te - M + m;
        if (s >= tb) {  // uniform
            const uint4 r = *reinterpret_cast<const uint4 *>(static_cast<const char *>(p.x) +
                                                             ((size_t)s * p.channels + c0) * IO::ESZ);
            IO::unpack(r, v[m]);
        } else {  // old entry m + len, with len < M - m: one static case per length
#pragma unroll
            for (int L = 0; L < M - m; ++L)
                if (len == L) {
#pragma unroll
                    for (int e = 0; e < V; ++e) v[m][e] = old[e * M + m + L];
                }
        }
    }
#pragma unroll
    for (int q = 0; q < M; ++q) {
        float f[V];
#pragma unroll
        for (int i = 0; i < V; ++i) f[i] = v[(q * V + i) % M][(q * V + i) / M];
        IO::store_vec(p.state, ((size_t)dst * p.channels + c0) * M + (size_t)q * V, f);
    }
}

template <class IO, int K>
hipError_t launch_k(const ConvParams &p, hipStream_t s) {
    const int64_t vblocks = (p.channels / IO::VEC + kConvThreads - 1) / kConvThreads;
    // sequences averaging under 4 tokens (decode): one token per thread
    const bool shortseq = p.total_tokens < 4 * (int64_t)p.n_seqs;
    const int tok = shortseq ? 1 : 16;
    const int64_t tgroups = (p.total_tokens + tok - 1) / tok;
    void *args[] = {const_cast<ConvParams *>(&p)};
    if (tgroups > 0) {
        const void *fn = shortseq ? reinterpret_cast<const void *>(&gdn_conv_kernel<IO, K, 1>)
                                  : reinterpret_cast<const void *>(&gdn_conv_kernel<IO, K, 16>);
        const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)(tgroups * vblocks)), dim3(kConvThreads), args, 0, s);
        if (e != hipSuccess) return e;
    }
    return hipLaunchKernel(reinterpret_cast<const void *>(&gdn_conv_state_kernel<IO, K>),
                           dim3((unsigned)vblocks, (unsigned)p.n_seqs), dim3(kConvThreads), args, 0, s);
}

template <class IO>
hipError_t launch_io(const ConvParams &p, hipStream_t s) {
    switch (p.taps) {
        case 2: return launch_k<IO, 2>(p, s);
        case 3: return launch_k<IO, 3>(p, s);
        case 4: return launch_k<IO, 4>(p, s);
        case 5: return launch_k<IO, 5>(p, s);
        case 6: return launch_k<IO, 6>(p, s);
        case 7: return launch_k<IO, 7>(p, s);
        case 8: return launch_k<IO, 8>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_short_conv(const ConvParams &p, int io_dtype, hipStream_t s) {
    return io_dtype == GDN_BF16 ? launch_io<IoBf16>(p, s) : launch_io<IoF32>(p, s);
}

// ------------------------------------------------------------------------ backward
//
// Gradients of the convolution given dy = dL/dy (fp32):
//     dz(t) = dy(t) * (sigmoid(z) (1 + z (1 - sigmoid(z))))   (SiLU; else dz = dy)
//     dx(s) = sum_{i=0}^{K-1} w[K-1-i] dz(s + i)     (tokens of s's own sequence)
//     dw[c][j] = sum_t dz(t) x(t - (K-1) + j),  dbias[c] = sum_t dz(t)
//     dstate[n][c][m] = sum_{j<=m} w[j] dz(tb + m - j)   (the carried state's gradient)
// with z recomputed exactly as the forward does.  One thread per channel walks a
// block of kConvBwdTokens tokens and K - 1 more (so that the block's last tokens
// see the dz they need), keeping the last K values of the input window, of dz and
// of the sequence ends in registers.  dw and dbias are sums over all tokens: each
// block writes its partial sums, added block by block afterwards.

namespace {

constexpr int kConvBwdTokens = 64;

template <class IO, int K>
__device__ __forceinline__ float conv_dz(const ConvBwdParams &p, const float (&wc)[K], float bc, const float (&win)[K],
                                         float dy) {
    float z = bc;
#pragma unroll
    for (int j = 0; j < K; ++j) z = __builtin_fmaf(wc[j], win[j], z);
    if (!p.silu) return dy;
    const float sg = sigmoid_f32(z);
    return dy * (sg * (1.f + z * (1.f - sg)));
}

template <class IO>
__device__ __forceinline__ float state_at(const ConvBwdParams &p, int n, int64_t c, int m, int M) {
    const int64_t src = slot_of(p.src_idx, n, p.pool_size);
    return src >= 0 ? IO::load1(p.state, ((size_t)src * p.channels + c) * M + m) : 0.f;
}

__device__ __forceinline__ int64_t bclamp_cu(const ConvBwdParams &p, int i) {
    int64_t v = p.cu_seqlens[i];
    return v < 0 ? 0 : (v > p.total_tokens ? p.total_tokens : v);
}

__device__ int bseq_of(const ConvBwdParams &p, int64_t t) {
    int lo = 0, hi = p.n_seqs;  // the last n with cu[n] <= t, in [lo, hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (bclamp_cu(p, mid) <= t) lo = mid; else hi = mid;
    }
    return lo;
}

template <class IO, int K>
__global__ __launch_bounds__(kConvThreads) void gdn_conv_bwd_kernel(ConvBwdParams p) {
    constexpr int M = K - 1;
    const int64_t c = (int64_t)blockIdx.y * kConvThreads + threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * kConvBwdTokens;
    if (c >= p.channels || t0 >= p.total_tokens) return;
    const int64_t T = p.total_tokens, C = p.channels;
    const int64_t t1 = t0 + kConvBwdTokens < T ? t0 + kConvBwdTokens : T;
    float wc[K];
#pragma unroll
    for (int j = 0; j < K; ++j) wc[j] = p.w[c * K + j];
    const float bc = p.bias ? p.bias[c] : 0.f;

    int n = bseq_of(p, t0);
    int64_t tb = bclamp_cu(p, n), te = bclamp_cu(p, n + 1);
    // win[j] = input of token t - M + j (the state before the sequence's first token)
    float win[K];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        const int64_t s = t0 - M + j;
        win[j] = s >= tb ? IO::load1(p.x, (size_t)s * C + c) : state_at<IO>(p, n, c, (int)(s - tb + M), M);
    }
    // dzr[i] = dz of token t - M + i and er[i] = the end of its sequence (dz of tokens
    // before the block is never used: their dx belongs to the block before)
    float dzr[K];
    int64_t er[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
        dzr[i] = 0.f;
        er[i] = 0;
    }
    float pw[K], pb = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) pw[j] = 0.f;
    const int steps = (int)(t1 - t0) + M;
    for (int i = 0; i < steps; ++i) {
        const int64_t t = t0 + i;
        float dz = 0.f;
        int64_t et = T;
        if (t < T) {
            if (t >= te) {  // a new sequence (empty ones skipped): its state fills the window
                while (n + 1 < p.n_seqs && bclamp_cu(p, n + 1) <= t) ++n;
                tb = bclamp_cu(p, n);
                te = bclamp_cu(p, n + 1);
#pragma unroll
                for (int j = 0; j < M; ++j) win[j] = state_at<IO>(p, n, c, j, M);
            }
            win[M] = IO::load1(p.x, (size_t)t * C + c);
            dz = conv_dz<IO, K>(p, wc, bc, win, p.dy[(size_t)t * C + c]);
            et = te;
            if (t < t1) {  // this block's share of dw and dbias
#pragma unroll
                for (int j = 0; j < K; ++j) pw[j] = __builtin_fmaf(dz, win[j], pw[j]);
                pb = pb + dz;
            }
#pragma unroll
            for (int j = 0; j < M; ++j) win[j] = win[j + 1];
        }
#pragma unroll
        for (int j = 0; j < M; ++j) {
            dzr[j] = dzr[j + 1];
            er[j] = er[j + 1];
        }
        dzr[M] = dz;
        er[M] = et;
        const int64_t s = t - M;  // its dz and those of the M tokens after it are known
        if (s >= t0 && s < t1) {
            float dx = 0.f;
#pragma unroll
            for (int q = 0; q <= M; ++q)
                if (s + q < er[0]) dx = __builtin_fmaf(wc[M - q], dzr[q], dx);
            p.dx[(size_t)s * C + c] = dx;
        }
    }
    float *part = p.partial + ((size_t)blockIdx.x * C + c) * (K + 1);
#pragma unroll
    for (int j = 0; j < K; ++j) part[j] = pw[j];
    part[K] = pb;
}

// dw and dbias: the blocks' partial sums, block by block.
template <int K>
__global__ __launch_bounds__(kConvThreads) void gdn_conv_bwd_sum_kernel(ConvBwdParams p) {
    const int64_t c = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
    if (c >= p.channels) return;
    const int64_t nblk = (p.total_tokens + kConvBwdTokens - 1) / kConvBwdTokens;
    float acc[K + 1];
#pragma unroll
    for (int j = 0; j <= K; ++j) acc[j] = 0.f;
    for (int64_t b = 0; b < nblk; ++b) {
        const float *part = p.partial + ((size_t)b * p.channels + c) * (K + 1);
#pragma unroll
        for (int j = 0; j <= K; ++j) acc[j] = acc[j] + part[j];
    }
#pragma unroll
    for (int j = 0; j < K; ++j) p.dw[c * K + j] = acc[j];
    if (p.dbias) p.dbias[c] = acc[K];
}

// The carried state's gradient of (sequence blockIdx.y, channel): the window of its
// first K - 1 tokens, dz recomputed as above.
template <class IO, int K>
__global__ __launch_bounds__(kConvThreads) void gdn_conv_bwd_state_kernel(ConvBwdParams p) {
    constexpr int M = K - 1;
    const int64_t c = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
    const int n = blockIdx.y;
    if (c >= p.channels) return;
    const int64_t C = p.channels;
    const int64_t tb = bclamp_cu(p, n);
    int64_t te = bclamp_cu(p, n + 1);
    te = te < tb ? tb : te;
    const int64_t len = te - tb;
    float wc[K];
#pragma unroll
    for (int j = 0; j < K; ++j) wc[j] = p.w[c * K + j];
    const float bc = p.bias ? p.bias[c] : 0.f;
    float win[K], dz[M];
#pragma unroll
    for (int j = 0; j < M; ++j) win[j] = state_at<IO>(p, n, c, j, M);
#pragma unroll
    for (int i = 0; i < M; ++i) {
        dz[i] = 0.f;
        if (i < len) {
            win[M] = IO::load1(p.x, (size_t)(tb + i) * C + c);
            dz[i] = conv_dz<IO, K>(p, wc, bc, win, p.dy[(size_t)(tb + i) * C + c]);
#pragma unroll
            for (int j = 0; j < M; ++j) win[j] = win[j + 1];
        }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        float v = 0.f;
#pragma unroll
        for (int j = 0; j <= m; ++j)
            if (m - j < len) v = __builtin_fmaf(wc[j], dz[m - j], v);
        p.dstate[((size_t)n * C + c) * M + m] = v;
    }
}

template <class IO, int K>
hipError_t conv_bwd_launch(const ConvBwdParams &p, hipStream_t s) {
    const unsigned cblocks = (unsigned)((p.channels + kConvThreads - 1) / kConvThreads);
    if (p.total_tokens > 0) {
        const unsigned tblocks = (unsigned)((p.total_tokens + kConvBwdTokens - 1) / kConvBwdTokens);
        hipLaunchKernelGGL((gdn_conv_bwd_kernel<IO, K>), dim3(tblocks, cblocks), dim3(kConvThreads), 0, s, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((gdn_conv_bwd_sum_kernel<K>), dim3(cblocks), dim3(kConvThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.dstate || p.n_seqs == 0) return e;
    hipLaunchKernelGGL((gdn_conv_bwd_state_kernel<IO, K>), dim3(cblocks, (unsigned)p.n_seqs), dim3(kConvThreads), 0,
                       s, p);
    return hipGetLastError();
}

template <class IO>
hipError_t conv_bwd_io(const ConvBwdParams &p, hipStream_t s) {
    switch (p.taps) {
        case 2: return conv_bwd_launch<IO, 2>(p, s);
        case 3: return conv_bwd_launch<IO, 3>(p, s);
        case 4: return conv_bwd_launch<IO, 4>(p, s);
        case 5: return conv_bwd_launch<IO, 5>(p, s);
        case 6: return conv_bwd_launch<IO, 6>(p, s);
        case 7: return conv_bwd_launch<IO, 7>(p, s);
        case 8: return conv_bwd_launch<IO, 8>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

uint64_t conv_bwd_workspace_bytes(int64_t T, int64_t C, int K) {
    return (uint64_t)((T + kConvBwdTokens - 1) / kConvBwdTokens) * C * (K + 1) * 4;
}

hipError_t launch_short_conv_backward(const ConvBwdParams &p, int io_dtype, hipStream_t s) {
    return io_dtype == GDN_BF16 ? conv_bwd_io<IoBf16>(p, s) : conv_bwd_io<IoF32>(p, s);
}

}  // namespace gdn
