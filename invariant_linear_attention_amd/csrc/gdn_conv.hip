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
// with z recomputed exactly as the forward does.  One thread takes four consecutive
// channels (one, where rows do not start on a four-channel boundary) and walks a
// block of kConvBwdTokens tokens and K - 1 more (so that the block's last tokens
// see the dz they need), keeping the last K values of the input window, of dz and
// of the sequence ends in registers.  dw and dbias are sums over all tokens: each
// block writes its partial sums, added afterwards in a fixed order.

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

// V consecutive channels of one input element (V = 4: one 8- or 16-byte load).
template <class IO, int V>
__device__ __forceinline__ void load_chan(const void *base, size_t idx, float (&f)[V]) {
    if constexpr (V == 4) {
        const float4 r = IO::load4(base, idx);
        f[0] = r.x;
        f[1] = r.y;
        f[2] = r.z;
        f[3] = r.w;
    } else {
#pragma unroll
        for (int v = 0; v < V; ++v) f[v] = IO::load1(base, idx + v);
    }
}

template <int V>
__device__ __forceinline__ void load_chan_f32(const float *base, size_t idx, float (&f)[V]) {
    if constexpr (V == 4) {
        const float4 r = *reinterpret_cast<const float4 *>(base + idx);
        f[0] = r.x;
        f[1] = r.y;
        f[2] = r.z;
        f[3] = r.w;
    } else {
#pragma unroll
        for (int v = 0; v < V; ++v) f[v] = base[idx + v];
    }
}

template <int V>
__device__ __forceinline__ void store_chan_f32(float *base, size_t idx, const float (&f)[V]) {
    if constexpr (V == 4) {
        *reinterpret_cast<float4 *>(base + idx) = make_float4(f[0], f[1], f[2], f[3]);
    } else {
#pragma unroll
        for (int v = 0; v < V; ++v) base[idx + v] = f[v];
    }
}

// A token block that lies inside one sequence together with the K - 1 tokens before
// it and the K - 1 after it: no sequence end to watch, so the window is indexed by
// position within a group of G tokens and only its last K - 1 entries carry over.
// Every row address is the token's (uniform) plus the lane's 32-bit byte offset;
// dy (read once) and dx (written once) go past the caches with nontemporal hints.
// The arithmetic, operation by operation, is the general path's.
template <class IO, int K, int G>
__device__ __forceinline__ void conv_bwd_interior(const ConvBwdParams &p, int64_t t0, int64_t c0,
                                                  const float (&wc)[4][K], const float (&bc)[4], float (&pw)[4][K],
                                                  float (&pb)[4]) {
    constexpr int M = K - 1, V = 4, W = M + (G > M ? G : M);
    const size_t C = (size_t)p.channels;
    const uint32_t xo = (uint32_t)c0 * IO::ESZ, fo = (uint32_t)c0 * 4;
    const char *xb = static_cast<const char *>(p.x);
    const char *db = reinterpret_cast<const char *>(p.dy);
    char *ob = reinterpret_cast<char *>(p.dx);
    auto ldx = [&](int64_t t, float (&f)[V]) {
        const float4 r = IO::load4(xb + (size_t)t * C * IO::ESZ + xo, 0);
        f[0] = r.x;
        f[1] = r.y;
        f[2] = r.z;
        f[3] = r.w;
    };
    auto lddy = [&](int64_t t, float (&f)[V]) {
        const float4 *q = reinterpret_cast<const float4 *>(db + (size_t)t * C * 4 + fo);
        const float4 r = make_float4(__builtin_nontemporal_load(&q->x), __builtin_nontemporal_load(&q->y),
                                     __builtin_nontemporal_load(&q->z), __builtin_nontemporal_load(&q->w));
        f[0] = r.x;
        f[1] = r.y;
        f[2] = r.z;
        f[3] = r.w;
    };
    auto stdx = [&](int64_t s, const float (&f)[V]) {
        float4 *q = reinterpret_cast<float4 *>(ob + (size_t)s * C * 4 + fo);
        __builtin_nontemporal_store(f[0], &q->x);
        __builtin_nontemporal_store(f[1], &q->y);
        __builtin_nontemporal_store(f[2], &q->z);
        __builtin_nontemporal_store(f[3], &q->w);
    };
    // xs[v][i] = x(tg - M + i), ds[v][i] = dz(tg - M + i) for the group starting at tg
    float xs[V][W], ds[V][W];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        float f[V];
        ldx(t0 - M + j, f);
#pragma unroll
        for (int v = 0; v < V; ++v) {
            xs[v][j] = f[v];
            ds[v][j] = 0.f;
        }
    }
    for (int g0 = 0; g0 < kConvBwdTokens; g0 += G) {
        const int64_t tg = t0 + g0;
        float dr[G][V];
#pragma unroll
        for (int u = 0; u < G; ++u) {
            float f[V];
            ldx(tg + u, f);
            lddy(tg + u, dr[u]);
#pragma unroll
            for (int v = 0; v < V; ++v) xs[v][M + u] = f[v];
        }
#pragma unroll
        for (int u = 0; u < G; ++u) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
                float win[K];
#pragma unroll
                for (int j = 0; j < K; ++j) win[j] = xs[v][u + j];
                const float dz = conv_dz<IO, K>(p, wc[v], bc[v], win, dr[u][v]);
                ds[v][M + u] = dz;
#pragma unroll
                for (int j = 0; j < K; ++j) pw[v][j] = __builtin_fmaf(dz, win[j], pw[v][j]);
                pb[v] = pb[v] + dz;
            }
            if (g0 + u >= M) {  // dx of s = tg + u - M: dz(s .. s + M) are ds[u .. u + M]
                float dx[V];
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    dx[v] = 0.f;
#pragma unroll
                    for (int q = 0; q <= M; ++q) dx[v] = __builtin_fmaf(wc[v][M - q], ds[v][u + q], dx[v]);
                }
                stdx(tg + u - M, dx);
            }
        }
#pragma unroll
        for (int v = 0; v < V; ++v) {
#pragma unroll
            for (int j = 0; j < M; ++j) {
                xs[v][j] = xs[v][G + j];
                ds[v][j] = ds[v][G + j];
            }
        }
    }
    // the M tokens after the block: their dz (outside this block's sums) completes
    // the dx of the block's last M tokens
    const int64_t t1 = t0 + kConvBwdTokens;
    float dr[M][V];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        float f[V];
        ldx(t1 + i, f);
        lddy(t1 + i, dr[i]);
#pragma unroll
        for (int v = 0; v < V; ++v) xs[v][M + i] = f[v];
    }
#pragma unroll
    for (int i = 0; i < M; ++i) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
            float win[K];
#pragma unroll
            for (int j = 0; j < K; ++j) win[j] = xs[v][i + j];
            ds[v][M + i] = conv_dz<IO, K>(p, wc[v], bc[v], win, dr[i][v]);
        }
    }
#pragma unroll
    for (int i = 0; i < M; ++i) {
        float dx[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            dx[v] = 0.f;
#pragma unroll
            for (int q = 0; q <= M; ++q) dx[v] = __builtin_fmaf(wc[v][M - q], ds[v][i + q], dx[v]);
        }
        stdx(t1 - M + i, dx);
    }
}

// Any token block: the window refills from a state slot where a sequence starts, and
// dx sums only the dz of its own sequence.
template <class IO, int K, int V>
__device__ __forceinline__ void conv_bwd_general(const ConvBwdParams &p, int64_t t0, int64_t t1, int64_t c0, int n,
                                                 int64_t tb, int64_t te, const float (&wc)[V][K], const float (&bc)[V],
                                                 float (&pw)[V][K], float (&pb)[V]) {
    constexpr int M = K - 1, G = V == 4 ? 2 : (K <= 4 ? 8 : 4);
    const int64_t T = p.total_tokens, C = p.channels;
    // win[v][j] = input of token t - M + j (the state before the sequence's first token)
    float win[V][K];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        const int64_t s = t0 - M + j;
        if (s >= tb) {
            float f[V];
            load_chan<IO, V>(p.x, (size_t)s * C + c0, f);
#pragma unroll
            for (int v = 0; v < V; ++v) win[v][j] = f[v];
        } else {
#pragma unroll
            for (int v = 0; v < V; ++v) win[v][j] = state_at<IO>(p, n, c0 + v, (int)(s - tb + M), M);
        }
    }
    // dzr[v][i] = dz of token t - M + i and er[i] = the end of its sequence (dz of
    // tokens before the block is never used: their dx belongs to the block before)
    float dzr[V][K];
    int64_t er[K];
#pragma unroll
    for (int i = 0; i < K; ++i) er[i] = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
#pragma unroll
        for (int i = 0; i < K; ++i) dzr[v][i] = 0.f;
    }
    const int steps = (int)(t1 - t0) + M;
    for (int g0 = 0; g0 < steps; g0 += G) {
        float xr[G][V], dr[G][V];
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const int64_t t = t0 + g0 + u;
            if (g0 + u < steps && t < T) {
                load_chan<IO, V>(p.x, (size_t)t * C + c0, xr[u]);
                load_chan_f32<V>(p.dy, (size_t)t * C + c0, dr[u]);
            } else {
#pragma unroll
                for (int v = 0; v < V; ++v) xr[u][v] = dr[u][v] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < G; ++u) {
            if (g0 + u < steps) {
                const int64_t t = t0 + g0 + u;
                float dz[V];
                int64_t et = T;
#pragma unroll
                for (int v = 0; v < V; ++v) dz[v] = 0.f;
                if (t < T) {
                    if (t >= te) {  // a new sequence (empty ones skipped): its state fills the window
                        while (n + 1 < p.n_seqs && bclamp_cu(p, n + 1) <= t) ++n;
                        tb = bclamp_cu(p, n);
                        te = bclamp_cu(p, n + 1);
#pragma unroll
                        for (int v = 0; v < V; ++v) {
#pragma unroll
                            for (int j = 0; j < M; ++j) win[v][j] = state_at<IO>(p, n, c0 + v, j, M);
                        }
                    }
                    et = te;
#pragma unroll
                    for (int v = 0; v < V; ++v) {
                        win[v][M] = xr[u][v];
                        dz[v] = conv_dz<IO, K>(p, wc[v], bc[v], win[v], dr[u][v]);
                        if (t < t1) {  // this block's share of dw and dbias
#pragma unroll
                            for (int j = 0; j < K; ++j) pw[v][j] = __builtin_fmaf(dz[v], win[v][j], pw[v][j]);
                            pb[v] = pb[v] + dz[v];
                        }
#pragma unroll
                        for (int j = 0; j < M; ++j) win[v][j] = win[v][j + 1];
                    }
                }
#pragma unroll
                for (int j = 0; j < M; ++j) er[j] = er[j + 1];
                er[M] = et;
#pragma unroll
                for (int v = 0; v < V; ++v) {
#pragma unroll
                    for (int j = 0; j < M; ++j) dzr[v][j] = dzr[v][j + 1];
                    dzr[v][M] = dz[v];
                }
                const int64_t s = t - M;  // its dz and those of the M tokens after it are known
                if (s >= t0 && s < t1) {
                    float dx[V];
#pragma unroll
                    for (int v = 0; v < V; ++v) {
                        dx[v] = 0.f;
#pragma unroll
                        for (int q = 0; q <= M; ++q)
                            if (s + q < er[0]) dx[v] = __builtin_fmaf(wc[v][M - q], dzr[v][q], dx[v]);
                    }
                    store_chan_f32<V>(p.dx, (size_t)s * C + c0, dx);
                }
            }
        }
    }
}

// One thread: V consecutive channels of one token block.  In both paths the x and
// dy rows of G tokens are loaded together ahead of their use (the token loop's
// branches depend only on the token, so they are uniform across the workgroup).
template <class IO, int K, int V>
__global__ __launch_bounds__(kConvThreads) void gdn_conv_bwd_kernel(ConvBwdParams p) {
    constexpr int M = K - 1;
    const int64_t c0 = ((int64_t)blockIdx.y * kConvThreads + threadIdx.x) * V;
    const int64_t t0 = (int64_t)blockIdx.x * kConvBwdTokens;
    if (c0 >= p.channels || t0 >= p.total_tokens) return;
    const int64_t T = p.total_tokens, C = p.channels;
    const int64_t t1 = t0 + kConvBwdTokens < T ? t0 + kConvBwdTokens : T;
    float wc[V][K], bc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
#pragma unroll
        for (int j = 0; j < K; ++j) wc[v][j] = p.w[(c0 + v) * K + j];
        bc[v] = p.bias ? p.bias[c0 + v] : 0.f;
    }

    int n = bseq_of(p, t0);
    int64_t tb = bclamp_cu(p, n), te = bclamp_cu(p, n + 1);
    float pw[V][K], pb[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
#pragma unroll
        for (int i = 0; i < K; ++i) pw[v][i] = 0.f;
        pb[v] = 0.f;
    }
    if (V == 4 && tb <= t0 - M && t0 + kConvBwdTokens + M <= te) {
        if constexpr (V == 4) conv_bwd_interior<IO, K, 4>(p, t0, c0, wc, bc, pw, pb);
    } else {
        conv_bwd_general<IO, K, V>(p, t0, t1, c0, n, tb, te, wc, bc, pw, pb);
    }
    // partial sums, [block][K + 1][C]: the summing kernel reads them channel-contiguous
    float *part = p.partial + (size_t)blockIdx.x * (K + 1) * C + c0;
#pragma unroll
    for (int j = 0; j <= K; ++j) {
        float f[V];
#pragma unroll
        for (int v = 0; v < V; ++v) f[v] = j < K ? pw[v][j] : pb[v];
        store_chan_f32<V>(part + (size_t)j * C, 0, f);
    }
}

// dw and dbias from the blocks' partial sums: a workgroup takes 64 channels of one
// sum (a tap or the bias); its four waves add a quarter of the blocks each, in block
// order, and the quarters meet as (q0 + q1) + (q2 + q3).
template <int K>
__global__ __launch_bounds__(kConvThreads) void gdn_conv_bwd_sum_kernel(ConvBwdParams p) {
    __shared__ float qs[4][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, j = blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * 64 + lane, C = p.channels;
    const int64_t nblk = (p.total_tokens + kConvBwdTokens - 1) / kConvBwdTokens;
    const int64_t b0 = nblk * wv / 4, b1 = nblk * (wv + 1) / 4;
    float acc = 0.f;
    if (c < C) {
        const float *part = p.partial + (size_t)j * C + c;
#pragma unroll 8
        for (int64_t b = b0; b < b1; ++b) acc = acc + part[(size_t)b * (K + 1) * C];
    }
    qs[wv][lane] = acc;
    __syncthreads();
    if (wv != 0 || c >= C) return;
    const float s = (qs[0][lane] + qs[1][lane]) + (qs[2][lane] + qs[3][lane]);
    if (j < K) p.dw[c * K + j] = s;
    else if (p.dbias) p.dbias[c] = s;
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
        // four channels a thread where every row starts on a 4-channel boundary
        const bool vec4 = p.channels % 4 == 0 && (uintptr_t)p.x % (4 * IO::ESZ) == 0 &&
                          (uintptr_t)p.dy % 16 == 0 && (uintptr_t)p.dx % 16 == 0 && (uintptr_t)p.partial % 16 == 0;
        const unsigned tblocks = (unsigned)((p.total_tokens + kConvBwdTokens - 1) / kConvBwdTokens);
        if (vec4) {
            const unsigned c4 = (unsigned)((p.channels / 4 + kConvThreads - 1) / kConvThreads);
            hipLaunchKernelGGL((gdn_conv_bwd_kernel<IO, K, 4>), dim3(tblocks, c4), dim3(kConvThreads), 0, s, p);
        } else {
            hipLaunchKernelGGL((gdn_conv_bwd_kernel<IO, K, 1>), dim3(tblocks, cblocks), dim3(kConvThreads), 0, s,
                               p);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((gdn_conv_bwd_sum_kernel<K>), dim3((unsigned)((p.channels + 63) / 64), (unsigned)(K + 1)),
                       dim3(kConvThreads), 0, s, p);
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
