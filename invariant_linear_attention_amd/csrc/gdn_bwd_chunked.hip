// gdn_bwd_chunked.hip -- gradients of the gated delta rule in the chunked (WY) form,
// on the matrix cores (gdn_bwd_chunked).
//
// The page "Defending Against the Training-Inference Numeric Mismatch in RL
// (Especially Linear Attention)" (section 3.2, "Solution") runs the recurrence token
// by token in every forward and keeps the chunked kernel for the training backward.
// This is that backward: the gradients of the same recurrence, taken chunk by chunk
// (16 tokens at positions 16c .. 16c + 15 of a sequence) with every product against a
// state on fp32 MFMA.
//
// Within a chunk (notation of gdn_chunked.hip: S0 the state at its start, Gam_{m,s}
// the decay products, Gam_m = Gam_{m,0} a_0, T = (I + A)^-1, B[m][s] = Gam_{m,s}
// (q_m . k_s), x_m = v_m - Gam_m S0 k_m, R = beta x, U = T R, O = Gam S0 Q + B U, and
// the state after the chunk's last token l: S1 = Gam_l S0 + sum_s Gam_{l,s} u_s k_s^T),
// given D = dL/dS1 and dO:
//
//     E     = K D^T                          dU = B^T dO + Gam_{l,.} E
//     dR    = T^T dU                         dv = beta dR
//     dB    = dO U^T  (s <= m)               dA = -dR U^T  (s < m)
//     dq_m  = Gam_m S0^T dO_m + sum_s dB[m][s] Gam_{m,s} k_s
//     dk_s  = -beta_s Gam_s S0^T dR_s + Gam_{l,s} D^T u_s + sum_m dB[m][s] Gam_{m,s} q_m
//             + sum_r (H[s][r] + H[r][s]) k_r,        H[m][r] = dA[m][r] beta_m Gam_{m,r}
//     dbeta_m = dR_m . x_m + sum_r dA[m][r] Gam_{m,r} (k_m . k_r)
//     dL/dS0 = Gam_l D + sum_m Gam_m dO_m q_m^T - sum_m beta_m Gam_m dR_m k_m^T
//
// and the gate gradient needs no derivative of the decay products: with Phi_t =
// <dL/dS_t, S_t>, dg_t = <dhT, hT> + sum_{s >= t} (dO_s . o_s - dv_s . v_s) over the
// sequence, and dO_s . o_s = q_s . dq_s (dq of this value head).
//
// Launches: the chunked form's prep kernel (records with T, B, Gam and the two extra
// tables), its main kernel as a forward walk that stores the state at every chunk's
// start and x = v - Gam P, then the reverse walk below (one workgroup per sequence and
// value head, all of its state in the workgroup) and, when value heads share key
// heads, a fixed-order sum of dq and dk over them.  Every sum has a fixed order and
// nothing crosses sequences, so the gradients are deterministic and batch-invariant.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.hpp"
#include "gdn_mfma.hpp"

#pragma clang fp contract(off)

namespace gdn {
namespace {

constexpr int kCk = kChunkLen;

// What one chunk of the reverse walk reads from global memory, per lane.
template <int DK, int DV, class IO, int P>
struct RevFetch {
    static constexpr int NW = DV / 16 / P, NT = DK / 16, CTW = (NT + NW - 1) / NW, RT = NW;
    static constexpr int KITEMS = kCk * DK / 4;                      // 4-element items of a K (or Q) tile
    static constexpr int KIT = (KITEMS + 64 * NW - 1) / (64 * NW);   // per lane
    static constexpr int EPT = (kCk * kCk + 64 * NW - 1) / (64 * NW);  // 16 x 16 entries per lane
    typename Raw4<IO>::T kr[KIT], qr[KIT];
    uint32_t dor[4], vr[4];   // dO and v bits, token 4 g + c, row r0 + x
    float xr[4];              // x = v - Gam P, same place
    float4 bet, gam, wl;      // beta, Gam_m and Gam_{l,m} of tokens 4 g .. 4 g + 3
    float bx, gx, wx, gl;     // beta, Gam and Gam_{l,x} of token x; Gam_l
    float4 trow;              // T[x][4 g ..]
    float tcol[4], bcol[4];   // T[4 g + c][x], B[4 g + c][x]
    float ge[EPT], ae[EPT], be[EPT];  // Gam_{m,s}, Gam_{m,s} (k_m . k_s) and beta_m of entries tid + 64 NW e
};

// P workgroups per (sequence, value head), each of dv / (16 P) waves: part p owns the
// adjoint state's rows p dv/P .. (p + 1) dv/P - 1, wave w of it rows 16 w .. 16 w + 15
// of those (all dk columns, as MFMA accumulators) and, for the products over the
// part's rows, the column tiles w, w + NW, ...  The state rows of D are independent of
// one another; only the sums over rows (dB, dA, dq, dk, dbeta and the terms of dg)
// couple them, and each of those is linear in its rows' contributions, so each part
// writes its own partial results and a last kernel adds the parts in order (P = 1:
// the results themselves).  Per chunk, from the last:
//   P1  E, dU, dR, U on the wave's rows; dv; the token rows of dO, dR and U and D into
//       LDS; D moved to the chunk's start; (wave 0) the previous chunk's per-token results
//   P2  the wave's partial dB, dA over its rows; dq0 and dk1 on its column tiles
//   P3  dB, dA summed over the waves; the dA part of dbeta
//   P4  the in-chunk terms of dq and dk; stores; q . dq
// with one LDS barrier between phases.  Keys and queries and the per-token sums are
// double-buffered by chunk parity, so no barrier is needed between P4 and the next
// chunk's staging.
template <int DK, int DV, class IO, int P>
__global__ __launch_bounds__(64 * (DV / 16 / P)) void gdn_bwd_chunk_rev_kernel(BwdChunkParams p) {
    using RF = RevFetch<DK, DV, IO, P>;
    using RW = Raw4<IO>;
    constexpr int NW = RF::NW, NT = RF::NT, CTW = RF::CTW, RT = RF::RT;
    constexpr int DVP = DV / P;  // state rows of one part
    constexpr int KP = DK + 4, VP = DVP + 4;
    constexpr int NTH = 64 * NW;
    // (16-byte aligned: read and written as float4)
    __shared__ __align__(16) float Ks[2][kCk][KP];
    __shared__ __align__(16) float Qs[2][kCk][KP];
    __shared__ __align__(16) float dOs[kCk][VP];  // token rows of dO, dR and U
    __shared__ __align__(16) float dRs[kCk][VP];
    __shared__ __align__(16) float Us[kCk][VP];
    __shared__ __align__(16) float Ds[DVP][KP];   // D = dL/dS at the chunk's end (the part's rows)
    __shared__ float dBp[NW][kCk][kCk + 1], dAp[NW][kCk][kCk + 1];
    __shared__ float Ms[kCk][kCk + 1], Hs[kCk][kCk + 1];  // dB Gam (s <= m), dA beta Gam (s < m)
    __shared__ float abrow[kCk];                          // sum_s dA[m][s] Gam_{m,s} (k_m . k_s)
    __shared__ __align__(16) float red[2][NW][kCk][4];    // per parity, wave and token: dR.x, dv.v, q.dq
    __shared__ __align__(16) float phis[kCk];             // wave 0: the chunk's phi of every token

    // (the wave index as a uniform value, so that tests on it are scalar branches)
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int x = lane & 15, g = lane >> 4;
    // Workgroups that read the same keys and queries (one sequence and key head) get
    // ids equal modulo 8, so they run on one XCD and share its L2.
    int rank, h, part;
    {
        const int G = p.hv / p.hk * P;  // (value head, part) pairs of a key head
        const int ngroups = p.n_seqs * p.hk;
        const int full = (ngroups / 8) * 8 * G;
        const int id = blockIdx.x;
        int grp, member;
        if (id < full) {
            const int xcd = id % 8, slot = id / 8;
            grp = (slot / G) * 8 + xcd;
            member = slot % G;
        } else {
            grp = full / G + (id - full) / G;
            member = (id - full) % G;
        }
        rank = grp / p.hk;
        h = (grp % p.hk) * (G / P) + member / P;
        part = member % P;
    }
    const int n = p.rank_by_length ? seq_by_length_rank(p.cu_seqlens, p.n_seqs, rank, tid, NTH) : rank;
    const int kh = h / (p.hv / p.hk);
    const int r0 = 16 * wave;           // this wave's state rows within the part
    const int rg = part * DVP + r0;     // the same rows within the head
    int64_t tb = p.cu_seqlens[n], te = p.cu_seqlens[n + 1];
    tb = tb < 0 ? 0 : (tb > p.total_tokens ? p.total_tokens : tb);
    te = te < tb ? tb : (te > p.total_tokens ? p.total_tokens : te);
    const int64_t len = te - tb;
    const int64_t base = chunk_slot_base(tb, n);
    int nch = (int)((len + kCk - 1) / kCk);
    if (base + nch > p.ws_slots) nch = (int)(p.ws_slots - base > 0 ? p.ws_slots - base : 0);
    const size_t vrow = (size_t)p.hv * DV;
    constexpr uint32_t E = IO::ESZ;
    const uint32_t krow_b = (uint32_t)p.hk * DK * E, vrow_b = (uint32_t)vrow * E;

    // D = dL/dS, rows r0 .. r0 + 15, held transposed: lane x + 16 g, tile t, component c
    // is D[r0 + x][16 t + 4 g + c]
    f4 Dt[NT];
    {
        const float *src = p.dhT ? p.dhT + (((size_t)n * p.hv + h) * DV + rg + x) * DK : nullptr;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            Dt[t] = f4_zero();
            if (src) {
                const float4 v4 = *reinterpret_cast<const float4 *>(src + 16 * t + 4 * g);
                Dt[t] = f4{v4.x, v4.y, v4.z, v4.w};
            }
        }
    }
    // <dhT, hT> over the part's rows from the forward walk's partial sums (four per
    // 16-row tile), in order: the start of the part's dg running sum
    float carry = 0.f;
    if (p.dhT)
        for (int i = part * (DVP / 16) * 4; i < (part + 1) * (DVP / 16) * 4; ++i)
            carry = carry + p.hdot[((size_t)n * p.hv + h) * p.hdot_parts + i];

    auto chunk_m1 = [&](int j) {
        const int64_t left = len - (int64_t)kCk * j;
        return left < kCk ? (int)left : kCk;
    };
    auto fetch = [&](RF &F, int j_) {
        const int j = j_ < 0 ? 0 : j_;  // past the first chunk: repeat its reads
        const int m1 = chunk_m1(j);
        const int64_t t0 = tb + (int64_t)kCk * j;
        const char *kb = static_cast<const char *>(p.k) + ((size_t)t0 * p.hk + kh) * DK * E;
        const char *qb = static_cast<const char *>(p.q) + ((size_t)t0 * p.hk + kh) * DK * E;
#pragma unroll
        for (int s = 0; s < RF::KIT; ++s) {
            int it = tid + NTH * s;
            it = it < RF::KITEMS ? it : RF::KITEMS - 1;
            const int m = it / (DK / 4), c = 4 * (it % (DK / 4));
            const uint32_t off = (uint32_t)(m < m1 ? m : m1 - 1) * krow_b + (uint32_t)c * E;
            F.kr[s] = RW::load_at(kb, off);
            F.qr[s] = RW::load_at(qb, off);
        }
        const char *ob = static_cast<const char *>(p.dout) + ((size_t)t0 * p.hv + h) * DV * E;
        const char *vb = static_cast<const char *>(p.v) + ((size_t)t0 * p.hv + h) * DV * E;
        // x: the forward walk's [row][token] tile of this chunk and 16 rows (tokens
        // 4 g .. 4 g + 3 of row x in one 16-byte piece)
        const float4 x4 = *reinterpret_cast<const float4 *>(
            p.xv + (((size_t)(base + j) * p.hv + h) * DV + rg) * kCk + x * kCk + 4 * g);
        F.xr[0] = x4.x;
        F.xr[1] = x4.y;
        F.xr[2] = x4.z;
        F.xr[3] = x4.w;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t tm = (uint32_t)(4 * g + c < m1 ? 4 * g + c : m1 - 1);
            F.dor[c] = RW::load1_at(ob, tm * vrow_b + (uint32_t)(rg + x) * E);
            F.vr[c] = RW::load1_at(vb, tm * vrow_b + (uint32_t)(rg + x) * E);
        }
        const float *rec = p.rec + ((size_t)(base + j) * p.hv + h) * kChunkRecBwd;
        const int l = m1 - 1;
        F.bet = *reinterpret_cast<const float4 *>(rec + kRecBeta + 4 * g);
        F.gam = *reinterpret_cast<const float4 *>(rec + kRecGam + 4 * g);
        F.wl = *reinterpret_cast<const float4 *>(rec + kRecGm + l * kCk + 4 * g);
        F.bx = rec[kRecBeta + x];
        F.gx = rec[kRecGam + x];
        F.wx = rec[kRecGm + l * kCk + x];
        F.gl = rec[kRecGam + l];
        F.trow = *reinterpret_cast<const float4 *>(rec + kRecT + x * kCk + 4 * g);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            F.tcol[c] = rec[kRecT + (4 * g + c) * kCk + x];
            F.bcol[c] = rec[kRecB + (4 * g + c) * kCk + x];
        }
#pragma unroll
        for (int e = 0; e < RF::EPT; ++e) {
            int i = tid + NTH * e;
            i = i < kCk * kCk ? i : kCk * kCk - 1;
            F.ge[e] = rec[kRecGm + i];
            F.ae[e] = rec[kRecAb + i];
            F.be[e] = rec[kRecBeta + i / kCk];
        }
    };
    // The chunk's start state on this wave's column tiles, as MFMA B operands over the
    // part's rows: s0[rt][l2][c] = S0[part DVP + 16 rt + 4 g + c][16 (wave + NW l2) + x]
    // (read a chunk ahead, once the current one is no longer needed).
    f4 s0[RT][CTW];
    auto fetch_s0 = [&](int j_) {
        const int j = j_ < 0 ? 0 : j_;
        // (the forward walk stores it tile-major: [dk / 16 column tiles][dv rows][16])
        const float *ck = p.ck + ((size_t)(base + j) * p.hv + h) * DV * DK + (size_t)(part * DVP) * 16;
#pragma unroll
        for (int l2 = 0; l2 < CTW; ++l2) {
            const int ct = wave + NW * l2 < NT ? wave + NW * l2 : NT - 1;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int c = 0; c < 4; ++c) s0[rt][l2][c] = ck[((size_t)ct * DV + 16 * rt + 4 * g + c) * 16 + x];
        }
    };

    // The per-token results of a chunk (wave 0, lane m = token): dbeta, and dg as the
    // running sum from the sequence's end, carry + phi_15 + ... + phi_m in that order
    // (phi = dO . o - dv . v; tokens past the chunk's end hold exact zeros); with
    // P > 1, the part's share of each.
    float *const out_beta = P == 1 ? p.grad_beta : p.dbeta_part + (size_t)part * p.total_tokens * p.hv;
    float *const out_g = P == 1 ? p.grad_g : p.dg_part + (size_t)part * p.total_tokens * p.hv;
    auto per_token = [&](int j, int b) {
        if (wave != 0) return;
        const int m1 = chunk_m1(j);
        const int64_t t0 = tb + (int64_t)kCk * j;
        const int m = lane & 15;
        float4 rw[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) rw[w] = *reinterpret_cast<const float4 *>(&red[b][w][m][0]);
        float sbv = 0.f, svv = 0.f, sq = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            sbv = sbv + rw[w].x;
            svv = svv + rw[w].y;
            sq = sq + rw[w].z;
        }
        const float phi = sq - svv;
        // every token's phi to every lane (through LDS: one store, four broadcast reads),
        // then the running sum from token 15 down; lane m keeps it at token m
        if (lane < kCk) phis[m] = phi;
        float ph[kCk];
#pragma unroll
        for (int i = 0; i < kCk / 4; ++i) {
            const float4 v4 = *reinterpret_cast<const float4 *>(&phis[4 * i]);
            ph[4 * i] = v4.x;
            ph[4 * i + 1] = v4.y;
            ph[4 * i + 2] = v4.z;
            ph[4 * i + 3] = v4.w;
        }
        float run = carry, dg = carry;
#pragma unroll
        for (int s = kCk - 1; s >= 0; --s) {
            run = run + ph[s];
            dg = s == m ? run : dg;
        }
        carry = run;
        // unconditional buffer stores (out-of-range offset where there is nothing to
        // write), so that the memory counters stay exact and no wait drains the next
        // chunk's reads
        const uint32_t bytes = (uint32_t)m1 * (uint32_t)p.hv * 4u;
        const uint32_t off = lane < kCk && m < m1 ? ((uint32_t)m * (uint32_t)p.hv + (uint32_t)h) * 4u : kDropped;
        buf_store_f32(buf_rsrc(out_beta + (size_t)t0 * p.hv, bytes), off, sbv + abrow[m]);
        buf_store_f32(buf_rsrc(out_g + (size_t)t0 * p.hv, bytes), off, dg);
    };

    RF F;
    if (nch > 0) {
        fetch(F, nch - 1);
        fetch_s0(nch - 1);
    }
    for (int j = nch - 1; j >= 0; --j) {
        const int m1 = chunk_m1(j);
        const int64_t t0 = tb + (int64_t)kCk * j;
        const int b = j & 1;
        float(*Kc)[KP] = Ks[b];
        float(*Qc)[KP] = Qs[b];

        // ---- stage this chunk: keys and queries into LDS, the rest into registers
#pragma unroll
        for (int s = 0; s < RF::KIT; ++s) {
            const int it = tid + NTH * s;
            if (it < RF::KITEMS) {
                const int m = it / (DK / 4), c = 4 * (it % (DK / 4));
                const bool on = m < m1;
                *reinterpret_cast<float4 *>(&Kc[m][c]) = RW::widen(RW::keep(F.kr[s], on));
                *reinterpret_cast<float4 *>(&Qc[m][c]) = RW::widen(RW::keep(F.qr[s], on));
            }
        }
        float dO[4], vv[4], xx[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bool on = 4 * g + c < m1;
            dO[c] = on ? RW::widen1(F.dor[c]) : 0.f;
            vv[c] = on ? RW::widen1(F.vr[c]) : 0.f;
            xx[c] = on ? F.xr[c] : 0.f;
        }
        const float bt[4] = {F.bet.x, F.bet.y, F.bet.z, F.bet.w};
        const float gm[4] = {F.gam.x, F.gam.y, F.gam.z, F.gam.w};
        const float wl[4] = {F.wl.x, F.wl.y, F.wl.z, F.wl.w};
        const float bx = F.bx, gx = F.gx, wx = F.wx, gl = F.gl;
        const float4 trow = F.trow;
        float tcol[4], bcol[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            tcol[c] = F.tcol[c];
            bcol[c] = F.bcol[c];
        }
        float ge[RF::EPT], ae[RF::EPT], be[RF::EPT];
#pragma unroll
        for (int e = 0; e < RF::EPT; ++e) {
            ge[e] = F.ge[e];
            ae[e] = F.ae[e];
            be[e] = F.be[e];
        }
        fetch(F, j - 1);
        lds_barrier();

        // ---- P1.  E = K D^T on this wave's rows (token 4 g + c, row r0 + x); the key
        // tiles are all read before the products
        f4 Ev = f4_zero();
        float4 kav[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) kav[t] = *reinterpret_cast<const float4 *>(&Kc[x][16 * t + 4 * g]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            Ev = mfma_16x16x4(kav[t].x, Dt[t][0], Ev);
            Ev = mfma_16x16x4(kav[t].y, Dt[t][1], Ev);
            Ev = mfma_16x16x4(kav[t].z, Dt[t][2], Ev);
            Ev = mfma_16x16x4(kav[t].w, Dt[t][3], Ev);
        }
        // dU = Gam_{l,.} E + B^T dO;  dR = T^T dU;  U = T (beta x)
        f4 dU = f4{wl[0] * Ev[0], wl[1] * Ev[1], wl[2] * Ev[2], wl[3] * Ev[3]};
#pragma unroll
        for (int c = 0; c < 4; ++c) dU = mfma_16x16x4(bcol[c], dO[c], dU);
        f4 dR = f4_zero();
#pragma unroll
        for (int c = 0; c < 4; ++c) dR = mfma_16x16x4(tcol[c], dU[c], dR);
        f4 U = f4_zero();
        U = mfma_16x16x4(trow.x, bt[0] * xx[0], U);
        U = mfma_16x16x4(trow.y, bt[1] * xx[1], U);
        U = mfma_16x16x4(trow.z, bt[2] * xx[2], U);
        U = mfma_16x16x4(trow.w, bt[3] * xx[3], U);

        // the previous chunk's per-token results (its sums are complete: barrier above)
        if (j + 1 < nch) per_token(j + 1, b ^ 1);

        // dv = beta dR; the row sums dR . x and dv . v of this wave's rows; the token
        // rows of dO, dR and U and D at the chunk's end for the products over rows
        // (dR and U pass through vector registers first: stores straight from the MFMA
        // accumulators were merged with wrong offsets by the compiler)
        const auto dv_rsrc = buf_rsrc(p.grad_v + (size_t)t0 * vrow, (uint32_t)(m1 * vrow * 4));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int m = 4 * g + c;
            float dr = dR[c], uu = U[c];
            asm volatile("" : "+v"(dr), "+v"(uu));
            const float dvv = bt[c] * dr;
            buf_store_f32(dv_rsrc, m < m1 ? (uint32_t)((m * vrow + (size_t)h * DV + rg + x) * 4) : kDropped, dvv);
            const float sb = lane_sum<16>(dr * xx[c]);
            const float sv = lane_sum<16>(dvv * vv[c]);
            if (x == 0) {
                red[b][wave][m][0] = sb;
                red[b][wave][m][1] = sv;
            }
            dOs[m][r0 + x] = dO[c];
            dRs[m][r0 + x] = dr;
            Us[m][r0 + x] = uu;
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
            *reinterpret_cast<float4 *>(&Ds[r0 + x][16 * t + 4 * g]) = make_float4(Dt[t][0], Dt[t][1], Dt[t][2], Dt[t][3]);

        // D at the chunk's start: D^T = Gam_l D^T + Q^T (Gam dO) - K^T (beta Gam dR)
        {
            float bq[4], bk[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                bq[c] = gm[c] * dO[c];
                bk[c] = -(bt[c] * gm[c]) * dR[c];
            }
            // (the next tile's query and key columns are read while this tile's
            // products run)
            float qa[2][4], ka[2][4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                qa[0][c] = Qc[4 * g + c][x];
                ka[0][c] = Kc[4 * g + c][x];
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (t + 1 < NT) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        qa[(t + 1) & 1][c] = Qc[4 * g + c][16 * (t + 1) + x];
                        ka[(t + 1) & 1][c] = Kc[4 * g + c][16 * (t + 1) + x];
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                f4 C = f4{gl * Dt[t][0], gl * Dt[t][1], gl * Dt[t][2], gl * Dt[t][3]};
#pragma unroll
                for (int c = 0; c < 4; ++c) C = mfma_16x16x4(qa[t & 1][c], bq[c], C);
#pragma unroll
                for (int c = 0; c < 4; ++c) C = mfma_16x16x4(ka[t & 1][c], bk[c], C);
                Dt[t] = C;
            }
        }
        lds_barrier();

        // ---- P2.  partial dB = dO U^T and dA = -dR U^T over this wave's rows
        {
            const float4 o4 = *reinterpret_cast<const float4 *>(&dOs[x][r0 + 4 * g]);
            const float4 r4 = *reinterpret_cast<const float4 *>(&dRs[x][r0 + 4 * g]);
            const float4 u4 = *reinterpret_cast<const float4 *>(&Us[x][r0 + 4 * g]);
            f4 pb = f4_zero(), pa = f4_zero();
            pb = mfma_16x16x4(o4.x, u4.x, pb);
            pb = mfma_16x16x4(o4.y, u4.y, pb);
            pb = mfma_16x16x4(o4.z, u4.z, pb);
            pb = mfma_16x16x4(o4.w, u4.w, pb);
            pa = mfma_16x16x4(-r4.x, u4.x, pa);
            pa = mfma_16x16x4(-r4.y, u4.y, pa);
            pa = mfma_16x16x4(-r4.z, u4.z, pa);
            pa = mfma_16x16x4(-r4.w, u4.w, pa);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float vb = pb[r], va = pa[r];
                asm volatile("" : "+v"(vb), "+v"(va));
                dBp[wave][4 * g + r][x] = vb;
                dAp[wave][4 * g + r][x] = va;
            }
        }

        // products over the rows on this wave's column tiles:
        //   dq0 = dO S0,  dk1 = (-beta Gam dR) S0 + (Gam_{l,.} U) D
        f4 dq[CTW], dk[CTW];
        {
            const float fr = -(bx * gx), fu = wx;  // factors of A-operand row x (token x)
            // every operand read from LDS before the products, so that no product waits
            // on a read: the token rows of dO, dR and U over the part's rows (A operands)
            // and the D columns of this wave's tiles (B operands of the D term)
            float ao[RT][4], ar[RT][4], au[RT][4], dd[CTW][RT][4];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const float4 o4 = *reinterpret_cast<const float4 *>(&dOs[x][16 * rt + 4 * g]);
                const float4 r4 = *reinterpret_cast<const float4 *>(&dRs[x][16 * rt + 4 * g]);
                const float4 u4 = *reinterpret_cast<const float4 *>(&Us[x][16 * rt + 4 * g]);
                ao[rt][0] = o4.x; ao[rt][1] = o4.y; ao[rt][2] = o4.z; ao[rt][3] = o4.w;
                ar[rt][0] = r4.x; ar[rt][1] = r4.y; ar[rt][2] = r4.z; ar[rt][3] = r4.w;
                au[rt][0] = u4.x; au[rt][1] = u4.y; au[rt][2] = u4.z; au[rt][3] = u4.w;
            }
#pragma unroll
            for (int l2 = 0; l2 < CTW; ++l2) {
                const int ct = wave + NW * l2 < NT ? wave + NW * l2 : NT - 1;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int c = 0; c < 4; ++c) dd[l2][rt][c] = Ds[16 * rt + 4 * g + c][16 * ct + x];
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    ar[rt][c] = fr * ar[rt][c];
                    au[rt][c] = fu * au[rt][c];
                }
#pragma unroll
            for (int l2 = 0; l2 < CTW; ++l2) {
                const int ct = wave + NW * l2;
                f4 aq = f4_zero(), ak = f4_zero();
                if (NT % NW == 0 || ct < NT) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            aq = mfma_16x16x4(ao[rt][c], s0[rt][l2][c], aq);
                            ak = mfma_16x16x4(ar[rt][c], s0[rt][l2][c], ak);
                            ak = mfma_16x16x4(au[rt][c], dd[l2][rt][c], ak);
                        }
                    }
                }
                dq[l2] = f4{gm[0] * aq[0], gm[1] * aq[1], gm[2] * aq[2], gm[3] * aq[3]};
                dk[l2] = ak;
            }
        }
        fetch_s0(j - 1);
        lds_barrier();

        // ---- P3.  dB and dA summed over the waves (in order), masked and weighted; the
        // dA part of dbeta, sum_s dA[m][s] Gam_{m,s} (k_m . k_s), summed across a DPP row
        // (the 16 entries of row m sit in lanes 16 (m % 4) .. of one wave)
#pragma unroll
        for (int e = 0; e < RF::EPT; ++e) {
            const int i = tid + NTH * e;
            if (i < kCk * kCk) {
                const int m = i / kCk, s = i % kCk;
                float sbv = 0.f, sav = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    sbv = sbv + dBp[w][m][s];
                    sav = sav + dAp[w][m][s];
                }
                Ms[m][s] = sbv * ge[e];  // Gam is zero above the diagonal
                Hs[m][s] = s < m ? sav * (be[e] * ge[e]) : 0.f;
                const float ab = lane_sum<16>(sav * ae[e]);  // ae is zero unless s < m
                if (s == 0) abrow[m] = ab;
            }
        }
        lds_barrier();

        // ---- P4.  in-chunk terms: dq += Ms K;  dk += Ms^T Q + (H + H^T) K; q . dq
        {
            float mr[4], mc[4], hh[4], kcol[CTW][4], qcol[CTW][4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                mr[c] = Ms[x][4 * g + c];
                mc[c] = Ms[4 * g + c][x];
                hh[c] = Hs[x][4 * g + c] + Hs[4 * g + c][x];
            }
            // the key and query columns of this wave's tiles, read before the products
#pragma unroll
            for (int l2 = 0; l2 < CTW; ++l2) {
                const int ct = wave + NW * l2 < NT ? wave + NW * l2 : NT - 1;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    kcol[l2][c] = Kc[4 * g + c][16 * ct + x];
                    qcol[l2][c] = Qc[4 * g + c][16 * ct + x];
                }
            }
#pragma unroll
            for (int l2 = 0; l2 < CTW; ++l2) {
                if (NT % NW == 0 || wave + NW * l2 < NT) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) dq[l2] = mfma_16x16x4(mr[c], kcol[l2][c], dq[l2]);
#pragma unroll
                    for (int c = 0; c < 4; ++c) dk[l2] = mfma_16x16x4(mc[c], qcol[l2][c], dk[l2]);
#pragma unroll
                    for (int c = 0; c < 4; ++c) dk[l2] = mfma_16x16x4(hh[c], kcol[l2][c], dk[l2]);
                }
            }
            float qd[4] = {0.f, 0.f, 0.f, 0.f};
            // this chunk's rows of the part's dq and dk (stores every lane issues)
            const uint32_t qrow = (uint32_t)(p.hv * DK);
            const size_t qbase = ((size_t)part * p.total_tokens + t0) * p.hv * DK;
            const auto dq_rsrc = buf_rsrc(p.dqh + qbase, (uint32_t)m1 * qrow * 4u);
            const auto dk_rsrc = buf_rsrc(p.dkh + qbase, (uint32_t)m1 * qrow * 4u);
#pragma unroll
            for (int l2 = 0; l2 < CTW; ++l2) {
                const int ct = wave + NW * l2;
                if (NT % NW == 0 || ct < NT) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = 4 * g + r;
                        qd[r] = __builtin_fmaf(qcol[l2][r], dq[l2][r], qd[r]);
                        const uint32_t o = m < m1 ? ((uint32_t)m * qrow + (uint32_t)(h * DK + 16 * ct + x)) * 4u : kDropped;
                        buf_store_f32(dq_rsrc, o, dq[l2][r]);
                        buf_store_f32(dk_rsrc, o, dk[l2][r]);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = lane_sum<16>(qd[r]);
                if (x == 0) red[b][wave][4 * g + r][2] = v;
            }
        }
    }
    if (nch > 0) {
        lds_barrier();
        per_token(0, 0);
    }

    if (p.grad_h0) {
        float *dst = p.grad_h0 + (((size_t)n * p.hv + h) * DV + rg + x) * DK;
#pragma unroll
        for (int t = 0; t < NT; ++t)
            *reinterpret_cast<float4 *>(dst + 16 * t + 4 * g) = make_float4(Dt[t][0], Dt[t][1], Dt[t][2], Dt[t][3]);
    }
}

// The reverse walk for dv = 128 in two parts of 64 rows, with specialized waves.
// Only E, dU, dR and the move of D to the chunk's start lie on the recurrence; the
// products over rows (dB, dA, dq0, dk1), the in-chunk terms and the per-token sums
// of a chunk need its D and token rows but feed nothing back.  So four state waves
// (16 rows of D each) run chunk c while four gradient waves (dk/64 column tiles each)
// run the rest of chunk c + 1, and each SIMD holds one wave of each kind, whose
// instruction streams overlap.  A step has two barriers: after the keys and queries
// of the state waves' chunk are staged, and after both kinds of work.  What one kind
// writes for the other is double-buffered by chunk parity (the per-token sums, read
// two steps later, by chunk index mod 3).  The arithmetic and every order of
// summation are those of gdn_bwd_chunk_rev_kernel with P = 2, so the results are the
// same bits.
template <int DK, class IO>
__global__ __launch_bounds__(512) void gdn_bwd_chunk_ws_kernel(BwdChunkParams p) {
    using RW = Raw4<IO>;
    constexpr int DV = 128, P = 2, DVP = DV / P, NWD = DVP / 16;  // state waves: 16 rows each
    constexpr int NT = DK / 16, CTW = NT / NWD, RT = NWD;          // column tiles per gradient wave
    constexpr int KP = DK + 4, VP = DVP + 4;
    constexpr int KITEMS = kCk * DK / 4, KIT = (KITEMS + 511) / 512;  // key (query) items per thread
    static_assert(NT % NWD == 0, "column tiles");
    __shared__ __align__(16) float Ks[2][kCk][KP];
    __shared__ __align__(16) float Qs[2][kCk][KP];
    __shared__ __align__(16) float dOs[2][kCk][VP];  // token rows of dO, dR and U
    __shared__ __align__(16) float dRs[2][kCk][VP];
    __shared__ __align__(16) float Us[2][kCk][VP];
    __shared__ __align__(16) float Ds[2][DVP][KP];   // D at the chunk's end
    // the state waves' partial dB and dA, entry-major with the four waves' values
    // side by side (one 16-byte read gives an entry's four partials; rows padded by
    // one entry so that reads down a column spread over the banks)
    __shared__ __align__(16) float dBw[2][kCk][kCk + 1][NWD], dAw[2][kCk][kCk + 1][NWD];
    __shared__ float abrow[3][kCk];
    __shared__ __align__(16) float red[3][NWD][kCk][4];  // by chunk mod 3: dR.x, dv.v (state), q.dq (gradient)
    __shared__ __align__(16) float phis[kCk];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int x = lane & 15, g = lane >> 4;
    int rank, h, part;
    {
        const int G = p.hv / p.hk * P;  // (value head, part) pairs of a key head
        const int ngroups = p.n_seqs * p.hk;
        const int full = (ngroups / 8) * 8 * G;
        const int id = blockIdx.x;
        int grp, member;
        if (id < full) {
            const int xcd = id % 8, slot = id / 8;
            grp = (slot / G) * 8 + xcd;
            member = slot % G;
        } else {
            grp = full / G + (id - full) / G;
            member = (id - full) % G;
        }
        rank = grp / p.hk;
        h = (grp % p.hk) * (G / P) + member / P;
        part = member % P;
    }
    const int n = p.rank_by_length ? seq_by_length_rank(p.cu_seqlens, p.n_seqs, rank, tid, 512) : rank;
    const int kh = h / (p.hv / p.hk);
    int64_t tb = p.cu_seqlens[n], te = p.cu_seqlens[n + 1];
    tb = tb < 0 ? 0 : (tb > p.total_tokens ? p.total_tokens : tb);
    te = te < tb ? tb : (te > p.total_tokens ? p.total_tokens : te);
    const int64_t len = te - tb;
    const int64_t base = chunk_slot_base(tb, n);
    int nch = (int)((len + kCk - 1) / kCk);
    if (base + nch > p.ws_slots) nch = (int)(p.ws_slots - base > 0 ? p.ws_slots - base : 0);
    const size_t vrow = (size_t)p.hv * DV;
    constexpr uint32_t E = IO::ESZ;
    const uint32_t krow_b = (uint32_t)p.hk * DK * E, vrow_b = (uint32_t)vrow * E;
    auto chunk_m1 = [&](int j) {
        const int64_t left = len - (int64_t)kCk * j;
        return left < kCk ? (int)left : kCk;
    };
    auto rec_of = [&](int j) { return p.rec + ((size_t)(base + j) * p.hv + h) * kChunkRecBwd; };

    // keys and queries: every thread stages KIT items of a chunk (read a step ahead)
    typename RW::T kr[KIT], qr[KIT];
    auto fetch_kq = [&](int j_) {
        const int j = j_ < 0 ? 0 : j_;
        const int m1 = chunk_m1(j);
        const int64_t t0 = tb + (int64_t)kCk * j;
        const char *kb = static_cast<const char *>(p.k) + ((size_t)t0 * p.hk + kh) * DK * E;
        const char *qb = static_cast<const char *>(p.q) + ((size_t)t0 * p.hk + kh) * DK * E;
#pragma unroll
        for (int s = 0; s < KIT; ++s) {
            int it = tid + 512 * s;
            it = it < KITEMS ? it : KITEMS - 1;
            const int m = it / (DK / 4), c = 4 * (it % (DK / 4));
            const uint32_t off = (uint32_t)(m < m1 ? m : m1 - 1) * krow_b + (uint32_t)c * E;
            kr[s] = RW::load_at(kb, off);
            qr[s] = RW::load_at(qb, off);
        }
    };
    auto stage_kq = [&](int j) {
        const int m1 = chunk_m1(j);
#pragma unroll
        for (int s = 0; s < KIT; ++s) {
            const int it = tid + 512 * s;
            if (it < KITEMS) {
                const int m = it / (DK / 4), c = 4 * (it % (DK / 4));
                const bool on = m < m1;
                *reinterpret_cast<float4 *>(&Ks[j & 1][m][c]) = RW::widen(RW::keep(kr[s], on));
                *reinterpret_cast<float4 *>(&Qs[j & 1][m][c]) = RW::widen(RW::keep(qr[s], on));
            }
        }
    };
    if (nch > 0) fetch_kq(nch - 1);

    if (wave < NWD) {
        // ================================================================ state waves
        const int r0 = 16 * wave, rg = part * DVP + r0;
        f4 Dt[NT];  // D[rg + x][16 t + 4 g + c]
        {
            const float *src = p.dhT ? p.dhT + (((size_t)n * p.hv + h) * DV + rg + x) * DK : nullptr;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                Dt[t] = f4_zero();
                if (src) {
                    const float4 v4 = *reinterpret_cast<const float4 *>(src + 16 * t + 4 * g);
                    Dt[t] = f4{v4.x, v4.y, v4.z, v4.w};
                }
            }
        }
        struct {
            uint32_t dor[4], vr[4];
            float xr[4];
            float4 bet, gam, wl, trow;
            float gl, tcol[4], bcol[4];
        } F;
        auto fetch = [&](int j_) {
            const int j = j_ < 0 ? 0 : j_;
            const int m1 = chunk_m1(j);
            const int64_t t0 = tb + (int64_t)kCk * j;
            const char *ob = static_cast<const char *>(p.dout) + ((size_t)t0 * p.hv + h) * DV * E;
            const char *vb = static_cast<const char *>(p.v) + ((size_t)t0 * p.hv + h) * DV * E;
            // x: the forward walk's [row][token] tile (see gdn_bwd_chunk_rev_kernel)
            const float4 x4 = *reinterpret_cast<const float4 *>(
                p.xv + (((size_t)(base + j) * p.hv + h) * DV + rg) * kCk + x * kCk + 4 * g);
            F.xr[0] = x4.x;
            F.xr[1] = x4.y;
            F.xr[2] = x4.z;
            F.xr[3] = x4.w;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t tm = (uint32_t)(4 * g + c < m1 ? 4 * g + c : m1 - 1);
                F.dor[c] = RW::load1_at(ob, tm * vrow_b + (uint32_t)(rg + x) * E);
                F.vr[c] = RW::load1_at(vb, tm * vrow_b + (uint32_t)(rg + x) * E);
            }
            const float *rec = rec_of(j);
            const int l = m1 - 1;
            F.bet = *reinterpret_cast<const float4 *>(rec + kRecBeta + 4 * g);
            F.gam = *reinterpret_cast<const float4 *>(rec + kRecGam + 4 * g);
            F.wl = *reinterpret_cast<const float4 *>(rec + kRecGm + l * kCk + 4 * g);
            F.gl = rec[kRecGam + l];
            F.trow = *reinterpret_cast<const float4 *>(rec + kRecT + x * kCk + 4 * g);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                F.tcol[c] = rec[kRecT + (4 * g + c) * kCk + x];
                F.bcol[c] = rec[kRecB + (4 * g + c) * kCk + x];
            }
        };
        float carry = 0.f;  // (wave 0) the part's dg running sum, from <dhT, hT> over its rows
        if (p.dhT && wave == 0)
            for (int i = part * (DVP / 16) * 4; i < (part + 1) * (DVP / 16) * 4; ++i)
                carry = carry + p.hdot[((size_t)n * p.hv + h) * p.hdot_parts + i];
        float *const out_beta = p.dbeta_part + (size_t)part * p.total_tokens * p.hv;
        float *const out_g = p.dg_part + (size_t)part * p.total_tokens * p.hv;
        // (wave 0) the per-token results of chunk j: dbeta and dg as the running sum
        // from the sequence's end, as in gdn_bwd_chunk_rev_kernel
        auto per_token = [&](int j) {
            const int m1 = chunk_m1(j);
            const int64_t t0 = tb + (int64_t)kCk * j;
            const int m = lane & 15;
            float4 rw[NWD];
#pragma unroll
            for (int w = 0; w < NWD; ++w) rw[w] = *reinterpret_cast<const float4 *>(&red[j % 3][w][m][0]);
            float sbv = 0.f, svv = 0.f, sq = 0.f;
#pragma unroll
            for (int w = 0; w < NWD; ++w) {
                sbv = sbv + rw[w].x;
                svv = svv + rw[w].y;
                sq = sq + rw[w].z;
            }
            const float phi = sq - svv;
            if (lane < kCk) phis[m] = phi;
            float ph[kCk];
#pragma unroll
            for (int i = 0; i < kCk / 4; ++i) {
                const float4 v4 = *reinterpret_cast<const float4 *>(&phis[4 * i]);
                ph[4 * i] = v4.x;
                ph[4 * i + 1] = v4.y;
                ph[4 * i + 2] = v4.z;
                ph[4 * i + 3] = v4.w;
            }
            float run = carry, dg = carry;
#pragma unroll
            for (int s = kCk - 1; s >= 0; --s) {
                run = run + ph[s];
                dg = s == m ? run : dg;
            }
            carry = run;
            // unconditional buffer stores, as in gdn_bwd_chunk_rev_kernel
            const uint32_t bytes = (uint32_t)m1 * (uint32_t)p.hv * 4u;
            const uint32_t off = lane < kCk && m < m1 ? ((uint32_t)m * (uint32_t)p.hv + (uint32_t)h) * 4u : kDropped;
            buf_store_f32(buf_rsrc(out_beta + (size_t)t0 * p.hv, bytes), off, sbv + abrow[j % 3][m]);
            buf_store_f32(buf_rsrc(out_g + (size_t)t0 * p.hv, bytes), off, dg);
        };
        // (wave 1) the dA part of dbeta of chunk j, sum_s dA[m][s] Gam_{m,s} (k_m . k_s),
        // from the partials the state waves left a step before (a row's 16 entries sit
        // in 16 lanes); its Gam (k . k) entries are read a step ahead
        float aen[4];
        auto fetch_ab = [&](int j_) {
            const float *rec = rec_of(j_ < 0 ? 0 : j_);
#pragma unroll
            for (int e = 0; e < 4; ++e) aen[e] = rec[kRecAb + lane + 64 * e];
        };
        auto abrow_calc = [&](int j) {
            const int b = j & 1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = lane + 64 * e;
                const int m = i / kCk, s = i % kCk;
                const float ae = aen[e];
                const float4 a4 = *reinterpret_cast<const float4 *>(&dAw[b][m][s][0]);
                const float sav = (((0.f + a4.x) + a4.y) + a4.z) + a4.w;
                const float ab = lane_sum<16>(sav * ae);
                if (s == 0) abrow[j % 3][m] = ab;
            }
        };
        if (nch > 0) fetch(nch - 1);
        if (wave == 1 && nch > 0) fetch_ab(nch - 1);
        for (int st = 0; st <= nch; ++st) {
            const int j = nch - 1 - st;  // this step's chunk (none at the last step)
            if (j >= 0) {
                stage_kq(j);
                fetch_kq(j - 1);
            }
            lds_barrier();
            if (j >= 0) {
                const int m1 = chunk_m1(j);
                const int64_t t0 = tb + (int64_t)kCk * j;
                const int b = j & 1;
                float(*Kc)[KP] = Ks[b];
                float(*Qc)[KP] = Qs[b];
                float dO[4], vv[4], xx[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const bool on = 4 * g + c < m1;
                    dO[c] = on ? RW::widen1(F.dor[c]) : 0.f;
                    vv[c] = on ? RW::widen1(F.vr[c]) : 0.f;
                    xx[c] = on ? F.xr[c] : 0.f;
                }
                const float bt[4] = {F.bet.x, F.bet.y, F.bet.z, F.bet.w};
                const float gm[4] = {F.gam.x, F.gam.y, F.gam.z, F.gam.w};
                const float wl[4] = {F.wl.x, F.wl.y, F.wl.z, F.wl.w};
                const float gl = F.gl;
                const float4 trow = F.trow;
                float tcol[4], bcol[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    tcol[c] = F.tcol[c];
                    bcol[c] = F.bcol[c];
                }
                fetch(j - 1);

                // E = K D^T on this wave's rows; dU = Gam_{l,.} E + B^T dO; dR = T^T dU; U = T (beta x)
                f4 Ev = f4_zero();
                float4 kav[NT];
#pragma unroll
                for (int t = 0; t < NT; ++t) kav[t] = *reinterpret_cast<const float4 *>(&Kc[x][16 * t + 4 * g]);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    Ev = mfma_16x16x4(kav[t].x, Dt[t][0], Ev);
                    Ev = mfma_16x16x4(kav[t].y, Dt[t][1], Ev);
                    Ev = mfma_16x16x4(kav[t].z, Dt[t][2], Ev);
                    Ev = mfma_16x16x4(kav[t].w, Dt[t][3], Ev);
                }
                f4 dU = f4{wl[0] * Ev[0], wl[1] * Ev[1], wl[2] * Ev[2], wl[3] * Ev[3]};
#pragma unroll
                for (int c = 0; c < 4; ++c) dU = mfma_16x16x4(bcol[c], dO[c], dU);
                f4 dR = f4_zero();
#pragma unroll
                for (int c = 0; c < 4; ++c) dR = mfma_16x16x4(tcol[c], dU[c], dR);
                f4 U = f4_zero();
                U = mfma_16x16x4(trow.x, bt[0] * xx[0], U);
                U = mfma_16x16x4(trow.y, bt[1] * xx[1], U);
                U = mfma_16x16x4(trow.z, bt[2] * xx[2], U);
                U = mfma_16x16x4(trow.w, bt[3] * xx[3], U);

                // dv; the row sums dR . x and dv . v; the token rows for the gradient waves
                // (through vector registers: see gdn_bwd_chunk_rev_kernel)
                const auto dv_rsrc = buf_rsrc(p.grad_v + (size_t)t0 * vrow, (uint32_t)(m1 * vrow * 4));
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int m = 4 * g + c;
                    float dr = dR[c], uu = U[c];
                    asm volatile("" : "+v"(dr), "+v"(uu));
                    const float dvv = bt[c] * dr;
                    buf_store_f32(dv_rsrc, m < m1 ? (uint32_t)((m * vrow + (size_t)h * DV + rg + x) * 4) : kDropped, dvv);
                    const float sb = lane_sum<16>(dr * xx[c]);
                    const float sv = lane_sum<16>(dvv * vv[c]);
                    if (x == 0) {
                        red[j % 3][wave][m][0] = sb;
                        red[j % 3][wave][m][1] = sv;
                    }
                    dOs[b][m][r0 + x] = dO[c];
                    dRs[b][m][r0 + x] = dr;
                    Us[b][m][r0 + x] = uu;
                }
                // partial dB = dO U^T and dA = -dR U^T over this wave's rows (its own
                // token rows, just written)
                {
                    const float4 o4 = *reinterpret_cast<const float4 *>(&dOs[b][x][r0 + 4 * g]);
                    const float4 r4 = *reinterpret_cast<const float4 *>(&dRs[b][x][r0 + 4 * g]);
                    const float4 u4 = *reinterpret_cast<const float4 *>(&Us[b][x][r0 + 4 * g]);
                    f4 pb = f4_zero(), pa = f4_zero();
                    pb = mfma_16x16x4(o4.x, u4.x, pb);
                    pb = mfma_16x16x4(o4.y, u4.y, pb);
                    pb = mfma_16x16x4(o4.z, u4.z, pb);
                    pb = mfma_16x16x4(o4.w, u4.w, pb);
                    pa = mfma_16x16x4(-r4.x, u4.x, pa);
                    pa = mfma_16x16x4(-r4.y, u4.y, pa);
                    pa = mfma_16x16x4(-r4.z, u4.z, pa);
                    pa = mfma_16x16x4(-r4.w, u4.w, pa);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float vb = pb[r], va = pa[r];
                        asm volatile("" : "+v"(vb), "+v"(va));
                        dBw[b][4 * g + r][x][wave] = vb;
                        dAw[b][4 * g + r][x][wave] = va;
                    }
                }
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    *reinterpret_cast<float4 *>(&Ds[b][r0 + x][16 * t + 4 * g]) =
                        make_float4(Dt[t][0], Dt[t][1], Dt[t][2], Dt[t][3]);

                // D at the chunk's start: D^T = Gam_l D^T + Q^T (Gam dO) - K^T (beta Gam dR)
                float bq[4], bk[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    bq[c] = gm[c] * dO[c];
                    bk[c] = -(bt[c] * gm[c]) * dR[c];
                }
                float qa[2][4], ka[2][4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    qa[0][c] = Qc[4 * g + c][x];
                    ka[0][c] = Kc[4 * g + c][x];
                }
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    if (t + 1 < NT) {
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            qa[(t + 1) & 1][c] = Qc[4 * g + c][16 * (t + 1) + x];
                            ka[(t + 1) & 1][c] = Kc[4 * g + c][16 * (t + 1) + x];
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    f4 C = f4{gl * Dt[t][0], gl * Dt[t][1], gl * Dt[t][2], gl * Dt[t][3]};
#pragma unroll
                    for (int c = 0; c < 4; ++c) C = mfma_16x16x4(qa[t & 1][c], bq[c], C);
#pragma unroll
                    for (int c = 0; c < 4; ++c) C = mfma_16x16x4(ka[t & 1][c], bk[c], C);
                    Dt[t] = C;
                }
            }
            // the gradient waves run chunk j + 1 in this step; chunk j + 2 is complete
            if (wave == 1 && st >= 1) {
                abrow_calc(j + 1);
                fetch_ab(j);
            }
            if (wave == 0 && st >= 2) per_token(j + 2);
            lds_barrier();
        }
        if (wave == 0 && nch > 0) per_token(0);
        if (p.grad_h0) {
            float *dst = p.grad_h0 + (((size_t)n * p.hv + h) * DV + rg + x) * DK;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                *reinterpret_cast<float4 *>(dst + 16 * t + 4 * g) = make_float4(Dt[t][0], Dt[t][1], Dt[t][2], Dt[t][3]);
        }
    } else {
        // ============================================================= gradient waves
        const int gw = wave - NWD;
        struct {
            float4 gam, gmr, be4;       // Gam_{4 g + c}, Gam_{x, 4 g + c}, beta_{4 g + c}
            float bx, gx, wx;           // beta, Gam and Gam_{l,x} of token x
            float gmc[4];               // Gam_{4 g + c, x}
        } F;
        // S0[part DVP + 16 rt + 4 g + c][16 (gw + NWD l2) + x], read a chunk ahead once
        // the current one is no longer needed
        f4 s0[RT][CTW];
        auto fetch_s0 = [&](int j_) {
            const int j = j_ < 0 ? 0 : j_;
            // (tile-major, as the forward walk stores it)
            const float *ck = p.ck + ((size_t)(base + j) * p.hv + h) * DV * DK + (size_t)(part * DVP) * 16;
#pragma unroll
            for (int l2 = 0; l2 < CTW; ++l2)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        s0[rt][l2][c] = ck[((size_t)(gw + NWD * l2) * DV + 16 * rt + 4 * g + c) * 16 + x];
        };
        auto fetch = [&](int j_) {
            const int j = j_ < 0 ? 0 : j_;
            const float *rec = rec_of(j);
            const int l = chunk_m1(j) - 1;
            F.gam = *reinterpret_cast<const float4 *>(rec + kRecGam + 4 * g);
            F.gmr = *reinterpret_cast<const float4 *>(rec + kRecGm + x * kCk + 4 * g);
            F.be4 = *reinterpret_cast<const float4 *>(rec + kRecBeta + 4 * g);
            F.bx = rec[kRecBeta + x];
            F.gx = rec[kRecGam + x];
            F.wx = rec[kRecGm + l * kCk + x];
#pragma unroll
            for (int c = 0; c < 4; ++c) F.gmc[c] = rec[kRecGm + (4 * g + c) * kCk + x];
        };
        if (nch > 0) {
            fetch(nch - 1);
            fetch_s0(nch - 1);
        }
        for (int st = 0; st <= nch; ++st) {
            const int js = nch - 1 - st;  // the state waves' chunk
            const int j = js + 1;         // this step's chunk (none at the first step)
            if (js >= 0) {
                stage_kq(js);
                fetch_kq(js - 1);
            }
            lds_barrier();
            if (st >= 1) {
                const int m1 = chunk_m1(j);
                const int64_t t0 = tb + (int64_t)kCk * j;
                const int b = j & 1;
                float(*Kc)[KP] = Ks[b];
                float(*Qc)[KP] = Qs[b];
                const float gm[4] = {F.gam.x, F.gam.y, F.gam.z, F.gam.w};
                const float fr = -(F.bx * F.gx), fu = F.wx;  // factors of A-operand row x (token x)
                const float gmr[4] = {F.gmr.x, F.gmr.y, F.gmr.z, F.gmr.w};
                const float be4[4] = {F.be4.x, F.be4.y, F.be4.z, F.be4.w};
                const float bx = F.bx;
                float gmc[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) gmc[c] = F.gmc[c];
                fetch(j - 1);

                // the entries of Ms = dB Gam (s <= m) and H = dA beta Gam (s < m) this lane
                // needs, at (x, 4 g + c) and (4 g + c, x): dB and dA summed over the state
                // waves in order, then masked and weighted
                float mr[4], mc[4], hh[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float4 b1 = *reinterpret_cast<const float4 *>(&dBw[b][x][4 * g + c][0]);
                    const float4 b2 = *reinterpret_cast<const float4 *>(&dBw[b][4 * g + c][x][0]);
                    const float4 a1 = *reinterpret_cast<const float4 *>(&dAw[b][x][4 * g + c][0]);
                    const float4 a2 = *reinterpret_cast<const float4 *>(&dAw[b][4 * g + c][x][0]);
                    const float sb1 = (((0.f + b1.x) + b1.y) + b1.z) + b1.w;
                    const float sb2 = (((0.f + b2.x) + b2.y) + b2.z) + b2.w;
                    const float sa1 = (((0.f + a1.x) + a1.y) + a1.z) + a1.w;
                    const float sa2 = (((0.f + a2.x) + a2.y) + a2.z) + a2.w;
                    mr[c] = sb1 * gmr[c];
                    mc[c] = sb2 * gmc[c];
                    const float h1 = 4 * g + c < x ? sa1 * (bx * gmr[c]) : 0.f;
                    const float h2 = x < 4 * g + c ? sa2 * (be4[c] * gmc[c]) : 0.f;
                    hh[c] = h1 + h2;
                }

                // products over the part's rows on this wave's column tiles:
                //   dq0 = dO S0,  dk1 = (-beta Gam dR) S0 + (Gam_{l,.} U) D
                f4 dq[CTW], dk[CTW];
                {
                    float ao[RT][4], ar[RT][4], au[RT][4];
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        const float4 o4 = *reinterpret_cast<const float4 *>(&dOs[b][x][16 * rt + 4 * g]);
                        const float4 r4 = *reinterpret_cast<const float4 *>(&dRs[b][x][16 * rt + 4 * g]);
                        const float4 u4 = *reinterpret_cast<const float4 *>(&Us[b][x][16 * rt + 4 * g]);
                        ao[rt][0] = o4.x; ao[rt][1] = o4.y; ao[rt][2] = o4.z; ao[rt][3] = o4.w;
                        ar[rt][0] = r4.x; ar[rt][1] = r4.y; ar[rt][2] = r4.z; ar[rt][3] = r4.w;
                        au[rt][0] = u4.x; au[rt][1] = u4.y; au[rt][2] = u4.z; au[rt][3] = u4.w;
                    }
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            ar[rt][c] = fr * ar[rt][c];
                            au[rt][c] = fu * au[rt][c];
                        }
#pragma unroll
                    for (int l2 = 0; l2 < CTW; ++l2) {
                        // this column tile's D columns, read before its products
                        float dd[RT][4];
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                            for (int c = 0; c < 4; ++c) dd[rt][c] = Ds[b][16 * rt + 4 * g + c][16 * (gw + NWD * l2) + x];
                        f4 aq = f4_zero(), ak = f4_zero();
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
                            for (int c = 0; c < 4; ++c) {
                                aq = mfma_16x16x4(ao[rt][c], s0[rt][l2][c], aq);
                                ak = mfma_16x16x4(ar[rt][c], s0[rt][l2][c], ak);
                                ak = mfma_16x16x4(au[rt][c], dd[rt][c], ak);
                            }
                        }
                        dq[l2] = f4{gm[0] * aq[0], gm[1] * aq[1], gm[2] * aq[2], gm[3] * aq[3]};
                        dk[l2] = ak;
                    }
                }
                fetch_s0(j - 1);

                // in-chunk terms: dq += Ms K;  dk += Ms^T Q + (H + H^T) K; stores; q . dq
                {
                    float kcol[CTW][4], qcol[CTW][4];
#pragma unroll
                    for (int l2 = 0; l2 < CTW; ++l2)
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            kcol[l2][c] = Kc[4 * g + c][16 * (gw + NWD * l2) + x];
                            qcol[l2][c] = Qc[4 * g + c][16 * (gw + NWD * l2) + x];
                        }
#pragma unroll
                    for (int l2 = 0; l2 < CTW; ++l2) {
#pragma unroll
                        for (int c = 0; c < 4; ++c) dq[l2] = mfma_16x16x4(mr[c], kcol[l2][c], dq[l2]);
#pragma unroll
                        for (int c = 0; c < 4; ++c) dk[l2] = mfma_16x16x4(mc[c], qcol[l2][c], dk[l2]);
#pragma unroll
                        for (int c = 0; c < 4; ++c) dk[l2] = mfma_16x16x4(hh[c], kcol[l2][c], dk[l2]);
                    }
                    float qd[4] = {0.f, 0.f, 0.f, 0.f};
                    const uint32_t qrow = (uint32_t)(p.hv * DK);
                    const size_t qbase = ((size_t)part * p.total_tokens + t0) * p.hv * DK;
                    const auto dq_rsrc = buf_rsrc(p.dqh + qbase, (uint32_t)m1 * qrow * 4u);
                    const auto dk_rsrc = buf_rsrc(p.dkh + qbase, (uint32_t)m1 * qrow * 4u);
#pragma unroll
                    for (int l2 = 0; l2 < CTW; ++l2) {
                        const int ct = gw + NWD * l2;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int m = 4 * g + r;
                            qd[r] = __builtin_fmaf(qcol[l2][r], dq[l2][r], qd[r]);
                            const uint32_t o =
                                m < m1 ? ((uint32_t)m * qrow + (uint32_t)(h * DK + 16 * ct + x)) * 4u : kDropped;
                            buf_store_f32(dq_rsrc, o, dq[l2][r]);
                            buf_store_f32(dk_rsrc, o, dk[l2][r]);
                        }
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float v = lane_sum<16>(qd[r]);
                        if (x == 0) red[j % 3][gw][4 * g + r][2] = v;
                    }
                }
            }
            lds_barrier();
        }
    }
}

// dq and dk of each key head: the (value head, part) partials that read it, added
// value head by value head and within a head part by part.
__global__ __launch_bounds__(256) void gdn_bwd_chunk_gqa_kernel(BwdChunkParams p) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one 4-column item
    const int64_t per_tok = (int64_t)p.hk * p.dk / 4;
    if (i >= p.total_tokens * per_tok) return;
    const int64_t t = i / per_tok;
    const int rem = (int)(i % per_tok);
    const int kh = rem / (p.dk / 4), c = 4 * (rem % (p.dk / 4));
    const int G = p.hv / p.hk;
    const size_t src = ((size_t)t * p.hv + (size_t)kh * G) * p.dk + c;
    const size_t pstride = (size_t)p.total_tokens * p.hv * p.dk;
    float4 sq = make_float4(0.f, 0.f, 0.f, 0.f), sk = sq;
    for (int gi = 0; gi < G; ++gi) {
        for (int pt = 0; pt < p.parts; ++pt) {
            const size_t o = src + (size_t)gi * p.dk + (size_t)pt * pstride;
            const float4 a = *reinterpret_cast<const float4 *>(p.dqh + o);
            const float4 b = *reinterpret_cast<const float4 *>(p.dkh + o);
            if (gi == 0 && pt == 0) {
                sq = a;
                sk = b;
            } else {
                sq = make_float4(sq.x + a.x, sq.y + a.y, sq.z + a.z, sq.w + a.w);
                sk = make_float4(sk.x + b.x, sk.y + b.y, sk.z + b.z, sk.w + b.w);
            }
        }
    }
    const size_t dst = ((size_t)t * p.hk + kh) * p.dk + c;
    *reinterpret_cast<float4 *>(p.grad_q + dst) = sq;
    *reinterpret_cast<float4 *>(p.grad_k + dst) = sk;
}

// dbeta and dg of each (token, value head): the parts' shares, added part by part.
__global__ __launch_bounds__(256) void gdn_bwd_chunk_parts_kernel(BwdChunkParams p) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n = p.total_tokens * p.hv;
    if (i >= n) return;
    float b = p.dbeta_part[i], g = p.dg_part[i];
    for (int pt = 1; pt < p.parts; ++pt) {
        b = b + p.dbeta_part[(size_t)pt * n + i];
        g = g + p.dg_part[(size_t)pt * n + i];
    }
    p.grad_beta[i] = b;
    p.grad_g[i] = g;
}

template <int DK, int DV, class IO>
hipError_t rev_launch(const BwdChunkParams &p, hipStream_t s) {
    const unsigned grid = (unsigned)((int64_t)p.n_seqs * p.hv * p.parts);
    if constexpr (DV == 128) {
        if (p.parts == 2 && !p.plain) {
            hipLaunchKernelGGL((gdn_bwd_chunk_ws_kernel<DK, IO>), dim3(grid), dim3(512), 0, s, p);
            return hipGetLastError();
        }
    }
    if (p.parts == 1)
        hipLaunchKernelGGL((gdn_bwd_chunk_rev_kernel<DK, DV, IO, 1>), dim3(grid), dim3(64 * (DV / 16)), 0, s, p);
    else if constexpr (DV >= 64)
        hipLaunchKernelGGL((gdn_bwd_chunk_rev_kernel<DK, DV, IO, 2>), dim3(grid), dim3(64 * (DV / 32)), 0, s, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <class IO>
hipError_t rev_io(const BwdChunkParams &p, hipStream_t s) {
    if (p.dk == 128) {
        switch (p.dv) {
            case 32: return rev_launch<128, 32, IO>(p, s);
            case 64: return rev_launch<128, 64, IO>(p, s);
            case 128: return rev_launch<128, 128, IO>(p, s);
        }
    } else if (p.dk == 64) {
        switch (p.dv) {
            case 32: return rev_launch<64, 32, IO>(p, s);
            case 64: return rev_launch<64, 64, IO>(p, s);
            case 128: return rev_launch<64, 128, IO>(p, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd_chunked(const BwdChunkParams &p, int io_dtype, hipStream_t s) {
    if (p.parts != 1 && p.parts != 2) return hipErrorInvalidValue;
    hipError_t e = io_dtype == GDN_BF16 ? rev_io<IoBf16>(p, s) : rev_io<IoF32>(p, s);
    if (e != hipSuccess || p.total_tokens == 0) return e;
    if (p.hv > p.hk || p.parts > 1) {
        const int64_t items = p.total_tokens * p.hk * p.dk / 4;
        hipLaunchKernelGGL(gdn_bwd_chunk_gqa_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (p.parts > 1) {
        const int64_t items = p.total_tokens * p.hv;
        hipLaunchKernelGGL(gdn_bwd_chunk_parts_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, p);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace gdn
