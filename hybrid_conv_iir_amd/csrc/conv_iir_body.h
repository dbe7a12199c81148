// Conv/recurrent half of the block forward: short depthwise FIR -> outer
// depthwise FIR -> diagonal modal IIR scan that keeps every per-position
// state (EvSpark digest, Figure 1(d): the outer-FIR inputs u_i and the IIR
// states s_i are what slicing later selects from).
//
// One workgroup = 16 channels of one sequence, 256 threads, every candidate
// block of the sequence at once (rows r = c * P + i, R = nc * P rows); a
// 4096-channel layer spreads over 256 workgroups per sequence.
//  phase 0  one round of loads (every value to registers first, then to
//           LDS): the committed short window and the block inputs x of every
//           row (as fp32), the outer window and the short and outer taps of
//           the 16 channels go to LDS; the IIR parameters and the committed
//           IIR state stay in registers
//  phase 1  thread (row slot, channel) computes f_r (short FIR) for rows
//           r = slot, slot + 16, ...
//  phase 2  the same threads compute g_r = sum_j w_outer[j] * fbar[i - j]
//           from LDS, one fixed-order fma chain per output
//  phase 3  thread (channel, candidate, group of four poles) runs the IIR
//           recurrence in fp32 registers over the P positions and writes
//           s_i (16 bytes per thread, a contiguous kilobyte per channel group);
//           the readout y_i adds the group's terms, then the groups by a
//           fixed-order butterfly over ceil(N/4) lanes.
// All per-output arithmetic happens in a fixed order that does not depend
// on P or on the candidate count, so a block forward and P single-position
// forwards give identical bits for f, s and y.
#pragma once

#include "hci_internal.h"

namespace hci {

constexpr int kCG = 16;        // channels per workgroup
constexpr int kConvT = 256;    // threads per workgroup

// LDS floats: short window + x rows, outer window + f rows, g rows, outer taps, short taps
__host__ __device__ inline size_t conv_iir_lds_floats(int Ts, int To, int R) {
    return (size_t)((Ts - 1 + R) + (To - 1 + R) + R + To + Ts) * kCG;
}

// one workgroup: channel group cgi (16 channels) of sequence b, all nc candidate blocks
// (they share the committed windows, state and taps); lds holds conv_iir_lds_floats floats
template <int ACT>
__device__ __forceinline__ void conv_iir_block(
    const float* __restrict__ w_short, const float* __restrict__ w_outer,
    const float* __restrict__ lam, const float* __restrict__ beta, const float* __restrict__ cc,
    const typename Act<ACT>::T* __restrict__ short_win, const float* __restrict__ outer_win,
    const float* __restrict__ iir, const typename Act<ACT>::T* __restrict__ x,
    float* __restrict__ f_out, float* __restrict__ s_out, typename Act<ACT>::T* __restrict__ y_out,
    int d, int Ts, int To, int N, int nc, int P, int cgi, int b, float* lds)
{
    const int W = To - 1, Ws = Ts - 1, R = nc * P;
    float* xs = lds;                            // [Ws + R][kCG]: short window rows, then x rows
    float* fb = xs + (size_t)(Ws + R) * kCG;    // [W + R][kCG]: outer window rows, then f rows
    float* gl = fb + (size_t)(W + R) * kCG;     // [R][kCG]
    float* wl = gl + (size_t)R * kCG;           // [To][kCG]
    float* ws = wl + (size_t)To * kCG;          // [Ts][kCG]

    const int ch0 = cgi * kCG;
    const int tid = threadIdx.x;
    const int cl = tid & (kCG - 1), row = tid >> 4;     // 16 row slots of 16 channels
    const int ch = ch0 + cl;
    const bool live = ch < d;
    const typename Act<ACT>::T* sw = short_win + (size_t)b * Ws * d;
    const float* ow = outer_win + (size_t)b * W * d;
    const typename Act<ACT>::T* xb = x + (size_t)b * R * d;

    // IIR task of this thread: channel ch0 + tch, poles 4 * tg .. 4 * tg + 3 (G = ceil(N / 4) groups
    // per channel, rounded up to a power of two), candidates tc, tc + per, ... (see phase 3)
    const int G = N <= 4 ? 1 : N <= 8 ? 2 : N <= 16 ? 4 : N <= 32 ? 8 : 16;
    const int tg = tid % G, tch = (tid / G) % kCG, tc = tid / (G * kCG);
    const int chn = ch0 + tch;
    const bool scan = chn < d;                          // uniform across the G lanes of a task
    float lm[4], bt[4], cv[4], s0[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int n = 4 * tg + q;
        const bool ok = scan && n < N;
        const size_t o = (size_t)chn * N + n;
        lm[q] = ok ? lam[o] : 0.f;
        bt[q] = ok ? beta[o] : 0.f;
        cv[q] = ok ? cc[o] : 0.f;
        s0[q] = ok ? iir[(size_t)b * d * N + o] : 0.f;
    }

    // phase 0: every load of the workgroup in one round: all values go to registers first
    // (the common sizes: up to 128 window rows and taps, 64 block rows, 16 short taps), then
    // to LDS; rows beyond those sizes are staged by a plain loop afterwards
    {
        constexpr int SW = 8, SX = 4;                   // rows per thread of the register batch
        float vw[SW], vt[SW], vx[SX], vsw, vst;
#pragma unroll
        for (int u = 0; u < SW; ++u) {
            const int r = row + 16 * u;
            vw[u] = live && r < W ? ow[(size_t)r * d + ch] : 0.f;
            vt[u] = live && r < To ? w_outer[(size_t)r * d + ch] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < SX; ++u) {
            const int r = row + 16 * u;
            vx[u] = live && r < R ? Act<ACT>::load(xb, (size_t)r * d + ch) : 0.f;
        }
        vsw = live && row < Ws ? Act<ACT>::load(sw, (size_t)row * d + ch) : 0.f;
        vst = live && row < Ts ? w_short[(size_t)row * d + ch] : 0.f;
#pragma unroll
        for (int u = 0; u < SW; ++u) {
            const int r = row + 16 * u;
            if (r < W) fb[r * kCG + cl] = vw[u];
            if (r < To) wl[r * kCG + cl] = vt[u];
        }
#pragma unroll
        for (int u = 0; u < SX; ++u) {
            const int r = row + 16 * u;
            if (r < R) xs[(Ws + r) * kCG + cl] = vx[u];
        }
        if (row < Ws) xs[row * kCG + cl] = vsw;
        if (row < Ts) ws[row * kCG + cl] = vst;
        for (int r = row + 16 * SW; r < W; r += kConvT / kCG) fb[r * kCG + cl] = live ? ow[(size_t)r * d + ch] : 0.f;
        for (int r = row + 16 * SW; r < To; r += kConvT / kCG) wl[r * kCG + cl] = live ? w_outer[(size_t)r * d + ch] : 0.f;
        for (int r = row + 16 * SX; r < R; r += kConvT / kCG) xs[(Ws + r) * kCG + cl] = live ? Act<ACT>::load(xb, (size_t)r * d + ch) : 0.f;
        for (int r = row + 16; r < Ws; r += kConvT / kCG) xs[r * kCG + cl] = live ? Act<ACT>::load(sw, (size_t)r * d + ch) : 0.f;
        for (int r = row + 16; r < Ts; r += kConvT / kCG) ws[r * kCG + cl] = live ? w_short[(size_t)r * d + ch] : 0.f;
    }

    __syncthreads();

    // phase 1: short FIR, f_i = sum_{j<Ts} w_short[j] * xbar[i-j]
    for (int r = row; r < R; r += kConvT / kCG) {
        const int c = r / P, i = r - c * P;
        float acc = 0.f;
        for (int j = 0; j < Ts; ++j) {
            const int m = i - j;
            const float xv = m >= 0 ? xs[(Ws + c * P + m) * kCG + cl] : xs[(Ws + m) * kCG + cl];
            acc = fmaf(ws[j * kCG + cl], xv, acc);
        }
        if (live) f_out[((size_t)b * R + r) * d + ch] = acc;
        fb[(W + r) * kCG + cl] = acc;
    }
    __syncthreads();

    // phase 2: outer FIR, g_i = sum_{j<To} w_outer[j] * fbar[i-j], j ascending
    for (int r = row; r < R; r += kConvT / kCG) {
        const int c = r / P, i = r - c * P;
        const float* fblk = fb + (W + c * P) * kCG + cl;   // candidate c's f rows
        const float* fwin = fb + W * kCG + cl;             // fwin[-k * kCG] = outer window row W - k
        float acc = 0.f;
        int j = 0;
#pragma unroll 8
        for (; j <= i && j < To; ++j) acc = fmaf(wl[j * kCG + cl], fblk[(i - j) * kCG], acc);
#pragma unroll 8
        for (; j < To; ++j) acc = fmaf(wl[j * kCG + cl], fwin[(i - j) * kCG], acc);
        gl[r * kCG + cl] = acc;
    }
    __syncthreads();

    // phase 3: IIR scan from the committed state, in registers.  A task = (channel, candidate,
    // group of 4 poles); 256 / (16 G) candidates advance together.  y_i adds the group's four
    // terms in pole order, then the G groups by a fixed-order butterfly: the order depends on N
    // only, never on P or the candidates.
    {
        const int per = kConvT / (G * kCG);
        for (int c = tc; c - tc < nc; c += per) {
            const bool act = scan && c < nc;
            float st[4] = {s0[0], s0[1], s0[2], s0[3]};
            for (int i = 0; i < P; ++i) {
                const int r = c * P + i;
                const float g = act ? gl[r * kCG + tch] : 0.f;
                float py = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    st[q] = fmaf(lm[q], st[q], bt[q] * g);
                    py = fmaf(cv[q], st[q], py);
                }
                if (act) {
                    float* so = s_out + (((size_t)b * R + r) * d + chn) * N + 4 * tg;
                    if ((N & 3) == 0) {
                        *(float4*)so = make_float4(st[0], st[1], st[2], st[3]);
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (4 * tg + q < N) so[q] = st[q];
                    }
                }
                for (int off = G >> 1; off >= 1; off >>= 1) py += __shfl_xor(py, off, G);
                if (act && tg == 0) Act<ACT>::store(y_out, ((size_t)b * R + r) * d + chn, py);
            }
        }
    }
}

}  // namespace hci
