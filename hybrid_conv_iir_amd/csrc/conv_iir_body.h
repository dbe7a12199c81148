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
//  phase 2  outer FIR as kFirChunks fixed tap chunks: a task (channel,
//           candidate, chunk, block of 16 positions) sums its chunk's taps in
//           ascending order for 16 outputs at once over a 31-value register
//           window (16 taps x 16 outputs per step, two LDS reads per eight
//           multiply-adds); the chunk sums land in LDS and are added in chunk
//           order where phase 3 reads g
//  phase 3  thread (channel, candidate, group of four poles) runs the IIR
//           recurrence in fp32 registers over the P positions and writes
//           s_i (16 bytes per thread, a contiguous kilobyte per channel group);
//           the readout y_i adds the group's terms, then the groups by a
//           fixed-order butterfly over ceil(N/4) lanes (quad permutations on
//           the vector ALU); the next position's input is read ahead.
// All per-output arithmetic happens in a fixed order that does not depend
// on P or on the candidate count, so a block forward and P single-position
// forwards give identical bits for f, s and y.
#pragma once

#include "act_raw.h"
#include "hci_internal.h"

namespace hci {

constexpr int kCG = 16;        // channels per workgroup
constexpr int kConvT = 256;    // threads per workgroup
constexpr int kFirChunks = 4;  // tap chunks of the outer FIR (their sums are added in order)

// LDS floats: short window + x rows, outer window + f rows, chunk sums of g, outer taps,
// short taps
__host__ __device__ inline size_t conv_iir_lds_floats(int Ts, int To, int R) {
    return (size_t)((Ts - 1 + R) + (To - 1 + R) + kFirChunks * R + To + Ts) * kCG;
}

// Sum over the G lanes of an aligned group (G = 1, 2, 4, 8 or 16), the same bits on every
// lane of the group: lane offsets G/2, ..., 2, 1 in turn.  Offsets 2 and 1 are quad
// permutations on the vector ALU (no LDS round trip); wider groups use the LDS crossbar.
__device__ __forceinline__ float group_sum(float v, int G) {
    for (int off = G >> 1; off >= 4; off >>= 1) v += __shfl_xor(v, off, G);
    if (G >= 4) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
    if (G >= 2) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
    return v;
}

// v if keep, else +0.0, by masking the bits: the load behind v stays unconditional (a
// select on a loaded value can turn into a branch around the load)
__device__ __forceinline__ float keep_if(float v, bool keep) {
    return __int_as_float(__float_as_int(v) & (keep ? -1 : 0));
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
    float* gl = fb + (size_t)(W + R) * kCG;     // [kFirChunks][R][kCG]: chunk sums of g
    float* wl = gl + (size_t)kFirChunks * R * kCG;   // [To][kCG]
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
    // (loaded from clamped addresses, zeroed past the channels or poles before the scan)
    float lm[4], bt[4], cv[4], s0[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const size_t o = (size_t)min(chn, d - 1) * N + min(4 * tg + q, N - 1);
        lm[q] = lam[o];
        bt[q] = beta[o];
        cv[q] = cc[o];
        s0[q] = iir[(size_t)b * d * N + o];
    }

    // phase 0: every load of the workgroup in one round: all values go to registers first
    // (the common sizes: up to 128 window rows and taps, 64 block rows, 16 short taps), then
    // to LDS; rows beyond those sizes are staged by a plain loop afterwards.  The loads are
    // unconditional, from clamped (always valid) addresses, their values masked where they are
    // stored: with no branch around a load the compiler counts the loads in flight exactly and
    // waits for each one only where it is used; activations stay raw bits until then (a
    // conversion next to a load would wait for it there).
    {
        constexpr int SW = 8, SX = 4;                   // rows per thread of the register batch
        const int chc = min(ch, d - 1);
        float vw[SW], vt[SW], vst;
        typename ActRaw<ACT>::R rx[SX], rsw;
#pragma unroll
        for (int u = 0; u < SW; ++u) {
            const int r = row + 16 * u;
            vw[u] = (W > 0 ? ow + (size_t)min(r, W - 1) * d : w_outer)[chc];     // no window: any valid row
            vt[u] = w_outer[(size_t)min(r, To - 1) * d + chc];
        }
#pragma unroll
        for (int u = 0; u < SX; ++u) rx[u] = ActRaw<ACT>::load(xb, (size_t)min(row + 16 * u, R - 1) * d + chc);
        rsw = ActRaw<ACT>::load(Ws > 0 ? sw + (size_t)min(row, Ws - 1) * d : xb, chc);
        vst = w_short[(size_t)min(row, Ts - 1) * d + chc];
#pragma unroll
        for (int u = 0; u < SW; ++u) {
            const int r = row + 16 * u;
            if (r < W) fb[r * kCG + cl] = keep_if(vw[u], live);
            if (r < To) wl[r * kCG + cl] = keep_if(vt[u], live);
        }
#pragma unroll
        for (int u = 0; u < SX; ++u) {
            const int r = row + 16 * u;
            if (r < R) xs[(Ws + r) * kCG + cl] = keep_if(ActRaw<ACT>::cvt(rx[u]), live);
        }
        if (row < Ws) xs[row * kCG + cl] = keep_if(ActRaw<ACT>::cvt(rsw), live);
        if (row < Ts) ws[row * kCG + cl] = keep_if(vst, live);
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

    // phase 2: outer FIR, g_i = sum_{j<To} w_outer[j] * fbar[i-j].  Chunk k holds taps
    // [k CS, min((k + 1) CS, To)), CS = ceil(To / kFirChunks); a task sums its chunk in
    // ascending tap order for outputs i0 .. i0 + 15 of one candidate, 16 taps per step from a
    // register window win[q] = fbar[i0 - js - 15 + q].  Taps past the chunk's end enter with
    // weight 0.  Every output's order depends on To only (not on P or the candidate count).
    {
        // task t: channel t % 16, chunk (t / 64) % 4 (one chunk per wave, so the waves of a
        // workgroup run the four chunks side by side and a wave's lanes share their steps'
        // path), (candidate, position block) pair 4 (t / 256) + (t / 16) % 4
        static_assert(kFirChunks * 64 == kConvT, "one tap chunk per wave");
        const int CS = (To + kFirChunks - 1) / kFirChunks;
        const int IB = (P + 15) / 16;                   // 16-position blocks per candidate
        const int pairs = IB * nc;
        const int tasks = kConvT * ((pairs + 3) / 4);
        for (int t = tid; t < tasks; t += kConvT) {
            const int tcl = t % kCG;
            const int k = (t / 64) % kFirChunks;
            const int cb = 4 * (t / kConvT) + (t / kCG) % 4;
            if (cb >= pairs) continue;
            const int ib = cb % IB, c = cb / IB;
            const int i0 = 16 * ib, j0 = k * CS, j1 = min(j0 + CS, To);
            const int crow = W + c * P;                 // LDS row of candidate c's f_0
            const float* fcol = fb + tcl;
            // fbar[m] of candidate c (LDS row W + m for m < 0, crow + m for m >= 0); 0 outside
            // [-W, P) (only taps of weight 0 or outputs past P read there).  Branch-free: the
            // row is clamped into range and the value selected, so the 31 reads of a step
            // issue back to back.
            auto fbar = [&](int m) -> float {
                const int rw = m >= 0 ? crow + min(m, P - 1) : W + max(m, -W);
                return keep_if(fcol[rw * kCG], m >= -W && m < P);
            };
            float acc[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) acc[u] = 0.f;
            for (int js = j0; js < j1; js += 16) {
                float wv[16], win[31];
                const bool full = js + 16 <= j1;
                if (full && (js >= i0 + 16 || js == i0)) {
                    // full steps at fixed LDS offsets, no masks: the window m = i0 - js - 15 + q
                    // lies in the committed window rows (js >= i0 + 16; m >= -W since js + 15 < To)
                    // or straddles them and candidate c's rows at q = 15 (js == i0).  Rows at
                    // m >= P only reach outputs past P, which are not stored; they stay inside the
                    // LDS allocation (at most row W + R + 14).
                    const float* wrow = wl + (size_t)js * kCG + tcl;
#pragma unroll
                    for (int u = 0; u < 16; ++u) wv[u] = wrow[u * kCG];
                    if (js >= i0 + 16) {
                        const float* frow = fcol + (W + i0 - js - 15) * kCG;
#pragma unroll
                        for (int q = 0; q < 31; ++q) win[q] = frow[q * kCG];
                    } else {
                        const float* wrow0 = fcol + (W - 15) * kCG;      // q < 15: window row W + q - 15
                        const float* brow0 = fcol + (crow - 15) * kCG;   // q >= 15: block row q - 15
#pragma unroll
                        for (int q = 0; q < 31; ++q) win[q] = q < 15 ? wrow0[q * kCG] : brow0[q * kCG];
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < 16; ++u) wv[u] = keep_if(wl[min(js + u, To - 1) * kCG + tcl], js + u < j1);
#pragma unroll
                    for (int q = 0; q < 31; ++q) win[q] = fbar(i0 - js - 15 + q);
                }
#pragma unroll
                for (int u = 0; u < 16; ++u)
#pragma unroll
                    for (int o = 0; o < 16; ++o) acc[o] = fmaf(wv[u], win[o - u + 15], acc[o]);
            }
            float* gk = gl + ((size_t)k * R + c * P) * kCG + tcl;
#pragma unroll
            for (int o = 0; o < 16; ++o)
                if (i0 + o < P) gk[(i0 + o) * kCG] = acc[o];
        }
    }
    __syncthreads();

#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const bool ok = scan && 4 * tg + q < N;
        lm[q] = keep_if(lm[q], ok);
        bt[q] = keep_if(bt[q], ok);
        cv[q] = keep_if(cv[q], ok);
        s0[q] = keep_if(s0[q], ok);
    }

    // phase 3: IIR scan from the committed state, in registers.  A task = (channel, candidate,
    // group of 4 poles); 256 / (16 G) candidates advance together.  y_i adds the group's four
    // terms in pole order, then the G groups by a fixed-order butterfly: the order depends on N
    // only, never on P or the candidates.
    if (N == 16) {
        // 16 poles (G = 4): task (channel, candidate) per 4 lanes, one candidate per wave and
        // pass; pointers advance by one position per step, the quad sum runs on the vector ALU
        auto g_of = [&](int r) -> float {
            float g = gl[r * kCG + tch];
#pragma unroll
            for (int k = 1; k < kFirChunks; ++k) g += gl[((size_t)k * R + r) * kCG + tch];
            return g;
        };
        const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);      // == tc
        const size_t sstep = (size_t)d * 16;
        for (int c = wv; c < nc; c += kConvT / 64) {
            const int r0c = c * P;
            float st[4] = {s0[0], s0[1], s0[2], s0[3]};
            float* so = s_out + (((size_t)b * R + r0c) * d + chn) * 16 + 4 * tg;
            typename Act<ACT>::T* yo = y_out + ((size_t)b * R + r0c) * d + chn;
            float gn = g_of(r0c);
            for (int i = 0; i < P; ++i) {
                const float g = scan ? gn : 0.f;
                if (i + 1 < P) gn = g_of(r0c + i + 1);
                float py = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    st[q] = fmaf(lm[q], st[q], bt[q] * g);
                    py = fmaf(cv[q], st[q], py);
                }
                if (scan) *(float4*)so = make_float4(st[0], st[1], st[2], st[3]);
                py += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(py), 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
                py += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(py), 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
                if (scan && tg == 0) Act<ACT>::store(yo, 0, py);
                so += sstep;
                yo += d;
            }
        }
    } else {
        const int per = kConvT / (G * kCG);
        // g of row r: the chunk sums added in chunk order
        auto g_of = [&](int r) -> float {
            float g = gl[r * kCG + tch];
#pragma unroll
            for (int k = 1; k < kFirChunks; ++k) g += gl[((size_t)k * R + r) * kCG + tch];
            return g;
        };
        for (int c = tc; c - tc < nc; c += per) {
            const bool act = scan && c < nc;
            const int cr = min(c, nc - 1) * P;        // in-range rows for the reads of idle tasks
            float st[4] = {s0[0], s0[1], s0[2], s0[3]};
            float gn = g_of(cr);                       // the next position's input, read ahead
            for (int i = 0; i < P; ++i) {
                const int r = c * P + i;
                const float g = act ? gn : 0.f;
                if (i + 1 < P) gn = g_of(cr + i + 1);
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
                py = group_sum(py, G);
                if (act && tg == 0) Act<ACT>::store(y_out, ((size_t)b * R + r) * d + chn, py);
            }
        }
    }
}

}  // namespace hci
