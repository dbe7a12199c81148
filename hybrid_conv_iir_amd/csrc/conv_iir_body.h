// Conv/recurrent half of the block forward as a workgroup-level device
// function, shared by the stand-alone conv/IIR kernel and the fused
// verify kernel.  See conv_iir.hip for the description of the phases.
#pragma once

#include "hci_internal.h"

namespace hci {

constexpr int kCG = 16;        // channels per workgroup
constexpr int kConvT = 256;    // threads per workgroup

__host__ __device__ inline size_t conv_iir_lds_floats(int To, int P) {
    return (size_t)((To - 1 + P) + To + P) * kCG;
}

// one workgroup: channel group cgi (16 channels) of sequence b, for every
// candidate block c = 0..nc-1 in turn (they share the committed window and
// the taps, staged once); lds holds conv_iir_lds_floats(To, P) floats
template <int ACT>
__device__ __forceinline__ void conv_iir_block(
    const float* __restrict__ w_short, const float* __restrict__ w_outer,
    const float* __restrict__ lam, const float* __restrict__ beta, const float* __restrict__ cc,
    const typename Act<ACT>::T* __restrict__ short_win, const float* __restrict__ outer_win,
    const float* __restrict__ iir, const typename Act<ACT>::T* __restrict__ x,
    float* __restrict__ f_out, float* __restrict__ s_out, typename Act<ACT>::T* __restrict__ y_out,
    int d, int Ts, int To, int N, int nc, int P, int cgi, int b, float* lds)
{
    const int W = To - 1;
    float* fbar = lds;                          // [W + P][kCG]: row r holds fbar[r - W]
    float* wl = fbar + (size_t)(W + P) * kCG;   // [To][kCG]
    float* gl = wl + (size_t)To * kCG;          // [P][kCG]

    const int ch0 = cgi * kCG;
    const int tid = threadIdx.x;
    const int cl = tid & (kCG - 1), row = tid >> 4;     // 16 rows of 16 channels per pass
    const int ch = ch0 + cl;
    const bool live = ch < d;
    const typename Act<ACT>::T* sw = short_win + (size_t)b * (Ts - 1) * d;
    const float* ow = outer_win + (size_t)b * W * d;

    // phase 0: stage window rows and taps (once for all candidates)
    for (int r = row; r < W; r += kConvT / kCG) fbar[r * kCG + cl] = live ? ow[(size_t)r * d + ch] : 0.f;
    for (int j = row; j < To; j += kConvT / kCG) wl[j * kCG + cl] = live ? w_outer[(size_t)j * d + ch] : 0.f;

    // IIR parameters of thread (channel = tid / 16, lane n = tid % 16): poles n, n+16, ...
    const int lane16 = tid & 15;
    const int cg = tid >> 4;
    const int chn = ch0 + cg;
    const bool scan = chn < d;                          // uniform across the 16-lane group
    float lm[4], bt[4], cv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int n = lane16 + 16 * r;
        const bool ok = scan && n < N;
        const size_t o = (size_t)chn * N + n;
        lm[r] = ok ? lam[o] : 0.f;
        bt[r] = ok ? beta[o] : 0.f;
        cv[r] = ok ? cc[o] : 0.f;
    }

    for (int c = 0; c < nc; ++c) {
        const size_t blk = (size_t)b * nc + c;
        const typename Act<ACT>::T* xb = x + blk * P * d;

        // phase 1: short FIR, f_i = sum_{j<Ts} w_short[j] * xbar[i-j]
        for (int i = row; i < P; i += kConvT / kCG) {
            float acc = 0.f;
            if (live) {
                for (int j = 0; j < Ts; ++j) {
                    const int m = i - j;
                    const float xv = (m >= 0) ? Act<ACT>::load(xb, (size_t)m * d + ch)
                                              : Act<ACT>::load(sw, (size_t)(Ts - 1 + m) * d + ch);
                    acc = fmaf(w_short[(size_t)j * d + ch], xv, acc);
                }
                f_out[(blk * P + i) * d + ch] = acc;
            }
            fbar[(W + i) * kCG + cl] = acc;
        }
        __syncthreads();

        // phase 2: outer FIR, g_i = sum_{j<To} w_outer[j] * fbar[i-j], j ascending
        for (int i = row; i < P; i += kConvT / kCG) {
            float acc = 0.f;
            const float* fp = fbar + (W + i) * kCG + cl;
            const float* wp = wl + cl;
#pragma unroll 8
            for (int j = 0; j < To; ++j) acc = fmaf(wp[j * kCG], fp[-j * kCG], acc);
            gl[i * kCG + cl] = acc;
        }
        __syncthreads();

        // phase 3: IIR scan from the committed state, in registers
        if (scan) {
            float s[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int n = lane16 + 16 * r;
                s[r] = n < N ? iir[(size_t)b * d * N + (size_t)chn * N + n] : 0.f;
            }
            for (int i = 0; i < P; ++i) {
                const float g = gl[i * kCG + cg];
                float part_y = 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = lane16 + 16 * r;
                    s[r] = fmaf(lm[r], s[r], bt[r] * g);
                    if (n < N) s_out[((blk * P + i) * d + chn) * N + n] = s[r];
                    part_y = fmaf(cv[r], s[r], part_y);
                }
                // fixed-order butterfly over the 16 pole lanes of this channel
                part_y += __shfl_xor(part_y, 8, 16);
                part_y += __shfl_xor(part_y, 4, 16);
                part_y += __shfl_xor(part_y, 2, 16);
                part_y += __shfl_xor(part_y, 1, 16);
                if (lane16 == 0) Act<ACT>::store(y_out, (blk * P + i) * d + chn, part_y);
            }
        }
        __syncthreads();                             // f rows and g of this candidate are reused by the next
    }
}

}  // namespace hci
