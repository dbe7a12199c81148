// Conv/recurrent half of the block forward: short depthwise FIR -> outer
// depthwise FIR -> diagonal modal IIR scan that keeps every per-position
// state (EvSpark digest, Figure 1(d): the outer-FIR inputs u_i and the IIR
// states s_i are what slicing later selects from).
//
// One workgroup = 16 channels of one (sequence, candidate) block, 256
// threads, so a 4096-channel layer spreads over 256 workgroups.
//  phase 0  the outer window rows and the outer taps of the 16 channels are
//           staged in LDS
//  phase 1  thread (position, channel) computes f_i (short FIR)
//  phase 2  the same threads compute g_i = sum_j w_outer[j] * fbar[i-j]
//           from LDS, one fixed-order fma chain per output
//  phase 3  thread (channel, pole lane) runs the IIR recurrence in fp32
//           registers over the P positions and writes s_i (a contiguous
//           kilobyte per step), the readout y_i is a fixed-order butterfly
//           over the 16 pole lanes.
// All per-output arithmetic happens in a fixed order that does not depend
// on P, so a block forward and P single-position forwards give identical
// bits for f, s and y.
#include "hci_internal.h"

namespace hci {

constexpr int kCG = 16;        // channels per workgroup
constexpr int kConvT = 256;    // threads per workgroup

size_t conv_iir_lds_bytes(int To, int P) {
    return (size_t)((To - 1 + P) + To + P) * kCG * sizeof(float);
}

template <int ACT>
__global__ __launch_bounds__(kConvT) void k_conv_iir(
    const float* __restrict__ w_short, const float* __restrict__ w_outer,
    const float* __restrict__ lam, const float* __restrict__ beta, const float* __restrict__ cc,
    const typename Act<ACT>::T* __restrict__ short_win, const float* __restrict__ outer_win,
    const float* __restrict__ iir, const typename Act<ACT>::T* __restrict__ x,
    float* __restrict__ f_out, float* __restrict__ s_out, typename Act<ACT>::T* __restrict__ y_out,
    int d, int Ts, int To, int N, int nc, int P)
{
    extern __shared__ float lds[];
    const int W = To - 1;
    float* fbar = lds;                          // [W + P][kCG]: row r holds fbar[r - W]
    float* wl = fbar + (size_t)(W + P) * kCG;   // [To][kCG]
    float* gl = wl + (size_t)To * kCG;          // [P][kCG]

    const int ch0 = blockIdx.x * kCG;
    const int c = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int cl = tid & (kCG - 1), row = tid >> 4;     // 16 rows of 16 channels per pass
    const int ch = ch0 + cl;
    const bool live = ch < d;
    const size_t blk = (size_t)b * nc + c;
    const typename Act<ACT>::T* xb = x + blk * P * d;
    const typename Act<ACT>::T* sw = short_win + (size_t)b * (Ts - 1) * d;
    const float* ow = outer_win + (size_t)b * W * d;

    // phase 0: stage window rows and taps
    for (int r = row; r < W; r += kConvT / kCG) fbar[r * kCG + cl] = live ? ow[(size_t)r * d + ch] : 0.f;
    for (int j = row; j < To; j += kConvT / kCG) wl[j * kCG + cl] = live ? w_outer[(size_t)j * d + ch] : 0.f;

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

    // phase 3: IIR scan. thread (channel = tid / 16, lane n = tid % 16) owns poles n, n+16, ...
    const int lane16 = tid & 15;
    const int cg = tid >> 4;
    const int chn = ch0 + cg;
    if (chn >= d) return;                        // uniform across the 16-lane group
    float s[4], lm[4], bt[4], cv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int n = lane16 + 16 * r;
        const bool ok = n < N;
        const size_t o = (size_t)chn * N + n;
        s[r] = ok ? iir[(size_t)b * d * N + o] : 0.f;
        lm[r] = ok ? lam[o] : 0.f;
        bt[r] = ok ? beta[o] : 0.f;
        cv[r] = ok ? cc[o] : 0.f;
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

hipError_t launch_conv_iir(const hci_layer* L, const hci_state* S, const hci_block* blk,
                           int nb, int nc, int P, hipStream_t st)
{
    dim3 grid((L->d + kCG - 1) / kCG, nc, nb), block(kConvT);
    const size_t lds = conv_iir_lds_bytes(L->taps_outer, P);
    if (lds > 65536) {
        // allow the dynamic LDS request beyond the default 64 KiB (gfx950 has 160 KiB per CU)
        hipError_t e = hipFuncSetAttribute(L->act_dtype == HCI_BF16 ? (const void*)k_conv_iir<HCI_BF16>
                                                                    : (const void*)k_conv_iir<HCI_F32>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (L->act_dtype == HCI_BF16) {
        hipLaunchKernelGGL(k_conv_iir<HCI_BF16>, grid, block, lds, st,
            L->w_short, L->w_outer, L->lambda, L->beta, L->c,
            (const uint16_t*)S->short_win, S->outer_win, S->iir, (const uint16_t*)blk->x,
            blk->f, blk->s, (uint16_t*)blk->y, L->d, L->taps_short, L->taps_outer, L->poles, nc, P);
    } else {
        hipLaunchKernelGGL(k_conv_iir<HCI_F32>, grid, block, lds, st,
            L->w_short, L->w_outer, L->lambda, L->beta, L->c,
            (const float*)S->short_win, S->outer_win, S->iir, (const float*)blk->x,
            blk->f, blk->s, (float*)blk->y, L->d, L->taps_short, L->taps_outer, L->poles, nc, P);
    }
    return hipGetLastError();
}

}  // namespace hci
