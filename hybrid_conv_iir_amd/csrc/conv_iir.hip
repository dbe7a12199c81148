// Conv/recurrent half of the block forward: short depthwise FIR -> outer
// depthwise FIR -> diagonal modal IIR scan that keeps every per-position
// state (EvSpark digest, Figure 1(d): the outer-FIR inputs u_i and the IIR
// states s_i are what slicing later selects from).
//
// One workgroup = 64 channels of one (sequence, candidate) block.
//  phase 1  thread (channel, part) computes f_i for i = part, part+4, ...
//  phase 2  the same threads compute g_i = sum_j w_outer[j] * fbar[i-j]
//  phase 3  thread (channel, pole lane) runs the IIR recurrence in fp32
//           registers over the P positions and writes s_i (coalesced), the
//           readout y_i is a fixed-order reduction over the pole lanes.
// All per-output arithmetic happens in a fixed order that does not depend
// on P, so a block forward and P single-position forwards give identical
// bits for f, s and y.
#include "hci_internal.h"

namespace hci {

constexpr int kCG = 64;        // channels per workgroup
constexpr int kMaxP = 65;      // LDS rows for f and g

template <int ACT>
__global__ __launch_bounds__(256) void k_conv_iir(
    const float* __restrict__ w_short, const float* __restrict__ w_outer,
    const float* __restrict__ lam, const float* __restrict__ beta, const float* __restrict__ cc,
    const typename Act<ACT>::T* __restrict__ short_win, const float* __restrict__ outer_win,
    const float* __restrict__ iir, const typename Act<ACT>::T* __restrict__ x,
    float* __restrict__ f_out, float* __restrict__ s_out, typename Act<ACT>::T* __restrict__ y_out,
    int d, int Ts, int To, int N, int nc, int P)
{
    __shared__ float f_lds[kMaxP][kCG];
    __shared__ float g_lds[kMaxP][kCG];

    const int ch0 = blockIdx.x * kCG;
    const int c = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int cl = tid & (kCG - 1), part = tid >> 6;
    const int ch = ch0 + cl;
    const bool live = ch < d;
    const size_t blk = (size_t)b * nc + c;
    const typename Act<ACT>::T* xb = x + blk * P * d;
    const typename Act<ACT>::T* sw = short_win + (size_t)b * (Ts - 1) * d;
    const float* ow = outer_win + (size_t)b * (To - 1) * d;

    // phase 1: short FIR, f_i = sum_{j<Ts} w_short[j] * xbar[i-j]
    for (int i = part; i < P; i += 4) {
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
        f_lds[i][cl] = acc;
    }
    __syncthreads();

    // phase 2: outer FIR, g_i = sum_{j<To} w_outer[j] * fbar[i-j]
    for (int i = part; i < P; i += 4) {
        float acc = 0.f;
        if (live) {
            for (int j = 0; j < To; ++j) {
                const int m = i - j;
                const float fv = (m >= 0) ? f_lds[m][cl] : ow[(size_t)(To - 1 + m) * d + ch];
                acc = fmaf(w_outer[(size_t)j * d + ch], fv, acc);
            }
        }
        g_lds[i][cl] = acc;
    }
    __syncthreads();

    // phase 3: IIR scan. 16 lanes per channel, lane n owns poles n, n+16, ...
    const int lane16 = tid & 15;
    for (int cg = tid >> 4; cg < kCG; cg += 16) {
        const int chn = ch0 + cg;
        if (chn >= d) break;                     // uniform across the 16-lane group
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
            const float g = g_lds[i][cg];
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
}

hipError_t launch_conv_iir(const hci_layer* L, const hci_state* S, const hci_block* blk,
                           int nb, int nc, int P, hipStream_t st)
{
    dim3 grid((L->d + kCG - 1) / kCG, nc, nb), block(256);
    if (L->act_dtype == HCI_BF16) {
        hipLaunchKernelGGL(k_conv_iir<HCI_BF16>, grid, block, 0, st,
            L->w_short, L->w_outer, L->lambda, L->beta, L->c,
            (const uint16_t*)S->short_win, S->outer_win, S->iir, (const uint16_t*)blk->x,
            blk->f, blk->s, (uint16_t*)blk->y, L->d, L->taps_short, L->taps_outer, L->poles, nc, P);
    } else {
        hipLaunchKernelGGL(k_conv_iir<HCI_F32>, grid, block, 0, st,
            L->w_short, L->w_outer, L->lambda, L->beta, L->c,
            (const float*)S->short_win, S->outer_win, S->iir, (const float*)blk->x,
            blk->f, blk->s, (float*)blk->y, L->d, L->taps_short, L->taps_outer, L->poles, nc, P);
    }
    return hipGetLastError();
}

}  // namespace hci
