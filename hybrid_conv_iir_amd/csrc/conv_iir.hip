// Conv/recurrent half of the block forward: short depthwise FIR -> outer
// depthwise FIR -> diagonal modal IIR scan that keeps every per-position
// state (EvSpark digest, Figure 1(d): the outer-FIR inputs u_i and the IIR
// states s_i are what slicing later selects from).
//
// One workgroup = 16 channels of one sequence, 256 threads, so a
// 4096-channel layer spreads over 256 workgroups per sequence; the candidate
// blocks of the sequence share the committed window and taps and run phases
// 1-3 in turn.
//  phase 0  the outer window rows and the outer taps of the 16 channels are
//           staged in LDS (once)
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
#include "conv_iir_body.h"

namespace hci {

size_t conv_iir_lds_bytes(int To, int P) { return conv_iir_lds_floats(To, P) * sizeof(float); }

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
    conv_iir_block<ACT>(w_short, w_outer, lam, beta, cc, short_win, outer_win, iir, x, f_out, s_out, y_out,
                        d, Ts, To, N, nc, P, blockIdx.x, blockIdx.y, lds);
}

hipError_t launch_conv_iir(const hci_layer* L, const hci_state* S, const hci_block* blk,
                           int nb, int nc, int P, hipStream_t st)
{
    dim3 grid((L->d + kCG - 1) / kCG, nb), block(kConvT);
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
