// Prefill: run a prompt of T positions through the conv/recurrent path and
// append its K/V rows, leaving the committed state the first verify starts
// from.  By the block-forward contract (EvSpark digest, Interpretation: one
// block forward plus slicing restores the state sequential decoding would
// reach) this is a block forward over all T positions followed by a slice at
// T-1, restricted to the state; the prompt's attention outputs are not part
// of the state and are not computed.
//
// The IIR is linear and diagonal, so time is cut into chunks of 256
// positions (16 sub-chunks of 16) that scan independently from a zero state;
// the true start state of every chunk follows from a short carry scan over
// the chunk end states, and a fix-up adds its decayed contribution.
//   k_prefill_local  per (channel group, chunk): short FIR over the chunk and
//                    its halo into LDS, the outer FIR with a 31-value
//                    register window per thread (16 outputs x 16 taps per
//                    step, 2 LDS reads per 16 FMAs), the sub-chunk scans, the
//                    in-chunk carry, chunk-local readouts y and the chunk end
//                    state; the last To-1 f values of the prompt go to the
//                    workspace for the outer window
//   k_prefill_carry  per (sequence, channel, pole): chunk start states and
//                    the final IIR state (committed)
//   k_prefill_fixup  per (channel group, chunk): y += sum_n c lambda^(tau+1) S_chunk
//   k_prefill_commit FIR windows <- the prompt's last inputs
//   k_kv_pack        K/V rows appended in the tiled cache layout, then
//   k_len_add        kv_len += T.
#include "hci_internal.h"

namespace hci {

constexpr int kPfCG = 16;                  // channels per workgroup
constexpr int kPfS = 16;                   // positions per sub-chunk (outputs per thread)
constexpr int kPfSub = 16;                 // sub-chunks per chunk
constexpr int kPfC = kPfS * kPfSub;        // positions per chunk
constexpr int kPfT = kPfCG * kPfSub;       // threads per workgroup (channel, sub-chunk)
constexpr int kPfN = 16;                   // poles held in registers (N <= 16)

__host__ __device__ inline int pf_taps_padded(int To) { return (To + 15) / 16 * 16; }

size_t prefill_lds_bytes(int To) {
    const int Wp = pf_taps_padded(To) - 1;
    return ((size_t)(Wp + kPfC) * kPfCG + (size_t)pf_taps_padded(To) * kPfCG + (size_t)kPfSub * kPfCG * kPfN) * 4;
}

PrefillPlan plan_prefill(const hci_layer* L, int nb, int T, bool want_y) {
    PrefillPlan p{};
    p.nchunks = (T + kPfC - 1) / kPfC;
    p.s_elems = (size_t)nb * p.nchunks * L->d * kPfN;
    p.ftail_elems = (size_t)nb * (L->taps_outer - 1 > 0 ? L->taps_outer - 1 : 1) * L->d;
    p.yloc_elems = want_y ? (size_t)nb * T * L->d : 0;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    p.bytes = up(p.s_elems * 4) + up(p.ftail_elems * 4) + up(p.yloc_elems * 4);
    return p;
}

template <int ACT>
__global__ __launch_bounds__(kPfT) void k_prefill_local(
    const float* __restrict__ w_short, const float* __restrict__ w_outer,
    const float* __restrict__ lam, const float* __restrict__ beta, const float* __restrict__ cc,
    const typename Act<ACT>::T* __restrict__ short_win, const float* __restrict__ outer_win,
    const typename Act<ACT>::T* __restrict__ x, float* __restrict__ s_loc, float* __restrict__ f_tail,
    float* __restrict__ y_loc, int d, int Ts, int To, int N, int T, int nchunks)
{
    extern __shared__ float lds[];
    const int TP = pf_taps_padded(To);
    const int W = To - 1, Wp = TP - 1;
    float* fb = lds;                               // [Wp + C][16]: row r holds fbar[t0 - Wp + r]
    float* wl = fb + (size_t)(Wp + kPfC) * kPfCG;  // [TP][16], zero past To
    float* se = wl + (size_t)TP * kPfCG;           // [sub][16 ch][16 poles]

    const int cg = blockIdx.x, chunk = blockIdx.y, b = blockIdx.z;
    const int ch0 = cg * kPfCG;
    const int t0 = chunk * kPfC;
    const int tid = threadIdx.x;
    const typename Act<ACT>::T* xb = x + (size_t)b * T * d;
    const typename Act<ACT>::T* sw = short_win + (size_t)b * (Ts - 1) * d;
    const float* ow = outer_win + (size_t)b * W * d;

    // short FIR over the chunk and its halo: fbar[t] for t in [t0 - Wp, t0 + C)
    for (int e = tid; e < (Wp + kPfC) * kPfCG; e += kPfT) {
        const int r = e / kPfCG, c = e % kPfCG, ch = ch0 + c;
        const int t = t0 - Wp + r;
        float v = 0.f;
        if (ch < d) {
            if (t < 0) {
                v = (t >= -W) ? ow[(size_t)(W + t) * d + ch] : 0.f;     // committed outer-FIR inputs
            } else if (t < T) {
                for (int j = 0; j < Ts; ++j) {
                    const int m = t - j;
                    const float xv = (m >= 0) ? Act<ACT>::load(xb, (size_t)m * d + ch)
                                              : Act<ACT>::load(sw, (size_t)(Ts - 1 + m) * d + ch);
                    v = fmaf(w_short[(size_t)j * d + ch], xv, v);
                }
                if (r >= Wp && t >= T - W) f_tail[((size_t)b * W + (t - (T - W))) * d + ch] = v;
            }
        }
        fb[e] = v;
    }
    for (int e = tid; e < TP * kPfCG; e += kPfT) {
        const int j = e / kPfCG, c = e % kPfCG, ch = ch0 + c;
        wl[e] = (j < To && ch < d) ? w_outer[(size_t)j * d + ch] : 0.f;
    }
    __syncthreads();

    // outer FIR: thread (c, sub) computes g for its 16 positions, taps in blocks of 16:
    // R[m] = fbar[tau0 - jb - 15 + m], then g[tau] += w[jb+u] * R[tau - u + 15]
    const int c = tid % kPfCG, sub = tid / kPfCG;
    const int ch = ch0 + c;
    const int tau0 = sub * kPfS;
    float g[kPfS];
#pragma unroll
    for (int i = 0; i < kPfS; ++i) g[i] = 0.f;
    for (int jb = 0; jb < TP; jb += 16) {
        float R[31];
        const int base = Wp + tau0 - jb - 15;      // fb row of R[0]
#pragma unroll
        for (int m = 0; m < 31; ++m) R[m] = fb[(base + m) * kPfCG + c];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const float w = wl[(jb + u) * kPfCG + c];
#pragma unroll
            for (int i = 0; i < kPfS; ++i) g[i] = fmaf(w, R[i - u + 15], g[i]);
        }
    }

    // sub-chunk scan from a zero state, all poles in registers
    float lm[kPfN], bt[kPfN], cv[kPfN], s[kPfN];
#pragma unroll
    for (int n = 0; n < kPfN; ++n) {
        const bool ok = n < N && ch < d;
        const size_t o = (size_t)ch * N + n;
        lm[n] = ok ? lam[o] : 0.f;
        bt[n] = ok ? beta[o] : 0.f;
        cv[n] = ok ? cc[o] : 0.f;
        s[n] = 0.f;
    }
    const int valid = max(0, min(kPfS, T - (t0 + tau0)));       // positions of this sub-chunk inside the prompt
    float y[kPfS];
#pragma unroll
    for (int i = 0; i < kPfS; ++i) {
        float acc = 0.f;
        if (i < valid) {
#pragma unroll
            for (int n = 0; n < kPfN; ++n) {
                s[n] = fmaf(lm[n], s[n], bt[n] * g[i]);
                acc = fmaf(cv[n], s[n], acc);
            }
        }
        y[i] = acc;
    }
#pragma unroll
    for (int n = 0; n < kPfN; ++n) se[((size_t)sub * kPfCG + c) * kPfN + n] = s[n];
    __syncthreads();

    // in-chunk carry: thread (channel c2, pole n2) turns the 16 sub-chunk end states into start states
    {
        const int c2 = tid / kPfN, n2 = tid % kPfN, ch2 = ch0 + c2;
        const float l2 = (n2 < N && ch2 < d) ? lam[(size_t)ch2 * N + n2] : 0.f;
        float S = 0.f;
        for (int sb = 0; sb < kPfSub; ++sb) {
            const int len = max(0, min(kPfS, T - (t0 + sb * kPfS)));
            const float e = se[((size_t)sb * kPfCG + c2) * kPfN + n2];
            se[((size_t)sb * kPfCG + c2) * kPfN + n2] = S;                 // start state of sub-chunk sb
            float p = 1.f;
            for (int i = 0; i < len; ++i) p *= l2;
            S = fmaf(p, S, e);
        }
        if (ch2 < d) s_loc[(((size_t)b * nchunks + chunk) * d + ch2) * kPfN + n2] = S;   // chunk end (local)
    }
    __syncthreads();

    // chunk-local readouts: add the decayed sub-chunk start state
    if (y_loc != nullptr && ch < d) {
        float p[kPfN];
#pragma unroll
        for (int n = 0; n < kPfN; ++n) p[n] = se[((size_t)sub * kPfCG + c) * kPfN + n];
#pragma unroll
        for (int i = 0; i < kPfS; ++i) {
            if (i < valid) {
                float acc = 0.f;
#pragma unroll
                for (int n = 0; n < kPfN; ++n) {
                    p[n] *= lm[n];
                    acc = fmaf(cv[n], p[n], acc);
                }
                y_loc[((size_t)b * T + t0 + tau0 + i) * d + ch] = y[i] + acc;
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_prefill_carry(
    const float* __restrict__ lam, float* __restrict__ iir, float* __restrict__ s_loc,
    int d, int N, int T, int nchunks, int nb)
{
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;   // (b, ch, n), n fastest
    if (e >= (size_t)nb * d * kPfN) return;
    const int n = (int)(e % kPfN);
    const int ch = (int)((e / kPfN) % d);
    const int b = (int)(e / ((size_t)kPfN * d));
    if (n >= N) return;
    const float l = lam[(size_t)ch * N + n];
    float pc = 1.f;
    for (int i = 0; i < kPfC; ++i) pc *= l;                 // lambda^C for full chunks
    float S = iir[((size_t)b * d + ch) * N + n];
    float* sp = s_loc + ((size_t)b * nchunks * d + ch) * kPfN + n;
    const size_t stride = (size_t)d * kPfN;
    for (int k = 0; k < nchunks; ++k) {
        const float end = sp[k * stride];
        sp[k * stride] = S;                                  // start state of chunk k
        const int len = min(kPfC, T - k * kPfC);
        float p = pc;
        if (len < kPfC) {
            p = 1.f;
            for (int i = 0; i < len; ++i) p *= l;
        }
        S = fmaf(p, S, end);
    }
    iir[((size_t)b * d + ch) * N + n] = S;                   // committed IIR state after the prompt
}

template <int ACT>
__global__ __launch_bounds__(kPfT) void k_prefill_fixup(
    const float* __restrict__ lam, const float* __restrict__ cc, const float* __restrict__ s_loc,
    const float* __restrict__ y_loc, typename Act<ACT>::T* __restrict__ y, int d, int N, int T, int nchunks)
{
    const int cg = blockIdx.x, chunk = blockIdx.y, b = blockIdx.z;
    const int c = threadIdx.x % kPfCG, sub = threadIdx.x / kPfCG;
    const int ch = cg * kPfCG + c;
    if (ch >= d) return;
    const int t0 = chunk * kPfC + sub * kPfS;
    const int valid = max(0, min(kPfS, T - t0));
    float p[kPfN], lm[kPfN], cv[kPfN];
#pragma unroll
    for (int n = 0; n < kPfN; ++n) {
        const bool ok = n < N;
        lm[n] = ok ? lam[(size_t)ch * N + n] : 0.f;
        cv[n] = ok ? cc[(size_t)ch * N + n] : 0.f;
        float v = ok ? s_loc[(((size_t)b * nchunks + chunk) * d + ch) * kPfN + n] : 0.f;
        for (int i = 0; i < sub * kPfS; ++i) v *= lm[n];    // decay to the sub-chunk start
        p[n] = v;
    }
    for (int i = 0; i < valid; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int n = 0; n < kPfN; ++n) {
            p[n] *= lm[n];
            acc = fmaf(cv[n], p[n], acc);
        }
        const size_t o = ((size_t)b * T + t0 + i) * d + ch;
        Act<ACT>::store(y, o, y_loc[o] + acc);
    }
}

// FIR windows <- last inputs of the prompt: new[r] = concat(old, rows)[T + r]
template <int ACT>
__global__ __launch_bounds__(256) void k_prefill_commit(
    typename Act<ACT>::T* __restrict__ short_win, float* __restrict__ outer_win,
    const typename Act<ACT>::T* __restrict__ x, const float* __restrict__ f_tail, int d, int Ts, int To, int T)
{
    const int b = blockIdx.y;
    const int ch = blockIdx.x * blockDim.x + threadIdx.x;
    if (ch >= d) return;
    // every thread owns one channel column, rows ascending: new row r reads row T + r > r of the
    // concatenation, which this thread has not written yet
    const int Ws = Ts - 1;
    typename Act<ACT>::T* sw = short_win + (size_t)b * Ws * d;
    for (int r = 0; r < Ws; ++r) {
        const long long m = (long long)T + r;
        const float v = (m < Ws) ? Act<ACT>::load(sw, (size_t)m * d + ch)
                                 : Act<ACT>::load(x, ((size_t)b * T + (size_t)(m - Ws)) * d + ch);
        Act<ACT>::store(sw, (size_t)r * d + ch, v);
    }
    const int W = To - 1;
    float* ow = outer_win + (size_t)b * W * d;
    for (int r = 0; r < W; ++r) {
        const long long m = (long long)T + r;
        const float v = (m < W) ? ow[(size_t)m * d + ch] : f_tail[((size_t)b * W + r) * d + ch];
        ow[(size_t)r * d + ch] = v;
    }
}

hipError_t launch_prefill(const hci_layer* L, const hci_state* S, int nb, int T, const void* x, const void* k,
                          const void* v, void* y, const PrefillPlan& plan, void* ws, hipStream_t st)
{
    float* s_loc = (float*)ws;
    float* f_tail = (float*)((char*)ws + (plan.s_elems * 4 + 255) / 256 * 256);
    float* y_loc = y ? (float*)((char*)f_tail + (plan.ftail_elems * 4 + 255) / 256 * 256) : nullptr;
    const int d = L->d;
    const size_t lds = prefill_lds_bytes(L->taps_outer);
    dim3 grid((d + kPfCG - 1) / kPfCG, plan.nchunks, nb);
    hipError_t e;
    if (L->act_dtype == HCI_BF16) {
        if (lds > 65536 && (e = hipFuncSetAttribute((const void*)k_prefill_local<HCI_BF16>,
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
            return e;
        hipLaunchKernelGGL(k_prefill_local<HCI_BF16>, grid, dim3(kPfT), lds, st, L->w_short, L->w_outer, L->lambda,
                           L->beta, L->c, (const uint16_t*)S->short_win, S->outer_win, (const uint16_t*)x, s_loc,
                           f_tail, y_loc, d, L->taps_short, L->taps_outer, L->poles, T, plan.nchunks);
    } else {
        if (lds > 65536 && (e = hipFuncSetAttribute((const void*)k_prefill_local<HCI_F32>,
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
            return e;
        hipLaunchKernelGGL(k_prefill_local<HCI_F32>, grid, dim3(kPfT), lds, st, L->w_short, L->w_outer, L->lambda,
                           L->beta, L->c, (const float*)S->short_win, S->outer_win, (const float*)x, s_loc, f_tail,
                           y_loc, d, L->taps_short, L->taps_outer, L->poles, T, plan.nchunks);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t ncarry = (size_t)nb * d * kPfN;
    hipLaunchKernelGGL(k_prefill_carry, dim3((unsigned)((ncarry + 255) / 256)), dim3(256), 0, st, L->lambda, S->iir,
                       s_loc, d, L->poles, T, plan.nchunks, nb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (y) {
        if (L->act_dtype == HCI_BF16)
            hipLaunchKernelGGL(k_prefill_fixup<HCI_BF16>, grid, dim3(kPfT), 0, st, L->lambda, L->c, s_loc, y_loc,
                               (uint16_t*)y, d, L->poles, T, plan.nchunks);
        else
            hipLaunchKernelGGL(k_prefill_fixup<HCI_F32>, grid, dim3(kPfT), 0, st, L->lambda, L->c, s_loc, y_loc,
                               (float*)y, d, L->poles, T, plan.nchunks);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    dim3 cgrid((d + 255) / 256, nb);
    if (L->act_dtype == HCI_BF16)
        hipLaunchKernelGGL(k_prefill_commit<HCI_BF16>, cgrid, dim3(256), 0, st, (uint16_t*)S->short_win, S->outer_win,
                           (const uint16_t*)x, f_tail, d, L->taps_short, L->taps_outer, T);
    else
        hipLaunchKernelGGL(k_prefill_commit<HCI_F32>, cgrid, dim3(256), 0, st, (float*)S->short_win, S->outer_win,
                           (const float*)x, f_tail, d, L->taps_short, L->taps_outer, T);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // K/V rows at kv_len .. kv_len+T-1 of every sequence, then the lengths
    const size_t row_stride = (size_t)L->heads * L->head_dim;
    for (int b = 0; b < nb; ++b) {
        e = launch_kv_pack(L, S, b, -1, T, (const char*)k + (size_t)b * T * row_stride * (L->act_dtype == HCI_BF16 ? 2 : 4),
                           (const char*)v + (size_t)b * T * row_stride * (L->act_dtype == HCI_BF16 ? 2 : 4),
                           row_stride, (size_t)L->head_dim, st);
        if (e != hipSuccess) return e;
    }
    return launch_len_add(S, nb, T, st);
}

}  // namespace hci
