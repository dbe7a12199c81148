// The kernel that ends a verify: the conv/IIR scan and the merge of the
// prefix partials with the causal block part.
#include "conv_iir_body.h"
#include "verify_parts.h"
#include "worklist.h"

#include <math.h>

namespace hci {

constexpr int kF32Dh = 128;          // largest head dim of the per-state LDS rows

// ------------------------------------------------------------------ finish
//
// The kernel that ends a verify, once the prefix stream is done and HBM is
// quiet.  Its grid holds two kinds of workgroups:
//   conv    the conv/IIR scan of 16 channels of one sequence (every
//           candidate), conv_iir_body.h; it runs here rather than inside the
//           stream because its chain of dependent loads is short only when
//           the memory system is not saturated.
//   combine RG block rows of one (sequence, candidate, head): the four waves
//           each reduce a fixed subset of the prefix items of (b, h) (item j
//           of a phase goes to wave j mod 4) into a running softmax state per
//           row; then each row's causal block part (query i against the
//           block's own keys 0..i, fp32, from K/V rows staged in LDS) is
//           computed by one wave, and the five states of a row merge in a
//           fixed order:
//             M = max m_s,  o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// Lane l holds output dims l and l + 64.  RG (1..16 rows) is chosen by the
// host so that the grid has a few workgroups per CU.

template <int ACT, int RG>
__device__ __forceinline__ void combine_job(const FinishArgs& A, int c, int rg, int h, int b, float* lds)
{
    typedef typename Act<ACT>::T T;
    const T* q = (const T*)A.q;
    const T* kb = (const T*)A.kb;
    const T* vb = (const T*)A.vb;
    const int DH = A.DH, nq = A.nq, H = A.H, P = A.P;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int d0 = lane, d1 = lane + 64;
    const bool ok0 = d0 < DH, ok1 = d1 < DH;
    const int i0 = rg * RG, nr = min(RG, P - i0);      // rows i0 .. i0 + nr - 1 of candidate c
    const int r0 = c * P + i0;                         // their query-row index within the sequence

    T* ks = (T*)lds;
    T* vs = ks + (size_t)P * DH;
    float* st_o = lds + ((size_t)2 * P * DH * sizeof(T) + 3) / 4;   // [state][row][DH]
    float* st_ml = st_o + (size_t)(kCombW + 1) * RG * DH;           // [state][row][2]

    // stage the candidate's block K and V rows 0 .. i0 + nr - 1 in 16-byte pieces (a row is
    // Dh * act bytes, a multiple of 16); the first pieces of every thread are requested together
    {
        const int pr = DH * (int)sizeof(T) / 16;       // pieces per row
        const int half = (i0 + nr) * pr;               // K pieces, then as many V pieces
        const size_t krow0 = ((size_t)b * nq + (size_t)c * P) * H + h;
        auto src = [&](int e) -> const uint4* {
            const bool isv = e >= half;
            const int e2 = isv ? e - half : e, j = e2 / pr, u = e2 - j * pr;
            return (const uint4*)((isv ? vb : kb) + (krow0 + (size_t)j * H) * DH) + u;
        };
        auto dst = [&](int e) -> uint4* {
            return e >= half ? (uint4*)vs + (e - half) : (uint4*)ks + e;
        };
        constexpr int SB = 4;
        uint4 v[SB];
#pragma unroll
        for (int k = 0; k < SB; ++k) {
            const int e = tid + k * kCombT;
            v[k] = e < 2 * half ? *src(e) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < SB; ++k) {
            const int e = tid + k * kCombT;
            if (e < 2 * half) *dst(e) = v[k];
        }
        for (int e = tid + SB * kCombT; e < 2 * half; e += kCombT) *dst(e) = *src(e);
    }

    // ---- prefix items of (b, h): a running state per row
    const WorkList w = make_worklist(A.kv_len, A.nb, H, A.kv_lim, A.resident);
    float M[RG], l[RG], a0[RG], a1[RG];
#pragma unroll
    for (int k = 0; k < RG; ++k) { M[k] = -INFINITY; l[k] = 0.f; a0[k] = 0.f; a1[k] = 0.f; }
    long long base = 0;
    for (int p = 0; p < w.np; ++p) {
        long long off = 0, cnt = 0;
        int nn = 0;
        for (int bb = 0; bb < A.nb; ++bb) {
            const int n = phase_items(w, prefix_tiles(A.kv_len, bb, A.kv_lim), p);
            if (bb < b) off += (long long)n * H;
            if (bb == b) nn = n;
            cnt += (long long)n * H;
        }
        const long long first = base + off + (long long)h * nn;
        constexpr int B = RG >= 4 ? 1 : 4 / RG;        // items whose loads are in flight together
        for (int j0 = wave; j0 < nn; j0 += kCombW * B) {
            float2 ml[B][RG];
            float v0[B][RG], v1[B][RG];
#pragma unroll
            for (int u = 0; u < B; ++u) {
                const int j = j0 + u * kCombW;
#pragma unroll
                for (int k = 0; k < RG; ++k) {
                    ml[u][k] = make_float2(-INFINITY, 0.f);
                    v0[u][k] = v1[u][k] = 0.f;
                    if (j < nn && k < nr) {
                        const size_t row = (size_t)(first + j) * nq + r0 + k;
                        ml[u][k] = *(const float2*)(A.part_ml + row * 2);
                        if (ok0) v0[u][k] = A.part_o[row * DH + d0];
                        if (ok1) v1[u][k] = A.part_o[row * DH + d1];
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < B; ++u) {
                if (j0 + u * kCombW >= nn) break;
#pragma unroll
                for (int k = 0; k < RG; ++k) {
                    if (ml[u][k].x > M[k]) {           // wave-uniform
                        const float s = __builtin_amdgcn_exp2f(M[k] - ml[u][k].x);
                        l[k] *= s; a0[k] *= s; a1[k] *= s;
                        M[k] = ml[u][k].x;
                    }
                    const float wgt = __builtin_amdgcn_exp2f(ml[u][k].x - M[k]);
                    l[k] = fmaf(wgt, ml[u][k].y, l[k]);
                    a0[k] = fmaf(wgt, v0[u][k], a0[k]);
                    a1[k] = fmaf(wgt, v1[u][k], a1[k]);
                }
            }
        }
        base += cnt;
    }
#pragma unroll
    for (int k = 0; k < RG; ++k) {
        float* so = st_o + ((size_t)wave * RG + k) * DH;
        if (ok0) so[d0] = a0[k];
        if (ok1) so[d1] = a1[k];
        if (lane == 0) {
            st_ml[(wave * RG + k) * 2] = M[k];
            st_ml[(wave * RG + k) * 2 + 1] = l[k];
        }
    }
    __syncthreads();                                   // block rows staged

    // ---- causal block part: row k of the group by wave k mod 4, keys 0..i of the block
    for (int k = wave; k < nr; k += kCombW) {
        const int i = i0 + k;
        const size_t qrow = ((size_t)b * nq + r0 + k) * H + h;
        const float q0 = ok0 ? Act<ACT>::load(q, qrow * DH + d0) : 0.f;
        const float q1 = ok1 ? Act<ACT>::load(q, qrow * DH + d1) : 0.f;
        float my_s = -INFINITY;                        // lane j keeps score j
        for (int j = 0; j <= i; ++j) {
            float part = 0.f;
            if (ok0) part = fmaf(q0, Act<ACT>::load(ks, (size_t)j * DH + d0), part);
            if (ok1) part = fmaf(q1, Act<ACT>::load(ks, (size_t)j * DH + d1), part);
            for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);   // same bits on every lane
            if (lane == j) my_s = part * A.scale_log2;
        }
        float mb = my_s;
        for (int off = 32; off >= 1; off >>= 1) mb = fmaxf(mb, __shfl_xor(mb, off));
        const float pj = lane <= i ? __builtin_amdgcn_exp2f(my_s - mb) : 0.f;
        float lb = pj;
        for (int off = 32; off >= 1; off >>= 1) lb += __shfl_xor(lb, off);
        float b0 = 0.f, b1 = 0.f;
        for (int j = 0; j <= i; ++j) {
            const float pw = __shfl(pj, j);
            if (ok0) b0 = fmaf(pw, Act<ACT>::load(vs, (size_t)j * DH + d0), b0);
            if (ok1) b1 = fmaf(pw, Act<ACT>::load(vs, (size_t)j * DH + d1), b1);
        }
        float* so = st_o + ((size_t)kCombW * RG + k) * DH;
        if (ok0) so[d0] = b0;
        if (ok1) so[d1] = b1;
        if (lane == 0) {
            st_ml[(kCombW * RG + k) * 2] = mb;
            st_ml[(kCombW * RG + k) * 2 + 1] = lb;
        }
    }
    __syncthreads();

    // ---- fixed-order merge of the four wave states and the block part, per row
    for (int e = tid; e < nr * DH; e += kCombT) {
        const int k = e / DH, dd = e - k * DH;
        float Mt = st_ml[k * 2];
#pragma unroll
        for (int s = 1; s <= kCombW; ++s) Mt = fmaxf(Mt, st_ml[(s * RG + k) * 2]);
        float lt = 0.f, ot = 0.f;
#pragma unroll
        for (int s = 0; s <= kCombW; ++s) {
            const float wgt = __builtin_amdgcn_exp2f(st_ml[(s * RG + k) * 2] - Mt);
            lt = fmaf(wgt, st_ml[(s * RG + k) * 2 + 1], lt);
            ot = fmaf(wgt, st_o[((size_t)s * RG + k) * DH + dd], ot);
        }
        Act<ACT>::store((T*)A.o, (((size_t)b * nq + r0 + k) * H + h) * DH + dd, ot / lt);
    }
}

template <int ACT, int RG>
__global__ __launch_bounds__(kCombT) void k_verify_finish(FinishArgs A)
{
    extern __shared__ float lds[];
    typedef typename Act<ACT>::T T;
    const int id = blockIdx.x;
    if (id < A.n_conv) {
        const int groups = (A.d + kCG - 1) / kCG;
        conv_iir_block<ACT>(A.w_short, A.w_outer, A.lam, A.beta, A.cc, (const T*)A.short_win, A.outer_win, A.iir,
                            (const T*)A.x, A.f_out, A.s_out, (T*)A.y_out, A.d, A.Ts, A.To, A.N, A.nc, A.P,
                            id % groups, id / groups, lds);
        return;
    }
    const int j = id - A.n_conv;            // (rg, c, h, b), row group fastest
    const int rg = j % A.rg_count;
    const int t = j / A.rg_count;
    const int c = t % A.nc, h = (t / A.nc) % A.H, b = t / (A.nc * A.H);
    combine_job<ACT, RG>(A, c, rg, h, b, lds);
}

// rows per combine workgroup: the largest power of two (<= 16, <= P rounded up) that still
// leaves at least eight combine workgroups per CU
int combine_rows(int nb, int nc, int H, int P, int num_cus) {
    const long long blocks = (long long)nb * nc * H;
    int rg = 1;
    while (rg < 16 && rg < P && blocks * ((P + 2 * rg - 1) / (2 * rg)) >= 8LL * num_cus) rg *= 2;
    return rg;
}

template <int ACT>
static hipError_t launch_finish_t(const FinishArgs& F, int rg, int blocks, size_t lds, hipStream_t st) {
    const void* fn = nullptr;
    switch (rg) {
        case 1: fn = (const void*)k_verify_finish<ACT, 1>; break;
        case 2: fn = (const void*)k_verify_finish<ACT, 2>; break;
        case 4: fn = (const void*)k_verify_finish<ACT, 4>; break;
        case 8: fn = (const void*)k_verify_finish<ACT, 8>; break;
        default: fn = (const void*)k_verify_finish<ACT, 16>; break;
    }
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    switch (rg) {
        case 1: hipLaunchKernelGGL((k_verify_finish<ACT, 1>), dim3(blocks), dim3(kCombT), lds, st, F); break;
        case 2: hipLaunchKernelGGL((k_verify_finish<ACT, 2>), dim3(blocks), dim3(kCombT), lds, st, F); break;
        case 4: hipLaunchKernelGGL((k_verify_finish<ACT, 4>), dim3(blocks), dim3(kCombT), lds, st, F); break;
        case 8: hipLaunchKernelGGL((k_verify_finish<ACT, 8>), dim3(blocks), dim3(kCombT), lds, st, F); break;
        default: hipLaunchKernelGGL((k_verify_finish<ACT, 16>), dim3(blocks), dim3(kCombT), lds, st, F); break;
    }
    return hipGetLastError();
}

hipError_t launch_finish(const FinishArgs& F, int act_dtype, int rg, int blocks, size_t lds, hipStream_t st) {
    return act_dtype == HCI_BF16 ? launch_finish_t<HCI_BF16>(F, rg, blocks, lds, st)
                                 : launch_finish_t<HCI_F32>(F, rg, blocks, lds, st);
}

}  // namespace hci
