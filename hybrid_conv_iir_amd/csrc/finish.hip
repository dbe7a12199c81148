// The kernel that ends a verify: the conv/IIR scan and the merge of the
// prefix partials with the causal block part.
#include "conv_iir_body.h"
#include "tree.h"
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
//           each reduce a fixed subset of the prefix items of (b, h) (entry j
//           of the list of (b, h)'s items, phase by phase, goes to wave
//           j mod 4, up to 16 / RG entries' loads in flight at once) into a
//           running softmax state per row; then each row's causal block part (query i against the
//           block's own keys 0..i, fp32, from K/V rows staged in LDS) is
//           computed by one wave, and the five states of a row merge in a
//           fixed order:
//             M = max m_s,  o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// Lane l holds output dims l and l + 64.  RG (1..16 rows) is chosen by the
// host so that the grid has a few workgroups per CU.

// eight consecutive activations as floats from a 16-byte-aligned address (LDS or global)
template <int ACT>
__device__ __forceinline__ void load8(const typename Act<ACT>::T* p, float* v) {
    if constexpr (ACT == HCI_BF16) {
        const uint4 u = *(const uint4*)p;
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(w[e] << 16);
            v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    } else {
        const float4 x = *(const float4*)p, y = *(const float4*)(p + 4);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
    }
}

// fp32 all-reduce over the 16 lanes of a row of the wave by rotations (vector ALU, no LDS
// round trip); lane 0 of the row holds a fixed-order result
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));  // row_ror:8
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)));  // row_ror:4
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false)));  // row_ror:2
    return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false)));  // row_ror:1
}
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));
}

// orders one wave's LDS accesses across its lanes (a store by one lane before a load by
// another), with no workgroup barrier
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the same bits on all four) by two gfx950 lane swaps
__device__ __forceinline__ float sum_over_rows(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int ACT, int RG>
__device__ __forceinline__ void combine_job(const FinishArgs& A, int c, int rg, int h, int b, float* lds)
{
    typedef typename Act<ACT>::T T;
    const T* q = (const T*)A.q;
    const T* kb = (const T*)A.kb;
    const T* vb = (const T*)A.vb;
    const int DH = A.DH, nq = A.nq, H = A.H, P = A.P;
    // the wave index is uniform across the wave: said so, the item and row bookkeeping below
    // stays in scalar registers
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int d0 = lane, d1 = lane + 64;
    const bool ok0 = d0 < DH, ok1 = d1 < DH;
    const int i0 = rg * RG, nr = min(RG, P - i0);      // rows i0 .. i0 + nr - 1 of candidate c
    const int r0 = c * P + i0;                         // their query-row index within the sequence

    // LDS: block K rows, block V rows (row stride RS bytes, 16 bytes of padding so that the 16
    // keys a wave reads at once fall in distinct banks), the states, the block weights
    const int RS = combine_row_bytes(DH, (int)sizeof(T));
    char* ks = (char*)lds;
    char* vs = ks + (size_t)P * RS;
    float* st_o = lds + (size_t)2 * P * RS / 4;                    // [state][row][DH]
    float* st_ml = st_o + (size_t)(kCombW + 1) * RG * DH;           // [state][row][2]
    float* pwt = st_ml + (size_t)(kCombW + 1) * RG * 2 + 64 * wave; // [wave][64] block weights
    // token trees: ancestor masks [64] (8-byte aligned) and pointer-doubling jumps [64]
    // (an even float offset from the 16-byte aligned LDS base: 8-byte aligned; pointer arithmetic
    // on the LDS array, not on integers, so that the accesses stay LDS instructions)
    const size_t moff = ((size_t)(st_ml - lds) + (size_t)(kCombW + 1) * RG * 2 + 64 * kCombW + 1) & ~(size_t)1;
    uint64_t* tmask = (uint64_t*)(lds + moff);
    uint8_t* tjump = (uint8_t*)(tmask + 64);
    auto krow = [&](int j) { return (const T*)(ks + (size_t)j * RS); };
    auto vrow = [&](int j) { return (const T*)(vs + (size_t)j * RS); };

    // the candidate's block K and V rows 0 .. i0 + nr - 1 in 16-byte pieces (a row is Dh * act
    // bytes, a multiple of 16): the first pieces of every thread are requested here, before the
    // prefix items' loads, and land in LDS after the items are folded, so the two rounds of
    // loads overlap
    const int pr = DH * (int)sizeof(T) / 16;           // pieces per row
    const int half = (i0 + nr) * pr;                   // K pieces, then as many V pieces
    const size_t krow0 = ((size_t)b * nq + (size_t)c * P) * H + h;
    auto src = [&](int e) -> const uint4* {
        const bool isv = e >= half;
        const int e2 = isv ? e - half : e, j = e2 / pr, u = e2 - j * pr;
        return (const uint4*)((isv ? vb : kb) + (krow0 + (size_t)j * H) * DH) + u;
    };
    auto dst = [&](int e) -> uint4* {
        const bool isv = e >= half;
        const int e2 = isv ? e - half : e, j = e2 / pr, u = e2 - j * pr;
        return (uint4*)((isv ? vs : ks) + (size_t)j * RS) + u;
    };
    constexpr int SB = 4;
    uint4 sv[SB];
#pragma unroll
    for (int k = 0; k < SB; ++k) {
        const int e = tid + k * kCombT;
        sv[k] = e < 2 * half ? *src(e) : make_uint4(0, 0, 0, 0);
    }

    // ---- prefix items of (b, h): a running state per row.  The items of every phase form one
    // list (phase by phase, chunk order); wave w folds entries w, w + 4, ... in list order, the
    // loads of B entries in flight together, whatever phase they belong to.  Entry f of phase p
    // is item f + adj[p] (adj = the phase's first item of (b, h) minus the entries before it);
    // the table entries of (p, b) are read through the constant address space (scalar loads).
    const __attribute__((address_space(4))) int32_t* tab = (const __attribute__((address_space(4))) int32_t*)A.table;
    // adj[p] = adj[0] + sum of dadj[1..p]; an entry adds the steps of the phases it has passed
    // (a sum of selects, which the compiler keeps in registers)
    // (item indices stay below 2^30, so the bookkeeping is 32-bit)
    int adj0 = 0, dadj[kPhaseMax];
    int cum[kPhaseMax];                                // entries before phase p
    int total = 0;
    {
        int prev = 0;
#pragma unroll
        for (int p = 0; p < kPhaseMax; ++p) {
            const size_t e = ((size_t)p * A.nb + b) * 2;
            const int n = tab[e + 1];
            const int adj = tab[e] + h * n - total;
            if (p == 0) adj0 = adj;
            dadj[p] = adj - prev;
            prev = adj;
            cum[p] = total;
            total += n;
        }
    }
    auto item_of = [&](int f) -> long long {
        int a = adj0;
#pragma unroll
        for (int p = 1; p < kPhaseMax; ++p) a += f >= cum[p] ? dadj[p] : 0;
        return (long long)(f + a);
    };
    float M[RG], l[RG], a0[RG], a1[RG];
#pragma unroll
    for (int k = 0; k < RG; ++k) { M[k] = -INFINITY; l[k] = 0.f; a0[k] = 0.f; a1[k] = 0.f; }
    constexpr int B = RG >= 16 ? 1 : 16 / RG;          // entries whose loads are in flight together
    for (int f0 = wave; f0 < total; f0 += kCombW * B) {
        float2 ml[B][RG];
        float v0[B][RG], v1[B][RG];
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int f = f0 + u * kCombW;
            const long long it = item_of(f);
#pragma unroll
            for (int k = 0; k < RG; ++k) {
                ml[u][k] = make_float2(-INFINITY, 0.f);
                v0[u][k] = v1[u][k] = 0.f;
                if (f < total && k < nr) {
                    const size_t row = (size_t)it * nq + r0 + k;
                    ml[u][k] = *(const float2*)(A.part_ml + row * 2);
                    if (ok0) v0[u][k] = A.part_o[row * DH + d0];
                    if (ok1) v1[u][k] = A.part_o[row * DH + d1];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < B; ++u) {
            if (f0 + u * kCombW >= total) break;
#pragma unroll
            for (int k = 0; k < RG; ++k) {
                if (ml[u][k].x > M[k]) {               // wave-uniform
                    const float sc = __builtin_amdgcn_exp2f(M[k] - ml[u][k].x);
                    l[k] *= sc; a0[k] *= sc; a1[k] *= sc;
                    M[k] = ml[u][k].x;
                }
                const float wgt = __builtin_amdgcn_exp2f(ml[u][k].x - M[k]);
                l[k] = fmaf(wgt, ml[u][k].y, l[k]);
                a0[k] = fmaf(wgt, v0[u][k], a0[k]);
                a1[k] = fmaf(wgt, v1[u][k], a1[k]);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < SB; ++k) {
        const int e = tid + k * kCombT;
        if (e < 2 * half) *dst(e) = sv[k];
    }
    for (int e = tid + SB * kCombT; e < 2 * half; e += kCombT) *dst(e) = *src(e);
    const bool tree = A.parent != nullptr;
    if (tree) tree_masks(A.parent + (size_t)b * P, P, tmask, tjump);     // uniform branch; has a barrier
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

    // ---- causal block part: row k of the group by wave k mod 4, keys 0..i of the block.
    // Scores: lane (key jj, slice sl) takes the dot product over dims [sl DS, (sl + 1) DS) of a
    // 16-key block, the four slices are summed by lane swaps; max and normaliser over the keys
    // by row rotations; the weights go through LDS to the value product (lane = output dims).
    const int jj = lane & 15, sl = lane >> 4, DS = DH / 4;
    for (int k = wave; k < nr; k += kCombW) {
        const int i = i0 + k;
        // block keys query i sees: 0..i (a chain of candidate positions) or its ancestors and
        // itself (a token tree; every ancestor has a lower index)
        const uint64_t vis = tree ? tmask[i] : ~0ull;
        const T* qrow = q + (((size_t)b * nq + r0 + k) * H + h) * DH + sl * DS;
        // the query slice: every 16-byte piece requested first (from clamped, always valid
        // offsets; pieces past DS are not used), then converted, so the loads are in flight
        // together instead of one conversion waiting for each
        constexpr int QP = (kF32Dh / 4) * (int)sizeof(T) / 16;          // pieces of a full slice
        uint4 qr[QP];
#pragma unroll
        for (int pc = 0; pc < QP; ++pc)
            qr[pc] = *(const uint4*)(qrow + min(pc * 16 / (int)sizeof(T), DS - 16 / (int)sizeof(T)));
#pragma unroll
        for (int pc = 0; pc < QP; ++pc) asm volatile("" : "+v"(qr[pc].x), "+v"(qr[pc].y), "+v"(qr[pc].z), "+v"(qr[pc].w));
        float qv[kF32Dh / 4];
#pragma unroll
        for (int e0 = 0; e0 < kF32Dh / 4; e0 += 8) load8<ACT>((const T*)qr + e0, qv + e0);
        float mb = -INFINITY;
        for (int j0 = 0; j0 <= i; j0 += 16) {
            const int j = j0 + jj;
            const bool see = j <= i && ((vis >> (j & 63)) & 1ull);
            float part = 0.f;
            if (see) {
                const T* kr = krow(j) + sl * DS;
#pragma unroll
                for (int e0 = 0; e0 < kF32Dh / 4; e0 += 8) {
                    if (e0 < DS) {
                        float kv[8];
                        load8<ACT>(kr + e0, kv);
#pragma unroll
                        for (int e = 0; e < 8; ++e) part = fmaf(qv[e0 + e], kv[e], part);
                    }
                }
            }
            part = sum_over_rows(part);
            const float sj = see ? part * A.scale_log2 : -INFINITY;
            if (sl == 0) pwt[j] = sj;
            mb = fmaxf(mb, sj);
        }
        mb = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(row16_max(mb))));
        wave_lds_sync();                               // the scores are in pwt
        float lsum = 0.f;
        for (int j0 = 0; j0 <= i; j0 += 16) {
            const int j = j0 + jj;
            float pj = 0.f;
            if (j <= i) pj = __builtin_amdgcn_exp2f(pwt[j] - mb);      // 0 for keys it does not see
            lsum += pj;
            if (sl == 0 && j <= i) pwt[j] = pj;
        }
        const float lb = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(row16_sum(lsum))));
        wave_lds_sync();                               // the weights are in pwt
        float b0 = 0.f, b1 = 0.f;
        for (int j = 0; j <= i; ++j) {
            const float pw = pwt[j];
            if (ok0) b0 = fmaf(pw, Act<ACT>::load(vrow(j), d0), b0);
            if (ok1) b1 = fmaf(pw, Act<ACT>::load(vrow(j), d1), b1);
        }
        wave_lds_sync();                               // pwt is read before the next row reuses it
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
__global__ __launch_bounds__(kCombT, kFinishPerCu) void k_verify_finish(FinishArgs A)
{
    extern __shared__ float lds[];
    typedef typename Act<ACT>::T T;
    // the grid's first indices are dispatched first: the conv workgroups (the longer chain)
    // when the whole grid is resident at once, else the combine workgroups
    const int n_comb = (int)gridDim.x - A.n_conv;
    const int bid = blockIdx.x;
    const bool is_conv = A.comb_first ? bid >= n_comb : bid < A.n_conv;
    if (is_conv) {
        const int id = A.comb_first ? bid - n_comb : bid;
        const int groups = (A.d + kCG - 1) / kCG;
        if (A.parent) {
            const int cgi = id % groups, b = id / groups;
            const uint32_t bad = tree_conv_block<ACT>(A.w_short, A.w_outer, A.lam, A.beta, A.cc, (const T*)A.short_win,
                                                      A.outer_win, A.iir, (const T*)A.x, A.parent, A.f_out, A.s_out,
                                                      (T*)A.y_out, A.d, A.Ts, A.To, A.N, A.P, cgi, b, lds);
            if (bad && cgi == 0 && threadIdx.x == 0) report(A.status, b, bad);
            return;
        }
        conv_iir_block<ACT>(A.w_short, A.w_outer, A.lam, A.beta, A.cc, (const T*)A.short_win, A.outer_win, A.iir,
                            (const T*)A.x, A.f_out, A.s_out, (T*)A.y_out, A.d, A.Ts, A.To, A.N, A.nc, A.P,
                            id % groups, id / groups, lds);
        return;
    }
    const int j = A.comb_first ? bid : bid - A.n_conv;    // (rg, c, h, b), row group fastest
    const int rg = j % A.rg_count;
    const int t = j / A.rg_count;
    const int c = t % A.nc, h = (t / A.nc) % A.H, b = t / (A.nc * A.H);
    combine_job<ACT, RG>(A, c, rg, h, b, lds);
}

// rows per combine workgroup: the largest power of two (<= 16, <= P rounded up) that still
// leaves at least eight combine workgroups per CU; for a token tree at least four, since each
// workgroup stages the block rows up to its last row, most of the tree for its later rows (46-node
// tries of the 4 x 4 workload: finish 74 us with two rows, 66 with four, 83 with eight)
int combine_rows(int nb, int nc, int H, int P, int num_cus, bool tree) {
    const long long blocks = (long long)nb * nc * H;
    int rg = 1;
    while (rg < 16 && rg < P && blocks * ((P + 2 * rg - 1) / (2 * rg)) >= 8LL * num_cus) rg *= 2;
    if (tree && rg < 4) rg = P >= 3 ? 4 : (P >= 2 ? 2 : 1);
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
