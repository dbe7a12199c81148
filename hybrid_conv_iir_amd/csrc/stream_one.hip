// Prefix streaming: one persistent workgroup per CU takes prefix items from
// the job queue; its four waves split an item into contiguous runs of 32-key
// tiles, each streamed with non-temporal 16-byte loads and the next two tiles
// in flight, and merge their softmax states in LDS before one partial per
// query is written.  Every wave applies all NQT 16-query tiles of the sequence
// (nc * P <= 16 NQT queries, NQT <= 4) to each KV tile it streams, so a KV
// tile is read from HBM once, into the registers of one wave, and no LDS
// staging or per-tile barrier sits in the streaming loop.
#include "prefix_tile.h"

namespace hci {

template <int DH>
__host__ __device__ constexpr size_t prefix_merge_floats() {
    // per merged wave: O^T accumulators (16 queries x DH), running max, normaliser
    return (size_t)16 * DH + 2 * 16;
}

// One prefix item: tiles [t0, t1) of head h of sequence b, all nq <= 16 NQT
// queries, written to partial `slot`.  The four waves take contiguous runs of
// the item; each streams its run with the next two tiles' loads in flight
// while the current tile is consumed.  The waves' states merge in LDS in a
// fixed order (wave 0, 1, 2, 3).  Every wave returns (no early exit): the
// caller's barriers stay matched.
template <int DH, int NQT>
__device__ __forceinline__ void prefix_item(const StreamArgs& A, int b, int h, int t0, int t1, long long slot,
                                            float* merge, unsigned& next)
{
    constexpr int J = DH / 32, DT = DH / 16, KV4 = 4 * DH;
    constexpr size_t MF = prefix_merge_floats<DH>();
    const int L = prefix_len(A.kv_len, b, A.kv_lim);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
    const int per = (t1 - t0 + kPrefixWaves - 1) / kPrefixWaves;
    const int w0 = min(t0 + wave * per, t1), w1 = min(w0 + per, t1);

    PrefixAcc<DH, NQT> a;
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
        const int qi = 16 * nt + n;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (qi < A.nq) v = *(const uint4*)(A.q + (((size_t)b * A.nq + qi) * A.H + h) * DH + 32 * j + 8 * g);
            a.q[nt][j] = as_bf16x8(v);
        }
        a.m[nt] = -INFINITY;
        a.l[nt] = 0.f;
#pragma unroll
        for (int t = 0; t < DT; ++t) a.o[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const size_t slab = ((size_t)b * A.H + h) * (size_t)(A.kv_cap / kTile) * KV4;
    const uint4* kp = (const uint4*)A.kc + slab;
    const uint4* vp = (const uint4*)A.vc + slab;
    if (w0 < w1 && NQT >= 3) {
        // two register buffers, one tile in flight: with three or four query tiles a KV tile
        // takes several times longer to consume, and the registers go to the accumulators
        KvTile<DH> ta, tb;
        int T = w0;
        load_tile<DH>(ta, kp, vp, T, lane);
        for (; T + 2 < w1; T += 2) {
            load_tile<DH>(tb, kp, vp, T + 1, lane);
            consume_tile<DH, NQT>(a, ta, T, L, g, A.scale_log2);
            load_tile<DH>(ta, kp, vp, T + 2, lane);
            consume_tile<DH, NQT>(a, tb, T + 1, L, g, A.scale_log2);
        }
        // 1 or 2 tiles left: T (in ta) is loaded
        if (T + 1 < w1) load_tile<DH>(tb, kp, vp, T + 1, lane);
        consume_tile<DH, NQT>(a, ta, T, L, g, A.scale_log2);
        if (T + 1 < w1) consume_tile<DH, NQT>(a, tb, T + 1, L, g, A.scale_log2);
    } else if (w0 < w1) {
        // three register buffers, two tiles in flight ahead of the one consumed; the loads
        // inside the loop are unconditional, so the compiler's waits are exact
        KvTile<DH> ta, tb, tc;
        int T = w0;
        load_tile<DH>(ta, kp, vp, T, lane);
        if (T + 1 < w1) load_tile<DH>(tb, kp, vp, T + 1, lane);
        for (; T + 4 < w1; T += 3) {
            load_tile<DH>(tc, kp, vp, T + 2, lane);
            consume_tile<DH, NQT>(a, ta, T, L, g, A.scale_log2);
            load_tile<DH>(ta, kp, vp, T + 3, lane);
            consume_tile<DH, NQT>(a, tb, T + 1, L, g, A.scale_log2);
            load_tile<DH>(tb, kp, vp, T + 4, lane);
            consume_tile<DH, NQT>(a, tc, T + 2, L, g, A.scale_log2);
        }
        // 1..4 tiles left: T (in ta) and T+1 (in tb) are already loaded where they exist
        const int left = w1 - T;
        if (left >= 3) load_tile<DH>(tc, kp, vp, T + 2, lane);
        consume_tile<DH, NQT>(a, ta, T, L, g, A.scale_log2);
        if (left >= 4) load_tile<DH>(ta, kp, vp, T + 3, lane);
        if (left >= 2) consume_tile<DH, NQT>(a, tb, T + 1, L, g, A.scale_log2);
        if (left >= 3) consume_tile<DH, NQT>(a, tc, T + 2, L, g, A.scale_log2);
        if (left >= 4) consume_tile<DH, NQT>(a, ta, T + 3, L, g, A.scale_log2);
    }

    // the next ticket is taken once this item's loads are done: taken earlier, it would
    // hold the next item back for as long as this one still runs
    if (threadIdx.x == 0) next = atomicAdd(A.ticket, 1u);

    // every wave's state of every query tile goes to LDS; then wave w merges query tiles
    // w, w + 4, ... in the fixed order wave 0, 1, 2, 3.  An empty run contributes m = -inf,
    // l = 0, O = 0.
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
        float* mw = merge + ((size_t)wave * NQT + nt) * MF;
#pragma unroll
        for (int t = 0; t < DT; ++t)
            *(float4*)(mw + ((size_t)t * 64 + lane) * 4) =
                make_float4(a.o[t][nt][0], a.o[t][nt][1], a.o[t][nt][2], a.o[t][nt][3]);
        if (g == 0) {
            mw[16 * DH + n] = a.m[nt];
            mw[16 * DH + 16 + n] = a.l[nt];
        }
    }
    __syncthreads();
    const size_t pbase = (size_t)slot * A.nq;
    for (int nt = wave; nt < NQT; nt += kPrefixWaves) {
        const int qi = 16 * nt + n;
        auto st = [&](int w) { return merge + ((size_t)w * NQT + nt) * MF; };
        float mv[kPrefixWaves];
#pragma unroll
        for (int w = 0; w < kPrefixWaves; ++w) mv[w] = st(w)[16 * DH + n];
        float M = mv[0];
#pragma unroll
        for (int w = 1; w < kPrefixWaves; ++w) M = fmaxf(M, mv[w]);
        float sc[kPrefixWaves];
        sc[0] = __builtin_amdgcn_exp2f(mv[0] - M);
        float l = sc[0] * st(0)[16 * DH + 16 + n];
#pragma unroll
        for (int w = 1; w < kPrefixWaves; ++w) {
            sc[w] = __builtin_amdgcn_exp2f(mv[w] - M);
            l = fmaf(sc[w], st(w)[16 * DH + 16 + n], l);
        }
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            const float4 o0 = *(const float4*)(st(0) + ((size_t)t * 64 + lane) * 4);
            f32x4 acc = f32x4{o0.x, o0.y, o0.z, o0.w} * sc[0];
#pragma unroll
            for (int w = 1; w < kPrefixWaves; ++w) {
                const float4 o = *(const float4*)(st(w) + ((size_t)t * 64 + lane) * 4);
                acc[0] = fmaf(sc[w], o.x, acc[0]);
                acc[1] = fmaf(sc[w], o.y, acc[1]);
                acc[2] = fmaf(sc[w], o.z, acc[2]);
                acc[3] = fmaf(sc[w], o.w, acc[3]);
            }
            if (qi < A.nq) *(float4*)(A.part_o + (pbase + qi) * DH + 16 * t + 4 * g) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
        if (qi < A.nq && g == 0) *(float2*)(A.part_ml + (pbase + qi) * 2) = make_float2(M, l);
    }
}

// Persistent workgroup: prefix items from the queue.
template <int DH, int NQT>
__global__ __launch_bounds__(kRoleT, kStreamSlots) void k_verify_stream(StreamArgs A)
{
    __shared__ float merge[kPrefixWaves * NQT * prefix_merge_floats<DH>()];
    __shared__ unsigned s_ticket;
    const WorkList w = make_worklist(A.kv_len, A.nb, A.H, A.kv_lim, A.resident);
    const long long total = work_count(A.kv_len, w);
    if (threadIdx.x == 0) s_ticket = atomicAdd(A.ticket, 1u);
    __syncthreads();
    for (;;) {
        const long long t = s_ticket;
        __syncthreads();                               // every wave has read the ticket
        if (t >= total) break;
        unsigned next = 0xffffffffu;                   // past the end unless the item takes a ticket
        int b = 0, h = 0, t0 = 0, t1 = 0;
        if (work_item(A.kv_len, w, t, b, h, t0, t1)) prefix_item<DH, NQT>(A, b, h, t0, t1, t, merge, next);
        if (threadIdx.x == 0) s_ticket = next;
        __syncthreads();
    }
}

template <int DH>
static void launch_dh(const StreamArgs& A, int nqt, int blocks, hipStream_t st) {
    switch (nqt) {
        case 1: hipLaunchKernelGGL((k_verify_stream<DH, 1>), dim3(blocks), dim3(kRoleT), 0, st, A); break;
        case 2: hipLaunchKernelGGL((k_verify_stream<DH, 2>), dim3(blocks), dim3(kRoleT), 0, st, A); break;
        case 3: hipLaunchKernelGGL((k_verify_stream<DH, 3>), dim3(blocks), dim3(kRoleT), 0, st, A); break;
        default: hipLaunchKernelGGL((k_verify_stream<DH, 4>), dim3(blocks), dim3(kRoleT), 0, st, A); break;
    }
}

hipError_t launch_stream_one(const StreamArgs& A, int head_dim, int nqt, int blocks, hipStream_t st) {
    if (nqt < 1 || nqt > 4) return hipErrorInvalidValue;
    if (head_dim == 128) launch_dh<128>(A, nqt, blocks, st);
    else launch_dh<64>(A, nqt, blocks, st);
    return hipGetLastError();
}

}  // namespace hci
