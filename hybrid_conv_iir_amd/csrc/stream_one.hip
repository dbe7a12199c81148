// Prefix streaming for one 16-query tile (nc * P <= 16, the one-candidate
// verify): one persistent workgroup per CU takes prefix items from the job
// queue; its four waves split an item into contiguous runs of 32-key tiles,
// each streamed with non-temporal 16-byte loads and the next tile in flight,
// and merge their softmax states in LDS before one partial is written.
#include "prefix_tile.h"

namespace hci {

template <int DH>
__host__ __device__ constexpr size_t prefix_merge_floats() {
    // per merged wave: O^T accumulators (16 queries x DH), running max, normaliser
    return (size_t)16 * DH + 2 * 16;
}

// One prefix item of the one-tile kernel: tiles [t0, t1) of head h of sequence
// b, all nq <= 16 queries, written to partial `slot`.  The four waves take
// contiguous runs of the item; each streams its run with the next two tiles'
// loads in flight while the current tile is consumed.  The waves' states
// merge in LDS in a fixed order.  Every wave returns (no early exit): the
// caller's barriers stay matched.
template <int DH>
__device__ __forceinline__ void prefix_item(const StreamArgs& A, int b, int h, int t0, int t1, long long slot,
                                            float* merge, unsigned& next)
{
    constexpr int J = DH / 32, DT = DH / 16, KV4 = 4 * DH;
    constexpr size_t MF = prefix_merge_floats<DH>();
    const int L = prefix_len(A.kv_len, b, A.kv_lim);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
    const int per = (t1 - t0 + kPrefixWaves - 1) / kPrefixWaves;
    const int w0 = min(t0 + wave * per, t1), w1 = min(w0 + per, t1);

    PrefixAcc<DH, 1> a;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n < A.nq) v = *(const uint4*)(A.q + (((size_t)b * A.nq + n) * A.H + h) * DH + 32 * j + 8 * g);
        a.q[0][j] = as_bf16x8(v);
    }
    a.m[0] = -INFINITY;
    a.l[0] = 0.f;
#pragma unroll
    for (int t = 0; t < DT; ++t) a.o[t][0] = f32x4{0.f, 0.f, 0.f, 0.f};

    const size_t slab = ((size_t)b * A.H + h) * (size_t)(A.kv_cap / kTile) * KV4;
    const uint4* kp = (const uint4*)A.kc + slab;
    const uint4* vp = (const uint4*)A.vc + slab;
    if (w0 < w1) {
        // three register buffers, two tiles in flight ahead of the one consumed; the loads
        // inside the loop are unconditional, so the compiler's waits are exact
        KvTile<DH> ta, tb, tc;
        int T = w0;
        load_tile<DH>(ta, kp, vp, T, lane);
        if (T + 1 < w1) load_tile<DH>(tb, kp, vp, T + 1, lane);
        for (; T + 4 < w1; T += 3) {
            load_tile<DH>(tc, kp, vp, T + 2, lane);
            consume_tile<DH, 1>(a, ta, T, L, g, A.scale_log2);
            load_tile<DH>(ta, kp, vp, T + 3, lane);
            consume_tile<DH, 1>(a, tb, T + 1, L, g, A.scale_log2);
            load_tile<DH>(tb, kp, vp, T + 4, lane);
            consume_tile<DH, 1>(a, tc, T + 2, L, g, A.scale_log2);
        }
        // 1..4 tiles left: T (in ta) and T+1 (in tb) are already loaded where they exist
        const int left = w1 - T;
        if (left >= 3) load_tile<DH>(tc, kp, vp, T + 2, lane);
        consume_tile<DH, 1>(a, ta, T, L, g, A.scale_log2);
        if (left >= 4) load_tile<DH>(ta, kp, vp, T + 3, lane);
        if (left >= 2) consume_tile<DH, 1>(a, tb, T + 1, L, g, A.scale_log2);
        if (left >= 3) consume_tile<DH, 1>(a, tc, T + 2, L, g, A.scale_log2);
        if (left >= 4) consume_tile<DH, 1>(a, ta, T + 3, L, g, A.scale_log2);
    }

    // the next ticket is taken once this item's loads are done: taken earlier, it would
    // hold the next item back for as long as this one still runs
    if (threadIdx.x == 0) next = atomicAdd(A.ticket, 1u);

    // merge the four waves' states in LDS (fixed order: wave 0, 1, 2, 3); an empty run
    // contributes m = -inf, l = 0, O = 0
    if (wave > 0) {
        float* mw = merge + (size_t)(wave - 1) * MF;
#pragma unroll
        for (int t = 0; t < DT; ++t)
            *(float4*)(mw + ((size_t)t * 64 + lane) * 4) = make_float4(a.o[t][0][0], a.o[t][0][1], a.o[t][0][2], a.o[t][0][3]);
        if (g == 0) {
            mw[16 * DH + n] = a.m[0];
            mw[16 * DH + 16 + n] = a.l[0];
        }
    }
    __syncthreads();
    if (wave == 0) {
        const size_t pbase = (size_t)slot * A.nq;
        float M = a.m[0];
#pragma unroll
        for (int w = 1; w < kPrefixWaves; ++w) M = fmaxf(M, merge[(w - 1) * MF + 16 * DH + n]);
        float sc[kPrefixWaves];
        sc[0] = __builtin_amdgcn_exp2f(a.m[0] - M);
        float l = sc[0] * a.l[0];
#pragma unroll
        for (int w = 1; w < kPrefixWaves; ++w) {
            const float* mw = merge + (size_t)(w - 1) * MF;
            sc[w] = __builtin_amdgcn_exp2f(mw[16 * DH + n] - M);
            l = fmaf(sc[w], mw[16 * DH + 16 + n], l);
        }
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            f32x4 acc = a.o[t][0] * sc[0];
#pragma unroll
            for (int w = 1; w < kPrefixWaves; ++w) {
                const float4 o = *(const float4*)(merge + (size_t)(w - 1) * MF + ((size_t)t * 64 + lane) * 4);
                acc[0] = fmaf(sc[w], o.x, acc[0]);
                acc[1] = fmaf(sc[w], o.y, acc[1]);
                acc[2] = fmaf(sc[w], o.z, acc[2]);
                acc[3] = fmaf(sc[w], o.w, acc[3]);
            }
            if (n < A.nq) *(float4*)(A.part_o + (pbase + n) * DH + 16 * t + 4 * g) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
        if (n < A.nq && g == 0) *(float2*)(A.part_ml + (pbase + n) * 2) = make_float2(M, l);
    }
}

// Persistent workgroup of the one-tile kernel: prefix items from the queue.
template <int DH>
__global__ __launch_bounds__(kRoleT, kSlotsFused) void k_verify_stream(StreamArgs A)
{
    __shared__ float merge[(kPrefixWaves - 1) * prefix_merge_floats<DH>()];
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
        if (work_item(A.kv_len, w, t, b, h, t0, t1)) prefix_item<DH>(A, b, h, t0, t1, t, merge, next);
        if (threadIdx.x == 0) s_ticket = next;
        __syncthreads();
    }
}

hipError_t launch_stream_one(const StreamArgs& A, int head_dim, int blocks, hipStream_t st) {
    if (head_dim == 128)
        hipLaunchKernelGGL(k_verify_stream<128>, dim3(blocks), dim3(kRoleT), 0, st, A);
    else
        hipLaunchKernelGGL(k_verify_stream<64>, dim3(blocks), dim3(kRoleT), 0, st, A);
    return hipGetLastError();
}

}  // namespace hci
