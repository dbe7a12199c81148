// Prefix streaming: one persistent workgroup per CU runs prefix item
// blockIdx.x and then takes items from the job queue; its four waves share
// an item's 32-key tiles round-robin
// (wave w takes tiles t0 + w, t0 + w + 4, ..., so at any moment the
// workgroup reads four adjacent tiles, a contiguous 32 KB of keys and of
// values), each streamed with non-temporal 16-byte loads and the next two
// tiles in flight, and merge their softmax states in LDS before one partial
// per query is written.  Every wave applies all NQT 16-query tiles of the sequence
// (nc * P <= 16 NQT queries, NQT <= 4) to each KV tile it streams, so a KV
// tile is read from HBM once, by one wave, and no barrier sits in the
// streaming loop.  With one or two query tiles the tiles in flight sit in
// registers (three buffers); with three or four the query and accumulator
// registers leave no room for them, and each wave streams through a private
// two-slot LDS ring filled by direct global->LDS loads instead: it copies
// tile T from its slot into registers, refills the slot with tile T+2 and
// computes tile T, so two tiles stay in flight.
#include "prefix_tile.h"

namespace hci {

template <int DH>
__host__ __device__ constexpr size_t prefix_merge_floats() {
    // per merged wave: O^T accumulators (16 queries x DH), running max, normaliser
    return (size_t)16 * DH + 2 * 16;
}

// LDS pool of the kernel, in uint4: the merge states of every wave and query tile, which
// with three or four query tiles share the space of the waves' two-slot tile rings
template <int DH, int NQT>
__host__ __device__ constexpr size_t stream_pool_uint4() {
    const size_t merge = (kPrefixWaves * NQT * prefix_merge_floats<DH>() + 3) / 4;
    const size_t ring = NQT >= 3 ? (size_t)kPrefixWaves * 2 * (8 * DH) : 0;
    return merge > ring ? merge : ring;
}

// One prefix item: tiles [t0, t1) of head h of sequence b, all nq <= 16 NQT
// queries, written to partial `slot`.  The four waves take the item's tiles
// round-robin (measured against contiguous runs: adjacent tiles at the same
// time read 0.2% faster on a 262144-token prefix and 1.4% with four query
// tiles); each streams its share with the next two tiles' loads in flight
// while the current tile is consumed.  The waves' states merge in LDS in a
// fixed order (wave 0, 1, 2, 3).  Every wave returns (no early exit): the
// caller's barriers stay matched.
template <int DH, int NQT>
__device__ __forceinline__ void prefix_item(const StreamArgs& A, int b, int h, int t0, int t1, long long slot,
                                            uint4* lds_pool, unsigned& next)
{
    float* merge = (float*)lds_pool;
    constexpr int J = DH / 32, DT = DH / 16, KV4 = 4 * DH;
    constexpr size_t MF = prefix_merge_floats<DH>();
    const int L = prefix_len(A.kv_len, b, A.kv_lim);
    // the wave index is uniform across the wave: said so, every run bound and the waits on
    // them stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
    // wave w takes the tiles TT(k) = t0 + w + 4k, k in [w0, w1) = [0, nk); the loops below run
    // over k
    const int nk = t1 - t0 > wave ? (t1 - t0 - wave + kPrefixWaves - 1) / kPrefixWaves : 0;
    const int w0 = 0, w1 = nk;
    auto TT = [&](int k) { return t0 + wave + kPrefixWaves * k; };

    PrefixAcc<DH, NQT> a;
    auto load_q = [&]() {
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) {
            const int qi = 16 * nt + n;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                uint4 v = make_uint4(0, 0, 0, 0);
                if (qi < A.nq) v = *(const uint4*)(A.q + (((size_t)b * A.nq + qi) * A.H + h) * DH + 32 * j + 8 * g);
                a.q[nt][j] = as_bf16x8(v);
            }
        }
    };
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
        a.m[nt] = -INFINITY;
        a.l[nt] = 0.f;
#pragma unroll
        for (int t = 0; t < DT; ++t) a.o[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (NQT < 3) load_q();

    const size_t slab = ((size_t)b * A.H + h) * (size_t)(A.kv_cap / kTile) * KV4;
    const uint4* kp = (const uint4*)A.kc + slab;
    const uint4* vp = (const uint4*)A.vc + slab;
    if constexpr (NQT >= 3) {
        // the wave's ring: two slots of one tile (K then V, as stored) in the LDS pool
        constexpr int PT = 2 * KV4 / 64;               // direct loads per lane per tile
        const uint4* ring = lds_pool + (size_t)wave * 2 * (2 * KV4);
        const uint32_t ring0 = lds_offset(ring);
        auto issue = [&](int slot, int T) {
            const uint32_t dst = ring0 + (uint32_t)slot * (uint32_t)(2 * KV4 * sizeof(uint4));
            const size_t base = (size_t)T * KV4 + lane;
#pragma unroll
            for (int i = 0; i < PT; ++i) {
                const uint4* src = i < PT / 2 ? kp + base + i * 64 : vp + base + (i - PT / 2) * 64;
                dma16_nt(src, dst + (uint32_t)(i * 64 * sizeof(uint4)));
            }
        };
        // the queries are requested first (any wait the compiler places around them comes
        // before a direct load is in flight), then the item's first two tiles, so the three
        // latencies overlap.  One wait for every load follows (a count that never falls short,
        // whichever query loads the wave skipped; the two tiles arrive together anyway): the
        // compiler then knows its own loads are complete and never waits for a direct load.
        load_q();
        compiler_fence();
        if (w0 < w1) issue(0, TT(w0));
        if (w0 + 1 < w1) issue(1, TT(w0 + 1));
        compiler_fence();
        HCI_WAIT_VM(0);
        compiler_fence();
        KvTile<DH> cur;
        int slot = 0;
        for (int T = w0; T < w1; ++T) {
            // this wave's loads of tile T are done once at most tile T+1's are outstanding
            if (T > w0) {
                if (T + 1 < w1) HCI_WAIT_VM(PT); else HCI_WAIT_VM(0);
            }
            compiler_fence();
            const uint4* src = ring + (size_t)slot * (2 * KV4);
#pragma unroll
            for (int i = 0; i < DH / 16; ++i) cur.k[i] = src[i * 64 + lane];
#pragma unroll
            for (int i = 0; i < DH / 16; ++i) cur.v[i] = src[KV4 + i * 64 + lane];
            compiler_fence();
            HCI_WAIT_LGKM0();                          // the slot is read: refill it
            compiler_fence();
            if (T + 2 < w1) issue(slot, TT(T + 2));
            consume_tile<DH, NQT>(a, cur, TT(T), L, g, A.scale_log2);
            slot ^= 1;
        }
        // every wave is done with its ring before the merge states overwrite the pool
        __syncthreads();
    } else if (w0 < w1) {
        // three register buffers, two tiles in flight ahead of the one consumed; the loads
        // inside the loop are unconditional, so the compiler's waits are exact
        KvTile<DH> ta, tb, tc;
        int T = w0;
        load_tile<DH>(ta, kp, vp, TT(T), lane);
        if (T + 1 < w1) load_tile<DH>(tb, kp, vp, TT(T + 1), lane);
        for (; T + 4 < w1; T += 3) {
            load_tile<DH>(tc, kp, vp, TT(T + 2), lane);
            consume_tile<DH, NQT>(a, ta, TT(T), L, g, A.scale_log2);
            load_tile<DH>(ta, kp, vp, TT(T + 3), lane);
            consume_tile<DH, NQT>(a, tb, TT(T + 1), L, g, A.scale_log2);
            load_tile<DH>(tb, kp, vp, TT(T + 4), lane);
            consume_tile<DH, NQT>(a, tc, TT(T + 2), L, g, A.scale_log2);
        }
        // 1..4 tiles left: T (in ta) and T+1 (in tb) are already loaded where they exist
        const int left = w1 - T;
        if (left >= 3) load_tile<DH>(tc, kp, vp, TT(T + 2), lane);
        consume_tile<DH, NQT>(a, ta, TT(T), L, g, A.scale_log2);
        if (left >= 4) load_tile<DH>(ta, kp, vp, TT(T + 3), lane);
        if (left >= 2) consume_tile<DH, NQT>(a, tb, TT(T + 1), L, g, A.scale_log2);
        if (left >= 3) consume_tile<DH, NQT>(a, tc, TT(T + 2), L, g, A.scale_log2);
        if (left >= 4) consume_tile<DH, NQT>(a, ta, TT(T + 3), L, g, A.scale_log2);
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

// Persistent workgroup: its own index is its first item (no queue round trip before the first
// loads; the set-up kernel starts the queue past the grid), then items from the queue.
template <int DH, int NQT>
__global__ __launch_bounds__(kRoleT, kStreamSlots) void k_verify_stream(StreamArgs A)
{
    __shared__ uint4 lds_pool[stream_pool_uint4<DH, NQT>()];
    __shared__ unsigned s_ticket;
    const WorkTable wt = read_worktable(A.ws, A.nb, A.H, A.kv_lim);
    if (threadIdx.x == 0) s_ticket = blockIdx.x;
    __syncthreads();
    for (;;) {
        const unsigned t = s_ticket;
        __syncthreads();                               // every wave has read the ticket
        if (t >= (unsigned)wt.total) break;
        unsigned next = 0xffffffffu;                   // past the end unless the item takes a ticket
        int b = 0, h = 0, t0 = 0, t1 = 0;
        if (table_item(A.kv_len, wt, (int)t, b, h, t0, t1))
            prefix_item<DH, NQT>(A, b, h, t0, t1, t, lds_pool, next);
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
