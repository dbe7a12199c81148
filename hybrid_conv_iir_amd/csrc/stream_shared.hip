// Prefix streaming for several 16-query tiles (the multi-candidate verify):
// every wave of a persistent workgroup owns one query tile and the four walk
// the same KV tiles, staged once per workgroup in LDS.
#include "prefix_tile.h"

namespace hci {

// With more than 16 queries per sequence (several candidates) every wave of a
// prefix workgroup owns one 16-query tile and all four walk the same KV
// tiles.  Each 32-key tile is read from HBM once per workgroup, straight into
// LDS by the direct global->LDS loads of gfx950: lane l's 16 bytes land at the
// wave's LDS base + 16*l, so a wave-wide load copies one contiguous kilobyte
// of the tiled cache and no registers are spent on staging.  Four LDS stages
// keep three tiles in flight while the fourth is consumed, and every wave
// takes its matrix-core operands from LDS in the order they were stored (no
// bank conflicts).  A wave waits for its own direct loads with an explicit
// vector-memory count (loads complete in issue order); the barrier that
// follows publishes the tile to the other waves and also marks the stage
// read last time as free, so it is refilled as soon as the operands of the
// current tile are in registers.  Nothing else is in flight while the stages
// fill: the next ticket is taken after an item's last tile.

constexpr int kStages = 4;            // LDS stages of the several-tile kernel (16 KB each at Dh = 128; two workgroups per CU)

typedef __attribute__((address_space(3))) void lds_void;

// Direct global->LDS load of 16 bytes per lane, non-temporal: lane l's bytes
// land at lds_base + 16*l (lds_base wave-uniform, in M0).  Written as inline
// assembly so that the compiler's own wait insertion, which cannot follow a
// multi-stage LDS pipeline across loop iterations and would drain every load
// in flight, leaves it alone; the waits are explicit (HCI_WAIT_VM).  M0 is
// saved and restored, and one wait state separates its write from the load.
__device__ __forceinline__ void dma16_nt(const uint4* src, const uint4* lds_dst) {
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds_dst);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved) : "v"(src), "s"(base) : "memory");
}

// s_waitcnt that leaves n vector-memory operations outstanding (vmcnt in bits
// 3:0 and 15:14; expcnt and lgkmcnt at their no-wait maxima)
#define HCI_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | (((n) >> 4) << 14))

__device__ __forceinline__ void lds_read_barrier() {
    // this wave's LDS reads have completed, then the workgroup barrier; the memory
    // clobber keeps the compiler from moving any load or store across it
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int DH>
__global__ __launch_bounds__(kRoleT) void k_attn_prefix_shared(StreamArgs A, int nqt)
{
    constexpr int KV4 = 4 * DH;                        // uint4 of K (then of V) per tile
    constexpr int TU = 2 * KV4;                        // uint4 per tile
    constexpr int PER = TU / kRoleT;                   // direct loads per thread per tile
    static_assert(TU % kRoleT == 0 && KV4 % 64 == 0, "a tile splits into wave-wide loads");
    __shared__ uint4 stage[kStages][TU];
    __shared__ unsigned s_ticket;
    static_assert(kStages >= 3 && kStages <= 8, "the waits cover up to six tiles in flight");
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
    const bool has_q = wave < nqt;
    const int qi = 16 * wave + n;
    const WorkList w = make_worklist(A.kv_len, A.nb, A.H, A.kv_lim, A.resident);
    const long long total = work_count(A.kv_len, w);
    if (tid == 0) s_ticket = atomicAdd(A.ticket, 1u);
    __syncthreads();
    for (;;) {
        const long long t = s_ticket;
        __syncthreads();                               // every wave has read the ticket
        if (t >= total) break;
        int b = 0, h = 0, t0 = 0, t1 = 0;
        if (work_item(A.kv_len, w, t, b, h, t0, t1)) {
            const int L = prefix_len(A.kv_len, b, A.kv_lim);
            PrefixAcc<DH, 1> a;
#pragma unroll
            for (int j = 0; j < DH / 32; ++j) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (has_q && qi < A.nq) v = *(const u32x4*)(A.q + (((size_t)b * A.nq + qi) * A.H + h) * DH + 32 * j + 8 * g);
                // the query loads complete here, before any direct load is issued: the compiler
                // then has no load of its own pending inside the pipeline below
                asm volatile("" : "+v"(v));
                a.q[0][j] = __builtin_bit_cast(bf16x8, v);
            }
            a.m[0] = -INFINITY;
            a.l[0] = 0.f;
#pragma unroll
            for (int tt = 0; tt < DH / 16; ++tt) a.o[tt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
            const size_t slab = ((size_t)b * A.H + h) * (size_t)(A.kv_cap / kTile) * KV4;
            const uint4* kp = (const uint4*)A.kc + slab;
            const uint4* vp = (const uint4*)A.vc + slab;

            auto issue = [&](uint4* dst, int T) {
                const size_t base = (size_t)T * KV4;
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    const int e = tid + kRoleT * i;    // wave-uniform K/V choice: KV4 is a multiple of 64
                    const uint4* src = e < KV4 ? kp + base + e : vp + base + (e - KV4);
                    dma16_nt(src, dst + (e & ~63));
                }
            };
            auto wait_later = [&](int later) {             // leave `later` tiles' loads in flight
                switch (later) {
                    case 0: HCI_WAIT_VM(0); break;
                    case 1: HCI_WAIT_VM(1 * PER); break;
                    case 2: HCI_WAIT_VM(2 * PER); break;
                    case 3: HCI_WAIT_VM(3 * PER); break;
                    case 4: HCI_WAIT_VM(4 * PER); break;
                    case 5: HCI_WAIT_VM(5 * PER); break;
                    default: HCI_WAIT_VM(6 * PER); break;
                }
            };
            auto step = [&](const uint4* cur, uint4* refill, int T) {
                // loads issued after tile T's: tiles T+1 .. T+kStages-2, where they exist
                wait_later(min(t1 - 1 - T, kStages - 2));
                lds_read_barrier();                    // tile T complete for every wave; tile T-1 read by all
                KvTile<DH> tl;
                if (has_q) {
#pragma unroll
                    for (int i = 0; i < DH / 16; ++i) tl.k[i] = cur[i * 64 + lane];
#pragma unroll
                    for (int i = 0; i < DH / 16; ++i) tl.v[i] = cur[KV4 + i * 64 + lane];
                }
                // refill after the operand reads: the compiler then has no direct load to order them against
                if (T + kStages - 1 < t1) issue(refill, T + kStages - 1);
                if (has_q) consume_tile<DH, 1>(a, tl, T, L, g, A.scale_log2);
            };
            for (int i = 0; i < kStages - 1; ++i)
                if (t0 + i < t1) issue(stage[i], t0 + i);
            int cur = 0;
            for (int T = t0; T < t1; ++T) {
                // the stage read one step earlier is free once this step's barrier has passed
                step(stage[cur], stage[cur == 0 ? kStages - 1 : cur - 1], T);
                cur = cur + 1 == kStages ? 0 : cur + 1;
            }
            // the last step waited for every direct load: no LDS write is pending here
            if (has_q && qi < A.nq) {
                const size_t pbase = (size_t)t * A.nq;
#pragma unroll
                for (int tt = 0; tt < DH / 16; ++tt)
                    *(float4*)(A.part_o + (pbase + qi) * DH + 16 * tt + 4 * g) =
                        make_float4(a.o[tt][0][0], a.o[tt][0][1], a.o[tt][0][2], a.o[tt][0][3]);
                if (g == 0) *(float2*)(A.part_ml + (pbase + qi) * 2) = make_float2(a.m[0], a.l[0]);
            }
        }
        if (tid == 0) s_ticket = atomicAdd(A.ticket, 1u);
        __syncthreads();                               // the stages are free and the ticket is published
    }
}

hipError_t launch_stream_shared(const StreamArgs& A, int head_dim, int nqt, int blocks, hipStream_t st) {
    if (head_dim == 128)
        hipLaunchKernelGGL(k_attn_prefix_shared<128>, dim3(blocks), dim3(kRoleT), 0, st, A, nqt);
    else
        hipLaunchKernelGGL(k_attn_prefix_shared<64>, dim3(blocks), dim3(kRoleT), 0, st, A, nqt);
    return hipGetLastError();
}

}  // namespace hci
