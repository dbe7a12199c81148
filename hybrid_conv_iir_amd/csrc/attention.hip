// Attention half of the block forward, plus the fused streaming kernel.
//
// The block queries attend to the committed KV prefix and, causally, to the
// block's own keys.  EvSpark digest, Interpretation: the verify is one block
// forward from the committed state, so all nc*P queries of a sequence share
// a single read of its prefix; that read is the part of the verify that grows
// with context (ReaDy summary, section 5: token-wise KV traffic grows with the
// number of attended tokens).  The prefix is cut into work items (split-K);
// each item leaves a partial softmax state (running max in log2 units,
// normaliser, unnormalised output), and the combine kernel computes the
// causal block part and merges everything in a fixed order.
//
// Work distribution.  The streaming kernels run one persistent workgroup per
// resident slot (two per CU); every workgroup takes jobs from a queue (an
// atomic ticket counter in the workspace) until it is empty.  The queue holds
// first the conv/IIR jobs of the layer (conv_iir_body.h), then the prefix
// items in decreasing size: phase p covers the next half of what is left of
// every sequence's prefix in chunks of c0 / 2^p tiles, c0 being half of a
// slot's fair share.  Slots run at different speeds (the older of two
// workgroups on a CU issues first, and CUs differ), so a static split ends
// ragged; with the queue the fast slots take more items and the small last
// items let every slot finish within a few microseconds of the others.  An
// item always writes the same partial whichever slot runs it, so results do
// not depend on scheduling.
//
// bf16 layers:
//   k_verify_stream       one 16-query tile (nc*P <= 16): four waves split an
//                         item into contiguous runs of 32-key tiles, streamed
//                         with non-temporal 16-byte loads (a contiguous
//                         kilobyte per wave-wide load, thanks to the tiled
//                         cache layout), the next tile prefetched into
//                         registers; S^T = K Q^T and O^T += V^T P^T on
//                         v_mfma_f32_16x16x32_bf16 with the keys in M; online
//                         softmax in fp32 registers; the four waves merge in
//                         LDS before one partial is written.
//   k_attn_prefix_shared  several query tiles: every wave owns one tile and the
//                         four walk the same KV tiles, staged once per
//                         workgroup in LDS by direct global->LDS loads.
// fp32 layers (small shapes) use a vector-ALU prefix kernel with one item per
// workgroup.
#include "conv_iir_body.h"

#include <math.h>

namespace hci {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRoleT = 256;            // threads per workgroup of every streaming kernel
// resident streaming workgroups per CU.  The one-tile kernel keeps one, so that no two
// workgroups on a CU compete for issue (the older one would run up to twice as fast and
// finish its items late); its four waves keep enough loads in flight.  The several-tile
// kernel needs two to overlap one workgroup's matrix-core and softmax work with the
// other's barrier waits.
constexpr int kSlotsFused = 1;
constexpr int kSlotsShared = 2;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 ones_bf16x8() {
    return as_bf16x8(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));   // eight bf16 1.0
}

constexpr int kPrefixWaves = 4;      // waves per streaming workgroup

// Committed length of sequence b as the attention reads it: kv_len clamped to
// [0, lim], lim = min(kv_cap, max_kv_len), so that a length above the host's
// bound can never yield more work than the host planned for.
__device__ __forceinline__ int prefix_len(const int32_t* kv_len, int b, int lim) {
    const int L = kv_len[b];
    return L < 0 ? 0 : (L > lim ? lim : L);
}

__device__ __forceinline__ int prefix_tiles(const int32_t* kv_len, int b, int lim) {
    return (prefix_len(kv_len, b, lim) + kTile - 1) / kTile;
}

// ------------------------------------------------------------- work list
//
// Derived on the device from kv_len, identically by the streaming kernels
// and the combine.  With W = H * sum_b tiles_b and R resident slots,
// c0 = max(kChunkMin, ceil(W / 2R)) and np = the number of phases whose chunk
// c0 >> p stays >= kChunkMin (at most kPhaseMax).  Phase p of a prefix of T
// tiles covers [T - (T >> p), T - (T >> (p+1))) (the last phase runs to T)
// in chunks of c0 >> p tiles.  Items are numbered phase-major, then by
// sequence, head and chunk:
//   item = base_p + H * sum_{b' < b} n(p, b') + h * n(p, b) + j,
// n(p, b) = ceil(phase length / chunk).  Item i writes partial i.  Every
// phase holds at most 2R + 2 nb H items (the last one 4R + nb H), which is
// the bound the host sizes the workspace with.

constexpr int kChunkMin = 32;        // smallest item (tiles): eight per wave
constexpr int kPhaseMax = 8;

struct WorkList {
    int nb, H, lim, c0, np;
};

__host__ __device__ inline long long worklist_c0(long long total_tiles, int resident) {
    const long long half = 2LL * (resident > 0 ? resident : 1);
    long long c0 = (total_tiles + half - 1) / half;
    if (c0 < kChunkMin) c0 = kChunkMin;
    if (c0 > (1LL << 28)) c0 = 1LL << 28;
    return c0;
}

__host__ __device__ inline int worklist_np(long long c0) {
    int np = 1;
    while (np < kPhaseMax && (c0 >> np) >= kChunkMin) ++np;
    return np;
}

__device__ __forceinline__ WorkList make_worklist(const int32_t* kv_len, int nb, int H, int lim, int resident) {
    long long tot = 0;
    for (int b = 0; b < nb; ++b) tot += prefix_tiles(kv_len, b, lim);
    const long long c0 = worklist_c0(tot * H, resident);
    return WorkList{nb, H, lim, (int)c0, worklist_np(c0)};
}

__device__ __forceinline__ int phase_chunk(const WorkList& w, int p) { return w.c0 >> p; }

__device__ __forceinline__ void phase_range(const WorkList& w, int T, int p, int& s, int& e) {
    s = T - (T >> p);
    e = p + 1 < w.np ? T - (T >> (p + 1)) : T;
}

__device__ __forceinline__ int phase_items(const WorkList& w, int T, int p) {
    int s, e;
    phase_range(w, T, p, s, e);
    const int c = phase_chunk(w, p);
    return (e - s + c - 1) / c;
}

__device__ __forceinline__ long long work_count(const int32_t* kv_len, const WorkList& w) {
    long long n = 0;
    for (int p = 0; p < w.np; ++p)
        for (int b = 0; b < w.nb; ++b) n += (long long)phase_items(w, prefix_tiles(kv_len, b, w.lim), p) * w.H;
    return n;
}

// Locate item `item`: sequence b, head h, tiles [t0, t1); false past the last item.
__device__ __forceinline__ bool work_item(const int32_t* kv_len, const WorkList& w, long long item,
                                          int& b, int& h, int& t0, int& t1) {
    for (int p = 0; p < w.np; ++p) {
        for (int bb = 0; bb < w.nb; ++bb) {
            const int T = prefix_tiles(kv_len, bb, w.lim);
            const int n = phase_items(w, T, p);
            const long long cnt = (long long)n * w.H;
            if (item < cnt) {
                b = bb;
                h = (int)(item / n);
                const int j = (int)(item - (long long)h * n);
                int s, e;
                phase_range(w, T, p, s, e);
                t0 = s + j * phase_chunk(w, p);
                t1 = min(t0 + phase_chunk(w, p), e);
                return true;
            }
            item -= cnt;
        }
    }
    return false;
}

template <int DH, int NQT>
struct PrefixAcc {
    bf16x8 q[NQT][DH / 32];
    f32x4 o[DH / 16][NQT];
    float m[NQT], l[NQT];
};

template <int DH>
struct KvTile {
    uint4 k[2 * (DH / 32)];   // two 16-key halves x DH/32 k-steps
    uint4 v[DH / 16];         // DH/16 value-product tiles
};

template <int DH>
__device__ __forceinline__ void load_tile(KvTile<DH>& t, const uint4* kp, const uint4* vp, int T, int lane) {
    constexpr int KV4 = 4 * DH;
    const size_t base = (size_t)T * KV4;
#pragma unroll
    for (int i = 0; i < 2 * (DH / 32); ++i) t.k[i] = load_nt(kp + base + i * 64 + lane);
#pragma unroll
    for (int i = 0; i < DH / 16; ++i) t.v[i] = load_nt(vp + base + i * 64 + lane);
}

// One 32-key tile: S^T = K Q^T on the matrix cores, online softmax in fp32,
// O^T += V^T P^T on the matrix cores.  Keys >= L (the ragged end) are masked.
template <int DH, int NQT>
__device__ __forceinline__ void consume_tile(PrefixAcc<DH, NQT>& a, KvTile<DH>& t, int T, int L, int g,
                                             float scale_log2) {
    constexpr int J = DH / 32, DT = DH / 16;
    const int kbase = T * kTile;
    const bool tail = kbase + kTile > L;
    if (tail) {
        // zero value rows past the prefix so that 0 * (stale bits) cannot poison the sums
#pragma unroll
        for (int i = 0; i < DT; ++i) {
            uint32_t w[4] = {t.v[i].x, t.v[i].y, t.v[i].z, t.v[i].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = kbase + 16 * (e >> 2) + 4 * g + (e & 3);
                if (key >= L) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
            }
            t.v[i] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
        float s[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < J; ++j)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.k[u * J + j]), a.q[nt][j], acc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = acc[r] * scale_log2;
                if (tail && kbase + 16 * u + 4 * g + r >= L) v = -INFINITY;
                s[u][r] = v;
            }
        }
        float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(a.m[nt], mx);
        const float alpha = __builtin_amdgcn_exp2f(a.m[nt] - mnew);
        a.m[nt] = mnew;
        f32x2 pf[4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            pf[2 * u] = f32x2{__builtin_amdgcn_exp2f(s[u][0] - mnew), __builtin_amdgcn_exp2f(s[u][1] - mnew)};
            pf[2 * u + 1] = f32x2{__builtin_amdgcn_exp2f(s[u][2] - mnew), __builtin_amdgcn_exp2f(s[u][3] - mnew)};
        }
        const bf16x8 pb = __builtin_shufflevector(
            __builtin_shufflevector(__builtin_convertvector(pf[0], bf16x2), __builtin_convertvector(pf[1], bf16x2), 0, 1, 2, 3),
            __builtin_shufflevector(__builtin_convertvector(pf[2], bf16x2), __builtin_convertvector(pf[3], bf16x2), 0, 1, 2, 3),
            0, 1, 2, 3, 4, 5, 6, 7);                            // round to nearest even
        // the running max only grows now and then: skip the rescale when no lane of the wave needs it
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
            for (int i = 0; i < DT; ++i) a.o[i][nt] *= alpha;
            a.l[nt] *= alpha;
        }
#pragma unroll
        for (int i = 0; i < DT; ++i)
            a.o[i][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.v[i]), pb, a.o[i][nt], 0, 0, 0);
        // normaliser = the same product against a row of ones: it sums exactly the bf16
        // weights the value product used, and every lane of query n receives it
        const f32x4 lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_bf16x8(), pb, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        a.l[nt] += lsum[0];
    }
}


// ------------------------------------------------ fused kernel (one query tile)

template <int DH>
__host__ __device__ constexpr size_t prefix_merge_floats() {
    // per merged wave: O^T accumulators (16 queries x DH), running max, normaliser
    return (size_t)16 * DH + 2 * 16;
}

struct StreamArgs {
    const uint16_t *kc, *vc, *q; const int32_t* kv_len;
    float *part_o, *part_ml;
    unsigned* ticket;                  // the job queue's counter (zeroed before the launch)
    int H, kv_cap, kv_lim, nq, nb, resident;
    float scale_log2;
};

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

// ------------------------------------------- several query tiles per prefix
//
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

// ------------------------------------------------------------- f32 prefix
//
// fp32 layers (small shapes): 64 threads per work item, one item per
// workgroup (grid = the host's bound on the items; workgroups past the last
// item exit at once).  The tile is unpacked into LDS rows; thread tid scores
// query tid and accumulates output dims tid and tid+64 of every query, all
// in fp32 on the vector ALUs.  Limits: Dh <= 128, nq <= 64.

constexpr int kF32Dh = 128;
constexpr int kF32Nq = 64;

__global__ __launch_bounds__(64) void k_attn_prefix_f32(
    const float* __restrict__ kc, const float* __restrict__ vc,
    const int32_t* __restrict__ kv_len, const float* __restrict__ q,
    float* __restrict__ part_o, float* __restrict__ part_ml,
    int nb, int H, int DH, int kv_cap, int kv_lim, int nq, int resident, float scale_log2)
{
    __shared__ float ks[kTile][kF32Dh + 1];
    __shared__ float vs[kTile][kF32Dh + 1];
    __shared__ float ps[kF32Nq][kTile + 1];
    __shared__ float alpha_s[kF32Nq];

    const long long item = blockIdx.x;
    const WorkList w = make_worklist(kv_len, nb, H, kv_lim, resident);
    int b, h, t0, t1;
    if (!work_item(kv_len, w, item, b, h, t0, t1)) return;
    const int L = prefix_len(kv_len, b, kv_lim);
    const int tid = threadIdx.x;

    float qr[kF32Dh];
#pragma unroll
    for (int dd = 0; dd < kF32Dh; ++dd)
        qr[dd] = (tid < nq && dd < DH) ? q[(((size_t)b * nq + tid) * H + h) * DH + dd] : 0.f;
    float mrun = -INFINITY, lrun = 0.f;
    float oacc[kF32Nq][2];
#pragma unroll
    for (int qi = 0; qi < kF32Nq; ++qi) oacc[qi][0] = oacc[qi][1] = 0.f;

    const size_t slab = ((size_t)b * H + h) * (size_t)kv_cap * DH;
    for (int T = t0; T < t1; ++T) {
        __syncthreads();
        for (int e = tid; e < kTile * DH; e += 64) {
            const int wr = e / DH, dd = e % DH;
            const int key = T * kTile + wr;
            const bool ok = key < L;
            ks[wr][dd] = ok ? kc[slab + k_elem(key, dd, DH)] : 0.f;
            vs[wr][dd] = ok ? vc[slab + v_elem(key, dd, DH)] : 0.f;
        }
        __syncthreads();
        if (tid < nq) {
            float sc[kTile];
            float mx = -INFINITY;
#pragma unroll
            for (int wr = 0; wr < kTile; ++wr) {
                float acc = 0.f;
#pragma unroll
                for (int dd = 0; dd < kF32Dh; ++dd)
                    if (dd < DH) acc = fmaf(qr[dd], ks[wr][dd], acc);
                sc[wr] = (T * kTile + wr < L) ? acc * scale_log2 : -INFINITY;
                mx = fmaxf(mx, sc[wr]);
            }
            const float mnew = fmaxf(mrun, mx);
            const float alpha = exp2f(mrun - mnew);
            float psum = 0.f;
#pragma unroll
            for (int wr = 0; wr < kTile; ++wr) {
                const float p = exp2f(sc[wr] - mnew);
                ps[tid][wr] = p;
                psum += p;
            }
            lrun = fmaf(lrun, alpha, psum);
            mrun = mnew;
            alpha_s[tid] = alpha;
        }
        __syncthreads();
#pragma unroll
        for (int qi = 0; qi < kF32Nq; ++qi) {
            if (qi < nq) {
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int dd = tid + 64 * r;
                    if (dd < DH) {
                        float acc = oacc[qi][r] * alpha_s[qi];
                        for (int wr = 0; wr < kTile; ++wr) acc = fmaf(ps[qi][wr], vs[wr][dd], acc);
                        oacc[qi][r] = acc;
                    }
                }
            }
        }
    }
    const size_t pbase = (size_t)item * nq;
#pragma unroll
    for (int qi = 0; qi < kF32Nq; ++qi) {
        if (qi < nq) {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int dd = tid + 64 * r;
                if (dd < DH) part_o[(pbase + qi) * DH + dd] = oacc[qi][r];
            }
        }
    }
    if (tid < nq) {
        part_ml[(pbase + tid) * 2] = mrun;
        part_ml[(pbase + tid) * 2 + 1] = lrun;
    }
}

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

constexpr int kCombT = 256;
constexpr int kCombW = kCombT / 64;

struct FinishArgs {
    // conv / IIR
    const float *w_short, *w_outer, *lam, *beta, *cc;
    const void* short_win; const float* outer_win; const float* iir; const void* x;
    float* f_out; float* s_out; void* y_out;
    int d, Ts, To, N, nc, n_conv;
    // combine
    const int32_t* kv_len; const float *part_o, *part_ml;
    const void *q, *kb, *vb; void* o;
    int nb, H, DH, nq, P, kv_lim, resident, rg_count;
    float scale_log2;
};

// dynamic LDS floats of the combine role: the candidate's block K and V rows (raw
// activations), then per row and state (four waves + the block part) O [Dh] and (m, l)
__host__ __device__ inline size_t combine_lds_floats(int P, int DH, int act_bytes, int RG) {
    return ((size_t)2 * P * DH * act_bytes + 3) / 4 + (size_t)(kCombW + 1) * RG * (DH + 2);
}

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

    // stage the candidate's block K and V rows 0 .. i0 + nr - 1 (one round trip)
    const size_t krow0 = ((size_t)b * nq + (size_t)c * P) * H + h;
    for (int e = tid; e < (i0 + nr) * DH; e += kCombT) {
        const int j = e / DH, dd = e - j * DH;
        const size_t src = (krow0 + (size_t)j * H) * DH + dd;
        ks[e] = kb[src];
        vs[e] = vb[src];
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

__global__ void k_ticket_reset(unsigned* ticket) {
    if (threadIdx.x == 0) ticket[0] = 0u;
}

// -------------------------------------------------------------------- host

// Workspace: the queue's ticket counter (256 bytes), then the partials
// part_o [items][nq][Dh] and part_ml [items][nq][2].
AttnPlan plan_attention(const hci_layer* L, int nb, int nc, int gamma, int max_kv_len, int num_cus)
{
    AttnPlan p{};
    const int P = gamma + 1;
    p.nq = nc * P;
    p.resident = (num_cus > 0 ? num_cus : 1) * (p.nq > 16 ? kSlotsShared : kSlotsFused);
    p.kv_lim = max_kv_len;    // callers check max_kv_len + P <= kv_cap before any launch
    const long long tiles = (max_kv_len + kTile - 1) / kTile;
    const long long nbh = (long long)nb * L->heads;
    const int np = worklist_np(worklist_c0(tiles * nbh, p.resident));
    // every phase holds at most 2R + 2 nb H items, the last at most 4R + nb H
    const long long cap = tiles > 0 ? (long long)np * (4LL * p.resident + 2 * nbh) : 0;
    if (cap > (1LL << 30)) {               // beyond any launch: the caller reports it unsupported
        p.items_cap = -1;
        return p;
    }
    p.items_cap = (int)cap;
    p.part_o_elems = (size_t)cap * p.nq * L->head_dim;
    p.part_ml_elems = (size_t)cap * p.nq * 2;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    p.ticket_bytes = 256;
    p.bytes = p.ticket_bytes + up(p.part_o_elems * 4) + up(p.part_ml_elems * 4);
    return p;
}

// rows per combine workgroup: the largest power of two (<= 16, <= P rounded up) that still
// leaves at least eight combine workgroups per CU
static int combine_rows(int nb, int nc, int H, int P, int num_cus) {
    const long long blocks = (long long)nb * nc * H;
    int rg = 1;
    while (rg < 16 && rg < P && blocks * ((P + 2 * rg - 1) / (2 * rg)) >= 8LL * num_cus) rg *= 2;
    return rg;
}

// dynamic LDS of the finish kernel: the larger of its two roles
size_t stream_lds_bytes(const hci_layer* L, int nc, int P) {
    const int act_bytes = L->act_dtype == HCI_BF16 ? 2 : 4;
    const size_t conv = conv_iir_lds_floats(L->taps_short, L->taps_outer, nc * P);
    const size_t comb = combine_lds_floats(P, L->head_dim, act_bytes, 16);
    return (conv > comb ? conv : comb) * sizeof(float);
}

template <int ACT>
static hipError_t launch_finish(const FinishArgs& F, int rg, int blocks, size_t lds, hipStream_t st) {
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

// One verify: reset the queue, stream the prefix (bf16: persistent queue kernel; fp32: one
// workgroup per item), then the finish kernel (conv/IIR scan, causal block part, combine).
hipError_t launch_verify(const hci_layer* L, const hci_state* S, const hci_block* blk,
                         int nb, int nc, int P, const AttnPlan& plan, void* ws, hipStream_t st, hipEvent_t* ev,
                         bool conv)
{
    const int H = L->heads, DH = L->head_dim, nq = plan.nq;
    const float scale_log2 = kLog2e / sqrtf((float)DH);
    unsigned* ticket = (unsigned*)ws;
    float* part_o = (float*)((char*)ws + plan.ticket_bytes);
    float* part_ml = (float*)((char*)part_o + (plan.part_o_elems * 4 + 255) / 256 * 256);
    auto mark = [&](int i) { return (ev && ev[i]) ? hipEventRecord(ev[i], st) : hipSuccess; };
    hipError_t e = mark(0);
    if (e != hipSuccess) return e;

    if (plan.items_cap > 0) {
        if (L->act_dtype == HCI_BF16) {
            StreamArgs A{};
            A.kc = (const uint16_t*)S->k_cache; A.vc = (const uint16_t*)S->v_cache; A.q = (const uint16_t*)blk->q;
            A.kv_len = S->kv_len; A.part_o = part_o; A.part_ml = part_ml; A.ticket = ticket;
            A.H = H; A.kv_cap = S->kv_cap; A.kv_lim = plan.kv_lim; A.nq = nq; A.nb = nb; A.resident = plan.resident;
            A.scale_log2 = scale_log2;
            const int nqt = (nq + 15) / 16;
            hipLaunchKernelGGL(k_ticket_reset, dim3(1), dim3(64), 0, st, ticket);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            const int blocks = plan.items_cap < plan.resident ? plan.items_cap : plan.resident;
            if (nqt > 1) {
                if (DH == 128)
                    hipLaunchKernelGGL(k_attn_prefix_shared<128>, dim3(blocks), dim3(kRoleT), 0, st, A, nqt);
                else
                    hipLaunchKernelGGL(k_attn_prefix_shared<64>, dim3(blocks), dim3(kRoleT), 0, st, A, nqt);
            } else {
                if (DH == 128)
                    hipLaunchKernelGGL(k_verify_stream<128>, dim3(blocks), dim3(kRoleT), 0, st, A);
                else
                    hipLaunchKernelGGL(k_verify_stream<64>, dim3(blocks), dim3(kRoleT), 0, st, A);
            }
            if ((e = hipGetLastError()) != hipSuccess) return e;
        } else {
            hipLaunchKernelGGL(k_attn_prefix_f32, dim3(plan.items_cap), dim3(64), 0, st,
                               (const float*)S->k_cache, (const float*)S->v_cache, S->kv_len,
                               (const float*)blk->q, part_o, part_ml, nb, H, DH, S->kv_cap, plan.kv_lim, nq,
                               plan.resident, scale_log2);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    if ((e = mark(1)) != hipSuccess) return e;

    FinishArgs F{};
    F.w_short = L->w_short; F.w_outer = L->w_outer; F.lam = L->lambda; F.beta = L->beta; F.cc = L->c;
    F.short_win = S->short_win; F.outer_win = S->outer_win; F.iir = S->iir; F.x = blk->x;
    F.f_out = blk->f; F.s_out = blk->s; F.y_out = blk->y;
    F.d = L->d; F.Ts = L->taps_short; F.To = L->taps_outer; F.N = L->poles; F.nc = nc;
    F.n_conv = conv ? ((L->d + kCG - 1) / kCG) * nb : 0;
    F.kv_len = S->kv_len; F.part_o = part_o; F.part_ml = part_ml;
    F.q = blk->q; F.kb = blk->k; F.vb = blk->v; F.o = blk->o;
    F.nb = nb; F.H = H; F.DH = DH; F.nq = nq; F.P = P; F.kv_lim = plan.kv_lim; F.resident = plan.resident;
    F.scale_log2 = scale_log2;
    const int rg = combine_rows(nb, nc, H, P, plan.resident / (nq > 16 ? kSlotsShared : kSlotsFused));
    F.rg_count = (P + rg - 1) / rg;
    const long long blocks = (long long)F.n_conv + (long long)F.rg_count * nc * H * nb;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const int act_bytes = L->act_dtype == HCI_BF16 ? 2 : 4;
    const size_t conv_lds = conv ? conv_iir_lds_floats(L->taps_short, L->taps_outer, nc * P) : 0;
    const size_t comb_lds = combine_lds_floats(P, DH, act_bytes, rg);
    const size_t lds = (conv_lds > comb_lds ? conv_lds : comb_lds) * sizeof(float);
    e = L->act_dtype == HCI_BF16 ? launch_finish<HCI_BF16>(F, rg, (int)blocks, lds, st)
                                 : launch_finish<HCI_F32>(F, rg, (int)blocks, lds, st);
    if (e != hipSuccess) return e;
    return mark(2);
}

}  // namespace hci
