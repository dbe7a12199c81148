// One 32-key tile of the KV prefix against 16 queries on the matrix cores,
// shared by the prefix-streaming kernels.  The tiled cache layout (see
// hci_internal.h) makes every wave-wide 16-byte load a contiguous kilobyte and
// delivers the value operand already transposed: S^T = K Q^T and
// O^T += V^T P^T run on v_mfma_f32_16x16x32_bf16 with the keys in M; the
// online softmax (running max in log2 units, normaliser) stays in fp32
// registers, and the normaliser is one more product against a row of ones,
// so it sums exactly the bf16 weights the value product used.
#pragma once

#include "worklist.h"

namespace hci {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRoleT = 256;            // threads per workgroup of every streaming kernel
constexpr int kPrefixWaves = 4;        // waves per streaming workgroup
// resident streaming workgroups per CU: one, so that no two workgroups on a CU compete for
// issue (the older one would run up to twice as fast and finish its items late); its four
// waves keep enough loads in flight
constexpr int kStreamSlots = 1;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 ones_bf16x8() {
    return as_bf16x8(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));   // eight bf16 1.0
}

struct StreamArgs {
    const uint16_t *kc, *vc, *q; const int32_t* kv_len;
    float *part_o, *part_ml;
    const int32_t* ws;                 // the workspace header and work-list table (set-up kernel)
    unsigned* ticket;                  // the job queue's counter (zeroed by the set-up kernel)
    int H, kv_cap, kv_lim, nq, nb, resident;
    float scale_log2;
};

// Maximum over lanes l, l^16, l^32 and l^48 (the four 4-key row groups that hold one query
// column of a 16x16 product), on the vector ALU: two gfx950 lane swaps, each exchanging a
// value with the partner half (32 lanes apart) or row (16 lanes apart) of the wave.
__device__ __forceinline__ float max_over_row_groups(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// ------------------------------------------------ direct global->LDS loads
//
// LDS byte offset of a pointer into __shared__ memory: the LDS aperture of the flat address
// space starts at a 4 GiB boundary, so the low 32 bits of the flat address are the offset
// (no address-space cast, whose null check would keep 64-bit pointers alive).
__device__ __forceinline__ uint32_t lds_offset(const void* p) { return (uint32_t)(uintptr_t)p; }

// Direct global->LDS load of 16 bytes per lane, non-temporal: lane l's bytes land at LDS
// byte offset lds_base + 16*l (lds_base wave-uniform, in M0).  Inline assembly, so that the
// compiler's own wait insertion leaves it alone: the waits are explicit (HCI_WAIT_VM).  M0
// is saved and restored, and one wait state separates its write from the load.
__device__ __forceinline__ void dma16_nt(const uint4* src, uint32_t lds_base) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved) : "v"(src), "s"(base) : "memory");
}

// s_waitcnt that leaves n vector-memory operations outstanding (vmcnt in bits 3:0 and
// 15:14; expcnt and lgkmcnt at their no-wait maxima), and one for every LDS operation
#define HCI_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | (((n) >> 4) << 14))
#define HCI_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14))

// keeps the compiler from moving any memory access across this point
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

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

// Rescale threshold of the running maximum, in log2 units.  A query's reference
// maximum m moves only when a tile's top score exceeds it by more than this, so the
// accumulators are rescaled rarely (in practice on a run's first tiles); the weights
// exp2(s - m) then stay below 2^kLazyMax, far inside the range of bf16 and fp32, and
// the final division by the normaliser cancels the reference exactly.
constexpr float kLazyMax = 8.0f;

// One 32-key tile: S^T = K Q^T on the matrix cores, online softmax in fp32,
// O^T += V^T P^T on the matrix cores.  Keys >= L (the ragged end) are masked.
// The score products of every query tile are issued together (2 NQT independent
// accumulation chains), the maximum is taken on the raw products (the scale c is
// positive, so scaling the maximum is exact) and each weight is exp2(s c - m) with
// one fused multiply-add.
template <int DH, int NQT>
__device__ __forceinline__ void consume_tile(PrefixAcc<DH, NQT>& a, KvTile<DH>& t, int T, int L, int g,
                                             float c) {
    constexpr int J = DH / 32, DT = DH / 16;
    const int kbase = T * kTile;
    const bool tail = kbase + kTile > L;          // wave-uniform: only a prefix's last tile
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
    f32x4 acc[NQT][2];
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) acc[nt][0] = acc[nt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                acc[nt][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.k[u * J + j]), a.q[nt][j],
                                                                     acc[nt][u], 0, 0, 0);
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
        // element e of this lane: key kbase + 16 (e >> 2) + 4 g + (e & 3)
        float s[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = acc[nt][e >> 2][e & 3];
        if (tail) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (kbase + 16 * (e >> 2) + 4 * g + (e & 3) >= L) s[e] = -INFINITY;
        }
        float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
        mx = max_over_row_groups(mx);
        const float top = mx * c;
        const float mold = a.m[nt];
        const float mnew = top > mold + kLazyMax ? top : mold;
        const float alpha = __builtin_amdgcn_exp2f(mold - mnew);
        a.m[nt] = mnew;
        f32x2 pf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pf[i] = f32x2{__builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i], c, -mnew)),
                          __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i + 1], c, -mnew))};
        const bf16x8 pb = __builtin_shufflevector(
            __builtin_shufflevector(__builtin_convertvector(pf[0], bf16x2), __builtin_convertvector(pf[1], bf16x2), 0, 1, 2, 3),
            __builtin_shufflevector(__builtin_convertvector(pf[2], bf16x2), __builtin_convertvector(pf[3], bf16x2), 0, 1, 2, 3),
            0, 1, 2, 3, 4, 5, 6, 7);                            // round to nearest even
        // the reference maximum seldom moves: skip the rescale when no lane of the wave needs it
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

// launcher of the streaming kernel (grid = blocks persistent workgroups, nqt 16-query tiles)
hipError_t launch_stream_one(const StreamArgs& A, int head_dim, int nqt, int blocks, hipStream_t st);

}  // namespace hci
