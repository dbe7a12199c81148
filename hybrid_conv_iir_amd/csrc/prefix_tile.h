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
    unsigned* ticket;                  // the job queue's counter (zeroed before the launch)
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
        mx = max_over_row_groups(mx);
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

// launcher of the streaming kernel (grid = blocks persistent workgroups, nqt 16-query tiles)
hipError_t launch_stream_one(const StreamArgs& A, int head_dim, int nqt, int blocks, hipStream_t st);

}  // namespace hci
