// Attention half of the block forward, plus the fused streaming kernel.
//
// The block queries attend to the committed KV prefix and, causally, to the
// block's own keys.  EvSpark digest, Interpretation: the verify is one block
// forward from the committed state, so all nc*P queries of a sequence share
// a single read of its prefix; that read is the part of the verify that grows
// with context (ReaDy summary, section 5: token-wise KV traffic grows with the
// number of attended tokens).  The prefix is split into chunks (split-K); each
// chunk leaves a partial softmax state (running max in log2 units, normaliser,
// unnormalised output), the block part leaves one more, and a combine kernel
// merges them in a fixed order.
//
// bf16 layers run ONE streaming kernel with three workgroup roles, dispatched
// in this order so the short ones overlap the long KV stream:
//   conv   the conv/IIR scan of 16 channels (conv_iir_body.h)
//   tail   the causal block part of one (sequence, candidate, head)
// (with several 16-query tiles the prefix runs as its own kernel,
// k_attn_prefix_shared, one query tile per wave over LDS-shared KV tiles)
//   prefix one chunk of one (sequence, head): four waves, each streaming a
//          contiguous run of 32-key tiles with non-temporal 16-byte loads
//          (a contiguous kilobyte per wave-wide load, thanks to the tiled
//          cache layout) and one tile prefetched into registers; scores
//          S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 with the
//          keys in M and up to 16*NQT queries in N; online softmax in fp32
//          registers; the four waves' states merge in LDS before one partial
//          is written.
// fp32 layers (small shapes) use separate conv, tail, prefix (vector ALU)
// and combine kernels.
#include "conv_iir_body.h"

#include <math.h>

namespace hci {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRoleT = 256;            // threads per workgroup of every streaming role

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 ones_bf16x8() {
    return as_bf16x8(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));   // eight bf16 1.0
}

// ------------------------------------------------------------ bf16 prefix

constexpr int kPrefixWaves = 4;      // waves per workgroup; their partials merge in LDS

// ------------------------------------------------------------ split-K plan
//
// The prefix lengths live on the device, so the split of the committed
// prefixes into chunks is derived there, from kv_len, by every prefix
// workgroup and by the combine alike.  Work items (sequence b, head h,
// chunk c) are numbered consecutively, sequence-major:
//   item = base_b + h * n_b + c,  n_b = ceil(tiles_b / ct),
//   base_b = H * (n_0 + ... + n_{b-1}),
// with ct = max(ct_min, ceil(H * sum_b tiles_b / target)) tiles per chunk.
// Workgroup ids map one to one onto items and ids past the last item exit at
// once: real work occupies consecutive ids whatever the lengths, and since the
// dispatcher deals consecutive ids round-robin to the XCDs, every XCD gets an
// even share of a ragged batch.  The number of items never exceeds
// target + nb * H.  Partials: item i at index i; the block part of (b, h) at
// index tail_base + b * H + h.

// Committed length of sequence b as the attention reads it: kv_len clamped to
// [0, lim], lim = min(kv_cap, max_kv_len), so that a length above the host's
// bound can never yield more work items or chunks than the host planned for.
__device__ __forceinline__ int prefix_len(const int32_t* kv_len, int b, int lim) {
    const int L = kv_len[b];
    return L < 0 ? 0 : (L > lim ? lim : L);
}

__device__ __forceinline__ int prefix_tiles(const int32_t* kv_len, int b, int lim) {
    return (prefix_len(kv_len, b, lim) + kTile - 1) / kTile;
}

__device__ __forceinline__ int split_ct(const int32_t* kv_len, int nb, int H, int lim, int ct_min, int target) {
    long long w = 0;
    for (int b = 0; b < nb; ++b) w += prefix_tiles(kv_len, b, lim);
    w *= H;
    const long long ct = (w + target - 1) / target;
    return ct > ct_min ? (int)ct : ct_min;
}

// Locate work item `id`; false past the last item.
__device__ __forceinline__ bool split_item(const int32_t* kv_len, int nb, int H, int lim, int ct, int id,
                                           int& b, int& h, int& chunk) {
    int base = 0;
    for (int bb = 0; bb < nb; ++bb) {
        const int n = (prefix_tiles(kv_len, bb, lim) + ct - 1) / ct;
        if (id < base + n * H) {
            const int r = id - base;
            b = bb;
            h = r / n;
            chunk = r - h * n;
            return true;
        }
        base += n * H;
    }
    return false;
}

template <int DH, int NQT>
__host__ __device__ constexpr size_t prefix_merge_floats() {
    // per merged wave: O^T accumulators (16*NQT queries x DH), running max, normaliser
    return (size_t)NQT * 16 * DH + 2 * NQT * 16;
}

// Per-wave register state of the prefix kernel: queries (B operands), the
// O^T accumulators, running max (log2 units) and lane-partial normaliser.
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


// One prefix workgroup: chunk `chunk` of head h of sequence b, all nq queries.
// Partials: part_o [item][nq][DH], part_ml [item][nq][2].
template <int DH, int NQT>
__device__ __forceinline__ void prefix_block(
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc, int L,
    const uint16_t* __restrict__ q, float* __restrict__ part_o, float* __restrict__ part_ml,
    int H, int kv_cap, int nq, int chunk_tiles, int item, float scale_log2,
    int chunk, int h, int b, float* merge)
{
    constexpr int J = DH / 32;          // k-steps of the score product
    constexpr int DT = DH / 16;         // 16-wide output tiles of the value product
    constexpr int KV4 = 4 * DH;         // uint4 per tile (32 keys x DH bf16)
    constexpr size_t MF = prefix_merge_floats<DH, NQT>();

    const int tiles = (L + kTile - 1) / kTile;
    const int t0 = chunk * chunk_tiles;
    if (t0 >= tiles) return;                           // whole workgroup
    const int t1 = min(t0 + chunk_tiles, tiles);
    const int wave = threadIdx.x >> 6;
    const int per = (t1 - t0 + kPrefixWaves - 1) / kPrefixWaves;
    const int w0 = min(t0 + wave * per, t1), w1 = min(w0 + per, t1);   // wave 0 is never empty
    const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;

    PrefixAcc<DH, NQT> a;
    // queries as B operands: lane (g, n) holds Q[16nt+n][32j+8g .. 32j+8g+7]
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
        const int qi = 16 * nt + n;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (qi < nq) v = *(const uint4*)(q + (((size_t)b * nq + qi) * H + h) * DH + 32 * j + 8 * g);
            a.q[nt][j] = as_bf16x8(v);
        }
        a.m[nt] = -INFINITY;
        a.l[nt] = 0.f;
#pragma unroll
        for (int t = 0; t < DT; ++t) a.o[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const size_t slab = ((size_t)b * H + h) * (size_t)(kv_cap / kTile) * KV4;
    const uint4* kp = (const uint4*)kc + slab;
    const uint4* vp = (const uint4*)vc + slab;
    KvTile<DH> cur, nxt;
    if (w0 < w1) load_tile<DH>(cur, kp, vp, w0, lane);
    for (int T = w0; T < w1; ++T) {
        const bool more = T + 1 < w1;
        if (more) load_tile<DH>(nxt, kp, vp, T + 1, lane);
        consume_tile<DH, NQT>(a, cur, T, L, g, scale_log2);
        if (more) cur = nxt;
    }

    // merge the four waves' partial softmax states in LDS (fixed order: wave 0, 1, 2, 3)
    if (wave > 0) {
        float* mw = merge + (size_t)(wave - 1) * MF;
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) {
#pragma unroll
            for (int t = 0; t < DT; ++t)
                *(float4*)(mw + (((size_t)nt * DT + t) * 64 + lane) * 4) =
                    make_float4(a.o[t][nt][0], a.o[t][nt][1], a.o[t][nt][2], a.o[t][nt][3]);
            if (g == 0) {
                mw[(size_t)NQT * 16 * DH + nt * 16 + n] = a.m[nt];
                mw[(size_t)NQT * 16 * DH + NQT * 16 + nt * 16 + n] = a.l[nt];
            }
        }
    }
    __syncthreads();
    if (wave > 0) return;

    const size_t pbase = (size_t)item * nq;
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
        float M = a.m[nt];
#pragma unroll
        for (int w = 1; w < kPrefixWaves; ++w) M = fmaxf(M, merge[(w - 1) * MF + (size_t)NQT * 16 * DH + nt * 16 + n]);
        float sc[kPrefixWaves];
        sc[0] = __builtin_amdgcn_exp2f(a.m[nt] - M);
        float l = sc[0] * a.l[nt];
#pragma unroll
        for (int w = 1; w < kPrefixWaves; ++w) {
            const float* mw = merge + (size_t)(w - 1) * MF;
            sc[w] = __builtin_amdgcn_exp2f(mw[(size_t)NQT * 16 * DH + nt * 16 + n] - M);
            l = fmaf(sc[w], mw[(size_t)NQT * 16 * DH + NQT * 16 + nt * 16 + n], l);
        }
        const int qi = 16 * nt + n;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            f32x4 acc = a.o[t][nt] * sc[0];
#pragma unroll
            for (int w = 1; w < kPrefixWaves; ++w) {
                const float4 o = *(const float4*)(merge + (size_t)(w - 1) * MF + (((size_t)nt * DT + t) * 64 + lane) * 4);
                acc[0] = fmaf(sc[w], o.x, acc[0]);
                acc[1] = fmaf(sc[w], o.y, acc[1]);
                acc[2] = fmaf(sc[w], o.z, acc[2]);
                acc[3] = fmaf(sc[w], o.w, acc[3]);
            }
            if (qi < nq) *(float4*)(part_o + (pbase + qi) * DH + 16 * t + 4 * g) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
        if (qi < nq && g == 0) *(float2*)(part_ml + (pbase + qi) * 2) = make_float2(M, l);
    }
}

// ------------------------------------------------------------- block part
//
// One workgroup per (sequence, candidate, head): the P block queries attend
// causally to the block's own keys (query i sees keys 0..i), in fp32.  The
// result is one more partial softmax state, at index tail_base + b * H + h.

constexpr int kMaxP = 64;

// LDS floats of the block part: scores [P][P+1], row max and sum, and the
// q and k rows of the block staged as raw activations
__host__ __device__ constexpr size_t tail_lds_floats(int P, int DH, int act_bytes) {
    return (size_t)P * (P + 1) + 2 * P + ((size_t)2 * P * DH * act_bytes + 3) / 4;
}

template <int ACT>
__device__ __forceinline__ void tail_block(
    const typename Act<ACT>::T* __restrict__ q, const typename Act<ACT>::T* __restrict__ kb,
    const typename Act<ACT>::T* __restrict__ vb, float* __restrict__ part_o, float* __restrict__ part_ml,
    int H, int DH, int P, int nq, int tail_base, float scale_log2, int c, int h, int b, float* lds)
{
    typedef typename Act<ACT>::T T;
    float* S = lds;                                   // [P][P + 1] scores, then weights
    float* mrow = S + P * (P + 1);                    // [P]
    float* lrow = mrow + P;                           // [P]
    T* qs = (T*)(lrow + P);                           // [P][DH]
    T* ks = qs + (size_t)P * DH;                      // [P][DH]
    const int tid = threadIdx.x, nthr = blockDim.x;
    const size_t row0 = (size_t)b * nq + (size_t)c * P;          // block row of position 0
    for (int e = tid; e < P * DH; e += nthr) {
        const int i = e / DH, dd = e % DH;
        const size_t o = ((row0 + i) * H + h) * DH + dd;
        qs[e] = q[o];
        ks[e] = kb[o];
    }
    __syncthreads();
    // scores s_ij = q_i . k_j * scale (log2 units), j <= i
    const int npairs = P * (P + 1) / 2;
    for (int p = tid; p < npairs; p += nthr) {
        int i = (int)((sqrtf(8.f * p + 1.f) - 1.f) * 0.5f);
        while ((i + 1) * (i + 2) / 2 <= p) ++i;
        while (i * (i + 1) / 2 > p) --i;
        const int j = p - i * (i + 1) / 2;
        float acc = 0.f;
        for (int dd = 0; dd < DH; ++dd) acc = fmaf(Act<ACT>::load(qs, (size_t)i * DH + dd), Act<ACT>::load(ks, (size_t)j * DH + dd), acc);
        S[i * (P + 1) + j] = acc * scale_log2;
    }
    __syncthreads();
    if (tid < P) {
        const int i = tid;
        float m = -INFINITY;
        for (int j = 0; j <= i; ++j) m = fmaxf(m, S[i * (P + 1) + j]);
        float l = 0.f;
        for (int j = 0; j <= i; ++j) {
            const float w = __builtin_amdgcn_exp2f(S[i * (P + 1) + j] - m);
            S[i * (P + 1) + j] = w;
            l += w;
        }
        mrow[i] = m;
        lrow[i] = l;
    }
    __syncthreads();
    const size_t pbase = ((size_t)tail_base + (size_t)b * H + h) * nq + (size_t)c * P;
    for (int e = tid; e < P * DH; e += nthr) {
        const int i = e / DH, dd = e % DH;
        float acc = 0.f;
        for (int j = 0; j <= i; ++j)
            acc = fmaf(S[i * (P + 1) + j], Act<ACT>::load(vb, ((row0 + j) * H + h) * DH + dd), acc);
        part_o[(pbase + i) * DH + dd] = acc;
    }
    for (int i = tid; i < P; i += nthr) *(float2*)(part_ml + (pbase + i) * 2) = make_float2(mrow[i], lrow[i]);
}

// ------------------------------------------------------ fused bf16 kernel

struct StreamArgs {
    // conv / IIR
    const float *w_short, *w_outer, *lam, *beta, *cc;
    const uint16_t* short_win; const float* outer_win; const float* iir; const uint16_t* x;
    float* f_out; float* s_out; uint16_t* y_out;
    int d, Ts, To, N;
    // attention
    const uint16_t *kc, *vc, *q, *kb, *vb; const int32_t* kv_len;
    float *part_o, *part_ml;
    int H, kv_cap, kv_lim, nq, nb, ct_min, target, tail_base, P, nc;
    float scale_log2;
    // role layout: prefix workgroups first (one per possible work item), then conv, then the block part
    int prefix_blocks, n_conv, n_tail;
};

// The short roles of a streaming kernel, workgroup r past the prefix items:
// first the conv/IIR scan of 16 channels of one sequence (all its
// candidates), then the causal block part of one (sequence, candidate, head).
__device__ __forceinline__ void short_role(const StreamArgs& A, int r, int DH, float* lds)
{
    if (r < A.n_conv) {
        const int groups = (A.d + kCG - 1) / kCG;
        const int cgi = r % groups, b = r / groups;
        conv_iir_block<HCI_BF16>(A.w_short, A.w_outer, A.lam, A.beta, A.cc, A.short_win, A.outer_win, A.iir, A.x,
                                 A.f_out, A.s_out, A.y_out, A.d, A.Ts, A.To, A.N, A.nc, A.P, cgi, b, lds);
        return;
    }
    const int t = r - A.n_conv;
    const int h = t % A.H, c = (t / A.H) % A.nc, b = t / (A.H * A.nc);
    tail_block<HCI_BF16>(A.q, A.kb, A.vb, A.part_o, A.part_ml, A.H, DH, A.P, A.nq, A.tail_base,
                         A.scale_log2, c, h, b, lds);
}

template <int DH, int NQT>
__global__ __launch_bounds__(kRoleT) void k_verify_stream(StreamArgs A)
{
    extern __shared__ float lds[];
    const int id = blockIdx.x;
    if (id < A.prefix_blocks) {
        const int ct = split_ct(A.kv_len, A.nb, A.H, A.kv_lim, A.ct_min, A.target);
        int b, h, chunk;
        if (!split_item(A.kv_len, A.nb, A.H, A.kv_lim, ct, id, b, h, chunk)) return;
        const int L = prefix_len(A.kv_len, b, A.kv_lim);
        prefix_block<DH, NQT>(A.kc, A.vc, L, A.q, A.part_o, A.part_ml, A.H, A.kv_cap, A.nq, ct, id,
                              A.scale_log2, chunk, h, b, lds);
        return;
    }
    // the short roles come last: they fill the slots the KV stream frees as it drains
    short_role(A, id - A.prefix_blocks, DH, lds);
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
// current tile are in registers.

constexpr int kStages = 4;

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
    uint4 *st0 = stage[0], *st1 = stage[1], *st2 = stage[2], *st3 = stage[3];
    const int id = blockIdx.x;
    if (id >= A.prefix_blocks) {
        // the short roles ride at the end of the grid (the host lets them only when their
        // LDS fits the stages) and fill the slots the KV stream frees as it drains
        short_role(A, id - A.prefix_blocks, DH, (float*)&stage[0][0]);
        return;
    }
    const int ct = split_ct(A.kv_len, A.nb, A.H, A.kv_lim, A.ct_min, A.target);
    int b, h, chunk;
    if (!split_item(A.kv_len, A.nb, A.H, A.kv_lim, ct, id, b, h, chunk)) return;   // whole workgroup
    const int L = prefix_len(A.kv_len, b, A.kv_lim);
    const int tiles = (L + kTile - 1) / kTile;
    const int t0 = chunk * ct;
    if (t0 >= tiles) return;                           // cannot happen for an item; kept as a guard
    const int t1 = min(t0 + ct, tiles);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
    const bool has_q = wave < nqt;

    PrefixAcc<DH, 1> a;
    {
        const int qi = 16 * wave + n;
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
        for (int t = 0; t < DH / 16; ++t) a.o[t][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const size_t slab = ((size_t)b * A.H + h) * (size_t)(A.kv_cap / kTile) * KV4;
    const uint4* kp = (const uint4*)A.kc + slab;
    const uint4* vp = (const uint4*)A.vc + slab;

    auto issue = [&](uint4* dst, int T) {
        const size_t base = (size_t)T * KV4;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + kRoleT * i;            // wave-uniform K/V choice: KV4 is a multiple of 64
            const uint4* src = e < KV4 ? kp + base + e : vp + base + (e - KV4);
            dma16_nt(src, dst + (e & ~63));
        }
    };
    auto step = [&](const uint4* cur, uint4* refill, int T) {
        // loads issued after tile T's: tiles T+1 and T+2, where they exist
        const int later = min(t1 - 1 - T, kStages - 2);
        if (later >= 2) HCI_WAIT_VM(2 * PER);
        else if (later == 1) HCI_WAIT_VM(PER);
        else HCI_WAIT_VM(0);
        lds_read_barrier();                            // tile T complete for every wave; tile T-1 read by all
        KvTile<DH> t;
        if (has_q) {
#pragma unroll
            for (int i = 0; i < DH / 16; ++i) t.k[i] = cur[i * 64 + lane];
#pragma unroll
            for (int i = 0; i < DH / 16; ++i) t.v[i] = cur[KV4 + i * 64 + lane];
        }
        // refill after the operand reads: the compiler then has no direct load to order them against
        if (T + kStages - 1 < t1) issue(refill, T + kStages - 1);
        if (has_q) consume_tile<DH, 1>(a, t, T, L, g, A.scale_log2);
    };
    issue(st0, t0);
    if (t0 + 1 < t1) issue(st1, t0 + 1);
    if (t0 + 2 < t1) issue(st2, t0 + 2);
    for (int T = t0; T < t1; T += kStages) {
        step(st0, st3, T);
        if (T + 1 >= t1) break;
        step(st1, st0, T + 1);
        if (T + 2 >= t1) break;
        step(st2, st1, T + 2);
        if (T + 3 >= t1) break;
        step(st3, st2, T + 3);
    }
    // the last step waited for every direct load: no LDS write is pending at exit
    if (!has_q) return;
    const int qi = 16 * wave + n;
    if (qi >= A.nq) return;
    const size_t pbase = (size_t)id * A.nq;
#pragma unroll
    for (int t = 0; t < DH / 16; ++t)
        *(float4*)(A.part_o + (pbase + qi) * DH + 16 * t + 4 * g) =
            make_float4(a.o[t][0][0], a.o[t][0][1], a.o[t][0][2], a.o[t][0][3]);
    if (g == 0) *(float2*)(A.part_ml + (pbase + qi) * 2) = make_float2(a.m[0], a.l[0]);
}

// -------------------------------------------------- stand-alone fp32 parts

template <int ACT>
__global__ __launch_bounds__(kRoleT) void k_attn_tail(
    const typename Act<ACT>::T* __restrict__ q, const typename Act<ACT>::T* __restrict__ kb,
    const typename Act<ACT>::T* __restrict__ vb, float* __restrict__ part_o, float* __restrict__ part_ml,
    int H, int DH, int P, int nq, int tail_base, float scale_log2)
{
    extern __shared__ float lds[];
    tail_block<ACT>(q, kb, vb, part_o, part_ml, H, DH, P, nq, tail_base, scale_log2,
                    blockIdx.y, blockIdx.x, blockIdx.z, lds);
}

// ------------------------------------------------------------- f32 prefix
//
// fp32 layers (small shapes): 64 threads per work item (chunk, head, sequence).  The
// tile is unpacked into LDS rows; thread tid scores query tid and accumulates
// output dims tid and tid+64 of every query, all in fp32 on the vector ALUs.
// Limits: Dh <= 128, nq <= 64.

constexpr int kF32Dh = 128;
constexpr int kF32Nq = 64;

__global__ __launch_bounds__(64) void k_attn_prefix_f32(
    const float* __restrict__ kc, const float* __restrict__ vc,
    const int32_t* __restrict__ kv_len, const float* __restrict__ q,
    float* __restrict__ part_o, float* __restrict__ part_ml,
    int nb, int H, int DH, int kv_cap, int kv_lim, int nq, int ct_min, int target, float scale_log2)
{
    __shared__ float ks[kTile][kF32Dh + 1];
    __shared__ float vs[kTile][kF32Dh + 1];
    __shared__ float ps[kF32Nq][kTile + 1];
    __shared__ float alpha_s[kF32Nq];

    const int item = blockIdx.x;
    const int chunk_tiles = split_ct(kv_len, nb, H, kv_lim, ct_min, target);
    int b, h, chunk;
    if (!split_item(kv_len, nb, H, kv_lim, chunk_tiles, item, b, h, chunk)) return;
    const int L = prefix_len(kv_len, b, kv_lim);
    const int tiles = (L + kTile - 1) / kTile;
    const int t0 = chunk * chunk_tiles;
    if (t0 >= tiles) return;
    const int t1 = min(t0 + chunk_tiles, tiles);
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
            const int w = e / DH, dd = e % DH;
            const int key = T * kTile + w;
            const bool ok = key < L;
            ks[w][dd] = ok ? kc[slab + k_elem(key, dd, DH)] : 0.f;
            vs[w][dd] = ok ? vc[slab + v_elem(key, dd, DH)] : 0.f;
        }
        __syncthreads();
        if (tid < nq) {
            float sc[kTile];
            float mx = -INFINITY;
#pragma unroll
            for (int w = 0; w < kTile; ++w) {
                float acc = 0.f;
#pragma unroll
                for (int dd = 0; dd < kF32Dh; ++dd)
                    if (dd < DH) acc = fmaf(qr[dd], ks[w][dd], acc);
                sc[w] = (T * kTile + w < L) ? acc * scale_log2 : -INFINITY;
                mx = fmaxf(mx, sc[w]);
            }
            const float mnew = fmaxf(mrun, mx);
            const float alpha = exp2f(mrun - mnew);
            float psum = 0.f;
#pragma unroll
            for (int w = 0; w < kTile; ++w) {
                const float p = exp2f(sc[w] - mnew);
                ps[tid][w] = p;
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
                        for (int w = 0; w < kTile; ++w) acc = fmaf(ps[qi][w], vs[w][dd], acc);
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

// ----------------------------------------------------------------- combine
//
// One workgroup of 256 threads per (query, head, sequence) merges the chunk
// partials (items base_b + h*n_b + 0..n_b-1, derived from kv_len exactly as the
// prefix kernels derive them) and the block part:  M = max m_s, w_s = 2^(m_s - M),
//   o = sum_s w_s O_s / sum_s w_s l_s,
// with the chunks taken in a fixed interleave and the group sums merged in a
// fixed order, so the result does not depend on scheduling.

constexpr int kCombT = 256;
constexpr int kMaxChunks = 4096;     // the split-K plan never exceeds this

template <int ACT>
__global__ __launch_bounds__(kCombT) void k_attn_combine(
    const int32_t* __restrict__ kv_len, const float* __restrict__ part_o, const float* __restrict__ part_ml,
    typename Act<ACT>::T* __restrict__ o,
    int nb, int H, int DH, int nq, int kv_lim, int ct_min, int target, int tail_base)
{
    __shared__ float wts[kMaxChunks + 1];
    __shared__ float red[kCombT / 64][2];
    __shared__ float acc_s[kCombT];

    const int qi = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, ln = tid & 63;
    const int nw = kCombT / 64;

    const int ct = split_ct(kv_len, nb, H, kv_lim, ct_min, target);
    int base = 0;
    for (int bb = 0; bb < b; ++bb) base += (prefix_tiles(kv_len, bb, kv_lim) + ct - 1) / ct * H;
    const int nch = (prefix_tiles(kv_len, b, kv_lim) + ct - 1) / ct;
    const size_t first = (size_t)base + (size_t)h * nch;
    const size_t tail = (size_t)tail_base + (size_t)b * H + h;
    auto slot_of = [&](int s) { return s < nch ? first + s : tail; };    // s == nch is the block part
    const int ns = nch + 1;

    float mloc = -INFINITY;
    for (int s = tid; s < ns; s += kCombT) mloc = fmaxf(mloc, part_ml[(slot_of(s) * nq + qi) * 2]);
    for (int off = 32; off >= 1; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
    if (ln == 0) red[wave][0] = mloc;
    __syncthreads();
    float M = red[0][0];
    for (int w = 1; w < nw; ++w) M = fmaxf(M, red[w][0]);

    float lloc = 0.f;
    for (int s = tid; s < ns; s += kCombT) {
        const float2 ml = *(const float2*)(part_ml + (slot_of(s) * nq + qi) * 2);
        const float w = exp2f(ml.x - M);
        wts[s] = w;
        lloc = fmaf(w, ml.y, lloc);
    }
    for (int off = 32; off >= 1; off >>= 1) lloc += __shfl_xor(lloc, off);
    if (ln == 0) red[wave][1] = lloc;
    __syncthreads();
    float l = 0.f;
    for (int w = 0; w < nw; ++w) l += red[w][1];

    // thread (group, d) accumulates slots group, group+ng, ...
    const int ng = kCombT / DH;
    const int grp = tid / DH, dd = tid % DH;
    float acc = 0.f;
    if (grp < ng) {
        int s = grp;
        for (; s + 3 * ng < ns; s += 4 * ng) {
            const float o0 = part_o[(slot_of(s) * nq + qi) * DH + dd];
            const float o1 = part_o[(slot_of(s + ng) * nq + qi) * DH + dd];
            const float o2 = part_o[(slot_of(s + 2 * ng) * nq + qi) * DH + dd];
            const float o3 = part_o[(slot_of(s + 3 * ng) * nq + qi) * DH + dd];
            acc = fmaf(wts[s], o0, acc);
            acc = fmaf(wts[s + ng], o1, acc);
            acc = fmaf(wts[s + 2 * ng], o2, acc);
            acc = fmaf(wts[s + 3 * ng], o3, acc);
        }
        for (; s < ns; s += ng) acc = fmaf(wts[s], part_o[(slot_of(s) * nq + qi) * DH + dd], acc);
    }
    acc_s[tid] = acc;
    __syncthreads();
    if (tid < DH) {
        float tot = 0.f;
        for (int g2 = 0; g2 < ng; ++g2) tot += acc_s[g2 * DH + tid];
        Act<ACT>::store(o, (((size_t)b * nq + qi) * H + h) * DH + tid, tot / l);
    }
}

// -------------------------------------------------------------------- host

AttnPlan plan_attention(const hci_layer* L, int nb, int nc, int gamma, int max_kv_len, int num_cus)
{
    AttnPlan p{};
    const int P = gamma + 1;
    p.nq = nc * P;
    const int tiles = (max_kv_len + kTile - 1) / kTile;
    // The device splits the real prefixes into about `target` chunks (work
    // items) over the whole batch.  With one query tile the fused kernel keeps
    // two 4-wave workgroups per CU: two rounds of them keep every CU streaming
    // until the end.  With several query tiles a workgroup walks its chunk with
    // all four waves, so twice as many (shorter) chunks keep the same number of
    // tiles in flight.  A chunk holds at least 8 tiles per wave, so that
    // partials stay a small fraction of the traffic, and a sequence never has
    // more than kMaxChunks chunks (the combine's weight table).
    const int nqt = (p.nq + 15) / 16;
    p.target = num_cus * (nqt > 1 ? 8 : 4);
    if (p.target < 1) p.target = 1;
    int ct_min = 8 * kPrefixWaves;
    const int min_ct = (tiles + kMaxChunks - 1) / kMaxChunks;
    if (ct_min < min_ct) ct_min = min_ct;
    p.ct_min = ct_min;
    p.kv_lim = max_kv_len;    // callers check max_kv_len + P <= kv_cap before any launch
    // items <= H * sum_b (tiles_b / ct + 1) <= target + nb * H, since ct >= H * sum_b tiles_b / target;
    // no items at all when every prefix is empty
    const long long nbh = (long long)nb * L->heads;
    if (p.target + 2 * nbh > (1LL << 30)) {            // beyond any launch: the caller reports it unsupported
        p.items_cap = -1;
        return p;
    }
    p.items_cap = tiles > 0 ? p.target + (int)nbh : 0;
    p.tail_base = p.items_cap;
    const size_t parts = (size_t)p.items_cap + (size_t)nbh;   // + the block part of each (b, h)
    p.part_o_elems = parts * p.nq * L->head_dim;
    p.part_ml_elems = parts * p.nq * 2;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    p.bytes = up(p.part_o_elems * 4) + up(p.part_ml_elems * 4);
    return p;
}

size_t stream_lds_bytes(const hci_layer* L, int nc, int P) {
    (void)nc;    // the fused kernel runs with one query tile only
    const size_t pre = (kPrefixWaves - 1) * (size_t)(16 * L->head_dim + 32);
    const int act_bytes = L->act_dtype == HCI_BF16 ? 2 : 4;
    size_t f = conv_iir_lds_floats(L->taps_outer, P);
    const size_t t = tail_lds_floats(P, L->head_dim, act_bytes);
    f = f > t ? f : t;
    f = f > pre ? f : pre;
    return f * sizeof(float);
}

template <int DH>
static hipError_t launch_stream(const StreamArgs& A, int blocks, size_t lds, hipStream_t st) {
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)k_verify_stream<DH, 1>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_verify_stream<DH, 1>), dim3(blocks), dim3(kRoleT), lds, st, A);
    return hipGetLastError();
}

hipError_t launch_verify(const hci_layer* L, const hci_state* S, const hci_block* blk,
                         int nb, int nc, int P, const AttnPlan& plan, void* ws, hipStream_t st, hipEvent_t* ev,
                         bool conv)
{
    const int H = L->heads, DH = L->head_dim, nq = plan.nq;
    const float scale_log2 = kLog2e / sqrtf((float)DH);
    float* part_o = (float*)ws;
    float* part_ml = (float*)((char*)ws + (plan.part_o_elems * 4 + 255) / 256 * 256);
    auto mark = [&](int i) { return (ev && ev[i]) ? hipEventRecord(ev[i], st) : hipSuccess; };
    hipError_t e = mark(0);
    if (e != hipSuccess) return e;

    if (L->act_dtype == HCI_BF16) {
        StreamArgs A{};
        A.w_short = L->w_short; A.w_outer = L->w_outer; A.lam = L->lambda; A.beta = L->beta; A.cc = L->c;
        A.short_win = (const uint16_t*)S->short_win; A.outer_win = S->outer_win; A.iir = S->iir;
        A.x = (const uint16_t*)blk->x; A.f_out = blk->f; A.s_out = blk->s; A.y_out = (uint16_t*)blk->y;
        A.d = L->d; A.Ts = L->taps_short; A.To = L->taps_outer; A.N = L->poles;
        A.kc = (const uint16_t*)S->k_cache; A.vc = (const uint16_t*)S->v_cache; A.q = (const uint16_t*)blk->q;
        A.kb = (const uint16_t*)blk->k; A.vb = (const uint16_t*)blk->v; A.kv_len = S->kv_len;
        A.part_o = part_o; A.part_ml = part_ml;
        A.H = H; A.kv_cap = S->kv_cap; A.kv_lim = plan.kv_lim; A.nq = nq; A.nb = nb; A.ct_min = plan.ct_min; A.target = plan.target;
        A.tail_base = plan.tail_base; A.P = P; A.nc = nc; A.scale_log2 = scale_log2;
        A.prefix_blocks = plan.items_cap;
        const int nqt = (nq + 15) / 16;
        // With one query tile the streaming kernel keeps two workgroups per CU and the
        // short roles ride along at the end of its grid.  With more query tiles it holds
        // a whole CU per workgroup, so the short roles run as their own light kernels.
        // With one query tile the streaming kernel keeps two workgroups per CU and the short
        // roles ride along at the end of its grid.  With several, the shared-prefix kernel
        // carries them when their LDS fits its stages, else they run as their own kernels first.
        const bool fuse = nqt == 1;
        const size_t stage_bytes = (size_t)kStages * 128 * DH;
        const size_t tail_lds = tail_lds_floats(P, DH, 2) * sizeof(float);
        const bool ride = fuse || (conv_iir_lds_bytes(L->taps_outer, P) <= stage_bytes && tail_lds <= stage_bytes);
        if (!ride) {
            if (conv && (e = launch_conv_iir(L, S, blk, nb, nc, P, st)) != hipSuccess) return e;
            if (tail_lds > 65536) {
                e = hipFuncSetAttribute((const void*)k_attn_tail<HCI_BF16>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                        (int)tail_lds);
                if (e != hipSuccess) return e;
            }
            hipLaunchKernelGGL(k_attn_tail<HCI_BF16>, dim3(H, nc, nb), dim3(kRoleT), tail_lds, st,
                               (const uint16_t*)blk->q, (const uint16_t*)blk->k, (const uint16_t*)blk->v, part_o,
                               part_ml, H, DH, P, nq, plan.tail_base, scale_log2);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        A.n_conv = ride && conv ? ((L->d + kCG - 1) / kCG) * nb : 0;
        A.n_tail = ride ? nb * nc * H : 0;
        const long long blocks = (long long)A.prefix_blocks + A.n_conv + A.n_tail;
        if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
        if (blocks > 0) {
            if (!fuse) {
                if (DH == 128)
                    hipLaunchKernelGGL(k_attn_prefix_shared<128>, dim3((int)blocks), dim3(kRoleT), 0, st, A, nqt);
                else
                    hipLaunchKernelGGL(k_attn_prefix_shared<64>, dim3((int)blocks), dim3(kRoleT), 0, st, A, nqt);
                e = hipGetLastError();
            } else {
                const size_t lds = stream_lds_bytes(L, nc, P);
                e = DH == 128 ? launch_stream<128>(A, (int)blocks, lds, st) : launch_stream<64>(A, (int)blocks, lds, st);
            }
            if (e != hipSuccess) return e;
        }
    } else {
        if (conv && (e = launch_conv_iir(L, S, blk, nb, nc, P, st)) != hipSuccess) return e;
        const size_t tail_lds = tail_lds_floats(P, DH, 4) * sizeof(float);
        if (tail_lds > 65536) {
            e = hipFuncSetAttribute((const void*)k_attn_tail<HCI_F32>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)tail_lds);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(k_attn_tail<HCI_F32>, dim3(H, nc, nb), dim3(kRoleT), tail_lds, st,
                           (const float*)blk->q, (const float*)blk->k, (const float*)blk->v, part_o, part_ml,
                           H, DH, P, nq, plan.tail_base, scale_log2);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (plan.items_cap > 0) {
            hipLaunchKernelGGL(k_attn_prefix_f32, dim3(plan.items_cap), dim3(64), 0, st,
                               (const float*)S->k_cache, (const float*)S->v_cache, S->kv_len,
                               (const float*)blk->q, part_o, part_ml, nb, H, DH, S->kv_cap, plan.kv_lim, nq,
                               plan.ct_min, plan.target, scale_log2);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    if ((e = mark(1)) != hipSuccess) return e;

    dim3 cgrid(nq, H, nb), cblock(kCombT);
    if (L->act_dtype == HCI_BF16) {
        hipLaunchKernelGGL(k_attn_combine<HCI_BF16>, cgrid, cblock, 0, st, S->kv_len, part_o, part_ml,
                           (uint16_t*)blk->o, nb, H, DH, nq, plan.kv_lim, plan.ct_min, plan.target, plan.tail_base);
    } else {
        hipLaunchKernelGGL(k_attn_combine<HCI_F32>, cgrid, cblock, 0, st, S->kv_len, part_o, part_ml,
                           (float*)blk->o, nb, H, DH, nq, plan.kv_lim, plan.ct_min, plan.target, plan.tail_base);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return mark(2);
}

}  // namespace hci
