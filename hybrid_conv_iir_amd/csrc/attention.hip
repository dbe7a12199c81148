// Attention half of the block forward: the block queries attend to the
// committed KV prefix (split-K over the prefix, one partial softmax state per
// chunk) and causally to the block's own keys; a combine kernel merges the
// partials in a fixed order.  EvSpark digest, Interpretation: the verify is
// one block forward from the committed state, so all nc*P queries of a
// sequence share a single read of its prefix; the prefix read is the part of
// the verify that grows with context (ReaDy summary, section 5: token-wise KV
// traffic grows with the number of attended tokens).
//
// Prefix kernel (bf16): one wave per (chunk, head, sequence).  Per 32-key
// tile the wave issues 2*Dh/32 + Dh/16 sixteen-byte loads per lane, each a
// contiguous kilobyte thanks to the tiled cache layout, prefetching the next
// tile while the current one is consumed.  Scores S^T = K Q^T and the value
// product O^T += V^T P^T run on v_mfma_f32_16x16x32_bf16 with the keys in
// the M dimension and up to 16*NQT queries in N; the online softmax (max,
// rescale, exp2) runs in fp32 registers with a 4-lane exchange per query.
#include "hci_internal.h"

#include <math.h>

namespace hci {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// ------------------------------------------------------------ bf16 prefix

constexpr int kPrefixWaves = 4;      // waves per workgroup; their partials merge in LDS

template <int DH, int NQT>
constexpr size_t prefix_merge_floats() {
    // per merged wave: O^T accumulators (16*NQT queries x DH), running max, normaliser
    return (size_t)NQT * 16 * DH + 2 * NQT * 16;
}

template <int DH, int NQT>
__global__ __launch_bounds__(64 * kPrefixWaves) void k_attn_prefix_bf16(
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ kv_len, const uint16_t* __restrict__ q,
    float* __restrict__ part_o, float* __restrict__ part_ml,
    int H, int kv_cap, int nq, int chunk_tiles, int n_chunks, float scale_log2)
{
    constexpr int J = DH / 32;          // k-steps of the score product
    constexpr int DT = DH / 16;         // 16-wide output tiles of the value product
    constexpr int KV4 = 4 * DH;         // uint4 per tile (32 keys x DH bf16)
    constexpr size_t MF = prefix_merge_floats<DH, NQT>();
    extern __shared__ float merge[];    // [kPrefixWaves-1][MF]

    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    int L = kv_len[b];
    L = L < 0 ? 0 : (L > kv_cap ? kv_cap : L);
    const int tiles = (L + kTile - 1) / kTile;
    const int t0 = chunk * chunk_tiles;
    if (t0 >= tiles) return;                           // whole workgroup
    const int t1 = min(t0 + chunk_tiles, tiles);
    const int wave = threadIdx.x >> 6;
    const int per = (t1 - t0 + kPrefixWaves - 1) / kPrefixWaves;
    const int w0 = min(t0 + wave * per, t1), w1 = min(w0 + per, t1);   // wave 0 is never empty

    const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;

    // queries as B operands: lane (g, n) holds Q[16nt+n][32j+8g .. 32j+8g+7]
    bf16x8 qreg[NQT][J];
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
        const int qi = 16 * nt + n;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (qi < nq) v = *(const uint4*)(q + (((size_t)b * nq + qi) * H + h) * DH + 32 * j + 8 * g);
            qreg[nt][j] = as_bf16x8(v);
        }
    }

    f32x4 oacc[DT][NQT];
    float mrun[NQT], lrun[NQT];
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
        mrun[nt] = -INFINITY;
        lrun[nt] = 0.f;
#pragma unroll
        for (int t = 0; t < DT; ++t) oacc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const size_t slab = ((size_t)b * H + h) * (size_t)(kv_cap / kTile) * KV4;
    const uint4* kp = (const uint4*)kc + slab;
    const uint4* vp = (const uint4*)vc + slab;

    uint4 kr[2 * J], vr[DT];
    if (w0 < w1) {
#pragma unroll
        for (int i = 0; i < 2 * J; ++i) kr[i] = kp[(size_t)w0 * KV4 + i * 64 + lane];
#pragma unroll
        for (int t = 0; t < DT; ++t) vr[t] = vp[(size_t)w0 * KV4 + t * 64 + lane];
    }

    for (int T = w0; T < w1; ++T) {
        uint4 kn[2 * J], vn[DT];
        const bool more = T + 1 < w1;
        if (more) {
            const size_t base = (size_t)(T + 1) * KV4;
#pragma unroll
            for (int i = 0; i < 2 * J; ++i) kn[i] = kp[base + i * 64 + lane];
#pragma unroll
            for (int t = 0; t < DT; ++t) vn[t] = vp[base + t * 64 + lane];
        }

        const int kbase = T * kTile;
        const bool tail = kbase + kTile > L;
        if (tail) {
            // zero value rows past the prefix so that 0 * (stale bits) cannot poison the sums
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                uint32_t w[4] = {vr[t].x, vr[t].y, vr[t].z, vr[t].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int key = kbase + 16 * (e >> 2) + 4 * g + (e & 3);
                    if (key >= L) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
                }
                vr[t] = make_uint4(w[0], w[1], w[2], w[3]);
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
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[u * J + j]), qreg[nt][j], acc, 0, 0, 0);
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
            const float mnew = fmaxf(mrun[nt], mx);
            const float alpha = exp2f(mrun[nt] - mnew);
            mrun[nt] = mnew;
            uint32_t pk[4];
            float psum = 0.f;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const float p0 = exp2f(s[u][0] - mnew), p1 = exp2f(s[u][1] - mnew);
                const float p2 = exp2f(s[u][2] - mnew), p3 = exp2f(s[u][3] - mnew);
                pk[2 * u] = pack_bf16x2(p0, p1);
                pk[2 * u + 1] = pack_bf16x2(p2, p3);
                // the normaliser sums the same bf16-rounded weights the value product uses
                psum += (bf2f(pk[2 * u] & 0xffff) + bf2f(pk[2 * u] >> 16)) +
                        (bf2f(pk[2 * u + 1] & 0xffff) + bf2f(pk[2 * u + 1] >> 16));
            }
            lrun[nt] = fmaf(lrun[nt], alpha, psum);
            const bf16x8 pb = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                oacc[t][nt] *= alpha;
                oacc[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vr[t]), pb, oacc[t][nt], 0, 0, 0);
            }
        }

        if (more) {
#pragma unroll
            for (int i = 0; i < 2 * J; ++i) kr[i] = kn[i];
#pragma unroll
            for (int t = 0; t < DT; ++t) vr[t] = vn[t];
        }
    }

#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
        lrun[nt] += __shfl_xor(lrun[nt], 16);
        lrun[nt] += __shfl_xor(lrun[nt], 32);
    }

    // merge the four waves' partial softmax states in LDS (fixed order: wave 0, 1, 2, 3)
    if (wave > 0) {
        float* mw = merge + (size_t)(wave - 1) * MF;
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) {
#pragma unroll
            for (int t = 0; t < DT; ++t)
                *(float4*)(mw + (((size_t)nt * DT + t) * 64 + lane) * 4) =
                    make_float4(oacc[t][nt][0], oacc[t][nt][1], oacc[t][nt][2], oacc[t][nt][3]);
            if (g == 0) {
                mw[(size_t)NQT * 16 * DH + nt * 16 + n] = mrun[nt];
                mw[(size_t)NQT * 16 * DH + NQT * 16 + nt * 16 + n] = lrun[nt];
            }
        }
    }
    __syncthreads();
    if (wave > 0) return;

    // partial softmax state of this chunk: part_o [nb][H][n_chunks][nq][DH] (unnormalised),
    // part_ml [..][nq][2] = (running max in log2 units, normaliser)
    const size_t pbase = (((size_t)b * H + h) * n_chunks + chunk) * nq;
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
        float M = mrun[nt];
#pragma unroll
        for (int w = 1; w < kPrefixWaves; ++w) M = fmaxf(M, merge[(w - 1) * MF + (size_t)NQT * 16 * DH + nt * 16 + n]);
        float sc[kPrefixWaves];
        sc[0] = exp2f(mrun[nt] - M);
        float l = sc[0] * lrun[nt];
#pragma unroll
        for (int w = 1; w < kPrefixWaves; ++w) {
            const float* mw = merge + (size_t)(w - 1) * MF;
            sc[w] = exp2f(mw[(size_t)NQT * 16 * DH + nt * 16 + n] - M);
            l = fmaf(sc[w], mw[(size_t)NQT * 16 * DH + NQT * 16 + nt * 16 + n], l);
        }
        const int qi = 16 * nt + n;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            f32x4 acc = oacc[t][nt] * sc[0];
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

// ------------------------------------------------------------- f32 prefix
//
// fp32 layers (small shapes): 64 threads per (chunk, head, sequence).  The
// tile is unpacked into LDS rows; thread tid scores query tid and accumulates
// output dims tid and tid+64 of every query, all in fp32 on the vector ALUs.
// Limits: Dh <= 128, nq <= 64.

constexpr int kF32Dh = 128;
constexpr int kF32Nq = 64;

__global__ __launch_bounds__(64) void k_attn_prefix_f32(
    const float* __restrict__ kc, const float* __restrict__ vc,
    const int32_t* __restrict__ kv_len, const float* __restrict__ q,
    float* __restrict__ part_o, float* __restrict__ part_ml,
    int H, int DH, int kv_cap, int nq, int chunk_tiles, int n_chunks, float scale_log2)
{
    __shared__ float ks[kTile][kF32Dh + 1];
    __shared__ float vs[kTile][kF32Dh + 1];
    __shared__ float ps[kF32Nq][kTile + 1];
    __shared__ float alpha_s[kF32Nq];

    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    int L = kv_len[b];
    L = L < 0 ? 0 : (L > kv_cap ? kv_cap : L);
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
    const size_t pbase = (((size_t)b * H + h) * n_chunks + chunk) * nq;
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
// One workgroup of 256 threads per (query, head, sequence).  First the
// causal part over the block's own keys 0..i is computed in fp32 (one
// partial softmax state), then the prefix partials are merged with it:
//   M = max(m_tail, m_c), w_c = 2^(m_c - M),
//   o = (sum_c w_c O_c + 2^(m_tail - M) O_tail) / (sum_c w_c l_c + 2^(m_tail - M) l_tail)
// Chunk weights are formed once per chunk in LDS; thread groups accumulate
// interleaved chunks and are merged in a fixed order, so the result does not
// depend on scheduling.

constexpr int kCombT = 256;
constexpr int kMaxChunks = 4096;     // the split-K plan never exceeds this

template <int ACT>
__global__ __launch_bounds__(kCombT) void k_attn_combine(
    const typename Act<ACT>::T* __restrict__ q, const typename Act<ACT>::T* __restrict__ kb,
    const typename Act<ACT>::T* __restrict__ vb, const int32_t* __restrict__ kv_len,
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    typename Act<ACT>::T* __restrict__ o,
    int H, int DH, int P, int nq, int kv_cap, int chunk_tiles, int n_chunks, float scale_log2)
{
    __shared__ float wts[kMaxChunks];
    __shared__ float red[kCombT / 64][64];
    __shared__ float sc[64];
    __shared__ float acc_s[kCombT];

    const int qi = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int c = qi / P, i = qi % P;
    const int tid = threadIdx.x, wave = tid >> 6, ln = tid & 63;
    const int nw = kCombT / 64;

    // ---- block part: scores of keys 0..i (two-level fixed-order reduction)
    const size_t rowq = (((size_t)b * nq + qi) * H + h) * DH;
    const size_t rowb = ((size_t)b * nq + (size_t)c * P) * H;   // + j*H + h for block row j
    const float qd = tid < DH ? Act<ACT>::load(q, rowq + tid) : 0.f;
    for (int j = 0; j <= i; ++j) {
        float v = tid < DH ? qd * Act<ACT>::load(kb, (rowb + (size_t)j * H + h) * DH + tid) : 0.f;
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (ln == 0) red[wave][j] = v;
    }
    __syncthreads();
    if (tid <= i) {
        float s = 0.f;
        for (int w = 0; w < nw; ++w) s += red[w][tid];
        sc[tid] = s * scale_log2;
    }
    __syncthreads();
    float mt = -INFINITY;
    for (int j = 0; j <= i; ++j) mt = fmaxf(mt, sc[j]);

    // ---- prefix partials: running max over chunks
    int L = kv_len[b];
    L = L < 0 ? 0 : (L > kv_cap ? kv_cap : L);
    const int tiles = (L + kTile - 1) / kTile;
    int nch = (tiles + chunk_tiles - 1) / chunk_tiles;
    nch = nch > n_chunks ? n_chunks : nch;
    const size_t pb = ((size_t)b * H + h) * n_chunks;
    float mloc = -INFINITY;
    for (int ck = tid; ck < nch; ck += kCombT) mloc = fmaxf(mloc, part_ml[((pb + ck) * nq + qi) * 2]);
    for (int off = 32; off >= 1; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
    if (ln == 0) red[wave][0] = mloc;
    __syncthreads();
    float M = mt;
    for (int w = 0; w < nw; ++w) M = fmaxf(M, red[w][0]);
    __syncthreads();

    // ---- chunk weights and the normaliser
    float lloc = 0.f;
    for (int ck = tid; ck < nch; ck += kCombT) {
        const float2 ml = *(const float2*)(part_ml + ((pb + ck) * nq + qi) * 2);
        const float w = exp2f(ml.x - M);
        wts[ck] = w;
        lloc = fmaf(w, ml.y, lloc);
    }
    for (int off = 32; off >= 1; off >>= 1) lloc += __shfl_xor(lloc, off);
    if (ln == 0) red[wave][1] = lloc;
    __syncthreads();
    float l = 0.f;
    for (int w = 0; w < nw; ++w) l += red[w][1];

    // ---- weighted sum of the chunk outputs: thread (group, d) takes chunks group, group+ng, ...
    const int ng = kCombT / DH;
    const int grp = tid / DH, dd = tid % DH;
    float acc = 0.f;
    if (grp < ng) {
        int ck = grp;
        for (; ck + 3 * ng < nch; ck += 4 * ng) {
            const float o0 = part_o[((pb + ck) * nq + qi) * DH + dd];
            const float o1 = part_o[((pb + ck + ng) * nq + qi) * DH + dd];
            const float o2 = part_o[((pb + ck + 2 * ng) * nq + qi) * DH + dd];
            const float o3 = part_o[((pb + ck + 3 * ng) * nq + qi) * DH + dd];
            acc = fmaf(wts[ck], o0, acc);
            acc = fmaf(wts[ck + ng], o1, acc);
            acc = fmaf(wts[ck + 2 * ng], o2, acc);
            acc = fmaf(wts[ck + 3 * ng], o3, acc);
        }
        for (; ck < nch; ck += ng) acc = fmaf(wts[ck], part_o[((pb + ck) * nq + qi) * DH + dd], acc);
    }
    acc_s[tid] = acc;
    __syncthreads();

    if (tid < DH) {
        float tot = 0.f;
        for (int g2 = 0; g2 < ng; ++g2) tot += acc_s[g2 * DH + tid];
        // block part: weights 2^(s_j - M) directly in the merged frame
        float lt = 0.f, ot = 0.f;
        for (int j = 0; j <= i; ++j) {
            const float p = exp2f(sc[j] - M);
            lt += p;
            ot = fmaf(p, Act<ACT>::load(vb, (rowb + (size_t)j * H + h) * DH + tid), ot);
        }
        Act<ACT>::store(o, rowq + tid, (tot + ot) / (l + lt));
    }
}

// -------------------------------------------------------------------- host

AttnPlan plan_attention(const hci_layer* L, int nb, int nc, int gamma, int max_kv_len, int num_cus)
{
    AttnPlan p{};
    const int P = gamma + 1;
    p.nq = nc * P;
    const int tiles = (max_kv_len + kTile - 1) / kTile;
    // Aim for about 16 waves (4 workgroups of 4 waves) per CU over the whole
    // grid so that every CU keeps several waves and their prefetched tiles in
    // flight, with at least 8 tiles per wave so that partials stay a small
    // fraction of the traffic.
    const long long total_tiles = (long long)tiles * nb * L->heads;
    const long long target_wgs = (long long)num_cus * 4;
    long long ct = (total_tiles + target_wgs - 1) / (target_wgs > 0 ? target_wgs : 1);
    if (ct < 8 * kPrefixWaves) ct = 8 * kPrefixWaves;
    const long long min_ct = (tiles + kMaxChunks - 1) / kMaxChunks;   // combine holds <= kMaxChunks weights
    if (ct < min_ct) ct = min_ct;
    if (ct > tiles && tiles > 0) ct = tiles;
    if (ct < 1) ct = 1;
    p.chunk_tiles = (int)ct;
    p.n_chunks = tiles > 0 ? (int)((tiles + ct - 1) / ct) : 0;
    p.part_o_elems = (size_t)nb * L->heads * p.n_chunks * p.nq * L->head_dim;
    p.part_ml_elems = (size_t)nb * L->heads * p.n_chunks * p.nq * 2;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    p.bytes = up(p.part_o_elems * 4) + up(p.part_ml_elems * 4);
    return p;
}

hipError_t launch_attention(const hci_layer* L, const hci_state* S, const hci_block* blk,
                            int nb, int nc, int P, const AttnPlan& plan, void* ws, hipStream_t st,
                            hipEvent_t* after_prefix)
{
    const int H = L->heads, DH = L->head_dim, nq = plan.nq;
    const float scale_log2 = kLog2e / sqrtf((float)DH);
    float* part_o = (float*)ws;
    float* part_ml = (float*)((char*)ws + (plan.part_o_elems * 4 + 255) / 256 * 256);

    if (plan.n_chunks > 0) {
        dim3 grid(plan.n_chunks, H, nb), block(64);
        if (L->act_dtype == HCI_BF16) {
            const int nqt = (nq + 15) / 16;
#define HCI_PREFIX(DHV, NQTV)                                                                      \
    do {                                                                                           \
        const size_t lds = (kPrefixWaves - 1) * prefix_merge_floats<DHV, NQTV>() * sizeof(float);  \
        if (lds > 65536) {                                                                         \
            hipError_t ea = hipFuncSetAttribute((const void*)k_attn_prefix_bf16<DHV, NQTV>,        \
                                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
            if (ea != hipSuccess) return ea;                                                       \
        }                                                                                          \
        hipLaunchKernelGGL((k_attn_prefix_bf16<DHV, NQTV>), grid, dim3(64 * kPrefixWaves), lds, st, \
                           (const uint16_t*)S->k_cache, (const uint16_t*)S->v_cache, S->kv_len,    \
                           (const uint16_t*)blk->q, part_o, part_ml, H, S->kv_cap, nq,             \
                           plan.chunk_tiles, plan.n_chunks, scale_log2);                           \
    } while (0)
            if (DH == 128) {
                switch (nqt) {
                    case 1: HCI_PREFIX(128, 1); break;
                    case 2: HCI_PREFIX(128, 2); break;
                    case 3: HCI_PREFIX(128, 3); break;
                    default: HCI_PREFIX(128, 4); break;
                }
            } else {
                switch (nqt) {
                    case 1: HCI_PREFIX(64, 1); break;
                    case 2: HCI_PREFIX(64, 2); break;
                    case 3: HCI_PREFIX(64, 3); break;
                    default: HCI_PREFIX(64, 4); break;
                }
            }
#undef HCI_PREFIX
        } else {
            hipLaunchKernelGGL(k_attn_prefix_f32, grid, block, 0, st,
                               (const float*)S->k_cache, (const float*)S->v_cache, S->kv_len,
                               (const float*)blk->q, part_o, part_ml, H, DH, S->kv_cap, nq,
                               plan.chunk_tiles, plan.n_chunks, scale_log2);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (after_prefix && *after_prefix) {
        hipError_t e = hipEventRecord(*after_prefix, st);
        if (e != hipSuccess) return e;
    }

    dim3 cgrid(nq, H, nb), cblock(kCombT);
    if (L->act_dtype == HCI_BF16) {
        hipLaunchKernelGGL(k_attn_combine<HCI_BF16>, cgrid, cblock, 0, st,
                           (const uint16_t*)blk->q, (const uint16_t*)blk->k, (const uint16_t*)blk->v,
                           S->kv_len, part_o, part_ml, (uint16_t*)blk->o, H, DH, P, nq, S->kv_cap,
                           plan.chunk_tiles, plan.n_chunks, scale_log2);
    } else {
        hipLaunchKernelGGL(k_attn_combine<HCI_F32>, cgrid, cblock, 0, st,
                           (const float*)blk->q, (const float*)blk->k, (const float*)blk->v,
                           S->kv_len, part_o, part_ml, (float*)blk->o, H, DH, P, nq, S->kv_cap,
                           plan.chunk_tiles, plan.n_chunks, scale_log2);
    }
    return hipGetLastError();
}

}  // namespace hci
