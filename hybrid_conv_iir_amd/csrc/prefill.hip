// Prefill: run a prompt of T positions through the conv/recurrent path and
// append its K/V rows, leaving the committed state the first verify starts
// from.  By the block-forward contract (EvSpark digest, Interpretation: one
// block forward plus slicing restores the state sequential decoding would
// reach) this is a block forward over all T positions followed by a slice at
// T-1, restricted to the state; the prompt's attention outputs are not part
// of the state and are not computed.
//
// The IIR is linear and diagonal, so time is cut into chunks of 256
// positions (16 sub-chunks of 16) that scan independently from a zero state;
// the true start state of every chunk follows from a short carry scan over
// the chunk end states, and a fix-up adds its decayed contribution.
//   k_prefill_local  per (channel group, chunk): short FIR over the chunk and
//                    its halo into LDS, the outer FIR with a 31-value
//                    register window per thread (16 outputs x 16 taps per
//                    step, 2 LDS reads per 16 FMAs), the sub-chunk scans, the
//                    in-chunk carry, chunk-local readouts y and the chunk end
//                    state; the last To-1 f values of the prompt go to the
//                    workspace for the outer window
//   k_prefill_carry  per (sequence, channel, pole): chunk start states and
//                    the final IIR state (committed)
//   k_prefill_fixup  per (channel group, chunk): y += sum_n c lambda^(tau+1) S_chunk
//   k_prefill_commit FIR windows <- the prompt's last inputs
//   k_kv_pack        K/V rows appended in the tiled cache layout, then
//   k_len_add        kv_len += T.
//
// With bf16 activations the outputs y take a third route, k_prefill_y (one
// pass over the prompt per 16 channels on the matrix cores, described with the
// kernel), and the state the folded path below; the chunked kernels above
// serve fp32 layers and the shapes k_prefill_y does not cover.
//
// When only the state is wanted (no per-position outputs y) the outer FIR
// is folded into the IIR instead.  Both are linear and time-invariant per
// channel, so the state after the prompt is a fixed linear functional of
// the short-FIR outputs f, and exchanging the order of the two sums gives,
// with W = To-1, M = T-W and per (channel, pole),
//   s_T = lam^T s_0 + beta * ( H V + lam^(T-To) A + B )
//   V = sum_{m<M} lam^(M-1-m) f_m               one multiply-add per position
//   H = sum_{j<=W} w_j lam^(W-j)
//   B = sum_{b<W} f_{T-1-b} P_b,   P_b = sum_{j<=b} w_j lam^(b-j)
//   A = sum_{1<=a<=W} fbar_{-a} lam^a Q_a,   Q_a = sum_{j>=a} w_j lam^(W-j)
// (fbar_{-a} the committed outer window).  The per-position work drops from
// To + 2N multiply-adds to N, which leaves prefill bound by HBM traffic
// (dominated by the K/V append).  Requires T >= To.
//   k_prefill_scan   per (64 channels, chunk): short FIR in registers and the
//                    V scan over the chunk from zero, 8 sub-chunks merged in LDS
//   k_prefill_state  per (16 channels): chunk carries -> V, one pass over the
//                    taps for H, B and A, the new IIR state and both windows
#include "hci_internal.h"
#include "wave_ops.h"

namespace hci {

constexpr int kPfCG = 16;                  // channels per workgroup
constexpr int kPfS = 16;                   // positions per sub-chunk (outputs per thread)
constexpr int kPfSub = 16;                 // sub-chunks per chunk
constexpr int kPfC = kPfS * kPfSub;        // positions per chunk
constexpr int kPfT = kPfCG * kPfSub;       // threads per workgroup (channel, sub-chunk)
constexpr int kPfN = 16;                   // poles held in registers (N <= 16)

__host__ __device__ inline int pf_taps_padded(int To) { return (To + 15) / 16 * 16; }

__device__ __forceinline__ float powi(float x, int e) {      // x^e, e >= 0, by squaring
    float r = 1.f;
    while (e > 0) {
        if (e & 1) r *= x;
        x *= x;
        e >>= 1;
    }
    return r;
}


// LDS row pitches of the chunk kernel: f rows and sub-chunk states padded by one float, so that
// the four sub-chunks a wave serves (rows 16 apart) and the 16 channels of a state row fall in
// different banks
constexpr int kFbP = kPfCG + 1;
constexpr int kSeP = kPfN + 1;

size_t prefill_lds_bytes(int To) {
    const int Wp = pf_taps_padded(To) - 1;
    return ((size_t)(Wp + kPfC) * kFbP + (size_t)pf_taps_padded(To) * kPfCG + (size_t)kPfSub * kPfCG * kSeP) * 4;
}

constexpr int kScCh = 64;                  // channels per scan workgroup (32 lanes x 2 channels)
constexpr int kScSub = 8;                  // sub-chunks (threads along time) per scan chunk
constexpr int kScTs = 4;                   // short taps held in registers on the state path
constexpr int kScU = 8;                    // positions loaded ahead per step
constexpr int kScPad = kPfN + 1;           // LDS row pitch of the sub-chunk states

bool prefill_y_mfma(const hci_layer* L, int T);

// the folded state path: the state only, or the state next to the outputs y on the matrix cores
bool prefill_state_path(const hci_layer* L, int T, bool want_y) {
    return (!want_y || prefill_y_mfma(L, T)) && T >= L->taps_outer && L->taps_short <= kScTs && L->d % 2 == 0 &&
           L->poles <= kPfN;
}

size_t prefill_state_lds_bytes(const hci_layer* L) {
    const size_t rows = 2 * (size_t)(L->taps_outer - 1) + (size_t)(L->taps_short - 1);
    return rows * kPfCG * 4 + 16;
}

PrefillPlan plan_prefill(const hci_layer* L, int nb, int T, bool want_y) {
    PrefillPlan p{};
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    if (prefill_state_path(L, T, want_y)) {
        p.state_only = true;
        p.y_mfma = want_y;
        const int M = T - L->taps_outer + 1;
        const long long ncg = (L->d + kScCh - 1) / kScCh;
        long long want = (4096 + ncg * nb - 1) / (ncg * nb);
        want = want < 1 ? 1 : (want > 256 ? 256 : want);
        long long sub = (M + want * kScSub - 1) / (want * kScSub);
        sub = (sub + kScU - 1) / kScU * kScU;
        if (sub < 2 * kScU) sub = 2 * kScU;
        p.sub_len = (int)sub;
        p.chunk_len = (int)(sub * kScSub);
        p.nchunks = (int)((M + p.chunk_len - 1) / p.chunk_len);
        p.s_elems = (size_t)nb * p.nchunks * L->d * kPfN;
        p.bytes = up(p.s_elems * 4);
        return p;
    }
    p.nchunks = (T + kPfC - 1) / kPfC;
    p.s_elems = (size_t)nb * p.nchunks * L->d * kPfN;
    p.ftail_elems = (size_t)nb * (L->taps_outer - 1 > 0 ? L->taps_outer - 1 : 1) * L->d;
    p.yloc_elems = want_y ? (size_t)nb * T * L->d : 0;
    p.bytes = up(p.s_elems * 4) + up(p.ftail_elems * 4) + up(p.yloc_elems * 4);
    return p;
}

template <int ACT>
__global__ __launch_bounds__(kPfT) void k_prefill_local(
    const float* __restrict__ w_short, const float* __restrict__ w_outer,
    const float* __restrict__ lam, const float* __restrict__ beta, const float* __restrict__ cc,
    const typename Act<ACT>::T* __restrict__ short_win, const float* __restrict__ outer_win,
    const typename Act<ACT>::T* __restrict__ x, float* __restrict__ s_loc, float* __restrict__ f_tail,
    float* __restrict__ y_loc, int d, int Ts, int To, int N, int T, int nchunks)
{
    extern __shared__ float lds[];
    const int TP = pf_taps_padded(To);
    const int W = To - 1, Wp = TP - 1;
    float* fb = lds;                               // [Wp + C][kFbP]: row r holds fbar[t0 - Wp + r]
    float* wl = fb + (size_t)(Wp + kPfC) * kFbP;   // [TP][16], zero past To
    float* se = wl + (size_t)TP * kPfCG;           // [sub][16 ch][kSeP]: sub-chunk states

    const int cg = blockIdx.x, chunk = blockIdx.y, b = blockIdx.z;
    const int ch0 = cg * kPfCG;
    const int t0 = chunk * kPfC;
    const int tid = threadIdx.x;
    const typename Act<ACT>::T* xb = x + (size_t)b * T * d;
    const typename Act<ACT>::T* sw = short_win + (size_t)b * (Ts - 1) * d;
    const float* ow = outer_win + (size_t)b * W * d;

    // short FIR over the chunk and its halo: fbar[t] for t in [t0 - Wp, t0 + C).  Thread (c, q)
    // takes the contiguous rows [q R, q R + R) in order, its previous Ts - 1 inputs in registers,
    // so x is loaded once per row (up to kScTs short taps; longer filters load every tap).
    {
        const int rows = Wp + kPfC, R = (rows + kPfSub - 1) / kPfSub;
        const int c = tid % kPfCG, q = tid / kPfCG, ch = ch0 + c;
        const bool live = ch < d;
        const int r0 = q * R, r1 = min(r0 + R, rows);
        // xbar(m): the short-FIR input at position m (the committed short window before the prompt)
        auto xbar = [&](int m) -> float {
            if (!live || m >= T || m < -(Ts - 1)) return 0.f;
            return m >= 0 ? Act<ACT>::load(xb, (size_t)m * d + ch) : Act<ACT>::load(sw, (size_t)(Ts - 1 + m) * d + ch);
        };
        auto emit = [&](int r, int t, float v) {
            if (live && r >= Wp && t >= T - W && t < T) f_tail[((size_t)b * W + (t - (T - W))) * d + ch] = v;
            fb[r * kFbP + c] = v;
        };
        if (Ts <= kScTs) {
            float ws_[kScTs], xw[kScTs];               // xw[j] = xbar(t - j) for the running t
#pragma unroll
            for (int j = 0; j < kScTs; ++j) ws_[j] = live && j < Ts ? w_short[(size_t)j * d + ch] : 0.f;
#pragma unroll
            for (int j = 1; j < kScTs; ++j) xw[j] = j < Ts ? xbar(t0 - Wp + r0 - j) : 0.f;
            for (int r = r0; r < r1; ++r) {
                const int t = t0 - Wp + r;
                xw[0] = xbar(t);
                float v = 0.f;
                if (t < 0) {
                    v = live && t >= -W ? ow[(size_t)(W + t) * d + ch] : 0.f;     // committed outer-FIR inputs
                } else if (t < T) {
#pragma unroll
                    for (int j = 0; j < kScTs; ++j)
                        if (j < Ts) v = fmaf(ws_[j], xw[j], v);
                }
                emit(r, t, v);
#pragma unroll
                for (int j = kScTs - 1; j > 0; --j) xw[j] = xw[j - 1];
            }
        } else {
            for (int r = r0; r < r1; ++r) {
                const int t = t0 - Wp + r;
                float v = 0.f;
                if (t < 0) {
                    v = live && t >= -W ? ow[(size_t)(W + t) * d + ch] : 0.f;
                } else if (t < T && live) {
                    for (int j = 0; j < Ts; ++j) v = fmaf(w_short[(size_t)j * d + ch], xbar(t - j), v);
                }
                emit(r, t, v);
            }
        }
    }
    for (int e = tid; e < TP * kPfCG; e += kPfT) {
        const int j = e / kPfCG, c = e % kPfCG, ch = ch0 + c;
        wl[e] = (j < To && ch < d) ? w_outer[(size_t)j * d + ch] : 0.f;
    }
    __syncthreads();

    // outer FIR: thread (c, sub) computes g for its 16 positions, taps in blocks of 16:
    // R[m] = fbar[tau0 - jb - 15 + m], then g[tau] += w[jb+u] * R[tau - u + 15]
    const int c = tid % kPfCG, sub = tid / kPfCG;
    const int ch = ch0 + c;
    const int tau0 = sub * kPfS;
    float g[kPfS];
#pragma unroll
    for (int i = 0; i < kPfS; ++i) g[i] = 0.f;
    for (int jb = 0; jb < TP; jb += 16) {
        float R[31];
        const int base = Wp + tau0 - jb - 15;      // fb row of R[0]
#pragma unroll
        for (int m = 0; m < 31; ++m) R[m] = fb[(base + m) * kFbP + c];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const float w = wl[(jb + u) * kPfCG + c];
#pragma unroll
            for (int i = 0; i < kPfS; ++i) g[i] = fmaf(w, R[i - u + 15], g[i]);
        }
    }

    // sub-chunk scan from a zero state, all poles in registers
    float lm[kPfN], bt[kPfN], cv[kPfN], s[kPfN];
#pragma unroll
    for (int n = 0; n < kPfN; ++n) {
        const bool ok = n < N && ch < d;
        const size_t o = (size_t)ch * N + n;
        lm[n] = ok ? lam[o] : 0.f;
        bt[n] = ok ? beta[o] : 0.f;
        cv[n] = ok ? cc[o] : 0.f;
        s[n] = 0.f;
    }
    const int valid = max(0, min(kPfS, T - (t0 + tau0)));       // positions of this sub-chunk inside the prompt
    float y[kPfS];
#pragma unroll
    for (int i = 0; i < kPfS; ++i) {
        float acc = 0.f;
        if (i < valid) {
#pragma unroll
            for (int n = 0; n < kPfN; ++n) {
                s[n] = fmaf(lm[n], s[n], bt[n] * g[i]);
                acc = fmaf(cv[n], s[n], acc);
            }
        }
        y[i] = acc;
    }
#pragma unroll
    for (int n = 0; n < kPfN; ++n) se[((size_t)sub * kPfCG + c) * kSeP + n] = s[n];
    __syncthreads();

    // in-chunk carry: thread (channel c2, pole n2) turns the 16 sub-chunk end states into start states
    {
        const int c2 = tid / kPfN, n2 = tid % kPfN, ch2 = ch0 + c2;
        const float l2 = (n2 < N && ch2 < d) ? lam[(size_t)ch2 * N + n2] : 0.f;
        float S = 0.f;
        for (int sb = 0; sb < kPfSub; ++sb) {
            const int len = max(0, min(kPfS, T - (t0 + sb * kPfS)));
            const float e = se[((size_t)sb * kPfCG + c2) * kSeP + n2];
            se[((size_t)sb * kPfCG + c2) * kSeP + n2] = S;                 // start state of sub-chunk sb
            S = fmaf(powi(l2, len), S, e);
        }
        if (ch2 < d) s_loc[(((size_t)b * nchunks + chunk) * d + ch2) * kPfN + n2] = S;   // chunk end (local)
    }
    __syncthreads();

    // chunk-local readouts: add the decayed sub-chunk start state
    if (y_loc != nullptr && ch < d) {
        float p[kPfN];
#pragma unroll
        for (int n = 0; n < kPfN; ++n) p[n] = se[((size_t)sub * kPfCG + c) * kSeP + n];
#pragma unroll
        for (int i = 0; i < kPfS; ++i) {
            if (i < valid) {
                float acc = 0.f;
#pragma unroll
                for (int n = 0; n < kPfN; ++n) {
                    p[n] *= lm[n];
                    acc = fmaf(cv[n], p[n], acc);
                }
                y_loc[((size_t)b * T + t0 + tau0 + i) * d + ch] = y[i] + acc;
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_prefill_carry(
    const float* __restrict__ lam, float* __restrict__ iir, float* __restrict__ s_loc,
    const int32_t* __restrict__ kv_len, int d, int N, int T, int nchunks, int nb, int lim)
{
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;   // (b, ch, n), n fastest
    if (e >= (size_t)nb * d * kPfN) return;
    const int n = (int)(e % kPfN);
    const int ch = (int)((e / kPfN) % d);
    const int b = (int)(e / ((size_t)kPfN * d));
    if (n >= N) return;
    const float l = lam[(size_t)ch * N + n];
    const float pc = powi(l, kPfC);                          // lambda^C for full chunks
    float S = iir[((size_t)b * d + ch) * N + n];
    float* sp = s_loc + ((size_t)b * nchunks * d + ch) * kPfN + n;
    const size_t stride = (size_t)d * kPfN;
    for (int k = 0; k < nchunks; ++k) {
        const float end = sp[k * stride];
        sp[k * stride] = S;                                  // start state of chunk k
        const int len = min(kPfC, T - k * kPfC);
        S = fmaf(len < kPfC ? powi(l, len) : pc, S, end);
    }
    // committed IIR state after the prompt, unless the sequence's kv_len is out of contract (it
    // then keeps its state; the chunk start states above still serve its outputs y)
    const int L = kv_len[b];
    if (L >= 0 && L <= lim) iir[((size_t)b * d + ch) * N + n] = S;
}

template <int ACT>
__global__ __launch_bounds__(kPfT) void k_prefill_fixup(
    const float* __restrict__ lam, const float* __restrict__ cc, const float* __restrict__ s_loc,
    const float* __restrict__ y_loc, typename Act<ACT>::T* __restrict__ y, int d, int N, int T, int nchunks)
{
    const int cg = blockIdx.x, chunk = blockIdx.y, b = blockIdx.z;
    const int c = threadIdx.x % kPfCG, sub = threadIdx.x / kPfCG;
    const int ch = cg * kPfCG + c;
    if (ch >= d) return;
    const int t0 = chunk * kPfC + sub * kPfS;
    const int valid = max(0, min(kPfS, T - t0));
    float p[kPfN], lm[kPfN], cv[kPfN];
#pragma unroll
    for (int n = 0; n < kPfN; ++n) {
        const bool ok = n < N;
        lm[n] = ok ? lam[(size_t)ch * N + n] : 0.f;
        cv[n] = ok ? cc[(size_t)ch * N + n] : 0.f;
        const float v = ok ? s_loc[(((size_t)b * nchunks + chunk) * d + ch) * kPfN + n] : 0.f;
        p[n] = v * powi(lm[n], sub * kPfS);                // decay to the sub-chunk start
    }
    for (int i = 0; i < valid; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int n = 0; n < kPfN; ++n) {
            p[n] *= lm[n];
            acc = fmaf(cv[n], p[n], acc);
        }
        const size_t o = ((size_t)b * T + t0 + i) * d + ch;
        Act<ACT>::store(y, o, y_loc[o] + acc);
    }
}

// FIR windows <- last inputs of the prompt: new[r] = concat(old, rows)[T + r]
template <int ACT>
__global__ __launch_bounds__(256) void k_prefill_commit(
    typename Act<ACT>::T* __restrict__ short_win, float* __restrict__ outer_win,
    const typename Act<ACT>::T* __restrict__ x, const float* __restrict__ f_tail, const int32_t* __restrict__ kv_len,
    int d, int Ts, int To, int T, int lim)
{
    const int b = blockIdx.y;
    const int ch = blockIdx.x * blockDim.x + threadIdx.x;
    const int L = kv_len[b];
    if (ch >= d || L < 0 || L > lim) return;       // out-of-contract kv_len: the windows are kept
    // every thread owns one channel column, rows ascending: new row r reads row T + r > r of the
    // concatenation, which this thread has not written yet
    const int Ws = Ts - 1;
    typename Act<ACT>::T* sw = short_win + (size_t)b * Ws * d;
    for (int r = 0; r < Ws; ++r) {
        const long long m = (long long)T + r;
        const float v = (m < Ws) ? Act<ACT>::load(sw, (size_t)m * d + ch)
                                 : Act<ACT>::load(x, ((size_t)b * T + (size_t)(m - Ws)) * d + ch);
        Act<ACT>::store(sw, (size_t)r * d + ch, v);
    }
    const int W = To - 1;
    float* ow = outer_win + (size_t)b * W * d;
    for (int r = 0; r < W; ++r) {
        const long long m = (long long)T + r;
        const float v = (m < W) ? ow[(size_t)m * d + ch] : f_tail[((size_t)b * W + r) * d + ch];
        ow[(size_t)r * d + ch] = v;
    }
}

// ------------------------------------------------------------ state path

template <int ACT> struct PairLoad;
template <> struct PairLoad<HCI_BF16> {       // two consecutive bf16 channels
    __device__ static __forceinline__ void get(const uint16_t* p, float& a, float& b) {
        const uint32_t w = __builtin_nontemporal_load((const uint32_t*)p);
        a = __uint_as_float(w << 16);
        b = __uint_as_float(w & 0xffff0000u);
    }
};
template <> struct PairLoad<HCI_F32> {
    __device__ static __forceinline__ void get(const float* p, float& a, float& b) {
        a = __builtin_nontemporal_load(p);
        b = __builtin_nontemporal_load(p + 1);
    }
};

// V over the chunk's positions from a zero start, per (channel, pole).
// Thread (cp, sub) owns channels ch, ch+1 and sub_len consecutive positions.
template <int ACT>
__global__ __launch_bounds__(256) void k_prefill_scan(
    const float* __restrict__ w_short, const float* __restrict__ lam,
    const typename Act<ACT>::T* __restrict__ short_win, const typename Act<ACT>::T* __restrict__ x,
    float* __restrict__ e_out, int d, int Ts, int N, int T, int M, int sub_len, int nchunks)
{
    typedef typename Act<ACT>::T AT;
    __shared__ float es[kScSub * kScCh * kScPad];
    const int cg = blockIdx.x, chunk = blockIdx.y, b = blockIdx.z;
    const int cp = threadIdx.x % (kScCh / 2), sub = threadIdx.x / (kScCh / 2);
    const int ch = cg * kScCh + 2 * cp;                 // d is even, so ch + 1 < d whenever ch < d
    const bool live = ch < d;
    const int chunk_len = kScSub * sub_len;
    const int t_begin = chunk * chunk_len + sub * sub_len;
    const int t_end = min(t_begin + sub_len, M);
    const AT* xb = x + (size_t)b * T * d;
    const AT* sw = short_win + (size_t)b * (Ts - 1) * d;

    float wa[kScTs], wb[kScTs];
#pragma unroll
    for (int j = 0; j < kScTs; ++j) {
        wa[j] = (live && j < Ts) ? w_short[(size_t)j * d + ch] : 0.f;
        wb[j] = (live && j < Ts) ? w_short[(size_t)j * d + ch + 1] : 0.f;
    }
    float la[kPfN], lb[kPfN], sa[kPfN], sb[kPfN];
#pragma unroll
    for (int n = 0; n < kPfN; ++n) {
        la[n] = (live && n < N) ? lam[(size_t)ch * N + n] : 0.f;
        lb[n] = (live && n < N) ? lam[(size_t)(ch + 1) * N + n] : 0.f;
        sa[n] = 0.f;
        sb[n] = 0.f;
    }
    // xa[j] / xb_[j] = xbar[t - 1 - j]: the previous inputs of the running position t
    float xa[kScTs - 1], xq[kScTs - 1];
#pragma unroll
    for (int j = 0; j < kScTs - 1; ++j) {
        const int tp = t_begin - 1 - j;
        float va = 0.f, vb = 0.f;
        if (live && t_begin < t_end) {
            if (tp >= 0) {
                va = Act<ACT>::load(xb, (size_t)tp * d + ch);
                vb = Act<ACT>::load(xb, (size_t)tp * d + ch + 1);
            } else if (tp >= -(Ts - 1)) {
                va = Act<ACT>::load(sw, (size_t)(Ts - 1 + tp) * d + ch);
                vb = Act<ACT>::load(sw, (size_t)(Ts - 1 + tp) * d + ch + 1);
            }
        }
        xa[j] = va;
        xq[j] = vb;
    }

    auto step = [&](float ua, float ub) {
        float fa = wa[0] * ua, fb = wb[0] * ub;
#pragma unroll
        for (int j = 1; j < kScTs; ++j) {
            fa = fmaf(wa[j], xa[j - 1], fa);
            fb = fmaf(wb[j], xq[j - 1], fb);
        }
#pragma unroll
        for (int j = kScTs - 2; j > 0; --j) {
            xa[j] = xa[j - 1];
            xq[j] = xq[j - 1];
        }
        xa[0] = ua;
        xq[0] = ub;
#pragma unroll
        for (int n = 0; n < kPfN; ++n) {
            sa[n] = fmaf(la[n], sa[n], fa);
            sb[n] = fmaf(lb[n], sb[n], fb);
        }
    };

    if (live) {
        int t = t_begin;
        for (; t + kScU <= t_end; t += kScU) {
            float ua[kScU], ub[kScU];
#pragma unroll
            for (int u = 0; u < kScU; ++u) PairLoad<ACT>::get(xb + (size_t)(t + u) * d + ch, ua[u], ub[u]);
#pragma unroll
            for (int u = 0; u < kScU; ++u) step(ua[u], ub[u]);
        }
        for (; t < t_end; ++t) {
            float ua, ub;
            PairLoad<ACT>::get(xb + (size_t)t * d + ch, ua, ub);
            step(ua, ub);
        }
    }
#pragma unroll
    for (int n = 0; n < kPfN; ++n) {
        es[(sub * kScCh + 2 * cp) * kScPad + n] = sa[n];
        es[(sub * kScCh + 2 * cp + 1) * kScPad + n] = sb[n];
    }
    __syncthreads();
    // merge the sub-chunk states in time order: acc <- lam^len(sub) acc + state(sub)
    for (int e = threadIdx.x; e < kScCh * kPfN; e += blockDim.x) {
        const int c = e / kPfN, n = e % kPfN, chc = cg * kScCh + c;
        if (chc >= d) continue;
        const float l = n < N ? lam[(size_t)chc * N + n] : 0.f;
        const float l_full = powi(l, sub_len);
        float acc = 0.f;
        for (int q = 0; q < kScSub; ++q) {
            const int len = max(0, min(sub_len, M - (chunk * chunk_len + q * sub_len)));
            const float p = len == sub_len ? l_full : powi(l, len);
            acc = fmaf(p, acc, es[(q * kScCh + c) * kScPad + n]);
        }
        e_out[(((size_t)b * nchunks + chunk) * d + chc) * kPfN + n] = acc;
    }
}

// Carries, the tap pass and the commit, per 16 channels of one sequence.
template <int ACT>
__global__ __launch_bounds__(256) void k_prefill_state(
    const float* __restrict__ w_short, const float* __restrict__ w_outer, const float* __restrict__ lam,
    const float* __restrict__ beta, typename Act<ACT>::T* __restrict__ short_win, float* __restrict__ outer_win,
    float* __restrict__ iir, const typename Act<ACT>::T* __restrict__ x, const float* __restrict__ e_in,
    const int32_t* __restrict__ kv_len, int d, int Ts, int To, int N, int T, int M, int chunk_len, int nchunks,
    int lim)
{
    typedef typename Act<ACT>::T AT;
    extern __shared__ float lds[];
    {
        const int L = kv_len[blockIdx.y];
        if (L < 0 || L > lim) return;              // out-of-contract kv_len: the state is kept (reported later)
    }
    const int W = To - 1, Ws = Ts - 1;
    float* ft = lds;                       // [W][16]  f at positions T-W .. T-1
    float* ow = ft + (size_t)W * kPfCG;    // [W][16]  committed outer window, oldest first
    float* sw = ow + (size_t)W * kPfCG;    // [Ws][16] committed short window, oldest first
    const int cg = blockIdx.x, b = blockIdx.y, ch0 = cg * kPfCG;
    const AT* xb = x + (size_t)b * T * d;
    AT* swg = short_win + (size_t)b * Ws * d;
    float* owg = outer_win + (size_t)b * W * d;

    for (int e = threadIdx.x; e < Ws * kPfCG; e += blockDim.x) {
        const int r = e / kPfCG, ch = ch0 + e % kPfCG;
        sw[e] = ch < d ? Act<ACT>::load(swg, (size_t)r * d + ch) : 0.f;
    }
    for (int e = threadIdx.x; e < W * kPfCG; e += blockDim.x) {
        const int r = e / kPfCG, ch = ch0 + e % kPfCG;
        ow[e] = ch < d ? owg[(size_t)r * d + ch] : 0.f;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < W * kPfCG; e += blockDim.x) {
        const int r = e / kPfCG, c = e % kPfCG, ch = ch0 + c;
        const int t = T - W + r;                     // >= 1 because T >= To
        float f = 0.f;
        if (ch < d) {
            for (int j = 0; j < Ts; ++j) {
                const int m = t - j;
                const float xv = m >= 0 ? Act<ACT>::load(xb, (size_t)m * d + ch) : sw[(Ws + m) * kPfCG + c];
                f = fmaf(w_short[(size_t)j * d + ch], xv, f);
            }
        }
        ft[e] = f;
    }
    __syncthreads();

    {
        const int c = threadIdx.x / kPfN, n = threadIdx.x % kPfN, ch = ch0 + c;
        if (ch < d && n < N) {
            const size_t o = (size_t)ch * N + n;
            const float l = lam[o];
            const float l_chunk = powi(l, chunk_len);
            float V = 0.f;
            const float* ep = e_in + ((size_t)b * nchunks * d + ch) * kPfN + n;
#pragma unroll 8
            for (int k = 0; k < nchunks; ++k) {
                const int len = min(chunk_len, M - k * chunk_len);
                const float p = len == chunk_len ? l_chunk : powi(l, len);
                V = fmaf(p, V, ep[(size_t)k * d * kPfN]);
            }
            float P = 0.f, B = 0.f, pa = 1.f, R = 0.f, A = 0.f;
            for (int j = 0; j <= W; ++j) {
                const float w = w_outer[(size_t)j * d + ch];
                P = fmaf(P, l, w);                                        // P_j
                if (j < W) B = fmaf(ft[(W - 1 - j) * kPfCG + c], P, B);   // f_{T-1-j} P_j
                if (j >= 1) {
                    pa *= l;                                              // lam^j
                    R = fmaf(ow[(W - j) * kPfCG + c], pa, R);             // R_j = sum_{a<=j} fbar_{-a} lam^a
                    A = fmaf(A, l, w * R);                                // Horner: sum_j w_j R_j lam^(W-j)
                }
            }
            const float bt = beta[o];
            const float l_to = pa * l;                                    // lam^To
            const float l_rest = powi(l, T - To);
            float* sp = iir + (size_t)b * d * N + o;
            *sp = fmaf(l_rest, fmaf(l_to, *sp, bt * A), bt * fmaf(P, V, B));
        }
    }

    // windows: every read of the committed windows went to LDS above
    for (int e = threadIdx.x; e < W * kPfCG; e += blockDim.x) {
        const int r = e / kPfCG, ch = ch0 + e % kPfCG;
        if (ch < d) owg[(size_t)r * d + ch] = ft[e];
    }
    for (int e = threadIdx.x; e < Ws * kPfCG; e += blockDim.x) {
        const int r = e / kPfCG, c = e % kPfCG, ch = ch0 + c;
        if (ch >= d) continue;
        const int m = T + r;                         // row of [window ; x] that becomes row r
        const float v = m < Ws ? sw[m * kPfCG + c] : Act<ACT>::load(xb, (size_t)(m - Ws) * d + ch);
        Act<ACT>::store(swg, (size_t)r * d + ch, v);
    }
}

// ------------------------------------------------------------ outputs y on the matrix cores
//
// With bf16 activations the prompt's outputs y come from one pass per 16
// channels over the whole prompt, in tiles of 256 positions (16 blocks of 16),
// the IIR state carried from tile to tile in registers; the committed state
// itself is left to the folded state path, which runs afterwards.  Per channel
// and tile (block n, position i inside a block, pole p):
//   g[16n+i] = sum_k Wt[i][k] F[k][n],  F[k][n] = f[t0+16n-Wh+k],  Wt[i][k] = w[i+Wh-k]
//              (the outer FIR as a Toeplitz product over a window of Wh+16 inputs)
//   E[p][n]  = sum_m beta_p lam_p^(15-m) g[16n+m]      block n's inputs, at its end
//   sig_n    = lam^(16n) sig_0 + sum_{k<n} lam^(16(n-1-k)) E[.][k]   state before block n
//   y[16n+i] = sum_{m<=i} h[i-m] g[16n+m] + sum_p c_p lam_p^(i+1) sig_n[p],
//              h[k] = sum_p c_p beta_p lam_p^k
// The products run on v_mfma (16x16x32 bf16 for the FIR, 16x16x16 bf16 for the
// others) with every fp32 operand split into two bf16 terms (hi + lo) and the
// lo x lo term dropped, so each sum carries a relative error of about 2^-14 of
// the magnitudes of its terms before y is rounded to bf16.  In the accumulator
// layout lane (q, n) holds rows 4q..4q+3 of column n, which is also the B-operand
// layout of the 16x16x16 products: g and the states feed the next product in
// place, and the scan over the 16 blocks runs across the 16 lanes of a row.

constexpr int kYC = 16;                    // channels per workgroup
constexpr int kYW = 8;                     // waves; wave w owns channels 2w and 2w + 1
constexpr int kYT = 64 * kYW;
constexpr int kYTile = 256;                // positions per tile
constexpr int kYH = kScTs - 1;             // x rows kept before the tile (short FIR history)
constexpr int kYKs = 5;                    // FIR window steps of 32 inputs at most (To <= 144)
constexpr int kYysP = kYTile + 4;          // LDS pitch of the staged outputs (floats)

typedef short s16x4 __attribute__((ext_vector_type(4)));

__host__ __device__ inline int y_halo(int To) { return (To - 1 + 7) / 8 * 8; }     // Wh: >= To - 1, multiple of 8
__host__ __device__ inline int y_ksteps(int To) { return (y_halo(To) + 16 + 31) / 32; }
__host__ __device__ inline int y_ring(int To) { return y_halo(To) + kYTile; }       // f ring length (positions)
// ring row pitch: 16 bytes past the length, so that the 16 channel rows start in different banks
__host__ __device__ inline int y_ring_pitch(int To) { return y_ring(To) + 8; }

size_t prefill_y_lds_bytes(int To) {
    return (size_t)(kYH + kYTile) * kYC * 2 + (size_t)2 * kYC * y_ring_pitch(To) * 2 + (size_t)kYC * kYysP * 4;
}

bool prefill_y_mfma(const hci_layer* L, int T) {
    return L->act_dtype == HCI_BF16 && L->d % 8 == 0 && y_ksteps(L->taps_outer) <= kYKs && T >= L->taps_outer &&
           L->taps_short <= kScTs && L->poles <= kPfN;
}

__device__ __forceinline__ double powi_d(double x, int e) {
    double r = 1.0;
    while (e > 0) {
        if (e & 1) r *= x;
        x *= x;
        e >>= 1;
    }
    return r;
}

// v = hi + lo in bf16 (round to nearest even twice)
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
    hi = f2bf(v);
    lo = f2bf(v - bf2f(hi));
}
__device__ __forceinline__ void split_bf16_d(double v, uint16_t& hi, uint16_t& lo) {
    hi = f2bf((float)v);
    lo = f2bf((float)(v - (double)bf2f(hi)));
}

typedef float pf_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 pf_bf16x2 __attribute__((ext_vector_type(2)));

// two fp32 values -> two bf16 (round to nearest even, one v_cvt_pk_bf16_f32), a in the low half
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    const pf_f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, pf_bf16x2));
}
// the split of two values: hi = bf16(v), lo = bf16(v - hi), packed in pairs
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = pk_bf16(a, b);
    lo = pk_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int KS>
__global__ __launch_bounds__(kYT) void k_prefill_y(
    const float* __restrict__ w_short, const float* __restrict__ w_outer, const float* __restrict__ lam,
    const float* __restrict__ beta, const float* __restrict__ cc, const uint16_t* __restrict__ short_win,
    const float* __restrict__ outer_win, const float* __restrict__ iir, const uint16_t* __restrict__ x,
    uint16_t* __restrict__ y, int d, int Ts, int To, int N, int T, int ncg, int nb)
{
    extern __shared__ __align__(16) unsigned char ylds[];
    const int Wh = y_halo(To), RL = y_ring(To), RP = y_ring_pitch(To), W = To - 1;
    uint16_t* xs = (uint16_t*)ylds;                        // [kYH + 256][16]: x at t0 - kYH ..
    uint16_t* fh = xs + (kYH + kYTile) * kYC;              // [16][RP]: f, bf16 hi terms, ring
    uint16_t* fl = fh + kYC * RP;                          // [16][RP]: lo terms
    float* ys = (float*)(fl + kYC * RP);                   // [16][kYysP]: outputs of the tile

    // neighbouring channel groups on one XCD (workgroups are dealt to the 8 XCDs in turn), so
    // that the 32-byte row pieces of x and y of adjacent groups meet in one L2
    const int total = ncg * nb;
    int wg = blockIdx.x;
    if (total % 8 == 0) wg = (wg % 8) * (total / 8) + wg / 8;
    const int cg = wg % ncg, b = wg / ncg, ch0 = cg * kYC;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const uint16_t* xb = x + (size_t)b * T * d;
    uint16_t* yb = y + (size_t)b * T * d;

    // ---- per-channel operands of the wave's two channels
    bf16x8 Ah[2][KS], Al[2][KS];                   // Toeplitz FIR operand: lane (i, q) holds Wt[i][32s + 8q + e]
    s16x4 Bh[2], Bl[2], Hh[2], Hl[2], Chh[2], Cl[2];
    f32x4 L1[2], Ln[2], sig[2];                    // lane (q, n): poles 4q + r
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int ch = ch0 + 2 * wv + u;
        const bool live = ch < d;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint16_t h8[8], l8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = li + Wh - (32 * s + 8 * lq + e);
                const float w = (live && j >= 0 && j < To) ? w_outer[(size_t)j * d + ch] : 0.f;
                split_bf16(w, h8[e], l8[e]);
            }
            uint4 ph, pl;
            ph.x = h8[0] | ((uint32_t)h8[1] << 16); ph.y = h8[2] | ((uint32_t)h8[3] << 16);
            ph.z = h8[4] | ((uint32_t)h8[5] << 16); ph.w = h8[6] | ((uint32_t)h8[7] << 16);
            pl.x = l8[0] | ((uint32_t)l8[1] << 16); pl.y = l8[2] | ((uint32_t)l8[3] << 16);
            pl.z = l8[4] | ((uint32_t)l8[5] << 16); pl.w = l8[6] | ((uint32_t)l8[7] << 16);
            Ah[u][s] = __builtin_bit_cast(bf16x8, ph);
            Al[u][s] = __builtin_bit_cast(bf16x8, pl);
        }
        const float* lp = lam + (size_t)ch * N;
        const float* bp = beta + (size_t)ch * N;
        const float* cp = cc + (size_t)ch * N;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 4 * lq + e;              // operand column
            double bl = 0.0, hv = 0.0, cv = 0.0;
            if (live && li < N) bl = (double)bp[li] * powi_d(lp[li], 15 - m);           // [p = li][m]
            if (live && m <= li)                                                         // [i = li][m]
                for (int p = 0; p < N; ++p) hv += (double)cp[p] * bp[p] * powi_d(lp[p], li - m);
            if (live && m < N) cv = (double)cp[m] * powi_d(lp[m], li + 1);             // [i = li][p = m]
            uint16_t h, l;
            split_bf16_d(bl, h, l); Bh[u][e] = (short)h; Bl[u][e] = (short)l;
            split_bf16_d(hv, h, l); Hh[u][e] = (short)h; Hl[u][e] = (short)l;
            split_bf16_d(cv, h, l); Chh[u][e] = (short)h; Cl[u][e] = (short)l;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int p = 4 * lq + r;
            const bool ok = live && p < N;
            const double l = ok ? (double)lp[p] : 0.0;
            L1[u][r] = (float)powi_d(l, 16);
            Ln[u][r] = (float)powi_d(l, 16 * li);
            sig[u][r] = ok ? iir[((size_t)b * d + ch) * N + p] : 0.f;
        }
    }

    // ---- LDS: x history (the committed short window before the prompt), f ring (the committed
    // outer window at positions -W .. -1, zeros elsewhere); ring slot of position t: (t + Wh) mod RL
    for (int e = tid; e < kYH * kYC; e += kYT) {
        const int t = e / kYC - kYH, ch = ch0 + e % kYC;
        xs[e] = (ch < d && t >= -(Ts - 1)) ? short_win[((size_t)b * (Ts - 1) + (Ts - 1 + t)) * d + ch] : (uint16_t)0;
    }
    for (int e = tid; e < kYC * RP; e += kYT) {
        const int t = e % RP - Wh, ch = ch0 + e / RP;
        const float v = (ch < d && t < 0 && t >= -W) ? outer_win[((size_t)b * W + (W + t)) * d + ch] : 0.f;
        uint16_t h, l;
        split_bf16(v, h, l);
        fh[e] = h;
        fl[e] = l;
    }

    // x rows of a tile: thread (row, half) loads channels 8 half .. 8 half + 7 of one row.  Loads
    // and output stores run unconditionally, so that the compiler can count them in flight: a
    // row past the prompt reads row T - 1 (x there only reaches outputs past the prompt: both
    // filters are causal) and writes row T - 1's outputs, a half past d takes half 0 (same data,
    // same values written twice; d % 8 == 0, so a half lies wholly inside or outside)
    const int xrow = tid >> 1, xhalf = (ch0 + 8 * (tid & 1) < d) ? (tid & 1) : 0;
    auto load_x = [&](int t0) -> uint4 {
        const int t = min(t0 + xrow, T - 1);
        return load_nt((const uint4*)(xb + (size_t)t * d + ch0 + 8 * xhalf));
    };
    *(uint4*)(xs + (kYH + xrow) * kYC + 8 * xhalf) = load_x(0);
    // tiles t + 1 and t + 2 in flight in two register sets with fixed roles (a copy from one
    // set to the other would wait for the load)
    uint4 xq1 = load_x(kYTile), xq2 = load_x(2 * kYTile);

    // short FIR: thread (ac, ablk) makes positions 8 ablk .. 8 ablk + 7 of channel ac
    const int ac = tid & 15, ablk = tid >> 4;
    float wsr[kScTs];
#pragma unroll
    for (int j = 0; j < kScTs; ++j) wsr[j] = (ch0 + ac < d && j < Ts) ? w_short[(size_t)j * d + ch0 + ac] : 0.f;

    const int ntiles = (T + kYTile - 1) / kYTile;
    int base = 0;                                  // t0 mod RL
    // ring slot of window row 8 lq of block li in the current tile, reduced mod RL
    int rs = 16 * li + 8 * lq;
    if (rs >= RL) rs -= RL;                        // RL >= 256, rs < 264
    // body of one tile; xn holds the next tile's x rows and is refilled with the rows 3 tiles ahead
    auto tile_step = [&](int tile, uint4& xn) {
        const int t0 = tile * kYTile;
        // A: f of the tile into the ring, split into bf16 terms
        {
            float xv[8 + kYH];
#pragma unroll
            for (int k = 0; k < 8 + kYH; ++k) xv[k] = bf2f(xs[(8 * ablk + k) * kYC + ac]);
            float fv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float f = 0.f;
#pragma unroll
                for (int j = 0; j < kScTs; ++j) f = fmaf(wsr[j], xv[kYH + e - j], f);
                fv[e] = f;
            }
            int sl = base + Wh + 8 * ablk;
            if (sl >= RL) sl -= RL;
            uint4 ph, pl;
            split2(fv[0], fv[1], ph.x, pl.x);
            split2(fv[2], fv[3], ph.y, pl.y);
            split2(fv[4], fv[5], ph.z, pl.z);
            split2(fv[6], fv[7], ph.w, pl.w);
            *(uint4*)(fh + ac * RP + sl) = ph;
            *(uint4*)(fl + ac * RP + sl) = pl;
        }
        __syncthreads();

        // B: the wave's two channels through the four products
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = 2 * wv + u;
            f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0;
            // window rows past Wh + 15 meet only zero taps; they read ring slots of other positions,
            // finite unless an earlier input was not (and then every later output is not either)
            int sl = rs;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const uint4 vh = *(const uint4*)(fh + c * RP + sl);
                const uint4 vl = *(const uint4*)(fl + c * RP + sl);
                sl += 32;
                if (sl >= RL) sl -= RL;
                const bf16x8 bh = __builtin_bit_cast(bf16x8, vh), bl = __builtin_bit_cast(bf16x8, vl);
                a1 = mfma32(Ah[u][s], bl, a1);
                a2 = mfma32(Al[u][s], bh, a2);
                a0 = mfma32(Ah[u][s], bh, a0);
            }
            uint2 gh2, gl2;
            split2(a0[0] + (a1[0] + a2[0]), a0[1] + (a1[1] + a2[1]), gh2.x, gl2.x);
            split2(a0[2] + (a1[2] + a2[2]), a0[3] + (a1[3] + a2[3]), gh2.y, gl2.y);
            const s16x4 gh = __builtin_bit_cast(s16x4, gh2), gl = __builtin_bit_cast(s16x4, gl2);
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            f32x4 E = mfma16(Bh[u], gl, z);
            E = mfma16(Bl[u], gh, E);
            E = mfma16(Bh[u], gh, E);
            // inclusive scan over the blocks: I_n = sum_{k<=n} lam^(16(n-k)) E_k
            f32x4 I = E, Lp = L1[u];
#pragma unroll
            for (int r = 0; r < 4; ++r) I[r] = fmaf(Lp[r], dpp_f32<kRowShr1>(I[r]), I[r]);
            Lp *= Lp;
#pragma unroll
            for (int r = 0; r < 4; ++r) I[r] = fmaf(Lp[r], dpp_f32<kRowShr2>(I[r]), I[r]);
            Lp *= Lp;
#pragma unroll
            for (int r = 0; r < 4; ++r) I[r] = fmaf(Lp[r], dpp_f32<kRowShr4>(I[r]), I[r]);
            Lp *= Lp;
#pragma unroll
            for (int r = 0; r < 4; ++r) I[r] = fmaf(Lp[r], dpp_f32<kRowShr8>(I[r]), I[r]);
            Lp *= Lp;                              // lam^256
            float sg[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sg[r] = fmaf(Ln[u][r], sig[u][r], dpp_f32<kRowShr1>(I[r]));           // state before block n
                const float i15 = __int_as_float(__builtin_amdgcn_ds_bpermute((lq * 16 + 15) * 4, __float_as_int(I[r])));
                sig[u][r] = fmaf(Lp[r], sig[u][r], i15);                                // state after the tile
            }
            uint2 sh2, sl2;
            split2(sg[0], sg[1], sh2.x, sl2.x);
            split2(sg[2], sg[3], sh2.y, sl2.y);
            const s16x4 sh_ = __builtin_bit_cast(s16x4, sh2), sl_ = __builtin_bit_cast(s16x4, sl2);
            f32x4 Y = mfma16(Hh[u], gl, z);
            Y = mfma16(Hl[u], gh, Y);
            Y = mfma16(Chh[u], sl_, Y);
            Y = mfma16(Cl[u], sh_, Y);
            Y = mfma16(Hh[u], gh, Y);
            Y = mfma16(Chh[u], sh_, Y);
            *(f32x4*)(ys + c * kYysP + 16 * li + 4 * lq) = Y;
        }
        __syncthreads();

        // C: outputs of the tile (rows of 8 channels, bf16), the x history for the next tile
        {
            const int t = min(t0 + xrow, T - 1);
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = ys[(8 * xhalf + e) * kYysP + (t - t0)];
            uint4 pk;
            pk.x = pk_bf16(o[0], o[1]);
            pk.y = pk_bf16(o[2], o[3]);
            pk.z = pk_bf16(o[4], o[5]);
            pk.w = pk_bf16(o[6], o[7]);
            *(uint4*)(yb + (size_t)t * d + ch0 + 8 * xhalf) = pk;
        }
        uint4 hist = make_uint4(0u, 0u, 0u, 0u);
        if (tid < 2 * kYH) hist = *(const uint4*)(xs + (kYTile + (tid >> 1)) * kYC + 8 * (tid & 1));
        __syncthreads();
        if (tid < 2 * kYH) *(uint4*)(xs + (tid >> 1) * kYC + 8 * (tid & 1)) = hist;
        *(uint4*)(xs + (kYH + xrow) * kYC + 8 * xhalf) = xn;
        xn = load_x(t0 + 3 * kYTile);
        base += kYTile;
        if (base >= RL) base -= RL;
        rs += kYTile;
        if (rs >= RL) rs -= RL;
        __syncthreads();
    };
    // every load issued so far has landed before the loop: registers loaded above and used in
    // the loop (taps, states) then leave no wait at the loop head, which would also wait for the
    // prefetched tiles on every pass
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();                               // the LDS set-up above is complete
    // pairs of tiles with no branch between them (the count of loads and stores in flight is
    // then the same on every path into a wait), an odd last tile after the loop
    int tile = 0;
    for (; tile + 1 < ntiles; tile += 2) {
        tile_step(tile, xq1);
        tile_step(tile + 1, xq2);
    }
    if (tile < ntiles) tile_step(tile, xq1);
}

template <int KS>
static hipError_t launch_y_ks(const hci_layer* L, const hci_state* S, int nb, int T, const uint16_t* x, uint16_t* y,
                              hipStream_t st)
{
    const int d = L->d, ncg = (d + kYC - 1) / kYC;
    const size_t lds = prefill_y_lds_bytes(L->taps_outer);
    hipError_t e;
    if (lds > 65536 && (e = hipFuncSetAttribute((const void*)k_prefill_y<KS>,
                                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_prefill_y<KS>, dim3((unsigned)(ncg * nb)), dim3(kYT), lds, st, L->w_short, L->w_outer,
                       L->lambda, L->beta, L->c, (const uint16_t*)S->short_win, S->outer_win, S->iir, x, y, d,
                       L->taps_short, L->taps_outer, L->poles, T, ncg, nb);
    return hipGetLastError();
}

static hipError_t launch_y_mfma(const hci_layer* L, const hci_state* S, int nb, int T, const void* x, void* y,
                                hipStream_t st)
{
    const uint16_t* xa = (const uint16_t*)x;
    uint16_t* ya = (uint16_t*)y;
    switch (y_ksteps(L->taps_outer)) {
        case 1: return launch_y_ks<1>(L, S, nb, T, xa, ya, st);
        case 2: return launch_y_ks<2>(L, S, nb, T, xa, ya, st);
        case 3: return launch_y_ks<3>(L, S, nb, T, xa, ya, st);
        case 4: return launch_y_ks<4>(L, S, nb, T, xa, ya, st);
        case 5: return launch_y_ks<5>(L, S, nb, T, xa, ya, st);
        default: return hipErrorInvalidValue;
    }
}

// K/V rows at kv_len .. kv_len+T-1 of every sequence, then the lengths
static hipError_t append_kv(const hci_layer* L, const hci_state* S, int nb, int T, int lim, const void* k,
                            const void* v, hipStream_t st)
{
    const size_t row_stride = (size_t)L->heads * L->head_dim;
    const size_t esz = L->act_dtype == HCI_BF16 ? 2 : 4;
    for (int b = 0; b < nb; ++b) {
        const hipError_t e = launch_kv_pack(L, S, b, -1, T, (const char*)k + (size_t)b * T * row_stride * esz,
                                            (const char*)v + (size_t)b * T * row_stride * esz, row_stride,
                                            (size_t)L->head_dim, st, lim);
        if (e != hipSuccess) return e;
    }
    return launch_len_add(S, nb, T, lim, st);
}

template <int ACT>
static hipError_t launch_state_path(const hci_layer* L, const hci_state* S, int nb, int T, int lim,
                                    const typename Act<ACT>::T* x, const PrefillPlan& plan, void* ws, hipStream_t st)
{
    typedef typename Act<ACT>::T AT;
    const int d = L->d, M = T - L->taps_outer + 1;
    float* e = (float*)ws;
    hipLaunchKernelGGL(k_prefill_scan<ACT>, dim3((d + kScCh - 1) / kScCh, plan.nchunks, nb), dim3(256), 0, st,
                       L->w_short, L->lambda, (const AT*)S->short_win, x, e, d, L->taps_short, L->poles, T, M,
                       plan.sub_len, plan.nchunks);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_prefill_state<ACT>, dim3((d + kPfCG - 1) / kPfCG, nb), dim3(256),
                       prefill_state_lds_bytes(L), st, L->w_short, L->w_outer, L->lambda, L->beta, (AT*)S->short_win,
                       S->outer_win, S->iir, x, (const float*)e, S->kv_len, d, L->taps_short, L->taps_outer, L->poles,
                       T, M, plan.chunk_len, plan.nchunks, lim);
    return hipGetLastError();
}

hipError_t launch_prefill(const hci_layer* L, const hci_state* S, int nb, int T, int lim, const void* x,
                          const void* k, const void* v, void* y, const PrefillPlan& plan, void* ws, hipStream_t st)
{
    float* s_loc = (float*)ws;
    float* f_tail = (float*)((char*)ws + (plan.s_elems * 4 + 255) / 256 * 256);
    float* y_loc = y ? (float*)((char*)f_tail + (plan.ftail_elems * 4 + 255) / 256 * 256) : nullptr;
    const int d = L->d;
    hipError_t e;
    if (plan.state_only) {
        // outputs first: they start from the committed state the state path then replaces
        if (plan.y_mfma && (e = launch_y_mfma(L, S, nb, T, x, y, st)) != hipSuccess) return e;
        e = L->act_dtype == HCI_BF16
                ? launch_state_path<HCI_BF16>(L, S, nb, T, lim, (const uint16_t*)x, plan, ws, st)
                : launch_state_path<HCI_F32>(L, S, nb, T, lim, (const float*)x, plan, ws, st);
        if (e != hipSuccess) return e;
        return append_kv(L, S, nb, T, lim, k, v, st);
    }
    const size_t lds = prefill_lds_bytes(L->taps_outer);
    dim3 grid((d + kPfCG - 1) / kPfCG, plan.nchunks, nb);
    if (L->act_dtype == HCI_BF16) {
        if (lds > 65536 && (e = hipFuncSetAttribute((const void*)k_prefill_local<HCI_BF16>,
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
            return e;
        hipLaunchKernelGGL(k_prefill_local<HCI_BF16>, grid, dim3(kPfT), lds, st, L->w_short, L->w_outer, L->lambda,
                           L->beta, L->c, (const uint16_t*)S->short_win, S->outer_win, (const uint16_t*)x, s_loc,
                           f_tail, y_loc, d, L->taps_short, L->taps_outer, L->poles, T, plan.nchunks);
    } else {
        if (lds > 65536 && (e = hipFuncSetAttribute((const void*)k_prefill_local<HCI_F32>,
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
            return e;
        hipLaunchKernelGGL(k_prefill_local<HCI_F32>, grid, dim3(kPfT), lds, st, L->w_short, L->w_outer, L->lambda,
                           L->beta, L->c, (const float*)S->short_win, S->outer_win, (const float*)x, s_loc, f_tail,
                           y_loc, d, L->taps_short, L->taps_outer, L->poles, T, plan.nchunks);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t ncarry = (size_t)nb * d * kPfN;
    hipLaunchKernelGGL(k_prefill_carry, dim3((unsigned)((ncarry + 255) / 256)), dim3(256), 0, st, L->lambda, S->iir,
                       s_loc, S->kv_len, d, L->poles, T, plan.nchunks, nb, lim);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (y) {
        if (L->act_dtype == HCI_BF16)
            hipLaunchKernelGGL(k_prefill_fixup<HCI_BF16>, grid, dim3(kPfT), 0, st, L->lambda, L->c, s_loc, y_loc,
                               (uint16_t*)y, d, L->poles, T, plan.nchunks);
        else
            hipLaunchKernelGGL(k_prefill_fixup<HCI_F32>, grid, dim3(kPfT), 0, st, L->lambda, L->c, s_loc, y_loc,
                               (float*)y, d, L->poles, T, plan.nchunks);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    dim3 cgrid((d + 255) / 256, nb);
    if (L->act_dtype == HCI_BF16)
        hipLaunchKernelGGL(k_prefill_commit<HCI_BF16>, cgrid, dim3(256), 0, st, (uint16_t*)S->short_win, S->outer_win,
                           (const uint16_t*)x, f_tail, S->kv_len, d, L->taps_short, L->taps_outer, T, lim);
    else
        hipLaunchKernelGGL(k_prefill_commit<HCI_F32>, cgrid, dim3(256), 0, st, (float*)S->short_win, S->outer_win,
                           (const float*)x, f_tail, S->kv_len, d, L->taps_short, L->taps_outer, T, lim);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return append_kv(L, S, nb, T, lim, k, v, st);
}

}  // namespace hci
