// Token trees: the ancestor table shared by the tree kernels, and the
// conv/recurrent half of a tree block forward (every node's short FIR, outer
// FIR and modal IIR over its own root-to-node history).
//
// A tree of n <= 64 nodes per sequence: node 0 is the anchor, node m > 0 has a
// parent p(m) < m.  Node m stands for the positions along the path root -> m
// (EvSpark digest, Interpretation: several candidate blocks per step; ReaDy
// summary, section 5: tree verification with recovery of recurrent state), so
// its FIR windows read its ancestors, newest first, and then the committed
// window, and its IIR state starts from its parent's state.
//
// One workgroup = 16 channels of one sequence (the chain kernel's channel
// groups).  Every per-output sum is taken in the order the chain kernel
// (conv_iir_body.h) uses -- short FIR taps ascending; the outer FIR as
// kFirChunks tap chunks summed in ascending tap order and added in chunk
// order; s = fma(lambda, s_parent, beta * g); y per four-pole group, then the
// same lane butterfly -- so a node's f, s and y carry the same bits as the
// chain forward over its path.
#pragma once

#include "conv_iir_body.h"
#include "wave_ops.h"

namespace hci {

constexpr int kTreeMax = 64;       // nodes per tree (the attention path's query limit)
constexpr int kTreePoles = 16;     // poles per channel on the tree path

// LDS of the ancestor table: parents [64] bytes, depths [64] bytes, ancestors [64][64] bytes
constexpr size_t kTreeAncBytes = 2 * kTreeMax + (size_t)kTreeMax * kTreeMax;

struct TreeAnc {
    uint8_t* par;     // [n] parent (node 0: 0)
    uint8_t* depth;   // [n]
    uint8_t* anc;     // [n][64]: anc[m][j] = the node j steps above m, j <= depth[m]
};

__device__ __forceinline__ TreeAnc tree_anc_lds(void* base) {
    uint8_t* p = (uint8_t*)base;
    return TreeAnc{p, p + kTreeMax, p + 2 * kTreeMax};
}

// Whether parent entry m is valid: parent[0] == -1, 0 <= parent[m] < m for m > 0.
__device__ __forceinline__ bool tree_parent_ok(int m, int p) { return m == 0 ? p == -1 : (p >= 0 && p < m); }

// Builds the ancestor table of one tree (threads 0..n-1 each walk their own node; every parent
// precedes its child, so a walk ends at node 0 within m steps).  p is thread tid's parent entry,
// loaded by the caller (for tid < n).  An invalid parent entry is read as m - 1 (the tree's
// outputs are then those of that reading; callers report HCI_DS_TREE).  Returns whether every
// entry was valid (the same on every thread).  Ends with a barrier.
__device__ __forceinline__ bool tree_build(int p, int n, const TreeAnc& t, int* flag) {
    const int tid = threadIdx.x;
    if (tid == 0) *flag = 1;
    __syncthreads();
    if (tid < n) {
        const bool ok = tree_parent_ok(tid, p);
        if (!ok) *flag = 0;                          // every writer stores the same value
        t.par[tid] = (uint8_t)(tid == 0 ? 0 : (ok ? p : tid - 1));
    }
    __syncthreads();
    if (tid < n) {
        uint8_t* row = t.anc + tid * kTreeMax;
        int cur = tid, j = 0;
        row[0] = (uint8_t)tid;
        while (cur != 0) {
            cur = t.par[cur];
            row[++j] = (uint8_t)cur;
        }
        t.depth[tid] = (uint8_t)j;
    }
    __syncthreads();
    return *flag != 0;
}

// LDS of the tree conv role: the ancestor table, a flag word, the nodes of every depth as bit
// masks [64], the owner of every node [64] (u32) and whether it has a child [64] (bytes), then
// (16-byte aligned) floats: short window + x rows, outer window + f rows, chunk sums of g, outer
// taps, short taps.
__host__ __device__ inline size_t tree_conv_head_bytes() {
    return (kTreeAncBytes + 16 + kTreeMax * 8 + kTreeMax * 4 + kTreeMax + 15) / 16 * 16;
}
__host__ __device__ inline size_t tree_conv_lds_bytes(int Ts, int To, int n) {
    const size_t floats = (size_t)((Ts - 1 + n) + (To - 1 + n) + kFirChunks * n + To + Ts) * kCG;
    return tree_conv_head_bytes() + floats * sizeof(float);
}

// One workgroup: channel group cgi (16 channels) of sequence b; the tree's n nodes are the rows
// of x / f / s / y.  Returns the HCI_DS_* bits it found (HCI_DS_TREE), the same on every thread.
template <int ACT>
__device__ __forceinline__ uint32_t tree_conv_block(
    const float* __restrict__ w_short, const float* __restrict__ w_outer,
    const float* __restrict__ lam, const float* __restrict__ beta, const float* __restrict__ cc,
    const typename Act<ACT>::T* __restrict__ short_win, const float* __restrict__ outer_win,
    const float* __restrict__ iir, const typename Act<ACT>::T* __restrict__ x, const int32_t* __restrict__ parent,
    float* __restrict__ f_out, float* __restrict__ s_out, typename Act<ACT>::T* __restrict__ y_out,
    int d, int Ts, int To, int N, int n, int cgi, int b, void* lds_raw)
{
    const int W = To - 1, Ws = Ts - 1;
    const TreeAnc t = tree_anc_lds(lds_raw);
    int* flag = (int*)((char*)lds_raw + kTreeAncBytes);
    uint64_t* dmask = (uint64_t*)((char*)lds_raw + kTreeAncBytes + 16);   // [64]: the nodes of depth D
    uint32_t* owner = (uint32_t*)(dmask + kTreeMax);     // [64]: the first leaf (index order) below a node
    uint8_t* haschild = (uint8_t*)(owner + kTreeMax);    // [64]
    float* xs = (float*)((char*)lds_raw + tree_conv_head_bytes());  // [Ws + n][kCG]
    float* fb = xs + (size_t)(Ws + n) * kCG;          // [W + n][kCG]: outer window rows, then f rows
    float* gl = fb + (size_t)(W + n) * kCG;           // [kFirChunks][n][kCG]: chunk sums of g
    float* wl = gl + (size_t)kFirChunks * n * kCG;    // [To][kCG]
    float* ws = wl + (size_t)To * kCG;                // [Ts][kCG]

    const int ch0 = cgi * kCG;
    const int tid = threadIdx.x, lane = tid & 63;
    const int cl = tid & (kCG - 1), row = tid >> 4;
    const int ch = ch0 + cl;
    const bool live = ch < d;
    const typename Act<ACT>::T* sw = short_win + (size_t)b * Ws * d;
    const float* ow = outer_win + (size_t)b * W * d;
    const typename Act<ACT>::T* xb = x + (size_t)b * n * d;

    // The parent entries are requested first: loads return in order, so the ancestor table, the
    // leaves and the owners below are built while the window, tap, input and IIR parameter loads
    // are still in flight.
    const int pin = parent[(size_t)b * n + min(tid, n - 1)];     // used for tid < n only
    asm volatile("" ::: "memory");                  // issued before every load below

    // every other load of the workgroup in one round (values to registers first; the common
    // sizes, up to 128 window rows and taps and 64 nodes, then the rest by plain loops)
    // Every load is unconditional, from a clamped (always valid) address, its value masked where
    // it is stored: with no branch around a load the compiler counts the loads in flight exactly
    // and waits for each one only where it is used; activations stay raw bits until then (a
    // conversion next to a load would wait for it there).
    constexpr int SW = 8, SX = 4;                       // rows per thread of the register batch
    const int chc = min(ch, d - 1);
    float vw[SW], vt[SW], vst;
    typename ActRaw<ACT>::R rx[SX], rsw;
#pragma unroll
    for (int u = 0; u < SW; ++u) {
        const int r = row + 16 * u;
        vw[u] = (W > 0 ? ow + (size_t)min(r, W - 1) * d : w_outer)[chc];     // no window: any valid row
        vt[u] = w_outer[(size_t)min(r, To - 1) * d + chc];
    }
#pragma unroll
    for (int u = 0; u < SX; ++u) rx[u] = ActRaw<ACT>::load(xb, (size_t)min(row + 16 * u, n - 1) * d + chc);
    rsw = ActRaw<ACT>::load(Ws > 0 ? sw + (size_t)min(row, Ws - 1) * d : xb, chc);
    vst = w_short[(size_t)min(row, Ts - 1) * d + chc];

    // IIR task of this thread (channel ch0 + tch, poles 4 tg .. 4 tg + 3 of one root-to-leaf path
    // per wave and pass) and its parameters, used after the FIR
    const int G = N <= 4 ? 1 : N <= 8 ? 2 : 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tg = lane % G, tch = (lane / G) % kCG;
    const int chn = ch0 + tch;
    const bool task_lane = lane < kCG * G;
    const bool scan = task_lane && chn < d;
    float lm[4], bt[4], cv[4], s0[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const size_t o = (size_t)min(chn, d - 1) * N + min(4 * tg + q, N - 1);
        lm[q] = lam[o];
        bt[q] = beta[o];
        cv[q] = cc[o];
        s0[q] = iir[(size_t)b * d * N + o];
    }

    if (tid < kTreeMax) {
        owner[tid] = kTreeMax;
        haschild[tid] = 0;
    }
    const bool valid = tree_build(pin, n, t, flag);     // its first barrier publishes the two arrays
    // the nodes of every depth (n <= 64: one lane per node) and the leaves (no child)
    const int dl = lane < n ? (int)t.depth[lane] : -1;
    const int maxD = wave_max_i32(dl);
    for (int D = 0; D <= maxD; ++D) {
        const uint64_t mk = __ballot(dl == D);
        if (tid == 0) dmask[D] = mk;
    }
    if (tid > 0 && tid < n) haschild[t.par[tid]] = 1;
    __syncthreads();
    const bool is_leaf = lane < n && haschild[lane] == 0;
    const uint64_t leafmask = __ballot(is_leaf);
    const int nl = __popcll(leafmask);
    // a node is stored by the first leaf below it in index order: every leaf takes the minimum
    // over the nodes of its root path (published by the barrier after the LDS stores below)
    if (tid < n && is_leaf) {
        const uint8_t* am = t.anc + tid * kTreeMax;
        for (int j = 0; j <= dl; ++j) atomicMin(&owner[am[j]], (uint32_t)tid);
    }

#pragma unroll
    for (int u = 0; u < SW; ++u) {
        const int r = row + 16 * u;
        if (r < W) fb[r * kCG + cl] = keep_if(vw[u], live);
        if (r < To) wl[r * kCG + cl] = keep_if(vt[u], live);
    }
#pragma unroll
    for (int u = 0; u < SX; ++u) {
        const int r = row + 16 * u;
        if (r < n) xs[(Ws + r) * kCG + cl] = keep_if(ActRaw<ACT>::cvt(rx[u]), live);
    }
    if (row < Ws) xs[row * kCG + cl] = keep_if(ActRaw<ACT>::cvt(rsw), live);
    if (row < Ts) ws[row * kCG + cl] = keep_if(vst, live);
    for (int r = row + 16 * SW; r < W; r += kConvT / kCG) fb[r * kCG + cl] = live ? ow[(size_t)r * d + ch] : 0.f;
    for (int r = row + 16 * SW; r < To; r += kConvT / kCG) wl[r * kCG + cl] = live ? w_outer[(size_t)r * d + ch] : 0.f;
    for (int r = row + 16 * SX; r < n; r += kConvT / kCG) xs[(Ws + r) * kCG + cl] = live ? Act<ACT>::load(xb, (size_t)r * d + ch) : 0.f;
    for (int r = row + 16; r < Ws; r += kConvT / kCG) xs[r * kCG + cl] = live ? Act<ACT>::load(sw, (size_t)r * d + ch) : 0.f;
    for (int r = row + 16; r < Ts; r += kConvT / kCG) ws[r * kCG + cl] = live ? w_short[(size_t)r * d + ch] : 0.f;
    __syncthreads();

    // short FIR: f_m = sum_{j<Ts} w_short[j] * (input j positions before m on its path)
    for (int m = row; m < n; m += kConvT / kCG) {
        const int D = t.depth[m];
        const uint8_t* am = t.anc + m * kTreeMax;
        float acc = 0.f;
        for (int j = 0; j < Ts; ++j) {
            const int rw = j <= D ? Ws + am[j] : Ws - (j - D);
            acc = fmaf(ws[j * kCG + cl], xs[rw * kCG + cl], acc);
        }
        if (live) f_out[((size_t)b * n + m) * d + ch] = acc;
        fb[(W + m) * kCG + cl] = acc;
    }
    __syncthreads();

    // outer FIR in the chain kernel's order: chunk k sums taps [k CS, min((k + 1) CS, To)) in
    // ascending order from zero, and the IIR adds the chunk sums in chunk order.  Tap j of node m
    // (depth D) reads its ancestor j steps up for j <= D and the committed-window row W - (j - D)
    // past it, so a chunk that starts past D reads window rows only: its sum is the same for every
    // node of depth D, taken once per depth and stored for each of them; the other chunks are
    // summed per node.
    const int CS = (To + kFirChunks - 1) / kFirChunks;
    // per node: a node's chunk sum over taps [j0, j1), ancestors first, then window rows
    auto node_chunk = [&](int m, int k, int tcl) {
        const int D = t.depth[m];
        const int j0 = k * CS, j1 = min(j0 + CS, To);
        const uint8_t* am = t.anc + m * kTreeMax;
        const int ja = min(D, j1 - 1);                  // the last ancestor tap of the chunk
        float acc = 0.f;
#pragma unroll 4
        for (int j = j0; j <= ja; ++j) acc = fmaf(wl[j * kCG + tcl], fb[(W + am[j]) * kCG + tcl], acc);
#pragma unroll 8
        for (int j = ja + 1; j < j1; ++j) acc = fmaf(wl[j * kCG + tcl], fb[(W - (j - D)) * kCG + tcl], acc);
        gl[((size_t)k * n + m) * kCG + tcl] = acc;
    };
    // chunk 0 starts at tap 0 <= D: always per node, (node, channel) tasks
    for (int task = tid; task < n * kCG; task += kConvT) node_chunk(task / kCG, 0, task % kCG);
    // later chunks per node only in trees deeper than a chunk
    if (maxD >= CS)
        for (int task = tid; task < n * (kFirChunks - 1) * kCG; task += kConvT) {
            const int tcl = task % kCG, k = 1 + (task / kCG) % (kFirChunks - 1), m = task / (kCG * (kFirChunks - 1));
            if (k * CS <= (int)t.depth[m]) node_chunk(m, k, tcl);
        }
    // per depth: the chunks that start past D, stored for every node of depth D
    for (int task = tid; task < (maxD + 1) * (kFirChunks - 1) * kCG; task += kConvT) {
        const int tcl = task % kCG, k = 1 + (task / kCG) % (kFirChunks - 1), D = task / (kCG * (kFirChunks - 1));
        const int j0 = k * CS, j1 = min(j0 + CS, To);
        if (j0 <= D) continue;
        float acc = 0.f;
#pragma unroll 8
        for (int j = j0; j < j1; ++j) acc = fmaf(wl[j * kCG + tcl], fb[(W - (j - D)) * kCG + tcl], acc);
        for (uint64_t mk = dmask[D]; mk != 0; mk &= mk - 1)
            gl[((size_t)k * n + __builtin_ctzll(mk)) * kCG + tcl] = acc;
    }
    __syncthreads();

    // IIR along the tree, one root-to-leaf path per wave and pass: the path's nodes in order from
    // the root (lane j holds the node j steps above the leaf), each state s = fma(lambda, s_parent,
    // beta * g) kept in registers, the next node's input read ahead.  A node on several paths is
    // computed by each of them with the same arithmetic (the same bits) and stored by its owner.
    const int minleaf = lane < n ? (int)owner[lane] : kTreeMax;
    // the IIR parameters of a lane past the channels or poles are zero
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const bool ok = scan && 4 * tg + q < N;
        lm[q] = keep_if(lm[q], ok);
        bt[q] = keep_if(bt[q], ok);
        cv[q] = keep_if(cv[q], ok);
        s0[q] = keep_if(s0[q], ok);
    }
    // g of node m: the chunk sums in chunk order
    auto g_of = [&](int m) -> float {
        float g = gl[(size_t)m * kCG + tch];
#pragma unroll
        for (int k = 1; k < kFirChunks; ++k) g += gl[((size_t)k * n + m) * kCG + tch];
        return g;
    };
    for (int li = wv; li < nl; li += kConvT / 64) {
        uint64_t mk = leafmask;
        for (int i = 0; i < li; ++i) mk &= mk - 1;
        const int L = __builtin_ctzll(mk);               // the li-th leaf in index order
        const int D = t.depth[L];
        const int pv = t.anc[L * kTreeMax + lane];       // lane j: the node j steps above L
        if (task_lane) {
            float st[4] = {s0[0], s0[1], s0[2], s0[3]};
            float gn = g_of(__builtin_amdgcn_readlane(pv, D));
            for (int j = D; j >= 0; --j) {
                const int m = __builtin_amdgcn_readlane(pv, j);
                const float g = scan ? gn : 0.f;
                if (j > 0) gn = g_of(__builtin_amdgcn_readlane(pv, j - 1));
                float py = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    st[q] = fmaf(lm[q], st[q], bt[q] * g);
                    py = fmaf(cv[q], st[q], py);
                }
                const bool store = scan && __builtin_amdgcn_readlane(minleaf, m) == L;
                if (store) {
                    float* so = s_out + (((size_t)b * n + m) * d + chn) * N + 4 * tg;
                    if ((N & 3) == 0) {
                        *(float4*)so = make_float4(st[0], st[1], st[2], st[3]);
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (4 * tg + q < N) so[q] = st[q];
                    }
                }
                py = group_sum(py, G);
                if (store && tg == 0) Act<ACT>::store(y_out, ((size_t)b * n + m) * d + chn, py);
            }
        }
    }
    return valid ? 0u : HCI_DS_TREE;
}

// Ancestor sets of every node as bit masks (bit j of mask[m]: node j is m or one of its
// ancestors), by pointer doubling on one wave: lane m starts from {m, p(m)} and jumps to its
// ancestor 2^r steps up in round r.  Invalid parent entries are read as m - 1.  Called by
// every wave of the workgroup (the first does the work); ends with a barrier.
__device__ __forceinline__ void tree_masks(const int32_t* __restrict__ parent, int n, uint64_t* mask,
                                           uint8_t* jump) {
    const int tid = threadIdx.x;
    if (tid < 64) {
        const int m = tid;
        int p = 0;
        if (m < n) {
            const int v = parent[m];
            p = m == 0 ? 0 : (tree_parent_ok(m, v) ? v : m - 1);
        }
        uint64_t mk = m < n ? ((1ull << m) | (1ull << p)) : 0ull;
        mask[m] = mk;
        jump[m] = (uint8_t)p;
        for (int r = 0; r < 6; ++r) {                 // 2^6 = 64 >= any depth
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int jp = jump[m];
            const uint64_t add = mask[jp];
            const int jj = jump[jp];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            mk |= add;
            mask[m] = mk;
            jump[m] = (uint8_t)jj;
        }
    }
    __syncthreads();
}

}  // namespace hci
