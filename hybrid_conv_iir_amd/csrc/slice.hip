// State slicing to the accepted index (EvSpark digest, Figure 1(d) and
// Interpretation): the three state classes are restored by selecting values
// the block forward already produced -- no target computation is replayed.
//
// k_slice reads k and the winning candidate c* on the device, so no host
// synchronisation sits between acceptance and slicing.  Workgroup roles, by
// range of blockIdx.x (blockIdx.z = sequence):
//   0  FIR windows: 16 channels per workgroup; the new window rows are first
//      gathered into LDS, then written back (the update is in place)
//   1  IIR state <- s_k of c* (kSliceAux workgroups, 16-byte copies)
//   2  KV rows kv_len .. kv_len+k <- block k/v rows 0..k of c* (tiled layout;
//      kSliceAux workgroups)
// k_slice_len then advances kv_len; it runs after every role of k_slice has
// read the old length (stream order).
#include "act_raw.h"
#include "hci_internal.h"

namespace hci {

constexpr int kSliceCG = 16;         // channels per window workgroup
constexpr int kSliceRows = 256 / kSliceCG;   // window rows handled per pass of the 256 threads
constexpr int kSliceWinMax = 128;    // window rows staged in LDS per pass
// workgroups of each copy role per sequence: the IIR state (d N floats) and the accepted K/V rows
// are tens of kilobytes, so a few workgroups copy them, and a 4-sequence slice fits one round of
// resident workgroups
constexpr int kSliceAux = 64;

// The winning candidate c*, its accepted index k and the committed length L of sequence b,
// and the HCI_DS_* bits that stop the commit (0 when it may proceed): c* outside [0, nc), k
// outside [0, gamma], or kv_len outside [0, lim].  Nothing is clamped into range: a sequence
// with any of these is left exactly as it was.
__device__ __forceinline__ uint32_t slice_target(const int32_t* n_acc, const int32_t* best, const int32_t* kv_len,
                                                 int b, int nc, int gamma, int lim, int& cstar, int& k, int& L) {
    uint32_t bad = 0u;
    cstar = (best != nullptr && nc > 1) ? best[b] : 0;
    k = -1;
    if (cstar < 0 || cstar >= nc) bad |= HCI_DS_CAND_RANGE;
    else k = n_acc[(size_t)b * nc + cstar];
    if (bad == 0u && (k < 0 || k > gamma)) bad |= HCI_DS_K_RANGE;
    L = kv_len[b];
    if (L < 0 || L > lim) bad |= HCI_DS_KV_LEN;
    return bad;
}

// Token trees: whether the accepted path of sequence b (path [nb][n], entries 0..k) starts at
// the anchor and follows the tree (path[i] is a child of path[i-1], so the indices ascend).
// Threads i <= k check one step each; the answer is the same on every thread of the workgroup.
__device__ __forceinline__ bool tree_path_ok(const int32_t* __restrict__ path, const int32_t* __restrict__ parent,
                                             int n, int b, int k) {
    bool ok = true;
    for (int i = threadIdx.x; i <= k; i += blockDim.x) {
        const int v = path[(size_t)b * n + i];
        if (i == 0) {
            ok = ok && v == 0;
        } else {
            const int prev = path[(size_t)b * n + i - 1];
            ok = ok && v > prev && v < n && parent[(size_t)b * n + v] == prev;
        }
    }
    return __syncthreads_or(!ok) == 0;
}

// block row r of the committed rows: r itself (a chain of candidate positions) or the r-th node
// of the accepted path (a token tree)
__device__ __forceinline__ int row_of(const int32_t* rmap, int r) { return rmap ? rmap[r] : r; }

template <int ACT>
__device__ void window_update(typename Act<ACT>::T* win, const typename Act<ACT>::T* blk_rows,
                              int W, int d, int k, int ch0, float (*stage)[kSliceCG], const int32_t* rmap)
{
    // new[r] = concat(old[0..W), rows[0..k])[k+1+r] for r < W.  Rows are
    // processed in ascending chunks; chunk [r0, r0+128) reads old rows at or
    // above r0+k+1, which no earlier chunk has overwritten.  A thread's rows of
    // a chunk are loaded in one round (unconditional loads from clamped rows and
    // channels, raw bits until they are staged), so their latencies overlap.
    constexpr int RPT = kSliceWinMax / kSliceRows;     // rows per thread and chunk
    const int tid = threadIdx.x, cl = tid % kSliceCG, part = tid / kSliceCG;
    const int ch = ch0 + cl;
    const int chc = min(ch, d - 1);
    for (int r0 = 0; r0 < W; r0 += kSliceWinMax) {
        const int r1 = min(W, r0 + kSliceWinMax);
        // block rows first through the path (a token tree), all in one round
        int rb[RPT];
        if (rmap) {
#pragma unroll
            for (int u = 0; u < RPT; ++u) rb[u] = rmap[max(k + 1 + min(r0 + part + u * kSliceRows, r1 - 1) - W, 0)];
        } else {
#pragma unroll
            for (int u = 0; u < RPT; ++u) rb[u] = max(k + 1 + min(r0 + part + u * kSliceRows, r1 - 1) - W, 0);
        }
        typename ActRaw<ACT>::R v[RPT];
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            const int m = k + 1 + min(r0 + part + u * kSliceRows, r1 - 1);
            const typename Act<ACT>::T* src = m < W ? win + (size_t)m * d : blk_rows + (size_t)rb[u] * d;
            v[u] = ActRaw<ACT>::load(src, chc);
        }
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            const int r = r0 + part + u * kSliceRows;
            if (r < r1) stage[r - r0][cl] = ch < d ? ActRaw<ACT>::cvt(v[u]) : 0.f;
        }
        __syncthreads();
        for (int r = r0 + part; r < r1; r += kSliceRows)
            if (ch < d) Act<ACT>::store(win, (size_t)r * d + ch, stage[r - r0][cl]);
        __syncthreads();
    }
}

template <int ACT>
__global__ __launch_bounds__(256) void k_slice(
    typename Act<ACT>::T* __restrict__ short_win, float* __restrict__ outer_win,
    float* __restrict__ iir, typename Act<ACT>::T* __restrict__ kc, typename Act<ACT>::T* __restrict__ vc,
    const int32_t* __restrict__ kv_len, const typename Act<ACT>::T* __restrict__ x,
    const float* __restrict__ f, const float* __restrict__ s,
    const typename Act<ACT>::T* __restrict__ kb, const typename Act<ACT>::T* __restrict__ vb,
    const int32_t* __restrict__ n_acc, const int32_t* __restrict__ best,
    const int32_t* __restrict__ path, const int32_t* __restrict__ parent,
    int d, int Ts, int To, int N, int H, int DH, int kv_cap, int nc, int gamma, int lim)
{
    __shared__ float stage[kSliceWinMax][kSliceCG];
    const int b = blockIdx.z;
    const int win_blocks = (int)gridDim.x - 2 * kSliceAux;
    const int role = (int)blockIdx.x < win_blocks ? 0 : ((int)blockIdx.x < win_blocks + kSliceAux ? 1 : 2);
    const int wg = role == 0 ? (int)blockIdx.x : (int)blockIdx.x - win_blocks - (role - 1) * kSliceAux;
    const int P = gamma + 1;
    int cstar, k, L;
    // reported by the length kernel; the path check is workgroup-wide (every thread takes part)
    const bool bad = slice_target(n_acc, best, kv_len, b, nc, gamma, lim, cstar, k, L) != 0u;
    if (path != nullptr && !tree_path_ok(path, parent, P, b, bad ? -1 : k)) return;
    if (bad) return;
    const size_t blk = (size_t)b * nc + cstar;
    const int32_t* rmap = path ? path + (size_t)b * P : nullptr;     // a tree: nc = 1, P = its nodes

    if (role == 0) {
        const int ch0 = wg * kSliceCG;
        if (ch0 >= d) return;
        if (Ts > 1)
            window_update<ACT>(short_win + (size_t)b * (Ts - 1) * d, x + blk * P * d, Ts - 1, d, k, ch0, stage, rmap);
        if (To > 1)
            window_update<HCI_F32>(outer_win + (size_t)b * (To - 1) * d, f + blk * P * d, To - 1, d, k, ch0, stage,
                                   rmap);
    } else if (role == 1) {
        const size_t n = (size_t)d * N;
        const float* src = s + (blk * P + row_of(rmap, k)) * n;
        float* dst = iir + (size_t)b * n;
        const size_t t0 = (size_t)wg * blockDim.x + threadIdx.x, stride = (size_t)kSliceAux * blockDim.x;
        if (((uintptr_t)src % 16) == 0 && ((uintptr_t)dst % 16) == 0) {
            const size_t n4 = n / 4;
            for (size_t e = t0; e < n4; e += stride) ((float4*)dst)[e] = ((const float4*)src)[e];
            for (size_t e = 4 * n4 + t0; e < n; e += stride) dst[e] = src[e];
        } else {
            for (size_t e = t0; e < n; e += stride) dst[e] = src[e];
        }
    } else {
        const size_t per_row = (size_t)H * DH;
        const size_t n = (size_t)(k + 1) * per_row;
        const size_t slab = (size_t)kv_cap * DH;
        for (size_t e = (size_t)wg * blockDim.x + threadIdx.x; e < n; e += (size_t)kSliceAux * blockDim.x) {
            const int i = (int)(e / per_row);
            const int h = (int)((e / DH) % H);
            const int dd = (int)(e % DH);
            const int row = L + i;               // < lim + gamma + 1 <= kv_cap (host check)
            if (row >= kv_cap) continue;
            const size_t src = ((blk * P + row_of(rmap, i)) * H + h) * DH + dd;
            const size_t base = ((size_t)b * H + h) * slab;
            kc[base + k_elem(row, dd, DH)] = kb[src];
            vc[base + v_elem(row, dd, DH)] = vb[src];
        }
    }
}

__global__ void k_slice_len(int32_t* __restrict__ kv_len, const int32_t* __restrict__ n_acc,
                            const int32_t* __restrict__ best, uint32_t* __restrict__ status, int nb, int nc,
                            int gamma, int lim)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nb) return;
    int cstar, k, L;
    const uint32_t bad = slice_target(n_acc, best, kv_len, b, nc, gamma, lim, cstar, k, L);
    if (bad != 0u) {
        report(status, b, bad);
        return;
    }
    kv_len[b] = L + k + 1;
}

// kv_len += k + 1 for a token tree, after the path check (one 64-thread workgroup per sequence)
__global__ __launch_bounds__(64) void k_slice_len_tree(int32_t* __restrict__ kv_len, const int32_t* __restrict__ n_acc,
                                                       const int32_t* __restrict__ path,
                                                       const int32_t* __restrict__ parent, uint32_t* __restrict__ status,
                                                       int n, int lim)
{
    const int b = blockIdx.x;
    int cstar, k, L;
    uint32_t bad = slice_target(n_acc, nullptr, kv_len, b, 1, n - 1, lim, cstar, k, L);
    if (!tree_path_ok(path, parent, n, b, bad ? -1 : k)) bad |= HCI_DS_TREE;
    if (threadIdx.x != 0) return;
    if (bad != 0u) {
        report(status, b, bad);
        return;
    }
    kv_len[b] = L + k + 1;
}

hipError_t launch_slice(const hci_layer* L, const hci_state* S, const hci_block* blk,
                        int nb, int nc, int P, int lim, const int32_t* n_acc, const int32_t* best, hipStream_t st,
                        const int32_t* path, const int32_t* parent)
{
    const int gamma = P - 1;
    const int win_blocks = (L->d + kSliceCG - 1) / kSliceCG;
    dim3 grid(win_blocks + 2 * kSliceAux, 1, nb), block(256);
    if (L->act_dtype == HCI_BF16) {
        hipLaunchKernelGGL(k_slice<HCI_BF16>, grid, block, 0, st,
            (uint16_t*)S->short_win, S->outer_win, S->iir, (uint16_t*)S->k_cache, (uint16_t*)S->v_cache,
            S->kv_len, (const uint16_t*)blk->x, blk->f, blk->s, (const uint16_t*)blk->k,
            (const uint16_t*)blk->v, n_acc, best, path, parent, L->d, L->taps_short, L->taps_outer, L->poles,
            L->heads, L->head_dim, S->kv_cap, nc, gamma, lim);
    } else {
        hipLaunchKernelGGL(k_slice<HCI_F32>, grid, block, 0, st,
            (float*)S->short_win, S->outer_win, S->iir, (float*)S->k_cache, (float*)S->v_cache,
            S->kv_len, (const float*)blk->x, blk->f, blk->s, (const float*)blk->k,
            (const float*)blk->v, n_acc, best, path, parent, L->d, L->taps_short, L->taps_outer, L->poles,
            L->heads, L->head_dim, S->kv_cap, nc, gamma, lim);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (path)
        hipLaunchKernelGGL(k_slice_len_tree, dim3(nb), dim3(64), 0, st, S->kv_len, n_acc, path, parent, S->status, P,
                           lim);
    else
        hipLaunchKernelGGL(k_slice_len, dim3((nb + 63) / 64), dim3(64), 0, st,
                           S->kv_len, n_acc, best, S->status, nb, nc, gamma, lim);
    return hipGetLastError();
}

// ---------------------------------------------------------------- KV rows

template <typename T>
__global__ __launch_bounds__(256) void k_kv_copy(T* __restrict__ kc, T* __restrict__ vc,
                                                 const T* __restrict__ ksrc, const T* __restrict__ vsrc,
                                                 T* __restrict__ kdst, T* __restrict__ vdst,
                                                 int b, int row0, int nrows, int H, int DH, int kv_cap, int write)
{
    const size_t n = (size_t)H * nrows * DH;
    const size_t slab = (size_t)kv_cap * DH;
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const int h = (int)(e / ((size_t)nrows * DH));
        const int r = (int)((e / DH) % nrows);
        const int dd = (int)(e % DH);
        const size_t base = ((size_t)b * H + h) * slab;
        const size_t ko = base + k_elem(row0 + r, dd, DH), vo = base + v_elem(row0 + r, dd, DH);
        if (write) { kc[ko] = ksrc[e]; vc[vo] = vsrc[e]; }
        else { kdst[e] = kc[ko]; vdst[e] = vc[vo]; }
    }
}

// Append logical K/V rows to the tiled caches of sequence b: row i of the
// source (at k_rows + i * row_stride + h * head_stride) becomes cache row
// row0 + i, or kv_len[b] + i when row0 < 0 (read on the device).  One
// workgroup per (32-key tile, head): a K unit (8 consecutive dims of one key
// row) is one 16-byte load and store; V rows are staged in LDS and each V unit
// gathers one dim column of 8 keys.  Units whose keys fall partly outside the
// appended rows store element by element.  Sources and caches are 16-byte
// aligned and the row/head strides are multiples of 8 elements (checked on
// the host).
template <typename T>
struct Unit8 {                  // 8 consecutive elements
    u32x4 w[sizeof(T) / 2];
};

template <typename T>
__global__ __launch_bounds__(256) void k_kv_pack(T* __restrict__ kc, T* __restrict__ vc, const T* __restrict__ ks,
                                                 const T* __restrict__ vs, const int32_t* __restrict__ kv_len,
                                                 int b, int row0, int nrows, int H, int DH, int kv_cap,
                                                 size_t row_stride, size_t head_stride, int lim)
{
    constexpr int kMaxDh = 128, kPad = 8;
    __shared__ __align__(16) T vt[kTile * (kMaxDh + kPad)];
    const int L0 = row0 >= 0 ? row0 : kv_len[b];
    // an appended length outside the host's bound leaves the cache alone (k_len_add reports it);
    // the other conditions the host checks make unreachable
    if (L0 < 0 || (row0 < 0 && L0 > lim) || L0 + nrows > kv_cap || DH > kMaxDh) return;
    const int tile = L0 / kTile + (int)blockIdx.x;
    const int r0 = tile * kTile;
    if (r0 >= L0 + nrows) return;                                  // the grid covers an upper bound of tiles
    const int h = blockIdx.y;
    const int lo = max(L0, r0), hi = min(L0 + nrows, r0 + kTile);
    const bool full = lo == r0 && hi == r0 + kTile;
    const int pitch = DH + kPad, upr = DH / 8, J = DH / 32, units = 4 * DH;
    const size_t base = ((size_t)b * H + h) * (size_t)kv_cap * DH + (size_t)r0 * DH;
    T* kdst = kc + base;
    T* vdst = vc + base;
    const T* ksrc = ks + (size_t)h * head_stride;
    const T* vsrc = vs + (size_t)h * head_stride;
    for (int e = threadIdx.x; e < kTile * upr; e += blockDim.x) {
        const int r = e / upr, u = e % upr, row = r0 + r;
        if (row < lo || row >= hi) continue;
        const Unit8<T>* src = (const Unit8<T>*)(vsrc + (size_t)(row - L0) * row_stride + 8 * u);
        Unit8<T> val;
#pragma unroll
        for (int w = 0; w < (int)(sizeof(T) / 2); ++w) val.w[w] = __builtin_nontemporal_load(&src->w[w]);
        *(Unit8<T>*)(vt + r * pitch + 8 * u) = val;
    }
    for (int q = threadIdx.x; q < units; q += blockDim.x) {
        const int m = q & 15, g = (q >> 4) & 3, j = (q >> 6) % J, u = q / (64 * J);
        const int row = r0 + 16 * u + m;
        if (row < lo || row >= hi) continue;
        const Unit8<T>* src = (const Unit8<T>*)(ksrc + (size_t)(row - L0) * row_stride + 32 * j + 8 * g);
        Unit8<T> val;
#pragma unroll
        for (int w = 0; w < (int)(sizeof(T) / 2); ++w) val.w[w] = __builtin_nontemporal_load(&src->w[w]);
        *(Unit8<T>*)(kdst + (size_t)q * 8) = val;
    }
    __syncthreads();
    for (int q = threadIdx.x; q < units; q += blockDim.x) {
        const int m = q & 15, g = (q >> 4) & 3, dd = 16 * (q >> 6) + m;
        T vals[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) vals[i] = vt[(16 * (i >> 2) + 4 * g + (i & 3)) * pitch + dd];
        if (full) {
            Unit8<T> o;
            __builtin_memcpy(&o, vals, sizeof(o));
            *(Unit8<T>*)(vdst + (size_t)q * 8) = o;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = r0 + 16 * (i >> 2) + 4 * g + (i & 3);
                if (row >= lo && row < hi) vdst[(size_t)q * 8 + i] = vals[i];
            }
        }
    }
}

hipError_t launch_kv_pack(const hci_layer* L, const hci_state* S, int b, int row0, int nrows, const void* k_rows,
                          const void* v_rows, size_t row_stride, size_t head_stride, hipStream_t st, int lim)
{
    if (nrows <= 0) return hipSuccess;
    if (L->head_dim > 128 || L->head_dim % 32 || row_stride % 8 || head_stride % 8) return hipErrorInvalidValue;
    // tiles touched: at most nrows / 32 + 2 (row0 may be read on the device)
    const dim3 grid((unsigned)((nrows + 2 * kTile - 1) / kTile), (unsigned)L->heads);
    if (L->act_dtype == HCI_BF16)
        hipLaunchKernelGGL(k_kv_pack<uint16_t>, grid, dim3(256), 0, st, (uint16_t*)S->k_cache,
                           (uint16_t*)S->v_cache, (const uint16_t*)k_rows, (const uint16_t*)v_rows, S->kv_len, b, row0,
                           nrows, L->heads, L->head_dim, S->kv_cap, row_stride, head_stride, lim);
    else
        hipLaunchKernelGGL(k_kv_pack<float>, grid, dim3(256), 0, st, (float*)S->k_cache,
                           (float*)S->v_cache, (const float*)k_rows, (const float*)v_rows, S->kv_len, b, row0, nrows,
                           L->heads, L->head_dim, S->kv_cap, row_stride, head_stride, lim);
    return hipGetLastError();
}

__global__ void k_len_add(int32_t* __restrict__ kv_len, uint32_t* __restrict__ status, int nb, int add, int lim)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nb) return;
    const int L = kv_len[b];
    if (L < 0 || L > lim) {
        report(status, b, HCI_DS_KV_LEN);
        return;
    }
    kv_len[b] = L + add;                 // <= lim + add <= kv_cap (host check)
}

hipError_t launch_len_add(const hci_state* S, int nb, int add, int lim, hipStream_t st)
{
    hipLaunchKernelGGL(k_len_add, dim3((nb + 63) / 64), dim3(64), 0, st, S->kv_len, S->status, nb, add, lim);
    return hipGetLastError();
}

hipError_t launch_kv_copy(const hci_layer* L, const hci_state* S, int b, int row0, int nrows,
                          const void* k_rows, const void* v_rows, void* k_out, void* v_out,
                          bool write, hipStream_t st)
{
    if (write)   // logical rows [H][nrows][Dh]: row stride Dh, head stride nrows * Dh
        return launch_kv_pack(L, S, b, row0, nrows, k_rows, v_rows, (size_t)L->head_dim,
                              (size_t)nrows * L->head_dim, st);
    const size_t n = (size_t)L->heads * nrows * L->head_dim;
    size_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks == 0) return hipSuccess;
    if (L->act_dtype == HCI_BF16) {
        hipLaunchKernelGGL(k_kv_copy<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (uint16_t*)S->k_cache, (uint16_t*)S->v_cache, (const uint16_t*)k_rows,
                           (const uint16_t*)v_rows, (uint16_t*)k_out, (uint16_t*)v_out, b, row0, nrows,
                           L->heads, L->head_dim, S->kv_cap, write ? 1 : 0);
    } else {
        hipLaunchKernelGGL(k_kv_copy<float>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (float*)S->k_cache, (float*)S->v_cache, (const float*)k_rows,
                           (const float*)v_rows, (float*)k_out, (float*)v_out, b, row0, nrows,
                           L->heads, L->head_dim, S->kv_cap, write ? 1 : 0);
    }
    return hipGetLastError();
}

}  // namespace hci
