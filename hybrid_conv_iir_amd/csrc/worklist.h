// The split of the committed KV prefixes into work items, derived on the
// device from kv_len -- identically by the prefix-streaming kernels, which
// take the items from a queue, and by the finish kernel, which merges their
// partials.  Host code sizes the workspace with the bound stated below.
#pragma once

#include "hci_internal.h"

namespace hci {

// Committed length of sequence b as the attention reads it: kv_len clamped to
// [0, lim], lim = min(kv_cap, max_kv_len), so that a length above the host's
// bound can never yield more work than the host planned for.  kv_len does not
// change while the verify kernels run, so it is read through the constant
// address space: with a wave-uniform b that is a scalar load served by the
// scalar cache, not a vector load queued behind the prefix stream (the work
// list is decoded at every item start).
__device__ __forceinline__ int prefix_len(const int32_t* kv_len, int b, int lim) {
    const int L = ((const __attribute__((address_space(4))) int32_t*)kv_len)[b];
    return L < 0 ? 0 : (L > lim ? lim : L);
}

__device__ __forceinline__ int prefix_tiles(const int32_t* kv_len, int b, int lim) {
    return (prefix_len(kv_len, b, lim) + kTile - 1) / kTile;
}

// ------------------------------------------------------------- work list
//
// Derived on the device from kv_len, identically by the streaming kernels
// and the combine.  With W = H * sum_b tiles_b and R resident slots,
// c0 = max(kChunkMin, ceil(W / sR)) (s = 2, or 1 above 32 queries per
// sequence: worklist_split) and np = the number of phases whose chunk
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

// First-phase chunks: half of a slot's fair share, or the whole share when a sequence has more
// than 32 queries (the streaming kernel then runs its LDS-ring form, whose items end with a
// drained pipeline and a full merge, so fewer, larger items pay: measured on 4 sequences x 4
// candidates, 0.462 -> 0.451 ms; with 32 queries or fewer the larger items lose, 0.626 ->
// 0.655 ms on a 262144-token prefix)
__host__ __device__ inline int worklist_split(int nq) { return nq > 32 ? 1 : 2; }

__host__ __device__ inline long long worklist_c0(long long total_tiles, int resident, int nq) {
    const long long half = (long long)worklist_split(nq) * (resident > 0 ? resident : 1);
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

__device__ __forceinline__ WorkList make_worklist(const int32_t* kv_len, int nb, int H, int lim, int resident,
                                                  int nq) {
    long long tot = 0;
    for (int b = 0; b < nb; ++b) tot += prefix_tiles(kv_len, b, lim);
    const long long c0 = worklist_c0(tot * H, resident, nq);
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

// ------------------------------------------------------- work-list table
//
// Written once per verify by the set-up kernel, before the prefix stream, and read by the
// finish kernel: for phase p < kPhaseMax and sequence b, entry (p * nb + b) holds
//   base  the item index of (p, b, head 0): the items of (p, b, h) are base + h n .. + n - 1
//   n     items per head of sequence b in phase p (0 for phases past np)
// so a reader locates every item of (b, h) with 2 kPhaseMax scalar loads and no division.
constexpr size_t kWsTableOff = 256;                  // byte offset of the table in the workspace

__host__ __device__ inline size_t worklist_table_bytes(int nb) {
    return (size_t)kPhaseMax * (size_t)nb * 2 * sizeof(int32_t);
}

}  // namespace hci
