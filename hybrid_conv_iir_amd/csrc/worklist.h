// The split of the committed KV prefixes into work items, derived on the
// device from kv_len once per verify by the set-up kernel, which records it in
// the workspace (header and table below); the prefix-streaming kernels take
// the items from a queue and locate them through the table, and the finish
// kernel merges their partials through the same table.  Host code sizes the
// workspace with the bound stated below.
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
// With W = H * sum_b tiles_b and R resident slots,
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

// ------------------------------------------------------- work-list table
//
// Written once per verify by the set-up kernel, before the prefix stream, and read by the
// streaming kernels and the finish kernel.  The workspace starts with a header of int32 words
// (the job queue's ticket counter, the item count and the work list's c0 and np), and from
// byte kWsTableOff, for phase p < kPhaseMax and sequence b, entry (p * nb + b) holds
//   base  the item index of (p, b, head 0): the items of (p, b, h) are base + h n .. + n - 1
//   n     items per head of sequence b in phase p (0 for phases past np; base is then the
//         running total)
// so a reader locates every item of (b, h) with 2 kPhaseMax scalar loads and no division,
// and the streaming kernels find the (p, b) entry of an item by a binary search over the
// bases, which never decrease.
constexpr size_t kWsTableOff = 256;                  // byte offset of the table in the workspace
constexpr int kWsTicket = 0, kWsTotal = 1, kWsC0 = 2, kWsNp = 3;   // header words

__host__ __device__ inline size_t worklist_table_bytes(int nb) {
    return (size_t)kPhaseMax * (size_t)nb * 2 * sizeof(int32_t);
}

typedef const __attribute__((address_space(4))) int32_t* const_i32;

// The work list as the set-up kernel recorded it; read with scalar loads (the header and the
// table do not change while the kernels that read them run).
struct WorkTable {
    const_i32 tab;       // the table (2 words per entry)
    WorkList w;
    int total;           // items
};

__device__ __forceinline__ WorkTable read_worktable(const void* ws, int nb, int H, int lim) {
    const const_i32 hdr = (const_i32)ws;
    WorkTable t;
    t.tab = (const_i32)((const char*)ws + kWsTableOff);
    t.w = WorkList{nb, H, lim, hdr[kWsC0], hdr[kWsNp]};
    t.total = hdr[kWsTotal];
    return t;
}

// Locate item `item` through the table: sequence b, head h, tiles [t0, t1); false past the last
// item.  The entry holding it is the last one whose base is <= item (entries with no items
// share their base with the next entry, so the search skips them).
__device__ __forceinline__ bool table_item(const int32_t* kv_len, const WorkTable& t, int item,
                                           int& b, int& h, int& t0, int& t1) {
    if (item < 0 || item >= t.total) return false;
    int lo = 0, hi = kPhaseMax * t.w.nb - 1;           // tab base of entry 0 is 0 <= item
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (t.tab[2 * mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int p = lo / t.w.nb;
    b = lo - p * t.w.nb;
    const int n = t.tab[2 * lo + 1];
    const int rel = item - t.tab[2 * lo];
    h = rel / n;
    const int j = rel - h * n;
    int s, e;
    phase_range(t.w, prefix_tiles(kv_len, b, t.w.lim), p, s, e);
    t0 = s + j * phase_chunk(t.w, p);
    t1 = min(t0 + phase_chunk(t.w, p), e);
    return true;
}

}  // namespace hci
