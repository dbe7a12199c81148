// Attention half of the block forward: the plan, the launch sequence of a
// verify, and the fp32 prefix kernel used for small fp32 layers.
//
// The block queries attend to the committed KV prefix and, causally, to the
// block's own keys.  EvSpark digest, Interpretation: the verify is one block
// forward from the committed state, so all nc*P queries of a sequence share
// a single read of its prefix; that read is the part of the verify that grows
// with context (ReaDy summary, section 5: token-wise KV traffic grows with the
// number of attended tokens).  The prefix is cut into work items (split-K,
// worklist.h); each item leaves a partial softmax state (running max in log2
// units, normaliser, unnormalised output), and the finish kernel computes the
// causal block part and merges everything in a fixed order.
//
// Work distribution.  The bf16 streaming kernel (stream_one.hip; one to four
// 16-query tiles per wave) runs one persistent workgroup per CU that takes
// prefix items from a queue (an atomic ticket counter in the workspace,
// zeroed by a one-thread kernel before each launch) until it is empty.  Items
// come in decreasing size: phase p covers the next half of what is left of
// every sequence's prefix in chunks of c0 / 2^p tiles, c0 being half of a
// slot's fair share.  Slots run at different speeds (CUs differ, and of two
// workgroups on a CU the older issues first), so a static split ends ragged;
// with the queue the fast slots take more items and the small last items let
// every slot finish within a few microseconds of the others.  An item always
// writes the partial of its ticket whichever slot runs it, so results do not
// depend on scheduling.  fp32 layers (small shapes) use a vector-ALU prefix
// kernel with one item per workgroup.
#include "conv_iir_body.h"
#include "prefix_tile.h"
#include "tree.h"
#include "verify_parts.h"

#include <math.h>

namespace hci {

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
    float* __restrict__ part_o, float* __restrict__ part_ml, const int32_t* __restrict__ ws,
    int nb, int H, int DH, int kv_cap, int kv_lim, int nq, float scale_log2)
{
    __shared__ float ks[kTile][kF32Dh + 1];
    __shared__ float vs[kTile][kF32Dh + 1];
    __shared__ float ps[kF32Nq][kTile + 1];
    __shared__ float alpha_s[kF32Nq];

    const int item = blockIdx.x;
    const WorkTable wt = read_worktable(ws, nb, H, kv_lim);
    int b, h, t0, t1;
    if (!table_item(kv_len, wt, item, b, h, t0, t1)) return;
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

// Set-up of one verify (a kernel, so that graph capture records no memset): zero the job
// queue's counter, write the work-list header (item count, c0, np) and table, and report every
// sequence whose kv_len lies outside [0, lim] (it is read clamped).  Thread p < kPhaseMax owns
// phase p: it counts the phase's items of every sequence (the per-phase totals meet in LDS),
// then writes each sequence's base and count.  Runs for every verify, also when no sequence
// has a prefix (the finish kernel then reads an empty list, never a previous call's).
// first_ticket: the number of streaming workgroups (workgroup i runs item i first, so the queue
// hands out items from there on)
__global__ __launch_bounds__(64) void k_verify_setup(int32_t* ws, const int32_t* kv_len, uint32_t* status,
                                                     int nb, int H, int lim, int resident, int nq, int first_ticket)
{
    __shared__ long long cnt[kPhaseMax];
    int32_t* table = (int32_t*)((char*)ws + kWsTableOff);
    const int p = threadIdx.x;
    const WorkList w = make_worklist(kv_len, nb, H, lim, resident, nq);
    if (p < kPhaseMax) {
        long long c = 0;
        if (p < w.np)
            for (int b = 0; b < nb; ++b) c += (long long)phase_items(w, prefix_tiles(kv_len, b, lim), p) * H;
        cnt[p] = c;
    }
    __syncthreads();
    if (p < kPhaseMax) {
        long long base = 0;
        for (int q = 0; q < p; ++q) base += cnt[q];
        for (int b = 0; b < nb; ++b) {
            const int n = p < w.np ? phase_items(w, prefix_tiles(kv_len, b, lim), p) : 0;
            table[((size_t)p * nb + b) * 2] = (int32_t)base;
            table[((size_t)p * nb + b) * 2 + 1] = n;
            base += (long long)n * H;
        }
    }
    if (p == 0) {
        long long total = 0;
        for (int q = 0; q < kPhaseMax; ++q) total += cnt[q];
        ws[kWsTicket] = first_ticket;
        ws[kWsTotal] = (int32_t)total;
        ws[kWsC0] = w.c0;
        ws[kWsNp] = w.np;
    }
    for (int b = p; b < nb; b += blockDim.x) {
        const int L = kv_len[b];
        if (L < 0 || L > lim) report(status, b, HCI_DS_KV_LEN);
    }
}

// -------------------------------------------------------------------- host

// Workspace: the header (the queue's ticket counter; from byte kWsTableOff the work-list
// table), then the partials part_o [items][nq][Dh] and part_ml [items][nq][2].
AttnPlan plan_attention(const hci_layer* L, int nb, int nc, int gamma, int max_kv_len, int num_cus)
{
    AttnPlan p{};
    const int P = gamma + 1;
    p.nq = nc * P;
    p.resident = (num_cus > 0 ? num_cus : 1) * kStreamSlots;
    p.kv_lim = max_kv_len;    // callers check max_kv_len + P <= kv_cap before any launch
    const long long tiles = (max_kv_len + kTile - 1) / kTile;
    const long long nbh = (long long)nb * L->heads;
    const int np = worklist_np(worklist_c0(tiles * nbh, p.resident, p.nq));
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
    p.header_bytes = kWsTableOff + up(worklist_table_bytes(nb));
    p.bytes = p.header_bytes + up(p.part_o_elems * 4) + up(p.part_ml_elems * 4);
    return p;
}

// dynamic LDS of the finish kernel: the larger of its two roles
size_t stream_lds_bytes(const hci_layer* L, int nc, int P) {
    const int act_bytes = L->act_dtype == HCI_BF16 ? 2 : 4;
    const size_t conv = conv_iir_lds_floats(L->taps_short, L->taps_outer, nc * P);
    const size_t comb = combine_lds_floats(P, L->head_dim, act_bytes, 16);
    return (conv > comb ? conv : comb) * sizeof(float);
}

// One verify: reset the queue, stream the prefix (bf16: persistent queue kernel; fp32: one
// workgroup per item), then the finish kernel (conv/IIR scan, causal block part, combine).
size_t tree_finish_lds_bytes(const hci_layer* L, int n) {
    const int act_bytes = L->act_dtype == HCI_BF16 ? 2 : 4;
    const size_t conv = tree_conv_lds_bytes(L->taps_short, L->taps_outer, n);
    const size_t comb = combine_lds_floats(n, L->head_dim, act_bytes, 16) * sizeof(float);
    return conv > comb ? conv : comb;
}

hipError_t launch_verify(const hci_layer* L, const hci_state* S, const hci_block* blk,
                         int nb, int nc, int P, const AttnPlan& plan, void* ws, hipStream_t st, hipEvent_t* ev,
                         bool conv, const int32_t* parent)
{
    const int H = L->heads, DH = L->head_dim, nq = plan.nq;
    const float scale_log2 = kLog2e / sqrtf((float)DH);
    unsigned* ticket = (unsigned*)ws;
    int32_t* table = (int32_t*)((char*)ws + kWsTableOff);
    float* part_o = (float*)((char*)ws + plan.header_bytes);
    float* part_ml = (float*)((char*)part_o + (plan.part_o_elems * 4 + 255) / 256 * 256);
    auto mark = [&](int i) { return (ev && ev[i]) ? hipEventRecord(ev[i], st) : hipSuccess; };
    hipError_t e = mark(0);
    if (e != hipSuccess) return e;

    const int stream_blocks = plan.items_cap <= 0 || L->act_dtype != HCI_BF16 ? 0
                              : (plan.items_cap < plan.resident ? plan.items_cap : plan.resident);
    hipLaunchKernelGGL(k_verify_setup, dim3(1), dim3(64), 0, st, (int32_t*)ws, S->kv_len, S->status, nb, H,
                       plan.kv_lim, plan.resident, nq, stream_blocks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = mark(1)) != hipSuccess) return e;
    if (plan.items_cap > 0) {
        if (L->act_dtype == HCI_BF16) {
            StreamArgs A{};
            A.kc = (const uint16_t*)S->k_cache; A.vc = (const uint16_t*)S->v_cache; A.q = (const uint16_t*)blk->q;
            A.kv_len = S->kv_len; A.part_o = part_o; A.part_ml = part_ml; A.ws = (const int32_t*)ws;
            A.ticket = ticket;
            A.H = H; A.kv_cap = S->kv_cap; A.kv_lim = plan.kv_lim; A.nq = nq; A.nb = nb; A.resident = plan.resident;
            A.scale_log2 = scale_log2;
            const int nqt = (nq + 15) / 16;
            e = launch_stream_one(A, DH, nqt, stream_blocks, st);
            if (e != hipSuccess) return e;
        } else {
            hipLaunchKernelGGL(k_attn_prefix_f32, dim3(plan.items_cap), dim3(64), 0, st,
                               (const float*)S->k_cache, (const float*)S->v_cache, S->kv_len,
                               (const float*)blk->q, part_o, part_ml, (const int32_t*)ws, nb, H, DH, S->kv_cap,
                               plan.kv_lim, nq, scale_log2);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    if ((e = mark(2)) != hipSuccess) return e;

    FinishArgs F{};
    F.w_short = L->w_short; F.w_outer = L->w_outer; F.lam = L->lambda; F.beta = L->beta; F.cc = L->c;
    F.short_win = S->short_win; F.outer_win = S->outer_win; F.iir = S->iir; F.x = blk->x;
    F.f_out = blk->f; F.s_out = blk->s; F.y_out = blk->y;
    F.d = L->d; F.Ts = L->taps_short; F.To = L->taps_outer; F.N = L->poles; F.nc = nc;
    F.n_conv = conv ? ((L->d + kCG - 1) / kCG) * nb : 0;
    F.kv_len = S->kv_len; F.part_o = part_o; F.part_ml = part_ml; F.table = table;
    F.q = blk->q; F.kb = blk->k; F.vb = blk->v; F.o = blk->o;
    F.nb = nb; F.H = H; F.DH = DH; F.nq = nq; F.P = P; F.kv_lim = plan.kv_lim; F.resident = plan.resident;
    F.scale_log2 = scale_log2;
    F.parent = parent;
    F.status = S->status;
    const int rg = combine_rows(nb, nc, H, P, plan.resident / kStreamSlots, parent != nullptr);
    F.rg_count = (P + rg - 1) / rg;
    const long long blocks = (long long)F.n_conv + (long long)F.rg_count * nc * H * nb;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const int act_bytes = L->act_dtype == HCI_BF16 ? 2 : 4;
    const size_t conv_lds = !conv ? 0
                            : parent ? tree_conv_lds_bytes(L->taps_short, L->taps_outer, P)
                                     : conv_iir_lds_floats(L->taps_short, L->taps_outer, nc * P) * sizeof(float);
    const size_t comb_lds = combine_lds_floats(P, DH, act_bytes, rg) * sizeof(float);
    const size_t lds = conv_lds > comb_lds ? conv_lds : comb_lds;
    // combine workgroups first when the grid outgrows one round of resident workgroups (4 x 4
    // candidates: finish 45 -> 41 us); conv first when all are resident at once (its chain is
    // the longer one: long context 12.7 against 13.2 us)
    const long long per_cu = lds > 0 && kMaxLds / lds < (size_t)kFinishPerCu ? (long long)(kMaxLds / lds) : kFinishPerCu;
    F.comb_first = blocks > per_cu * (plan.resident / kStreamSlots) ? 1 : 0;
    e = launch_finish(F, L->act_dtype, rg, (int)blocks, lds, st);
    if (e != hipSuccess) return e;
    return mark(3);
}

}  // namespace hci
