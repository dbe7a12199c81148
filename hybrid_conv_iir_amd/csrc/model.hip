// A stack of full hybrid layers verified as one block and sliced layer by
// layer (the StripedHyena2 target of the EvSpark digest: Hyena layers with
// explicit or modal long filters interleaved with attention; Figure 1(a),
// Interpretation; slicing per state class as in Figure 1(d)).
//
// Per layer, on the block rows (nb * nc * P of them):
//   k_rmsnorm        a = bf16(RMSNorm(x) g)
//   k_linear         z = a W_in as three [rows][d] streams (fp32 for Hyena,
//                    bf16 q/k/v for attention)
//   k_hyena_mixer    short FIR of the 3d channels, u = zk * zv, the long
//                    filter (explicit FIR over the u window, or the modal
//                    IIR keeping every s_i), y = bf16(zq * h)
//   (attention)      the verify attention path (KV prefix stream, then the
//                    finish kernel's causal block part and fixed-order merge;
//                    no conv/IIR work)
//   k_linear         x' = bf16(x + y W_out)
// Slicing: k_model_slice (one launch for every layer: both windows, the
// IIR state, accepted K/V rows into the tiled cache, the drafter's window of
// target states), then k_model_slice_len (kv_len += k + 1, after every
// reader of kv_len).
#include "hci_internal.h"

namespace hci {

constexpr int kMxCG = 16;                   // channels per mixer workgroup (16 lanes each)

size_t mixer_lds_bytes(int kind, int Tl, int P) {
    size_t f = 3 * (size_t)P * kMxCG;                                       // zhat [3][P][16]
    if (kind == HCI_MIX_FIR) f += ((size_t)(Tl - 1) + P) * kMxCG + (size_t)Tl * kMxCG;   // u window + u, taps
    else f += (size_t)P * kMxCG;                                            // u
    return f * sizeof(float);
}

template <int KIND>
__global__ __launch_bounds__(256) void k_hyena_mixer(
    const float* __restrict__ z, const float* __restrict__ short_win, const float* __restrict__ long_win,
    const float* __restrict__ iir, const float* __restrict__ w_short, const float* __restrict__ w_long,
    const float* __restrict__ lam, const float* __restrict__ beta, const float* __restrict__ cc,
    uint16_t* __restrict__ y, float* __restrict__ u_out, float* __restrict__ s_out,
    int d, int Ts, int Tl, int N, int nc, int P)
{
    extern __shared__ float lds[];
    const int cg = blockIdx.x, cand = blockIdx.y, b = blockIdx.z;
    const int ch0 = cg * kMxCG;
    const size_t rows = (size_t)gridDim.z * nc * P;
    const size_t row0 = ((size_t)b * nc + cand) * P;
    const int Ws = Ts - 1, Wl = Tl - 1;
    float* zh = lds;                                                        // [3][P][16]
    float* ub = zh + (size_t)3 * P * kMxCG;                                 // FIR: [Wl + P][16], IIR: [P][16]
    float* hl = ub + (size_t)(KIND == HCI_MIX_FIR ? Wl + P : P) * kMxCG;   // FIR: [Tl][16]
    const int tid = threadIdx.x;

    // Every load of the workgroup in one round, to registers first: the short FIR's inputs and
    // taps of the thread's elements (three streams over [window ; block rows]), the long window
    // and taps (FIR kind), the IIR parameters and state (IIR kind).  The loads are unconditional,
    // from clamped (always valid) addresses, and the values are masked where they are used, so
    // they are in flight together (a load under a condition, or a value used right after its
    // load, makes the compiler wait for it there); the batches cover the common sizes, plain
    // loops the rest.
    constexpr int EZ = 3, JT = 4, EL = 8;               // short-FIR elements, short taps, long rows per thread
    const int nz = 3 * P * kMxCG;
    float zv[EZ][JT], zw[EZ][JT];
#pragma unroll
    for (int u = 0; u < EZ; ++u) {
        const int e = min(tid + u * (int)blockDim.x, nz - 1);
        const int c = e % kMxCG, i = (e / kMxCG) % P, sidx = e / (kMxCG * P);
        const int chc = min(ch0 + c, d - 1), col = sidx * d + chc;
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            const int jj = min(j, Ts - 1), m = i - jj;
            const float* src = m >= 0 ? z + ((size_t)sidx * rows + row0 + m) * d + chc
                                      : short_win + ((size_t)b * Ws + (Ws + m)) * 3 * d + col;
            zv[u][j] = *src;
            zw[u][j] = w_short[(size_t)jj * 3 * d + col];
        }
    }
    float lw[EL], lt[EL];
    if (KIND == HCI_MIX_FIR) {
        const int chc = min(ch0 + tid % kMxCG, d - 1);
#pragma unroll
        for (int u = 0; u < EL; ++u) {
            const int r = (tid + u * (int)blockDim.x) / kMxCG;
            lw[u] = Wl > 0 ? long_win[((size_t)b * Wl + min(r, Wl - 1)) * d + chc] : 0.f;
            lt[u] = w_long[(size_t)min(r, Tl - 1) * d + chc];
        }
    }
    // IIR kind: 16 channels x 16 pole lanes
    const int ic = tid >> 4, in = tid & 15, ich = ch0 + ic;
    float il = 0.f, ibt = 0.f, icv = 0.f, is0 = 0.f;
    if (KIND != HCI_MIX_FIR) {
        const size_t o = (size_t)min(ich, d - 1) * N + min(in, N - 1);
        il = lam[o];
        ibt = beta[o];
        icv = cc[o];
        is0 = iir[(size_t)b * d * N + o];
    }
#pragma unroll
    for (int u = 0; u < EZ; ++u) {
        const int e = tid + u * (int)blockDim.x;
        if (e >= nz) break;
        const int c = e % kMxCG, i = (e / kMxCG) % P, sidx = e / (kMxCG * P);
        const int ch = ch0 + c, col = sidx * d + ch;
        float acc = 0.f;
        if (ch < d) {
#pragma unroll
            for (int j = 0; j < JT; ++j)
                if (j < Ts) acc = fmaf(zw[u][j], zv[u][j], acc);
            for (int j = JT; j < Ts; ++j) {
                const int m = i - j;
                const float v = m >= 0 ? z[((size_t)sidx * rows + row0 + m) * d + ch]
                                       : short_win[((size_t)b * Ws + (Ws + m)) * 3 * d + col];
                acc = fmaf(w_short[(size_t)j * 3 * d + col], v, acc);
            }
        }
        zh[e] = acc;
    }
    for (int e = tid + EZ * (int)blockDim.x; e < nz; e += blockDim.x) {
        const int c = e % kMxCG, i = (e / kMxCG) % P, sidx = e / (kMxCG * P);
        const int ch = ch0 + c;
        float acc = 0.f;
        if (ch < d) {
            const int col = sidx * d + ch;
            for (int j = 0; j < Ts; ++j) {
                const int m = i - j;
                const float v = m >= 0 ? z[((size_t)sidx * rows + row0 + m) * d + ch]
                                       : short_win[((size_t)b * Ws + (Ws + m)) * 3 * d + col];
                acc = fmaf(w_short[(size_t)j * 3 * d + col], v, acc);
            }
        }
        zh[e] = acc;
    }
    if (KIND == HCI_MIX_FIR) {
        const bool live = ch0 + tid % kMxCG < d;
#pragma unroll
        for (int u = 0; u < EL; ++u) {
            const int e = tid + u * (int)blockDim.x;
            if (e < Wl * kMxCG) ub[e] = live ? lw[u] : 0.f;
            if (e < Tl * kMxCG) hl[e] = live ? lt[u] : 0.f;
        }
        for (int e = tid + EL * (int)blockDim.x; e < Wl * kMxCG; e += blockDim.x) {
            const int ch = ch0 + e % kMxCG, r = e / kMxCG;
            ub[e] = ch < d ? long_win[((size_t)b * Wl + r) * d + ch] : 0.f;
        }
        for (int e = tid + EL * (int)blockDim.x; e < Tl * kMxCG; e += blockDim.x) {
            const int ch = ch0 + e % kMxCG, j = e / kMxCG;
            hl[e] = ch < d ? w_long[(size_t)j * d + ch] : 0.f;
        }
    }
    __syncthreads();
    const int uo = KIND == HCI_MIX_FIR ? Wl : 0;
    for (int e = tid; e < P * kMxCG; e += blockDim.x) {
        const int c = e % kMxCG, i = e / kMxCG, ch = ch0 + c;
        const float u = zh[((size_t)P + i) * kMxCG + c] * zh[((size_t)2 * P + i) * kMxCG + c];
        ub[(uo + i) * kMxCG + c] = u;
        if (KIND == HCI_MIX_FIR && ch < d) u_out[(row0 + i) * d + ch] = u;
    }
    __syncthreads();
    if (KIND == HCI_MIX_FIR) {
        for (int e = tid; e < P * kMxCG; e += blockDim.x) {
            const int c = e % kMxCG, i = e / kMxCG, ch = ch0 + c;
            if (ch >= d) continue;
            float h = 0.f;
            for (int j = 0; j < Tl; ++j) h = fmaf(hl[j * kMxCG + c], ub[(Wl + i - j) * kMxCG + c], h);
            y[(row0 + i) * d + ch] = f2bf(zh[(size_t)i * kMxCG + c] * h);
        }
    } else {
        // 16 channels x 16 pole lanes (parameters loaded above); the readout sums the pole lanes
        // by butterfly
        const int c = ic, n = in, ch = ich;
        const bool ok = ch < d && n < N;
        const float l = ok ? il : 0.f, bt = ok ? ibt : 0.f, cv = ok ? icv : 0.f;
        float s = ok ? is0 : 0.f;
        for (int i = 0; i < P; ++i) {
            s = fmaf(l, s, bt * ub[i * kMxCG + c]);
            if (ok) s_out[((row0 + i) * d + ch) * N + n] = s;
            // the 16 pole lanes of a channel are one row of the wave: their sum by row rotations
            // on the vector ALU (lane 0 of the row holds a fixed-order result)
            float part = cv * s;
            part += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(part), 0x128, 0xF, 0xF, false));  // row_ror:8
            part += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(part), 0x124, 0xF, 0xF, false));  // row_ror:4
            part += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(part), 0x122, 0xF, 0xF, false));  // row_ror:2
            part += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(part), 0x121, 0xF, 0xF, false));  // row_ror:1
            if (n == 0 && ch < d) y[(row0 + i) * d + ch] = f2bf(zh[(size_t)i * kMxCG + c] * part);
        }
    }
}

// ------------------------------------------------------------------ slicing

__device__ __forceinline__ int accepted_rows(const int32_t* n_acc, const int32_t* best, int b, int nc, int P,
                                             int& cand) {
    int c = best ? best[b] : 0;
    c = c < 0 ? 0 : (c >= nc ? nc - 1 : c);
    int k = n_acc[(size_t)b * nc + c];
    k = k < 0 ? 0 : (k >= P ? P - 1 : k);
    cand = c;
    return k + 1;
}

// All of a slice's copies in one launch: a table of jobs (windows, IIR states, K/V rows, the
// feature buffer) for every layer; blockIdx.x walks the jobs' workgroup ranges, blockIdx.y is the
// sequence.  Windows follow new[r] = [old ; accepted rows][nrow + r]: a workgroup owns 16 columns,
// stages up to 128 rows of the result in LDS and writes them back; chunks go upward, and chunk
// [r0, r0 + 128) only reads old rows at or above r0 + nrow, which no earlier chunk has written.
constexpr int kJobMax = 24;
constexpr int kWinRows = 128;
enum { JOB_WIN_F32 = 0, JOB_WIN_BF16 = 1, JOB_COPY_F32 = 2, JOB_KV = 3 };

struct SliceJob {
    int type, wgs;
    void* dst;                   // window / state / K cache of sequence 0
    void* dst2;                  // V cache (JOB_KV)
    const void* src;             // block rows (row 0 of the block)
    long long dst_b;             // elements between sequences' windows / states
    int W, ncols;                // window rows, columns
    int seg, seg_stride_rows;    // source column t -> segment t / seg at t / seg * seg_stride_rows rows further
};

struct SliceJobs {
    SliceJob job[kJobMax];
    int njobs, nc, P, H, DH, kv_cap;
    long long rows;              // nb * nc * P
};

__global__ __launch_bounds__(256) void k_model_slice(SliceJobs J, const int32_t* __restrict__ n_acc,
                                                     const int32_t* __restrict__ best,
                                                     const int32_t* __restrict__ kv_len)
{
    __shared__ float stage[kWinRows][kMxCG];
    const int b = blockIdx.y;
    int wg = blockIdx.x, j = 0;
    while (j < J.njobs && wg >= J.job[j].wgs) wg -= J.job[j++].wgs;
    if (j >= J.njobs) return;
    const SliceJob& jb = J.job[j];
    int cand;
    const int nrow = accepted_rows(n_acc, best, b, J.nc, J.P, cand);
    const long long row0 = ((long long)b * J.nc + cand) * J.P;

    if (jb.type == JOB_WIN_F32 || jb.type == JOB_WIN_BF16) {
        const int cl = threadIdx.x % kMxCG, part = threadIdx.x / kMxCG;
        const int t = wg * kMxCG + cl;
        const bool live = t < jb.ncols;
        const long long src_col = live ? (long long)(t / jb.seg) * jb.seg_stride_rows * jb.seg + t % jb.seg : 0;
        const int sw = jb.seg;       // source row stride (one segment's width)
        for (int r0 = 0; r0 < jb.W; r0 += kWinRows) {
            const int r1 = min(jb.W, r0 + kWinRows);
            for (int r = r0 + part; r < r1; r += 256 / kMxCG) {
                const int m = nrow + r;
                float v = 0.f;
                if (live) {
                    if (jb.type == JOB_WIN_F32) {
                        const float* win = (const float*)jb.dst + b * jb.dst_b;
                        v = m < jb.W ? win[(long long)m * jb.ncols + t]
                                     : ((const float*)jb.src)[(row0 + m - jb.W) * sw + src_col];
                    } else {
                        const uint16_t* win = (const uint16_t*)jb.dst + b * jb.dst_b;
                        v = bf2f(m < jb.W ? win[(long long)m * jb.ncols + t]
                                          : ((const uint16_t*)jb.src)[(row0 + m - jb.W) * sw + src_col]);
                    }
                }
                stage[r - r0][cl] = v;
            }
            __syncthreads();
            for (int r = r0 + part; r < r1; r += 256 / kMxCG) {
                if (!live) continue;
                if (jb.type == JOB_WIN_F32)
                    ((float*)jb.dst + b * jb.dst_b)[(long long)r * jb.ncols + t] = stage[r - r0][cl];
                else
                    ((uint16_t*)jb.dst + b * jb.dst_b)[(long long)r * jb.ncols + t] = f2bf(stage[r - r0][cl]);
            }
            __syncthreads();
        }
    } else if (jb.type == JOB_COPY_F32) {
        const int e = wg * 256 + threadIdx.x;
        if (e < jb.ncols)
            ((float*)jb.dst + b * jb.dst_b)[e] = ((const float*)jb.src)[(row0 + nrow - 1) * jb.ncols + e];
    } else {
        const int d = J.H * J.DH;
        const int e = wg * 256 + threadIdx.x;                      // (i, h, dd)
        if (e >= J.P * d) return;
        const int i = e / d, hd = e % d, h = hd / J.DH, dd = hd % J.DH;
        const int row = kv_len[b] + i;
        if (i >= nrow || row < 0 || row >= J.kv_cap) return;
        const long long base = ((long long)b * J.H + h) * J.kv_cap * J.DH + (long long)(row & ~(kTile - 1)) * J.DH;
        const uint16_t* z = (const uint16_t*)jb.src;
        ((uint16_t*)jb.dst)[base + k_tile_offset(row & (kTile - 1), dd, J.DH)] = z[(J.rows + row0 + i) * d + hd];
        ((uint16_t*)jb.dst2)[base + v_tile_offset(row & (kTile - 1), dd, J.DH)] = z[(2 * J.rows + row0 + i) * d + hd];
    }
}

__global__ void k_model_slice_len(int32_t* __restrict__ kv_len, const int32_t* __restrict__ n_acc,
                                  const int32_t* __restrict__ best, int nb, int nc, int P, int kv_cap)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nb) return;
    int cand;
    const int L = kv_len[b] + accepted_rows(n_acc, best, b, nc, P, cand);
    kv_len[b] = L > kv_cap ? kv_cap : L;
}

// ------------------------------------------------------------------ host

static hci_layer attn_layer_view(const hci_model* M, const float* dummy) {
    hci_layer L{};
    L.d = M->d;
    L.taps_short = 1;
    L.taps_outer = 1;
    L.poles = 1;
    L.heads = M->heads;
    L.head_dim = M->head_dim;
    L.act_dtype = HCI_BF16;
    L.w_short = L.w_outer = L.lambda = L.beta = L.c = dummy;
    return L;
}

ModelPlan plan_model(const hci_model* M, int nb, int nc, int gamma, int max_kv_len, int num_cus) {
    ModelPlan p{};
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t rows = (size_t)nb * nc * (gamma + 1);
    p.rows = rows;
    p.a_off = 0;
    p.y_off = up(rows * M->d * 2);
    p.attn_off = p.y_off + up(rows * M->d * 2);
    bool has_attn = false;
    for (int l = 0; l < M->n_layers; ++l) has_attn = has_attn || M->layers[l].kind == HCI_MIX_ATTN;
    p.has_attn = has_attn;
    size_t attn = 0;
    if (has_attn) {
        const hci_layer L = attn_layer_view(M, nullptr);
        p.attn = plan_attention(&L, nb, nc, gamma, max_kv_len, num_cus);
        attn = p.attn.bytes;
    }
    p.bytes = p.attn_off + up(attn);
    return p;
}

hipError_t launch_model_verify(const hci_model* M, const hci_model_state* S, const hci_model_block* blk, int nb,
                               int nc, int P, const ModelPlan& plan, void* ws, hipStream_t st)
{
    const int d = M->d;
    const size_t rows = plan.rows;
    uint16_t* a = (uint16_t*)((char*)ws + plan.a_off);
    uint16_t* y = (uint16_t*)((char*)ws + plan.y_off);
    void* attn_ws = (char*)ws + plan.attn_off;
    hipError_t e;
    for (int l = 0; l < M->n_layers; ++l) {
        const hci_mixer& mx = M->layers[l];
        const hci_layer_state& ls = S->layers[l];
        const hci_layer_block& lb = blk->layers[l];
        const uint16_t* xl = (const uint16_t*)blk->x + (size_t)l * rows * d;
        uint16_t* xn = (uint16_t*)blk->x + (size_t)(l + 1) * rows * d;
        if ((e = launch_rmsnorm((int)rows, d, xl, mx.norm, M->eps, a, st)) != hipSuccess) return e;
        if (mx.kind == HCI_MIX_ATTN) {
            if ((e = launch_linear((int)rows, d, 3 * d, 3, a, mx.w_in, nullptr, lb.z, false, st)) != hipSuccess)
                return e;
            const hci_layer L = attn_layer_view(M, mx.norm);
            hci_state SA{};
            SA.kv_cap = S->kv_cap;
            SA.k_cache = ls.k_cache;
            SA.v_cache = ls.v_cache;
            SA.kv_len = S->kv_len;
            hci_block B{};
            B.q = lb.z;
            B.k = (uint16_t*)lb.z + rows * d;
            B.v = (uint16_t*)lb.z + 2 * rows * d;
            B.o = y;
            if ((e = launch_verify(&L, &SA, &B, nb, nc, P, plan.attn, attn_ws, st, nullptr, false)) != hipSuccess)
                return e;
        } else {
            if ((e = launch_linear((int)rows, d, 3 * d, 3, a, mx.w_in, nullptr, lb.z, true, st)) != hipSuccess)
                return e;
            const dim3 grid((d + kMxCG - 1) / kMxCG, nc, nb);
            const size_t lds = mixer_lds_bytes(mx.kind, mx.taps_long, P);
            if (mx.kind == HCI_MIX_FIR)
                hipLaunchKernelGGL(k_hyena_mixer<HCI_MIX_FIR>, grid, dim3(256), lds, st, (const float*)lb.z,
                                   ls.short_win, ls.long_win, ls.iir, mx.w_short, mx.w_long, mx.lambda, mx.beta, mx.c,
                                   y, lb.u, lb.s, d, mx.taps_short, mx.taps_long, mx.poles, nc, P);
            else
                hipLaunchKernelGGL(k_hyena_mixer<HCI_MIX_IIR>, grid, dim3(256), lds, st, (const float*)lb.z,
                                   ls.short_win, ls.long_win, ls.iir, mx.w_short, mx.w_long, mx.lambda, mx.beta, mx.c,
                                   y, lb.u, lb.s, d, mx.taps_short, 1, mx.poles, nc, P);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if ((e = launch_linear((int)rows, d, d, 1, y, mx.w_out, xl, xn, false, st)) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_model_slice(const hci_model* M, const hci_model_state* S, const hci_model_block* blk, int nb,
                              int nc, int P, const int32_t* n_acc, const int32_t* best, hipStream_t st)
{
    const int d = M->d;
    const long long rows = (long long)nb * nc * P;
    SliceJobs J{};
    J.nc = nc;
    J.P = P;
    J.H = M->heads;
    J.DH = M->head_dim;
    J.kv_cap = S->kv_cap;
    J.rows = rows;
    auto win = [&](int type, void* dst, long long dst_b, const void* src, int W, int ncols, int seg, int seg_rows) {
        SliceJob j{};
        j.type = type;
        j.wgs = (ncols + kMxCG - 1) / kMxCG;
        j.dst = dst;
        j.src = src;
        j.dst_b = dst_b;
        j.W = W;
        j.ncols = ncols;
        j.seg = seg;
        j.seg_stride_rows = seg_rows;
        J.job[J.njobs++] = j;
    };
    auto flush = [&]() -> hipError_t {
        if (J.njobs == 0) return hipSuccess;
        long long wgs = 0;
        for (int i = 0; i < J.njobs; ++i) wgs += J.job[i].wgs;
        hipLaunchKernelGGL(k_model_slice, dim3((unsigned)wgs, nb), dim3(256), 0, st, J, n_acc, best, S->kv_len);
        J.njobs = 0;
        return hipGetLastError();
    };
    hipError_t e;
    for (int l = 0; l < M->n_layers; ++l) {
        if (J.njobs + 2 > kJobMax && (e = flush()) != hipSuccess) return e;
        const hci_mixer& mx = M->layers[l];
        const hci_layer_state& ls = S->layers[l];
        const hci_layer_block& lb = blk->layers[l];
        if (mx.kind == HCI_MIX_ATTN) {
            SliceJob j{};
            j.type = JOB_KV;
            j.wgs = (int)((P * (long long)d + 255) / 256);
            j.dst = ls.k_cache;
            j.dst2 = ls.v_cache;
            j.src = lb.z;
            J.job[J.njobs++] = j;
            continue;
        }
        if (mx.taps_short > 1)       // window columns [s d, (s+1) d) come from stream s of z
            win(JOB_WIN_F32, ls.short_win, (long long)(mx.taps_short - 1) * 3 * d, lb.z, mx.taps_short - 1, 3 * d,
                d, (int)rows);
        if (mx.kind == HCI_MIX_FIR) {
            if (mx.taps_long > 1)
                win(JOB_WIN_F32, ls.long_win, (long long)(mx.taps_long - 1) * d, lb.u, mx.taps_long - 1, d, d, 0);
        } else {
            SliceJob j{};
            j.type = JOB_COPY_F32;
            j.ncols = d * mx.poles;
            j.wgs = (j.ncols + 255) / 256;
            j.dst = ls.iir;
            j.dst_b = (long long)d * mx.poles;
            j.src = lb.s;
            J.job[J.njobs++] = j;
        }
    }
    if (J.njobs + 1 > kJobMax && (e = flush()) != hipSuccess) return e;
    const uint16_t* xf = (const uint16_t*)blk->x + (size_t)(M->feature_layer + 1) * rows * d;
    win(JOB_WIN_BF16, S->feature, (long long)M->feature_window * d, xf, M->feature_window, d, d, 0);
    if ((e = flush()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_model_slice_len, dim3((nb + 63) / 64), dim3(64), 0, st, S->kv_len, n_acc, best, nb, nc, P,
                       S->kv_cap);
    return hipGetLastError();
}

}  // namespace hci
