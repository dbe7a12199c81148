// Dense projections for the layers around the conv/IIR/attention mixers:
// y = x W (+ residual) with few rows (the verified block: nb * nc * P rows)
// and a large weight, so the weight stream from HBM is the cost and every
// weight byte is read once per call.
//
// The weight is packed once in matrix-core operand order: tiles of 32 (K) x
// 16 (N), the tiles of one 16-column strip stored consecutively, and inside
// a tile element [g<4][n<16][e<8] holding W[32 kt + 8 g + e][16 nt + n], so
// the B operand of v_mfma_f32_16x16x32_bf16 is one contiguous 16-byte load
// per lane (a contiguous kilobyte per wave).  A workgroup owns CT column
// strips and up to 64 rows; its waves split K into contiguous ranges and
// stream their part of the strips with non-temporal loads, one batch of K
// steps in flight behind the one computed; the rows (A operands) come from
// L2; the wave partials are summed in a fixed order through LDS, so results
// do not depend on scheduling.
#include "hci_internal.h"

namespace hci {

constexpr int kLinMT = 4;              // 16-row tiles per workgroup (64 rows)
constexpr int kLinT = 512;             // threads per workgroup: 8 waves split K

__device__ __forceinline__ bf16x8 as_bf16x8_u(u32x4 v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

// K steps per register batch of one wave: BK steps of CT weight fragments and MT row fragments,
// about 64 registers per batch (two batches are held: the one computed and the one in flight)
__host__ __device__ constexpr int linear_batch(int CT, int MT) { return 16 / (CT + MT) > 0 ? 16 / (CT + MT) : 1; }

// One workgroup: CT column strips (16 columns each) x up to 16 * MT rows; its KW waves split
// K into contiguous ranges.  A wave streams its range in batches of BK K steps: the weight
// fragments (non-temporal, a contiguous kilobyte per wave and strip) and the row fragments (from
// L2) of batch i + 1 are requested before batch i's matrix-core products run, so a batch's loads
// are always in flight behind the arithmetic and the wave never waits for a load issued after
// the ones it needs.  Each row fragment feeds CT products.
template <int CT, int MT, bool OUT_F32>
__global__ __launch_bounds__(kLinT) void k_linear(const uint16_t* __restrict__ x, const u32x4* __restrict__ wp,
                                                const uint16_t* __restrict__ res, void* __restrict__ y,
                                                int M, int K, int N, int kspw, int parts, int act)
{
    constexpr int BK = linear_batch(CT, MT);
    constexpr int EPI = (CT * MT * 256 + kLinT - 1) / kLinT;   // epilogue elements per thread
    extern __shared__ float red[];                 // [KW][CT][mts][64][4]
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    constexpr int KW = kLinT / 64;
    const int nt0 = blockIdx.x * CT, row0 = blockIdx.y * 16 * MT;
    const int NT = N >> 4, KT = K >> 5;
    const int kt0 = wv * kspw, kt1 = min(KT, kt0 + kspw);
    const int rl = lane & 15, ko = 8 * (lane >> 4);
    int mts = (M - row0 + 15) >> 4;
    mts = mts > MT ? MT : mts;
    const u32x4* wcol[CT];
    bool cok[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        cok[c] = nt0 + c < NT;
        wcol[c] = wp + (size_t)(cok[c] ? nt0 + c : 0) * KT * 64 + lane;
    }
    f32x4 acc[CT][MT];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[c][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* xr[MT];
    bool ok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int row = row0 + 16 * mt + rl;
        ok[mt] = row < M && mt < mts;
        xr[mt] = x + (size_t)(ok[mt] ? row : 0) * K + ko;
    }
    const int Np = N / parts;
    // the residual of every output this thread writes, requested before the weight stream so it
    // has long arrived when the epilogue needs it
    float rv[EPI];
#pragma unroll
    for (int j = 0; j < EPI; ++j) {
        rv[j] = 0.f;
        const int e = threadIdx.x + kLinT * j;
        if (res && e < CT * MT * 256) {
            const int n = e & 15, g = (e >> 4) & 3, r = (e >> 6) & 3, mt = (e >> 8) % MT, c = e / (256 * MT);
            const int row = row0 + 16 * mt + 4 * g + r;
            if (mt < mts && row < M && nt0 + c < NT) {
                const int col = 16 * (nt0 + c) + n;
                const int p = col / Np;
                rv[j] = bf2f(res[((size_t)p * M + row) * Np + (col - p * Np)]);
            }
        }
    }
    struct Batch {
        u32x4 b[BK][CT];
        u32x4 a[BK][MT];
    };
    // K steps past the wave's range load nothing and contribute zero products
    auto load = [&](Batch& t, int kb) {
#pragma unroll
        for (int u = 0; u < BK; ++u) {
            const bool in = kb + u < kt1;
#pragma unroll
            for (int c = 0; c < CT; ++c)
                t.b[u][c] = in && cok[c] ? __builtin_nontemporal_load(wcol[c] + (size_t)(kb + u) * 64)
                                         : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                t.a[u][mt] = in && ok[mt] ? *(const u32x4*)(xr[mt] + 32 * (kb + u)) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto compute = [&](const Batch& t, int kb) {
#pragma unroll
        for (int u = 0; u < BK; ++u) {
            if (kb + u >= kt1) break;               // past the wave's range: zero fragments
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                if (mt < mts) {
#pragma unroll
                    for (int c = 0; c < CT; ++c)
                        acc[c][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_u(t.a[u][mt]),
                                                                             as_bf16x8_u(t.b[u][c]), acc[c][mt], 0, 0, 0);
                }
        }
    };
    Batch p, q;
    if (kt0 < kt1) load(p, kt0);
    for (int kb = kt0; kb < kt1; kb += 2 * BK) {
        if (kb + BK < kt1) load(q, kb + BK);
        compute(p, kb);
        if (kb + BK >= kt1) break;
        if (kb + 2 * BK < kt1) load(p, kb + 2 * BK);
        compute(q, kb + BK);
    }
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            if (mt < mts)
                *(f32x4*)(red + ((((size_t)wv * CT + c) * mts + mt) * 64 + lane) * 4) = acc[c][mt];
    __syncthreads();
    // element e -> (c, mt, r, g, n): row 16 mt + 4 g + r, column 16 (nt0 + c) + n (columns fastest)
#pragma unroll
    for (int j = 0; j < EPI; ++j) {
        const int e = threadIdx.x + kLinT * j;
        if (e >= CT * MT * 256) break;
        const int n = e & 15, g = (e >> 4) & 3, r = (e >> 6) & 3, mt = (e >> 8) % MT, c = e / (256 * MT);
        const int row = row0 + 16 * mt + 4 * g + r;
        if (mt >= mts || row >= M || nt0 + c >= NT) continue;
        const int ln = 16 * g + n;
        float v = 0.f;
        for (int w = 0; w < KW; ++w) v += red[((((size_t)w * CT + c) * mts + mt) * 64 + ln) * 4 + r];
        const int col = 16 * (nt0 + c) + n;
        const int p = col / Np;
        const size_t o = ((size_t)p * M + row) * Np + (col - p * Np);     // [parts][M][N / parts]
        if (res) v += rv[j];
        if (act == 1) v = v / (1.0f + __expf(-v));                   // SiLU
        if (OUT_F32) ((float*)y)[o] = v;
        else ((uint16_t*)y)[o] = f2bf(v);
    }
}

// w [K][N] bf16 row-major -> packed tiles
__global__ void k_linear_pack(const uint16_t* __restrict__ w, uint16_t* __restrict__ wp, int K, int N)
{
    const size_t total = (size_t)K * N;
    const int KT = K >> 5;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
        const int e = (int)(i & 7), n = (int)((i >> 3) & 15), g = (int)((i >> 7) & 3);
        const size_t tile = i >> 9;
        const int kt = (int)(tile % KT), nt = (int)(tile / KT);
        wp[i] = w[(size_t)(32 * kt + 8 * g + e) * N + 16 * nt + n];
    }
}

// y = x * g / sqrt(mean(x^2) + eps) per row, rounded to bf16; one workgroup per row.  With
// K % 8 == 0 every thread holds 8 consecutive values from one 16-byte load and the row is read
// once; the sum of squares is a fixed butterfly per wave, then the waves in order.
template <bool VEC>
__global__ __launch_bounds__(1024) void k_rmsnorm(const uint16_t* __restrict__ x, const float* __restrict__ gamma,
                                                  float eps, uint16_t* __restrict__ y, int K)
{
    __shared__ float part[16];
    const uint16_t* xr = x + (size_t)blockIdx.x * K;
    uint16_t* yr = y + (size_t)blockIdx.x * K;
    const int nw = blockDim.x >> 6;
    float v[8], g[8];
    float s = 0.f;
    if (VEC) {
        // the row's eight values and their eight gains requested together (clamped, always valid
        // offsets; a thread past K contributes zeros and stores nothing), so the gains are in hand
        // when the sum of squares is
        const int k0 = 8 * threadIdx.x, kc = min(k0, K - 8);
        const u32x4 w = *(const u32x4*)(xr + kc);
        const float4 g0 = *(const float4*)(gamma + kc), g1 = *(const float4*)(gamma + kc + 4);
        g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w;
        g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = k0 < K ? __uint_as_float(ws[i] << 16) : 0.f;
            v[2 * i + 1] = k0 < K ? __uint_as_float(ws[i] & 0xffff0000u) : 0.f;
        }
        for (int i = 0; i < 8; ++i) s = fmaf(v[i], v[i], s);
    } else {
        for (int k = threadIdx.x; k < K; k += blockDim.x) {
            const float t = bf2f(xr[k]);
            s = fmaf(t, t, s);
        }
    }
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < nw; ++w) tot += part[w];
    const float inv = 1.0f / sqrtf(tot / (float)K + eps);
    if (VEC) {
        const int k0 = 8 * threadIdx.x;
        if (k0 < K) {
            uint32_t o[4];
            for (int i = 0; i < 4; ++i)
                o[i] = (uint32_t)f2bf(v[2 * i] * inv * g[2 * i]) |
                       ((uint32_t)f2bf(v[2 * i + 1] * inv * g[2 * i + 1]) << 16);
            *(u32x4*)(yr + k0) = u32x4{o[0], o[1], o[2], o[3]};
        }
    } else {
        for (int k = threadIdx.x; k < K; k += blockDim.x) yr[k] = f2bf(bf2f(xr[k]) * inv * gamma[k]);
    }
}

// Launch shape: CT column strips per workgroup (the largest of 4, 3, 2, 1 that still gives every
// CU a workgroup), up to 64 rows, and eight waves splitting K.  Rows are split over fewer
// 16-row tiles per workgroup while one strip per workgroup would leave CUs idle (a 64-row window
// through a 1024-column weight: 64 workgroups with four row tiles each, or 256 with one): the
// row groups of a strip then read its weight again, from L2 (their workgroups are a multiple of
// eight apart in the grid, so they share an XCD when the strip count is a multiple of eight), and
// every sum keeps its order (the waves' K split does not depend on the rows).
LinearPlan plan_linear(int M, int K, int N) {
    LinearPlan p{};
    const int mts = (M + 15) / 16 < kLinMT ? (M + 15) / 16 : kLinMT;
    p.mt = mts <= 1 ? 1 : (mts <= 2 ? 2 : 4);
    const int NT = N / 16, KT = K / 32;
    const int cus = device_cu_count();
    while (p.mt > 1 && (long long)NT * ((M + 16 * p.mt - 1) / (16 * p.mt)) < cus) p.mt /= 2;
    const int gy = (M + 16 * p.mt - 1) / (16 * p.mt);
    p.ct = 1;
    const int ct_max = p.mt == 4 ? 2 : 4;
    for (int ct = ct_max; ct > 1; --ct)
        if ((long long)((NT + ct - 1) / ct) * gy >= cus) { p.ct = ct; break; }
    // a grid a little over one workgroup per CU runs in two rounds (one workgroup of this kernel
    // fits a CU): more strips per workgroup bring it back to one when that is enough
    // (a 76-row block through a 3072-column weight: 384 -> 192 workgroups)
    if ((long long)((NT + p.ct - 1) / p.ct) * gy > cus)
        for (int ct = p.ct + 1; ct <= ct_max; ++ct)
            if ((long long)((NT + ct - 1) / ct) * gy <= cus) { p.ct = ct; break; }
    p.kw = kLinT / 64;                             // waves past K's end stream nothing
    p.kspw = (KT + p.kw - 1) / p.kw;
    p.lds = (size_t)p.kw * p.ct * (mts < p.mt ? mts : p.mt) * 64 * 4 * sizeof(float);
    p.grid_x = (NT + p.ct - 1) / p.ct;
    p.grid_y = gy;
    return p;
}

template <int CT, int MT, bool OUT_F32>
static hipError_t launch_t(const LinearPlan& p, int M, int K, int N, int parts, const void* x, const void* wp,
                           const void* res, void* y, int act, hipStream_t st)
{
    const void* fn = (const void*)k_linear<CT, MT, OUT_F32>;
    if (p.lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_linear<CT, MT, OUT_F32>), dim3(p.grid_x, p.grid_y), dim3(kLinT), p.lds, st,
                       (const uint16_t*)x, (const u32x4*)wp, (const uint16_t*)res, y, M, K, N, p.kspw, parts, act);
    return hipGetLastError();
}

hipError_t launch_linear(int M, int K, int N, int parts, const void* x, const void* wp, const void* res, void* y,
                         bool out_f32, hipStream_t st, int act)
{
    const LinearPlan p = plan_linear(M, K, N);
#define HCI_LIN_CASE(CT_, MT_)                                                                                    \
    if (p.ct == CT_ && p.mt == MT_)                                                                               \
        return out_f32 ? launch_t<CT_, MT_, true>(p, M, K, N, parts, x, wp, res, y, act, st)                      \
                       : launch_t<CT_, MT_, false>(p, M, K, N, parts, x, wp, res, y, act, st);
    HCI_LIN_CASE(4, 1) HCI_LIN_CASE(4, 2)
    HCI_LIN_CASE(3, 1) HCI_LIN_CASE(3, 2)
    HCI_LIN_CASE(2, 1) HCI_LIN_CASE(2, 2) HCI_LIN_CASE(2, 4)
    HCI_LIN_CASE(1, 1) HCI_LIN_CASE(1, 2) HCI_LIN_CASE(1, 4)
#undef HCI_LIN_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_linear_pack(int K, int N, const void* w, void* wp, hipStream_t st)
{
    const size_t total = (size_t)K * N;
    size_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_linear_pack, dim3((unsigned)blocks), dim3(256), 0, st, (const uint16_t*)w, (uint16_t*)wp,
                       K, N);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(int M, int K, const void* x, const float* g, float eps, void* y, hipStream_t st)
{
    const bool vec = K % 8 == 0 && K <= 8 * 1024 && ((uintptr_t)x % 16) == 0 && ((uintptr_t)y % 16) == 0 &&
                     ((uintptr_t)g % 16) == 0;
    if (vec) {
        const int threads = ((K / 8 + 63) / 64) * 64;
        hipLaunchKernelGGL(k_rmsnorm<true>, dim3(M), dim3(threads), 0, st, (const uint16_t*)x, g, eps, (uint16_t*)y,
                           K);
    } else {
        hipLaunchKernelGGL(k_rmsnorm<false>, dim3(M), dim3(256), 0, st, (const uint16_t*)x, g, eps, (uint16_t*)y, K);
    }
    return hipGetLastError();
}

}  // namespace hci
