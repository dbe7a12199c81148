// Lossless acceptance of verified blocks (one workgroup per sequence, the
// candidates of a sequence in turn, then the best candidate).
//
// Greedy (ReaDy summary, section 3.1): keep the longest draft prefix equal
// to the target argmax, the next token is the argmax of row k.
// Sampling (ReaDy summary, section D.2; EvSpark digest, Figure 1(c)): the
// ratio test r * q(t) < p(t) left to right in fp64, correction from the
// residual max(0, p_k - q_{k+1}) or bonus from p_gamma, drawn by inverse
// CDF over ascending token ids.  All reductions are fixed-order butterflies
// and a fixed-order LDS pass, so the result does not depend on scheduling.
#include "hci_internal.h"

#include <math.h>
#include <float.h>

namespace hci {

constexpr int kAccT = 256;
constexpr int kAccW = kAccT / 64;

constexpr int kAccRows = 64;     // P <= 64

struct AccScratch {
    double d[kAccW];
    int i[kAccW];
    double d2[kAccW];
    double bcast[4];
    int ibcast[2];
    int arg[kAccRows];             // greedy: argmax per target row
    double gap[kAccRows];          // greedy: top-1 gap per target row
    double pm[kAccRows], ps[kAccRows];   // sampling: target row max / sum
    double qm[kAccRows], qs[kAccRows];   // sampling: draft row max / sum
};

__device__ __forceinline__ double block_sum(double v, AccScratch& sh) {
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.d[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = 0.0;
    for (int w = 0; w < kAccW; ++w) s += sh.d[w];
    return s;
}

__device__ __forceinline__ double block_max(double v, AccScratch& sh) {
    for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.d[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = sh.d[0];
    for (int w = 1; w < kAccW; ++w) s = fmax(s, sh.d[w]);
    return s;
}

__device__ __forceinline__ double block_min(double v, AccScratch& sh) {
    for (int off = 32; off >= 1; off >>= 1) v = fmin(v, __shfl_xor(v, off));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.d[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = sh.d[0];
    for (int w = 1; w < kAccW; ++w) s = fmin(s, sh.d[w]);
    return s;
}

__device__ __forceinline__ int block_imin(int v, AccScratch& sh) {
    for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.i[threadIdx.x >> 6] = v;
    __syncthreads();
    int s = sh.i[0];
    for (int w = 1; w < kAccW; ++w) s = min(s, sh.i[w]);
    return s;
}

__device__ __forceinline__ int block_imax(int v, AccScratch& sh) {
    for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.i[threadIdx.x >> 6] = v;
    __syncthreads();
    int s = sh.i[0];
    for (int w = 1; w < kAccW; ++w) s = max(s, sh.i[w]);
    return s;
}

constexpr int kLaneBatch = 8;   // row entries each lane loads before using any of them

// argmax / runner-up of one fp32 row by ONE wave (lanes stride the row, fixed butterfly)
__device__ void wave_row_argmax(const float* z, int V, int lane, int& arg, double& gap) {
    float b1 = -INFINITY, b2 = -INFINITY;
    int i1 = INT_MAX;
    for (int j0 = 0; j0 < V; j0 += 64 * kLaneBatch) {
        float v[kLaneBatch];
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e) {
            const int j = j0 + e * 64 + lane;
            v[e] = j < V ? z[j] : -INFINITY;
        }
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e) {     // ascending ids per lane
            const int j = j0 + e * 64 + lane;
            if (j < V) {
                if (v[e] > b1) { b2 = b1; b1 = v[e]; i1 = j; }
                else if (v[e] > b2) b2 = v[e];
            }
        }
    }
    for (int off = 32; off >= 1; off >>= 1) {
        const float o1 = __shfl_xor(b1, off), o2 = __shfl_xor(b2, off);
        const int oi = __shfl_xor(i1, off);
        float n1, n2; int ni;
        if (o1 > b1 || (o1 == b1 && oi < i1)) { n1 = o1; ni = oi; n2 = fmaxf(b1, o2); }
        else { n1 = b1; ni = i1; n2 = fmaxf(b2, o1); }
        b1 = n1; b2 = n2; i1 = ni;
    }
    arg = i1;
    gap = (b2 == -INFINITY) ? INFINITY : (double)b1 - (double)b2;
}

// softmax(z / T) statistics of one row by ONE wave: (max of z/T, sum of exp(z/T - max)) in fp64
__device__ void wave_row_stats(const float* z, int V, double T, int lane, double& mx, double& sum) {
    double m = -INFINITY;
    for (int j0 = 0; j0 < V; j0 += 64 * kLaneBatch) {
        float v[kLaneBatch];
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e) {
            const int j = j0 + e * 64 + lane;
            v[e] = j < V ? z[j] : -INFINITY;
        }
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e) m = fmax(m, (double)v[e] / T);
    }
    for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off));
    double s = 0.0;
    for (int j0 = 0; j0 < V; j0 += 64 * kLaneBatch) {
        float v[kLaneBatch];
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e) {
            const int j = j0 + e * 64 + lane;
            v[e] = j < V ? z[j] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e)
            if (j0 + e * 64 + lane < V) s += exp((double)v[e] / T - m);
    }
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    mx = m;
    sum = s;
}

__global__ __launch_bounds__(kAccT) void k_accept(
    int mode, int nc, int gamma, int V, double T,
    const float* __restrict__ zt, const float* __restrict__ zd, const int32_t* __restrict__ drafts,
    const double* __restrict__ uni, int32_t* __restrict__ n_acc, int32_t* __restrict__ next,
    int32_t* __restrict__ best, double* __restrict__ margin_out)
{
    __shared__ AccScratch sh;
    const int b = blockIdx.x;
    const int P = gamma + 1;
    int best_c = 0, best_k = -1;

    for (int c = 0; c < nc; ++c) {
        const size_t blk = (size_t)b * nc + c;
        const float* zt_c = zt + blk * P * V;
        const int32_t* dr = drafts + blk * gamma;
        int k = gamma, nxt = 0;
        double margin = INFINITY;

        const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
        if (mode == HCI_GREEDY) {
            // target rows four at a time (one per wave), stopping at the batch holding the first mismatch
            k = -1;
            for (int i0 = 0; i0 <= gamma && k < 0; i0 += kAccW) {
                const int i = i0 + wv;
                if (i <= gamma) {
                    int g; double gap;
                    wave_row_argmax(zt_c + (size_t)i * V, V, lane, g, gap);
                    if (lane == 0) { sh.arg[i] = g; sh.gap[i] = gap; }
                }
                __syncthreads();
                for (int r = i0; r < i0 + kAccW && r <= gamma; ++r)
                    if (r == gamma || dr[r] != sh.arg[r]) { k = r; break; }
            }
            nxt = sh.arg[k];
            for (int i = 0; i <= k; ++i) margin = fmin(margin, sh.gap[i]);
        } else {
            const float* zd_c = zd + blk * gamma * V;
            const double* u = uni + blk * P;
            // ratio tests two drafts at a time: waves 0,1 take target rows m-1, waves 2,3 draft rows m-1
            k = gamma;
            bool done = false;
            for (int m0 = 1; m0 <= gamma && !done; m0 += kAccW / 2) {
                const int m = m0 + (wv & 1);
                if (m <= gamma) {
                    double mx, sum;
                    if (wv < 2) {
                        wave_row_stats(zt_c + (size_t)(m - 1) * V, V, T, lane, mx, sum);
                        if (lane == 0) { sh.pm[m - 1] = mx; sh.ps[m - 1] = sum; }
                    } else {
                        wave_row_stats(zd_c + (size_t)(m - 1) * V, V, T, lane, mx, sum);
                        if (lane == 0) { sh.qm[m - 1] = mx; sh.qs[m - 1] = sum; }
                    }
                }
                __syncthreads();
                for (int mm = m0; mm < m0 + kAccW / 2 && mm <= gamma; ++mm) {
                    const int t = dr[mm - 1];
                    if (t < 0 || t >= V) { k = mm - 1; done = true; break; }
                    const double p_t = exp((double)zt_c[(size_t)(mm - 1) * V + t] / T - sh.pm[mm - 1]) / sh.ps[mm - 1];
                    const double q_t = exp((double)zd_c[(size_t)(mm - 1) * V + t] / T - sh.qm[mm - 1]) / sh.qs[mm - 1];
                    const double lhs = u[mm - 1] * q_t;
                    margin = fmin(margin, fabs(lhs - p_t) / fmax(p_t, 1e-300));
                    if (!(lhs < p_t)) { k = mm - 1; done = true; break; }
                }
            }
            if (k == gamma) {          // every draft kept: the bonus row p_gamma is still needed
                if (wv == 0) {
                    double mx, sum;
                    wave_row_stats(zt_c + (size_t)gamma * V, V, T, lane, mx, sum);
                    if (lane == 0) { sh.pm[gamma] = mx; sh.ps[gamma] = sum; }
                }
                __syncthreads();
            }
            // weights of the final draw: residual after a rejection, else p_gamma
            const double pm = sh.pm[k], ps = sh.ps[k];
            bool resid = k < gamma;
            const double qm = resid ? sh.qm[k] : 0.0, qs = resid ? sh.qs[k] : 1.0;
            const float* prow = zt_c + (size_t)k * V;
            const float* qrow = zd_c + (size_t)k * V;
            auto weight = [&](int j) {
                const double p = exp((double)prow[j] / T - pm) / ps;
                return resid ? fmax(0.0, p - exp((double)qrow[j] / T - qm) / qs) : p;
            };
            // each thread owns a contiguous run of token ids
            const int per = (V + kAccT - 1) / kAccT;
            const int j0 = min((int)threadIdx.x * per, V), j1 = min(j0 + per, V);
            double loc = 0.0;
            for (int j = j0; j < j1; ++j) loc += weight(j);
            if (resid && !(block_sum(loc, sh) > 0.0)) {   // cannot happen after a rejection; guard only
                resid = false;
                loc = 0.0;
                for (int j = j0; j < j1; ++j) loc += weight(j);
            }
            // exclusive scan of the per-thread totals: Hillis-Steele inside a wave, waves in order
            const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
            double incl = loc;
            for (int off = 1; off < 64; off <<= 1) {
                const double o = __shfl_up(incl, off);
                if (lane >= off) incl += o;
            }
            __syncthreads();
            if (lane == 63) sh.d[wv] = incl;
            __syncthreads();
            double excl = 0.0;
            for (int w = 0; w < wv; ++w) excl += sh.d[w];
            excl += incl - loc;
            // total = the running sum at the last token, exactly as the search below forms it
            double run = excl;
            for (int j = j0; j < j1; ++j) run += weight(j);
            __syncthreads();
            if (j0 < j1 && j1 == V) sh.bcast[0] = run;
            __syncthreads();
            const double total = sh.bcast[0];
            const double target = u[gamma] * total;
            int first = INT_MAX, lastpos = -1;
            double dmin = INFINITY;
            run = excl;
            for (int j = j0; j < j1; ++j) {
                const double w = weight(j);
                run += w;
                if (run > target && first == INT_MAX) first = j;
                if (w > 0.0) lastpos = j;
                dmin = fmin(dmin, fabs(run - target));
            }
            first = block_imin(first, sh);
            lastpos = block_imax(lastpos, sh);
            dmin = block_min(dmin, sh);
            nxt = first != INT_MAX ? first : lastpos;
            margin = fmin(margin, dmin / total);
        }
        if (threadIdx.x == 0) {
            n_acc[blk] = k;
            next[blk] = nxt;
            if (margin_out) margin_out[blk] = margin;
        }
        if (k > best_k) { best_k = k; best_c = c; }
        __syncthreads();
    }
    if (threadIdx.x == 0 && best) best[b] = best_c;
}

hipError_t launch_accept(int mode, int nb, int nc, int gamma, int V, float temperature,
                         const float* zt, const float* zd, const int32_t* drafts, const double* u,
                         int32_t* n_acc, int32_t* next, int32_t* best, double* margin, hipStream_t st)
{
    hipLaunchKernelGGL(k_accept, dim3(nb), dim3(kAccT), 0, st, mode, nc, gamma, V, (double)temperature,
                       zt, zd, drafts, u, n_acc, next, best, margin);
    return hipGetLastError();
}

}  // namespace hci
