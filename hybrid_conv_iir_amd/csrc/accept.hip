// Lossless acceptance of verified blocks: one workgroup per (sequence,
// candidate) block, then the best candidate of each sequence; recursive
// sampling over several candidates takes one workgroup per sequence.
//
// Greedy (ReaDy summary, section 3.1): keep the longest draft prefix equal
// to the target argmax, the next token is the argmax of row k.
// Sampling (ReaDy summary, section D.2; EvSpark digest, Figure 1(c)): the
// ratio test r * q(t) < p(t) left to right in fp64, correction from the
// residual max(0, p_k - q_{k+1}) or bonus from p_gamma, drawn by inverse
// CDF over ascending token ids.  Recursive sampling over several candidate
// blocks (multi-draft recursive rejection) keeps the target distribution
// when the candidates' drafts are independent.  All reductions are
// fixed-order butterflies and a fixed-order LDS pass, so the result does
// not depend on scheduling.
#include "hci_internal.h"
#include "wave_ops.h"

#include <math.h>
#include <float.h>

namespace hci {

constexpr int kAccT = 256;
constexpr int kAccW = kAccT / 64;

constexpr int kAccRows = 64;     // P <= 64

struct AccScratch {
    double d[kAccW];
    int i[kAccW];
    int i2[kAccW];
    double d2[kAccW];
    double bcast[4];
    int ibcast[2];
    int arg[kAccRows];             // greedy: argmax per target row
    double gap[kAccRows];          // greedy: top-1 gap per target row
    double pm[kAccRows], ps[kAccRows];   // sampling: target row max / sum
    double qm[kAccRows], qs[kAccRows];   // sampling: draft row max / sum
    float ztok[kAccRows], dtok[kAccRows]; // sampling: target / draft logit of row m's draft token
    double st[4];                  // recursive: (p max, p sum, q max, q sum) of the current depth
    double cm[kAccRows];           // recursive: per-candidate margin
    int na[kAccRows];              // recursive: per-candidate accepted count
    double zh[kAccRows + 1];       // recursive: residual totals z^(0..r)
    int zapp[kAccRows];            // recursive: whether rejection i changed the residual
    int badrow[kAccRows];          // greedy: row i holds NaN / +Inf or no finite entry
    double uu[kAccRows];           // sampling: the block's uniforms, staged at the start
};

// A row's softmax statistics are usable when its sum is >= 1 (the maximal entry contributes
// exactly 1; a NaN or +Inf entry, or a row with no finite entry, makes the sum NaN).
__device__ __forceinline__ bool row_finite(double sum) { return sum >= 1.0; }

__device__ __forceinline__ double qnan() { return __longlong_as_double(0x7ff8000000000000LL); }

__device__ __forceinline__ double block_sum(double v, AccScratch& sh) {
    v = wave_sum_f64(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.d[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = 0.0;
    for (int w = 0; w < kAccW; ++w) s += sh.d[w];
    return s;
}

__device__ __forceinline__ double block_max(double v, AccScratch& sh) {
    v = wave_max_f64(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.d[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = sh.d[0];
    for (int w = 1; w < kAccW; ++w) s = fmax(s, sh.d[w]);
    return s;
}

__device__ __forceinline__ double block_min(double v, AccScratch& sh) {
    v = wave_min_f64(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.d[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = sh.d[0];
    for (int w = 1; w < kAccW; ++w) s = fmin(s, sh.d[w]);
    return s;
}

__device__ __forceinline__ int block_imin(int v, AccScratch& sh) {
    v = wave_min_i32(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.i[threadIdx.x >> 6] = v;
    __syncthreads();
    int s = sh.i[0];
    for (int w = 1; w < kAccW; ++w) s = min(s, sh.i[w]);
    return s;
}

__device__ __forceinline__ int block_imax(int v, AccScratch& sh) {
    v = wave_max_i32(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.i[threadIdx.x >> 6] = v;
    __syncthreads();
    int s = sh.i[0];
    for (int w = 1; w < kAccW; ++w) s = max(s, sh.i[w]);
    return s;
}

constexpr int kLaneBatch = 8;   // row entries each lane loads before using any of them

// argmax / runner-up of one fp32 row by ONE wave (lanes stride the row, fixed butterfly);
// bad = the row holds a NaN or +Inf entry or no entry above -Inf
__device__ void wave_row_argmax(const float* z, int V, int lane, int& arg, double& gap, bool& bad) {
    float b1 = -INFINITY, b2 = -INFINITY;
    int i1 = INT_MAX;
    bool nonfin = false;
    for (int j0 = 0; j0 < V; j0 += 64 * kLaneBatch) {
        float v[kLaneBatch];
        // unconditional loads from clamped ids (no branch around a load, so the batch stays in
        // flight), masked afterwards
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e) v[e] = z[min(j0 + e * 64 + lane, V - 1)];
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e)
            if (j0 + e * 64 + lane >= V) v[e] = -INFINITY;
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e) {     // ascending ids per lane
            const int j = j0 + e * 64 + lane;
            if (j < V) {
                nonfin |= (v[e] != v[e]) | (v[e] == INFINITY);
                if (v[e] > b1) { b2 = b1; b1 = v[e]; i1 = j; }
                else if (v[e] > b2) b2 = v[e];
            }
        }
    }
    // merge with a partner lane's (best, index, runner-up): the same result on both lanes
    auto merge = [&](float o1, float o2, int oi) {
        float n1, n2; int ni;
        if (o1 > b1 || (o1 == b1 && oi < i1)) { n1 = o1; ni = oi; n2 = fmaxf(b1, o2); }
        else { n1 = b1; ni = i1; n2 = fmaxf(b2, o1); }
        b1 = n1; b2 = n2; i1 = ni;
    };
    merge(dpp_f32<kQuadSwap1>(b1), dpp_f32<kQuadSwap1>(b2), (int)dpp_u32<kQuadSwap1>((uint32_t)i1));
    merge(dpp_f32<kQuadSwap2>(b1), dpp_f32<kQuadSwap2>(b2), (int)dpp_u32<kQuadSwap2>((uint32_t)i1));
    merge(dpp_f32<kHalfMirror>(b1), dpp_f32<kHalfMirror>(b2), (int)dpp_u32<kHalfMirror>((uint32_t)i1));
    merge(dpp_f32<kRowMirror>(b1), dpp_f32<kRowMirror>(b2), (int)dpp_u32<kRowMirror>((uint32_t)i1));
    {
        // the row swaps return (own, partner) in even rows (halves) and (partner, own) in odd ones
        uint32_t a1, c1, a2, c2, ai, ci;
        swap_pair<false>(__float_as_uint(b1), a1, c1);
        swap_pair<false>(__float_as_uint(b2), a2, c2);
        swap_pair<false>((uint32_t)i1, ai, ci);
        const bool first_own = (threadIdx.x & 16) == 0;
        merge(__uint_as_float(first_own ? c1 : a1), __uint_as_float(first_own ? c2 : a2), (int)(first_own ? ci : ai));
        swap_pair<true>(__float_as_uint(b1), a1, c1);
        swap_pair<true>(__float_as_uint(b2), a2, c2);
        swap_pair<true>((uint32_t)i1, ai, ci);
        const bool first_own32 = (threadIdx.x & 32) == 0;
        merge(__uint_as_float(first_own32 ? c1 : a1), __uint_as_float(first_own32 ? c2 : a2),
              (int)(first_own32 ? ci : ai));
    }
    arg = i1;
    gap = (b2 == -INFINITY) ? INFINITY : (double)b1 - (double)b2;
    bad = __builtin_amdgcn_ballot_w64(nonfin) != 0ull || b1 == -INFINITY;
}

// softmax(z / T) statistics of one row by ONE wave: (max of z/T, sum of exp(z/T - max)) in fp64.
// A row of at most 64 kLaneBatch entries is loaded once (the same values in the same order as
// the two-pass form); the lane holding entry tok (if 0 <= tok < V) stores it to *ztok.
// ecache (rows of at most 64 kLaneBatch entries only; may be null): receives exp(z_j / T - max)
// for every entry j < V, the values the sum adds, for a later draw from the same row.
__device__ void wave_row_stats(const float* z, int V, double T, int lane, double& mx, double& sum,
                               int tok = -1, float* ztok = nullptr, double* ecache = nullptr) {
    if (V <= 64 * kLaneBatch) {
        // unconditional loads from clamped ids (no branch around a load and no use of a value
        // before the last load is issued, so the batch stays in flight), masked afterwards
        float v[kLaneBatch];
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e) v[e] = z[min(e * 64 + lane, V - 1)];
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e) {
            const int j = e * 64 + lane;
            if (j >= V) v[e] = -INFINITY;
            if (ztok && j == tok) *ztok = v[e];
        }
        double xs[kLaneBatch];
        double m = -INFINITY;
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e) {
            xs[e] = over_T((double)v[e], T);
            m = fmax(m, xs[e]);
        }
        m = wave_max_f64(m);
        double s = 0.0;
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e)
            if (e * 64 + lane < V) {
                const double ex = exp(xs[e] - m);
                s += ex;
                if (ecache) ecache[e * 64 + lane] = ex;
            }
        mx = m;
        sum = wave_sum_f64(s);
        return;
    }
    double m = -INFINITY;
    for (int j0 = 0; j0 < V; j0 += 64 * kLaneBatch) {
        float v[kLaneBatch];
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e) v[e] = z[min(j0 + e * 64 + lane, V - 1)];
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e)
            if (j0 + e * 64 + lane >= V) v[e] = -INFINITY;
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e) {
            m = fmax(m, over_T((double)v[e], T));
            if (ztok && j0 + e * 64 + lane == tok) *ztok = v[e];
        }
    }
    m = wave_max_f64(m);
    double s = 0.0;
    for (int j0 = 0; j0 < V; j0 += 64 * kLaneBatch) {
        float v[kLaneBatch];
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e) v[e] = z[min(j0 + e * 64 + lane, V - 1)];
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e)
            if (j0 + e * 64 + lane >= V) v[e] = 0.f;
#pragma unroll
        for (int e = 0; e < kLaneBatch; ++e)
            if (j0 + e * 64 + lane < V) s += exp(over_T((double)v[e], T) - m);
    }
    mx = m;
    sum = wave_sum_f64(s);
}


// Inverse-CDF draw over token ids with weights weight(j) >= 0: the smallest j whose running sum
// exceeds r x total (total = the running sum at the last token, formed exactly as the search
// forms it), else the last token with positive weight.  Every thread owns a contiguous run of
// ids; the run totals are scanned in a fixed order (a scan inside each wave, then the waves'
// totals in wave order).  Returns the token, the distance of the nearest running sum from the
// threshold relative to the total, and the total (0 when every weight is 0: no token is drawn
// then, token = -1).

// exclusive prefix of the thread's run total loc over the workgroup, in a fixed order
__device__ __forceinline__ double block_excl_scan(double loc, AccScratch& sh) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const double incl = wave_incl_scan_f64(loc, lane);
    __syncthreads();                                   // earlier readers of sh.d are done
    if (lane == 63) sh.d[wv] = incl;
    __syncthreads();
    double excl = 0.0;
    for (int w = 0; w < wv; ++w) excl += sh.d[w];
    return excl + (incl - loc);
}

// the draw's workgroup-wide result from every thread's (first crossing, last positive id,
// nearest distance): one exchange through LDS
__device__ __forceinline__ void draw_result(int first, int lastpos, double dmin, double total, AccScratch& sh,
                                            int& token, double& margin) {
    first = wave_min_i32(first);
    lastpos = wave_max_i32(lastpos);
    dmin = wave_min_f64(dmin);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    if (lane == 0) {
        sh.i[wv] = first;
        sh.i2[wv] = lastpos;
        sh.d2[wv] = dmin;
    }
    __syncthreads();
    first = sh.i[0];
    lastpos = sh.i2[0];
    dmin = sh.d2[0];
    for (int w = 1; w < kAccW; ++w) {
        first = min(first, sh.i[w]);
        lastpos = max(lastpos, sh.i2[w]);
        dmin = fmin(dmin, sh.d2[w]);
    }
    token = first != INT_MAX ? first : lastpos;
    margin = dmin / total;
}

template <typename F>
__device__ void draw_token(F weight, int V, double r, AccScratch& sh, int& token, double& margin,
                           double* total_out = nullptr)
{
    const int per = (V + kAccT - 1) / kAccT;
    const int j0 = min((int)threadIdx.x * per, V), j1 = min(j0 + per, V);
    double loc = 0.0;
    for (int j = j0; j < j1; ++j) loc += weight(j);
    const double excl = block_excl_scan(loc, sh);
    double run = excl;
    for (int j = j0; j < j1; ++j) run += weight(j);
    if (j0 < j1 && j1 == V) sh.bcast[0] = run;
    __syncthreads();
    const double total = sh.bcast[0];
    const double target = r * total;
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
    draw_result(first, lastpos, dmin, total, sh, token, margin);
    if (total_out) *total_out = total;
}


// draw_token with the weights of the thread's run of ids [j0, j1) (j1 - j0 <= kDrawCache,
// j0 = threadIdx.x * ceil(V / kAccT)) already in registers: the same sums in the same order
// as draw_token, without evaluating (and loading) every weight three times.
constexpr int kDrawCache = 4;
__device__ void draw_token_cached(const double (&wc)[kDrawCache], int V, double r, AccScratch& sh, int& token,
                                  double& margin, double* total_out = nullptr)
{
    const int per = (V + kAccT - 1) / kAccT;
    const int j0 = min((int)threadIdx.x * per, V), j1 = min(j0 + per, V);
    double loc = 0.0;
#pragma unroll
    for (int u = 0; u < kDrawCache; ++u)
        if (j0 + u < j1) loc += wc[u];
    const double excl = block_excl_scan(loc, sh);
    double run = excl;
#pragma unroll
    for (int u = 0; u < kDrawCache; ++u)
        if (j0 + u < j1) run += wc[u];
    if (j0 < j1 && j1 == V) sh.bcast[0] = run;
    __syncthreads();
    const double total = sh.bcast[0];
    const double target = r * total;
    int first = INT_MAX, lastpos = -1;
    double dmin = INFINITY;
    run = excl;
#pragma unroll
    for (int u = 0; u < kDrawCache; ++u) {
        const int j = j0 + u;
        if (j < j1) {
            const double w = wc[u];
            run += w;
            if (run > target && first == INT_MAX) first = j;
            if (w > 0.0) lastpos = j;
            dmin = fmin(dmin, fabs(run - target));
        }
    }
    draw_result(first, lastpos, dmin, total, sh, token, margin);
    if (total_out) *total_out = total;
}

// Residual weight of one token after r rejections at the current depth: w^(0) = p,
// w^(i+1) = max(0, w^(i) - z^(i) q) when rejection i changed the residual (z^(0) = 1,
// z^(i+1) = the total of w^(i+1)).  The product z q is rounded before the subtraction.
__device__ __forceinline__ double residual_weight(double p, double q, int r, const AccScratch& sh) {
    double w = p;
    for (int i = 0; i < r; ++i)
        if (sh.zapp[i]) w = fmax(0.0, w - __dmul_rn(sh.zh[i], q));
    return w;
}

// Recursive acceptance over the candidates of sequence b (several drafts per depth): at depth k
// the alive candidates share the accepted prefix and the lowest-index one supplies p and q; they
// are tried in index order against the running residual; the first kept draft extends the
// prefix, and if all are rejected the next token is drawn from the residual.  The multi-draft
// generalisation of the ReaDy summary's section D.2 rule (the pages give no rule for several
// candidates); with one candidate it is the one-candidate rule bit for bit.
__device__ void accept_recursive(int b, int nc, int gamma, int V, double T,
                                 const float* __restrict__ zt, const float* __restrict__ zd,
                                 const int32_t* __restrict__ drafts, const double* __restrict__ uni,
                                 int32_t* __restrict__ n_acc, int32_t* __restrict__ next,
                                 int32_t* __restrict__ best, double* __restrict__ margin_out,
                                 uint32_t* __restrict__ status, AccScratch& sh)
{
    const int P = gamma + 1;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    unsigned long long alive = nc == 64 ? ~0ull : ((1ull << nc) - 1ull);
    if (threadIdx.x < nc) {
        sh.cm[threadIdx.x] = INFINITY;
        sh.na[threadIdx.x] = 0;
    }
    int k = 0, nrej = 0, rep = 0;
    bool bad = false;
    uint32_t flags = 0u;
    const float* prow = nullptr;
    const float* qrow = nullptr;
    for (;;) {
        rep = __ffsll((long long)alive) - 1;
        const size_t rb = (size_t)b * nc + rep;
        prow = zt + (rb * P + k) * V;
        qrow = k < gamma ? zd + (rb * gamma + k) * V : nullptr;
        nrej = 0;
        __syncthreads();
        if (wv == 0 || (wv == 1 && k < gamma)) {
            double mx, sum;
            wave_row_stats(wv == 0 ? prow : qrow, V, T, lane, mx, sum);
            if (lane == 0) {
                sh.st[2 * wv] = mx;
                sh.st[2 * wv + 1] = sum;
            }
        }
        if (threadIdx.x == 0) sh.zh[0] = 1.0;
        __syncthreads();
        if (!row_finite(sh.st[1]) || (k < gamma && !row_finite(sh.st[3]))) {   // uniform: read from LDS
            bad = true;
            break;
        }
        if (k == gamma) break;                       // the alive path kept every draft: bonus from p_gamma
        const double pm = sh.st[0], ps = sh.st[1], qm = sh.st[2], qs = sh.st[3];
        int kept = -1;
        for (int c = 0; c < nc && kept < 0; ++c) {
            if (!((alive >> c) & 1ull)) continue;
            const int t = drafts[((size_t)b * nc + c) * gamma + k];
            if (t < 0 || t >= V) flags |= HCI_DS_DRAFT_ID;
            if (t >= 0 && t < V) {
                const double p_t = exp(over_T((double)prow[t], T) - pm) / ps;
                const double q_t = exp(over_T((double)qrow[t], T) - qm) / qs;
                const double lhs = uni[((size_t)b * nc + c) * P + k] * q_t * sh.zh[nrej];
                const double rhs = residual_weight(p_t, q_t, nrej, sh);
                if (threadIdx.x == 0) sh.cm[c] = fmin(sh.cm[c], fabs(lhs - rhs) / fmax(rhs, 1e-300));
                if (lhs < rhs) {
                    kept = t;
                    break;
                }
            }
            // rejection: total of max(0, w - z q) over the vocabulary
            const double z = sh.zh[nrej];
            double loc = 0.0;
            for (int j = threadIdx.x; j < V; j += kAccT) {
                const double q = exp(over_T((double)qrow[j], T) - qm) / qs;
                const double w = residual_weight(exp(over_T((double)prow[j], T) - pm) / ps, q, nrej, sh);
                loc += fmax(0.0, w - __dmul_rn(z, q));
            }
            const double tot = block_sum(loc, sh);
            __syncthreads();
            if (threadIdx.x == 0) {
                const bool ok = tot > 0.0;            // cannot fail after a rejection; guard only
                sh.zapp[nrej] = ok ? 1 : 0;
                sh.zh[nrej + 1] = ok ? tot : z;
            }
            __syncthreads();
            ++nrej;
        }
        if (kept < 0) break;
        for (int c = 0; c < nc; ++c) {
            if (((alive >> c) & 1ull) && drafts[((size_t)b * nc + c) * gamma + k] != kept) {
                if (threadIdx.x == 0) sh.na[c] = k;
                alive &= ~(1ull << c);
            }
        }
        ++k;
    }
    if (bad) {                                       // nothing is committed for this sequence
        for (int c = threadIdx.x; c < nc; c += kAccT) {
            const size_t o = (size_t)b * nc + c;
            n_acc[o] = -1;
            next[o] = -1;
            if (margin_out) margin_out[o] = qnan();
        }
        if (threadIdx.x == 0) {
            if (best) best[b] = -1;
            report(status, b, flags | HCI_DS_NONFINITE);
        }
        return;
    }
    if (threadIdx.x == 0) report(status, b, flags);
    const double pm = sh.st[0], ps = sh.st[1], qm = sh.st[2], qs = sh.st[3];
    const int r = nrej;
    auto weight = [&](int j) {
        const double p = exp(over_T((double)prow[j], T) - pm) / ps;
        return r == 0 ? p : residual_weight(p, exp(over_T((double)qrow[j], T) - qm) / qs, r, sh);
    };
    int tok;
    double m2;
    draw_token(weight, V, uni[(size_t)b * nc * P + gamma], sh, tok, m2);
    __syncthreads();
    if (threadIdx.x == 0) sh.cm[rep] = fmin(sh.cm[rep], m2);
    __syncthreads();
    for (int c = threadIdx.x; c < nc; c += kAccT) {
        const size_t o = (size_t)b * nc + c;
        n_acc[o] = ((alive >> c) & 1ull) ? k : sh.na[c];
        next[o] = tok;
        if (margin_out) margin_out[o] = sh.cm[c];
    }
    if (threadIdx.x == 0 && best) best[b] = rep;
}

// Recursive acceptance: one workgroup per sequence (the candidates are tried in turn at every depth).
__global__ __launch_bounds__(kAccT) void k_accept_recursive(
    int nc, int gamma, int V, double T,
    const float* __restrict__ zt, const float* __restrict__ zd, const int32_t* __restrict__ drafts,
    const double* __restrict__ uni, int32_t* __restrict__ n_acc, int32_t* __restrict__ next,
    int32_t* __restrict__ best, double* __restrict__ margin_out, uint32_t* __restrict__ status)
{
    __shared__ AccScratch sh;
    accept_recursive(blockIdx.x, nc, gamma, V, T, zt, zd, drafts, uni, n_acc, next, best, margin_out, status, sh);
}

// Greedy and one-candidate sampling: one workgroup per (sequence, candidate) block, blockIdx.x =
// b * nc + c; the candidates of a sequence are independent, so they run side by side.  With one
// candidate the best is candidate 0; otherwise k_accept_best picks it.
__global__ __launch_bounds__(kAccT) void k_accept(
    int mode, int nc, int gamma, int V, double T,
    const float* __restrict__ zt, const float* __restrict__ zd, const int32_t* __restrict__ drafts,
    const double* __restrict__ uni, int32_t* __restrict__ n_acc, int32_t* __restrict__ next,
    int32_t* __restrict__ best, double* __restrict__ margin_out, uint32_t* __restrict__ status)
{
    __shared__ AccScratch sh;
    // rows of at most 64 kLaneBatch tokens: the exp terms of the four rows a ratio step reads
    // (target rows m0 - 1, m0; draft rows m0 - 1, m0), kept for the final draw
    __shared__ double ecache[kAccW][64 * kLaneBatch];
    const int P = gamma + 1;
    {
        const size_t blk = blockIdx.x;
        const size_t b = blk / nc;
        const float* zt_c = zt + blk * P * V;
        const int32_t* dr = drafts + blk * gamma;
        int k = gamma, nxt = 0;
        double margin = INFINITY;
        bool bad = false;                  // a row the decision used is not finite
        uint32_t flags = 0u;

        const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
        if (mode == HCI_GREEDY) {
            // target rows four at a time (one per wave), stopping at the batch holding the first mismatch
            k = -1;
            for (int i0 = 0; i0 <= gamma && k < 0; i0 += kAccW) {
                const int i = i0 + wv;
                if (i <= gamma) {
                    int g; double gap; bool rb;
                    wave_row_argmax(zt_c + (size_t)i * V, V, lane, g, gap, rb);
                    if (lane == 0) { sh.arg[i] = g; sh.gap[i] = gap; sh.badrow[i] = rb ? 1 : 0; }
                }
                __syncthreads();
                for (int r = i0; r < i0 + kAccW && r <= gamma; ++r)
                    if (r == gamma || dr[r] != sh.arg[r]) { k = r; break; }
            }
            nxt = sh.arg[k];
            for (int i = 0; i <= k; ++i) {
                margin = fmin(margin, sh.gap[i]);
                bad |= sh.badrow[i] != 0;
            }
            if (k < gamma && (dr[k] < 0 || dr[k] >= V)) flags |= HCI_DS_DRAFT_ID;
        } else {
            const float* zd_c = zd + blk * gamma * V;
            const double* u = uni + blk * P;
            // ratio tests two drafts at a time: waves 0,1 take target rows m-1, waves 2,3 draft rows m-1
            const bool cached = V <= 64 * kLaneBatch;
            // the uniforms are staged before the first row statistics (whose barrier publishes
            // them), so neither the ratio tests nor the draw waits on a global load
            if ((int)threadIdx.x < P) sh.uu[threadIdx.x] = u[threadIdx.x];
            k = gamma;
            bool done = false;
            int m_last = 1;                    // m0 of the last ratio step (its rows are in ecache)
            for (int m0 = 1; m0 <= gamma && !done; m0 += kAccW / 2) {
                const int m = m0 + (wv & 1);
                m_last = m0;
                if (m <= gamma) {
                    double mx, sum;
                    const int tok = dr[m - 1];
                    if (wv < 2) {
                        wave_row_stats(zt_c + (size_t)(m - 1) * V, V, T, lane, mx, sum, tok, &sh.ztok[m - 1],
                                       cached ? ecache[wv] : nullptr);
                        if (lane == 0) { sh.pm[m - 1] = mx; sh.ps[m - 1] = sum; }
                    } else {
                        wave_row_stats(zd_c + (size_t)(m - 1) * V, V, T, lane, mx, sum, tok, &sh.dtok[m - 1],
                                       cached ? ecache[wv] : nullptr);
                        if (lane == 0) { sh.qm[m - 1] = mx; sh.qs[m - 1] = sum; }
                    }
                }
                __syncthreads();
                for (int mm = m0; mm < m0 + kAccW / 2 && mm <= gamma; ++mm) {
                    const int t = dr[mm - 1];
                    if (t < 0 || t >= V) { k = mm - 1; done = true; flags |= HCI_DS_DRAFT_ID; break; }
                    const double p_t = exp(over_T((double)sh.ztok[mm - 1], T) - sh.pm[mm - 1]) / sh.ps[mm - 1];
                    const double q_t = exp(over_T((double)sh.dtok[mm - 1], T) - sh.qm[mm - 1]) / sh.qs[mm - 1];
                    const double lhs = sh.uu[mm - 1] * q_t;
                    margin = fmin(margin, fabs(lhs - p_t) / fmax(p_t, 1e-300));
                    if (!(lhs < p_t)) { k = mm - 1; done = true; break; }
                }
            }
            if (k == gamma) {          // every draft kept: the bonus row p_gamma is still needed
                if (wv == 0) {
                    double mx, sum;
                    wave_row_stats(zt_c + (size_t)gamma * V, V, T, lane, mx, sum, -1, nullptr,
                                   cached ? ecache[0] : nullptr);
                    if (lane == 0) { sh.pm[gamma] = mx; sh.ps[gamma] = sum; }
                }
                __syncthreads();
            }
            // the cached exp terms of row k: target row k in slot k - (m_last - 1), draft row k two
            // slots further (the bonus row p_gamma in slot 0)
            const double* ct = cached ? ecache[k == gamma ? 0 : k - (m_last - 1)] : nullptr;
            const double* cq = cached && k < gamma ? ecache[2 + k - (m_last - 1)] : nullptr;
            // the rows the decision used: target rows 0..k, draft rows 0..min(k, gamma - 1)
            for (int i = 0; i <= k; ++i) bad |= !row_finite(sh.ps[i]) || (i < gamma && !row_finite(sh.qs[i]));
            // weights of the final draw: residual after a rejection, else p_gamma
            const double pm = sh.pm[k], ps = sh.ps[k];
            bool resid = k < gamma;
            const double qm = resid ? sh.qm[k] : 0.0, qs = resid ? sh.qs[k] : 1.0;
            const float* prow = zt_c + (size_t)k * V;
            const float* qrow = zd_c + (size_t)k * V;
            auto weight = [&](int j) {
                const double p = (ct ? ct[j] : exp(over_T((double)prow[j], T) - pm)) / ps;
                return resid ? fmax(0.0, p - (cq ? cq[j] : exp(over_T((double)qrow[j], T) - qm)) / qs) : p;
            };
            const int per = (V + kAccT - 1) / kAccT;
            const int j0 = min((int)threadIdx.x * per, V), j1 = min(j0 + per, V);
            int tok;
            double m2, tot;
            // an empty residual cannot follow a rejection (guard only): the draw then falls back
            // to p_k itself
            if (per <= kDrawCache) {
                // every weight of the thread's run evaluated once (its logits loaded once)
                double wc[kDrawCache];
#pragma unroll
                for (int uu = 0; uu < kDrawCache; ++uu) wc[uu] = j0 + uu < j1 ? weight(j0 + uu) : 0.0;
                draw_token_cached(wc, V, sh.uu[gamma], sh, tok, m2, &tot);
                if (resid && !(tot > 0.0)) {
                    resid = false;
#pragma unroll
                    for (int uu = 0; uu < kDrawCache; ++uu) wc[uu] = j0 + uu < j1 ? weight(j0 + uu) : 0.0;
                    draw_token_cached(wc, V, sh.uu[gamma], sh, tok, m2);
                }
            } else {
                draw_token(weight, V, sh.uu[gamma], sh, tok, m2, &tot);
                if (resid && !(tot > 0.0)) {
                    resid = false;
                    draw_token(weight, V, sh.uu[gamma], sh, tok, m2);
                }
            }
            nxt = tok;
            margin = fmin(margin, m2);
        }
        if (threadIdx.x == 0) {
            n_acc[blk] = bad ? -1 : k;
            next[blk] = bad ? -1 : nxt;
            if (margin_out) margin_out[blk] = bad ? qnan() : margin;
            if (nc == 1 && best) best[b] = bad ? -1 : 0;
            report(status, b, flags | (bad ? HCI_DS_NONFINITE : 0u));
        }
    }
}

// ------------------------------------------------------------------ token trees
//
// Acceptance over a token tree of n <= 64 nodes per sequence (node 0 the anchor, parent p(m) < m;
// several candidate blocks that share prefixes: EvSpark digest, Interpretation; tree verification:
// ReaDy summary, section 5).  One workgroup per sequence walks from the anchor:
//   greedy: at node m the target row's argmax is compared with m's children in index order and
//     the first child holding it becomes the current node; otherwise the argmax is emitted.
//   sampling: m's children are tried in index order against the running residual w / z of the
//     target row p (w = p, z = 1): child c, token t, drawn from q_c = softmax(draft row c / T), is
//     kept iff r_c q_c(t) z < w(t); a rejection sets w <- max(0, w - z q_c), z <- sum w.  A kept
//     child becomes the current node; if all are rejected the next token is drawn from w, and at
//     a node without children from p, with r* = u[b][0] (multi-step speculative sampling with one
//     draft distribution per child).
// Outputs per sequence: n_accepted = depth of the accepted node, path[0..k] = its nodes from the
// anchor (entries past k are -1), next_token, margin.

constexpr int kTreeNodes = 64;

struct TreeAccScratch {
    AccScratch a;
    int par[kTreeNodes], first[kTreeNodes], sib[kTreeNodes], path[kTreeNodes];
    int rnode[kTreeNodes];               // rejected children at the current node, in order
    double rqm[kTreeNodes], rqs[kTreeNodes];
    double zh[kTreeNodes + 1];
    int zapp[kTreeNodes];
    double pst[2], qst[2];
    int flag;
    // greedy: every target row's argmax, top-1 gap and bad-row flag, taken before the walk;
    // sampling: the row statistics (max, sum of exp) of the rows the walk visits, per node
    int garg[kTreeNodes], gbad[kTreeNodes];
    double ggap[kTreeNodes];
    double pm_[kTreeNodes], ps_[kTreeNodes], qm_[kTreeNodes], qs_[kTreeNodes];
    float zp_[kTreeNodes], zq_[kTreeNodes];  // node c's drafted token in its parent's target row / its draft row
};

__global__ __launch_bounds__(kAccT) void k_accept_tree(
    int mode, int n, int V, double T, const int32_t* __restrict__ parent, const int32_t* __restrict__ tokens,
    const float* __restrict__ zt, const float* __restrict__ zd, const double* __restrict__ uni,
    int32_t* __restrict__ n_acc, int32_t* __restrict__ path_out, int32_t* __restrict__ next,
    double* __restrict__ margin_out, uint32_t* __restrict__ status)
{
    __shared__ TreeAccScratch sh;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int32_t* tok = tokens + (size_t)b * n;
    // the tree in LDS: parents (validated), then first child / next sibling lists in index order
    if (tid == 0) sh.flag = 1;
    __syncthreads();
    if (tid < n) {
        const int p = parent[(size_t)b * n + tid];
        const bool ok = tid == 0 ? p == -1 : (p >= 0 && p < tid);
        if (!ok) sh.flag = 0;
        sh.par[tid] = ok ? p : -1;
        sh.first[tid] = -1;
        sh.sib[tid] = -1;
        sh.path[tid] = -1;
    }
    __syncthreads();
    if (tid == 0) {
        for (int c = n - 1; c >= 1; --c) {            // prepend in descending order: lists ascend
            const int p = sh.par[c];
            if (p >= 0) {
                sh.sib[c] = sh.first[p];
                sh.first[p] = c;
            }
        }
        sh.path[0] = 0;
    }
    const float* ztb = zt + (size_t)b * n * V;
    const float* zdb = zd ? zd + (size_t)b * n * V : nullptr;
    // greedy: every target row's argmax, the four waves side by side (none depends on the walk,
    // and without exponentials they are cheap); sampling: every drafted token's two logits
    if (mode == HCI_GREEDY) {
        for (int r = wv; r < n; r += kAccW) {
            int g; double gap; bool rb;
            wave_row_argmax(ztb + (size_t)r * V, V, lane, g, gap, rb);
            if (lane == 0) { sh.garg[r] = g; sh.ggap[r] = gap; sh.gbad[r] = rb ? 1 : 0; }
        }
    } else {
        if (tid > 0 && tid < n) {
            const int t = tok[tid], p = sh.par[tid];
            const bool ok = t >= 0 && t < V && p >= 0;
            sh.zp_[tid] = ok ? ztb[(size_t)p * V + t] : 0.f;
            sh.zq_[tid] = ok ? zdb[(size_t)tid * V + t] : 0.f;
        }
    }
    __syncthreads();
    bool bad = sh.flag == 0;
    uint32_t flags = bad ? HCI_DS_TREE : 0u;
    int m = 0, k = 0, nxt = -1;
    double margin = INFINITY;
    while (!bad) {
        const float* prow = ztb + (size_t)m * V;
        if (mode == HCI_GREEDY) {                     // every thread walks the same path: no barrier
            const int g = sh.garg[m];
            margin = fmin(margin, sh.ggap[m]);
            if (sh.gbad[m]) { bad = true; break; }
            int found = -1;
            for (int c = sh.first[m]; c >= 0; c = sh.sib[c]) {
                const int t = tok[c];
                if (t < 0 || t >= V) flags |= HCI_DS_DRAFT_ID;
                if (t == g) { found = c; break; }
            }
            if (found < 0) { nxt = g; break; }
            m = found;
            if (tid == 0) sh.path[k + 1] = m;
            ++k;
            continue;
        }
        // sampling: the statistics of the target row and of the children's draft rows in one round
        // (wave w: entries w, w + 4, ... of [target row m, draft rows of m's children in order]),
        // then the children in order
        {
            if (wv == 0) {
                double mx, sum;
                wave_row_stats(prow, V, T, lane, mx, sum);
                if (lane == 0) { sh.pm_[m] = mx; sh.ps_[m] = sum; sh.zh[0] = 1.0; }
            }
            int i = 1;
            for (int c = sh.first[m]; c >= 0; c = sh.sib[c], ++i)
                if (i % kAccW == wv) {
                    double mx, sum;
                    wave_row_stats(zdb + (size_t)c * V, V, T, lane, mx, sum);
                    if (lane == 0) { sh.qm_[c] = mx; sh.qs_[c] = sum; }
                }
        }
        __syncthreads();
        const double pm = sh.pm_[m], ps = sh.ps_[m];
        if (!row_finite(ps)) { bad = true; break; }
        int nrej = 0, kept = -1;
        for (int c = sh.first[m]; c >= 0 && !bad; c = sh.sib[c]) {
            const float* qrow = zdb + (size_t)c * V;
            const double qm = sh.qm_[c], qs = sh.qs_[c];
            if (!row_finite(qs)) { bad = true; break; }
            // residual weight of token j after the rejections so far at this node
            auto resid = [&](int j, double p) {
                double w = p;
                for (int i = 0; i < nrej; ++i)
                    if (sh.zapp[i])
                        w = fmax(0.0, w - __dmul_rn(sh.zh[i], exp(over_T((double)zdb[(size_t)sh.rnode[i] * V + j], T) -
                                                                  sh.rqm[i]) / sh.rqs[i]));
                return w;
            };
            const int t = tok[c];
            if (t >= 0 && t < V) {
                const double p_t = exp(over_T((double)sh.zp_[c], T) - pm) / ps;
                const double q_t = exp(over_T((double)sh.zq_[c], T) - qm) / qs;
                const double lhs = uni[(size_t)b * n + c] * q_t * sh.zh[nrej];
                const double rhs = resid(t, p_t);
                margin = fmin(margin, fabs(lhs - rhs) / fmax(rhs, 1e-300));
                if (lhs < rhs) { kept = c; break; }
            } else {
                flags |= HCI_DS_DRAFT_ID;
            }
            // rejection: total of max(0, w - z q_c) over the vocabulary
            const double z = sh.zh[nrej];
            double loc = 0.0;
            for (int j = tid; j < V; j += kAccT) {
                const double q = exp(over_T((double)qrow[j], T) - qm) / qs;
                loc += fmax(0.0, resid(j, exp(over_T((double)prow[j], T) - pm) / ps) - __dmul_rn(z, q));
            }
            const double tot = block_sum(loc, sh.a);
            __syncthreads();
            if (tid == 0) {
                const bool ok = tot > 0.0;            // cannot fail after a rejection; guard only
                sh.zapp[nrej] = ok ? 1 : 0;
                sh.zh[nrej + 1] = ok ? tot : z;
                sh.rnode[nrej] = c;
                sh.rqm[nrej] = qm;
                sh.rqs[nrej] = qs;
            }
            __syncthreads();
            ++nrej;
        }
        if (bad) break;
        if (kept >= 0) {
            m = kept;
            if (tid == 0) sh.path[k + 1] = m;
            ++k;
            __syncthreads();
            continue;
        }
        const int r = nrej;
        auto weight = [&](int j) {
            const double p = exp(over_T((double)prow[j], T) - pm) / ps;
            if (r == 0) return p;
            double w = p;
            for (int i = 0; i < r; ++i)
                if (sh.zapp[i])
                    w = fmax(0.0, w - __dmul_rn(sh.zh[i], exp(over_T((double)zdb[(size_t)sh.rnode[i] * V + j], T) -
                                                              sh.rqm[i]) / sh.rqs[i]));
            return w;
        };
        int tk;
        double m2;
        draw_token(weight, V, uni[(size_t)b * n], sh.a, tk, m2);
        nxt = tk;
        margin = fmin(margin, m2);
        break;
    }
    __syncthreads();
    if (tid < n) path_out[(size_t)b * n + tid] = (!bad && tid <= k) ? sh.path[tid] : -1;
    if (tid == 0) {
        n_acc[b] = bad ? -1 : k;
        next[b] = bad ? -1 : nxt;
        if (margin_out) margin_out[b] = bad ? qnan() : margin;
        report(status, b, flags | (bad && !(flags & HCI_DS_TREE) ? HCI_DS_NONFINITE : 0u));
    }
}

hipError_t launch_accept_tree(int mode, int nb, int n, int V, float temperature, const int32_t* parent,
                              const int32_t* tokens, const float* zt, const float* zd, const double* u, int32_t* n_acc,
                              int32_t* path, int32_t* next, double* margin, uint32_t* status, hipStream_t st)
{
    hipLaunchKernelGGL(k_accept_tree, dim3(nb), dim3(kAccT), 0, st, mode, n, V, (double)temperature, parent, tokens,
                       zt, zd, u, n_acc, path, next, margin, status);
    return hipGetLastError();
}

// best candidate of each sequence: the largest n_accepted, lowest index on ties; a candidate
// marked invalid (n_accepted -1) never wins, and -1 when none is valid
__global__ __launch_bounds__(256) void k_accept_best(int nb, int nc, const int32_t* __restrict__ n_acc,
                                                     int32_t* __restrict__ best)
{
    const size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= (size_t)nb) return;
    int bc = 0, bk = n_acc[b * nc];
    for (int c = 1; c < nc; ++c) {
        const int k = n_acc[b * nc + c];
        if (k > bk) { bk = k; bc = c; }
    }
    best[b] = bk < 0 ? -1 : bc;
}

// Serial drafting with the previous-token bias (EvSpark digest, Figure 1(b)): draft m draws from
// softmax(l / T), l = z[m] + B[prev] in fp32, by the same inverse-CDF rule as the acceptance
// draws.  One workgroup of four waves per sequence: each thread holds a contiguous run of
// ceil(V/256) token ids in registers; the row maximum, the sum and the scan of the run totals
// are wave collectives on the vector ALU whose four wave results meet in LDS (one barrier per
// exchange, each exchange with slots of its own, combined in wave order), and the thread whose
// run crosses u x total walks it.  A draw is bound by its fp64 exp and division work, which four
// waves split four ways.
constexpr int kDsW = 4;                    // waves per sequence
constexpr int kDsT = 64 * kDsW;
constexpr int kDsMaxPer = 16;              // V <= 4096 on this path

template <int PER>                         // ids per thread, a power of two >= ceil(V / 256)
__global__ __launch_bounds__(kDsT) void k_draft_sample(int gamma, int V, double T, const float* __restrict__ z,
                                                       const float* __restrict__ markov,
                                                       const int32_t* __restrict__ anchor,
                                                       const double* __restrict__ uni, int32_t* __restrict__ drafts,
                                                       float* __restrict__ dl, double* __restrict__ margin_out)
{
    // the four exchanges of a draw: maximum, sum, scan totals, and the crossing (first id,
    // last id with weight, smallest distance to the target)
    __shared__ double x_max[kDsW], x_sum[kDsW], x_tot[kDsW], x_dmin[kDsW];
    __shared__ int x_first[kDsW], x_last[kDsW];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (V + kDsT - 1) / kDsT;
    const int j0 = min(tid * per, V), j1 = min(j0 + per, V), n = j1 - j0;
    int prev = anchor[b];
    prev = prev < 0 ? 0 : (prev >= V ? V - 1 : prev);
    for (int m = 0; m < gamma; ++m) {
        const size_t r = ((size_t)b * gamma + m) * V;
        // the run's logits and bias entries in one batch: unconditional loads from clamped ids
        // (no branch around a load, no value used before the last load is issued), masked after
        float zl[PER], bl[PER], l[PER];
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            const int j = min(j0 + t, V - 1);
            zl[t] = z[r + j];
            bl[t] = markov[(size_t)prev * V + j];
        }
        // every value in hand before any is used under a condition (which would otherwise pull
        // its load into that branch)
#pragma unroll
        for (int t = 0; t < PER; ++t) asm volatile("" : "+v"(zl[t]), "+v"(bl[t]));
        double mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            const int j = j0 + t;
            l[t] = t < n ? zl[t] + bl[t] : -INFINITY;
            if (t < n) {
                dl[r + j] = l[t];
                mx = fmax(mx, over_T((double)l[t], T));
            }
        }
        mx = wave_max_f64(mx);
        if (lane == 0) x_max[wave] = mx;
        __syncthreads();
        mx = x_max[0];
#pragma unroll
        for (int w = 1; w < kDsW; ++w) mx = fmax(mx, x_max[w]);
        double e[PER];
        double loc = 0.0;
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            e[t] = t < n ? exp(over_T((double)l[t], T) - mx) : 0.0;
            loc += e[t];
        }
        loc = wave_sum_f64(loc);
        if (lane == 0) x_sum[wave] = loc;
        __syncthreads();
        double sum = x_sum[0];
#pragma unroll
        for (int w = 1; w < kDsW; ++w) sum += x_sum[w];
        // probabilities p_j = exp(l_j / T - mx) / sum; running sums over ascending ids
        double ploc = 0.0;
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            e[t] = e[t] / sum;
            ploc += e[t];
        }
        double wtot;
        double incl = wave_incl_scan_f64(ploc, lane, &wtot);
        if (lane == 0) x_tot[wave] = wtot;
        __syncthreads();
        double off = 0.0, total = x_tot[0];
#pragma unroll
        for (int w = 1; w < kDsW; ++w) {
            if (w == wave) off = total;
            total += x_tot[w];
        }
        incl += off;
        const double excl = incl - ploc;
        const double target = uni[(size_t)b * gamma + m] * total;
        int first = INT_MAX, lastpos = -1;
        double dmin = INFINITY, run = excl;
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            if (t < n) {
                const double w = e[t];
                run += w;
                if (run > target && first == INT_MAX) first = j0 + t;
                if (w > 0.0) lastpos = j0 + t;
                dmin = fmin(dmin, fabs(run - target));
            }
        }
        first = wave_min_i32(first);
        lastpos = wave_max_i32(lastpos);
        dmin = wave_min_f64(dmin);
        if (lane == 0) {
            x_first[wave] = first;
            x_last[wave] = lastpos;
            x_dmin[wave] = dmin;
        }
        __syncthreads();
        first = x_first[0];
        lastpos = x_last[0];
        dmin = x_dmin[0];
#pragma unroll
        for (int w = 1; w < kDsW; ++w) {
            first = min(first, x_first[w]);
            lastpos = max(lastpos, x_last[w]);
            dmin = fmin(dmin, x_dmin[w]);
        }
        const int tok = first != INT_MAX ? first : lastpos;
        if (tid == 0) {
            drafts[(size_t)b * gamma + m] = tok;
            if (margin_out) margin_out[(size_t)b * gamma + m] = dmin / total;
        }
        prev = tok;
    }
}

hipError_t launch_draft_sample(int nb, int gamma, int V, float temperature, const float* z, const float* markov,
                               const int32_t* anchor, const double* u, int32_t* drafts, float* dl, double* margin,
                               hipStream_t st)
{
    if (V > kDsT * kDsMaxPer) return hipErrorInvalidValue;
    const int per = (V + kDsT - 1) / kDsT;
#define HCI_DS(PER_)                                                                                            \
    if (per <= PER_) {                                                                                           \
        hipLaunchKernelGGL(k_draft_sample<PER_>, dim3(nb), dim3(kDsT), 0, st, gamma, V, (double)temperature, z,  \
                           markov, anchor, u, drafts, dl, margin);                                               \
        return hipGetLastError();                                                                                \
    }
    HCI_DS(1) HCI_DS(2) HCI_DS(4) HCI_DS(8) HCI_DS(16)
#undef HCI_DS
    return hipErrorInvalidValue;
}

hipError_t launch_accept(int mode, int nb, int nc, int gamma, int V, float temperature,
                         const float* zt, const float* zd, const int32_t* drafts, const double* u,
                         int32_t* n_acc, int32_t* next, int32_t* best, double* margin, uint32_t* status,
                         hipStream_t st)
{
    if (mode == HCI_SAMPLE_RECURSIVE) {
        hipLaunchKernelGGL(k_accept_recursive, dim3(nb), dim3(kAccT), 0, st, nc, gamma, V, (double)temperature,
                           zt, zd, drafts, u, n_acc, next, best, margin, status);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_accept, dim3((unsigned)((long long)nb * nc)), dim3(kAccT), 0, st, mode, nc, gamma, V,
                       (double)temperature, zt, zd, drafts, u, n_acc, next, best, margin, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nc == 1 || !best) return e;
    hipLaunchKernelGGL(k_accept_best, dim3((nb + 255) / 256), dim3(256), 0, st, nb, nc, n_acc, best);
    return hipGetLastError();
}

}  // namespace hci
