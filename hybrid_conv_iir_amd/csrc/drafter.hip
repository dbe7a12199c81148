// The drafter trunk (EvSpark digest, Figure 1(b)): a projected window of
// target states as the K/V prefix of two causal attention layers, the
// anchor and mask embeddings as the block rows, tied output embedding.
//
// Rows of the working buffer: [nb * W window rows ; nb * gamma block rows],
// so the normalisation and the q/k/v projection of a layer run over both in
// one call each, and the output projection and the MLP over the block rows.
//   k_linear           hw = window W_proj            (into the window rows)
//   k_draft_embed      block rows = E[anchor], mask, mask, ...
//   per layer: k_rmsnorm (all rows), k_linear q/k/v (all rows, 3 streams),
//     k_draft_attn (per sequence and head: scores over the window rows and
//     the causal block rows in LDS, softmax, weighted values),
//     k_linear o W_o + h, k_rmsnorm, k_linear SiLU(a W_up), k_linear m W_down + h
//   k_rmsnorm + k_linear  z = hf E^T (fp32)
#include "hci_internal.h"

namespace hci {

__global__ void k_draft_embed(uint16_t* __restrict__ h, const uint16_t* __restrict__ emb,
                              const uint16_t* __restrict__ mask, const int32_t* __restrict__ anchor, int d, int gamma,
                              int V)
{
    const int row = blockIdx.x;                   // b * gamma + i
    const int b = row / gamma, i = row % gamma;
    int a = anchor[b];
    a = a < 0 ? 0 : (a >= V ? V - 1 : a);
    const uint16_t* src = i == 0 ? emb + (size_t)a * d : mask;
    for (int c = threadIdx.x; c < d; c += blockDim.x) h[(size_t)row * d + c] = src[c];
}

size_t draft_attn_lds(int W, int gamma, int DH) {
    const int nk = W + gamma;
    return (size_t)2 * nk * DH * 2 + (size_t)gamma * DH * 2 + (size_t)gamma * nk * 4;
}

// one workgroup per (head, sequence); qkv = [3][rows_all][d] bf16
__global__ __launch_bounds__(256) void k_draft_attn(const uint16_t* __restrict__ qkv, uint16_t* __restrict__ o,
                                                    int nb, int W, int gamma, int H, int DH, float scale)
{
    extern __shared__ char smem[];
    const int h = blockIdx.x, b = blockIdx.y;
    const int d = H * DH, nk = W + gamma;
    const size_t rows = (size_t)nb * (W + gamma);
    uint16_t* ks = (uint16_t*)smem;                        // [nk][DH]
    uint16_t* vs = ks + (size_t)nk * DH;                   // [nk][DH]
    uint16_t* qs = vs + (size_t)nk * DH;                   // [gamma][DH]
    float* S = (float*)(qs + (size_t)gamma * DH);          // [gamma][nk]
    const uint16_t* kbase = qkv + rows * d;
    const uint16_t* vbase = qkv + 2 * rows * d;
    for (int e = threadIdx.x; e < nk * DH; e += blockDim.x) {
        const int j = e / DH, dd = e % DH;
        const size_t row = j < W ? (size_t)b * W + j : (size_t)nb * W + (size_t)b * gamma + (j - W);
        ks[e] = kbase[row * d + h * DH + dd];
        vs[e] = vbase[row * d + h * DH + dd];
    }
    for (int e = threadIdx.x; e < gamma * DH; e += blockDim.x) {
        const int i = e / DH, dd = e % DH;
        qs[e] = qkv[((size_t)nb * W + (size_t)b * gamma + i) * d + h * DH + dd];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < gamma * nk; e += blockDim.x) {
        const int i = e / nk, j = e % nk;
        float s = -INFINITY;
        if (j < W || j - W <= i) {
            s = 0.f;
            for (int dd = 0; dd < DH; ++dd) s = fmaf(bf2f(qs[i * DH + dd]), bf2f(ks[j * DH + dd]), s);
            s *= scale;
        }
        S[e] = s;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
    for (int i = wv; i < gamma; i += nw) {
        float m = -INFINITY;
        for (int j = lane; j < nk; j += 64) m = fmaxf(m, S[i * nk + j]);
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        float sum = 0.f;
        for (int j = lane; j < nk; j += 64) {
            const float p = __expf(S[i * nk + j] - m);
            S[i * nk + j] = p;
            sum += p;
        }
        for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
        const float inv = 1.0f / sum;
        for (int j = lane; j < nk; j += 64) S[i * nk + j] *= inv;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < gamma * DH; e += blockDim.x) {
        const int i = e / DH, dd = e % DH;
        float acc = 0.f;
        for (int j = 0; j < nk; ++j) acc = fmaf(S[i * nk + j], bf2f(vs[j * DH + dd]), acc);
        o[((size_t)b * gamma + i) * d + h * DH + dd] = f2bf(acc);
    }
}

DraftPlan plan_draft(const hci_drafter* D, int nb, int gamma) {
    DraftPlan p{};
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t rows = (size_t)nb * (D->window + gamma), brows = (size_t)nb * gamma;
    p.rows = rows;
    p.h_off = 0;
    p.a_off = p.h_off + up(rows * D->d * 2);
    p.qkv_off = p.a_off + up(rows * D->d * 2);
    p.o_off = p.qkv_off + up(3 * rows * D->d * 2);
    p.m_off = p.o_off + up(brows * D->d * 2);
    p.bytes = p.m_off + up(brows * D->ffn * 2);
    p.attn_lds = draft_attn_lds(D->window, gamma, D->head_dim);
    return p;
}

hipError_t launch_draft_logits(const hci_drafter* D, int nb, int gamma, const void* window, const int32_t* anchor,
                               float* z, const DraftPlan& p, void* ws, hipStream_t st)
{
    const int d = D->d, W = D->window;
    const size_t rows = p.rows, wrows = (size_t)nb * W, brows = (size_t)nb * gamma;
    uint16_t* h = (uint16_t*)((char*)ws + p.h_off);             // [window rows ; block rows][d]
    uint16_t* hb = h + wrows * d;                                // block rows
    uint16_t* a = (uint16_t*)((char*)ws + p.a_off);
    uint16_t* ab = a + wrows * d;
    uint16_t* qkv = (uint16_t*)((char*)ws + p.qkv_off);
    uint16_t* o = (uint16_t*)((char*)ws + p.o_off);
    uint16_t* m = (uint16_t*)((char*)ws + p.m_off);
    hipError_t e;
    if ((e = launch_linear((int)wrows, D->d_target, d, 1, window, D->w_proj, nullptr, h, false, st)) != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_draft_embed, dim3((unsigned)brows), dim3(256), 0, st, hb, (const uint16_t*)D->emb,
                       (const uint16_t*)D->mask, anchor, d, gamma, D->vocab);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.attn_lds > 65536 && (e = hipFuncSetAttribute((const void*)k_draft_attn,
                                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                                        (int)p.attn_lds)) != hipSuccess)
        return e;
    const float scale = 1.0f / sqrtf((float)D->head_dim);
    for (int l = 0; l < D->n_layers; ++l) {
        const hci_drafter_layer& L = D->layers[l];
        if ((e = launch_rmsnorm((int)rows, d, h, L.g1, D->eps, a, st)) != hipSuccess) return e;
        if ((e = launch_linear((int)rows, d, 3 * d, 3, a, L.w_qkv, nullptr, qkv, false, st)) != hipSuccess) return e;
        hipLaunchKernelGGL(k_draft_attn, dim3(D->heads, nb), dim3(256), p.attn_lds, st, qkv, o, nb, W, gamma, D->heads,
                           D->head_dim, scale);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_linear((int)brows, d, d, 1, o, L.w_o, hb, hb, false, st)) != hipSuccess) return e;
        if ((e = launch_rmsnorm((int)brows, d, hb, L.g2, D->eps, ab, st)) != hipSuccess) return e;
        if ((e = launch_linear((int)brows, d, D->ffn, 1, ab, L.w_up, nullptr, m, false, st, 1)) != hipSuccess) return e;
        if ((e = launch_linear((int)brows, D->ffn, d, 1, m, L.w_down, hb, hb, false, st)) != hipSuccess) return e;
    }
    if ((e = launch_rmsnorm((int)brows, d, hb, D->g_f, D->eps, ab, st)) != hipSuccess) return e;
    return launch_linear((int)brows, d, D->vocab, 1, ab, D->emb_t, nullptr, z, true, st);
}

}  // namespace hci
