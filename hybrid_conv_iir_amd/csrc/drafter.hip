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
//     k_draft_attn (one wave per query row, head and sequence: scores over
//     the window rows and the causal block rows, softmax, weighted values),
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
    (void)DH;
    return (size_t)(W + gamma) * sizeof(float);
}

// one wave per (query row, head, sequence); qkv = [3][rows_all][d] bf16, Dh = 128.  Lanes own
// keys (lane, lane + 64, ...) for the scores and two value columns each for the output.
__global__ __launch_bounds__(64) void k_draft_attn(const uint16_t* __restrict__ qkv, uint16_t* __restrict__ o,
                                                   int nb, int W, int gamma, int H, int DH, float scale)
{
    extern __shared__ float pr[];                         // [W + gamma] probabilities
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int d = H * DH, nk = W + i + 1;                  // the window and block keys 0..i
    const size_t rows = (size_t)nb * (W + gamma);
    const uint16_t* qrow = qkv + ((size_t)nb * W + (size_t)b * gamma + i) * d + h * DH;
    // The query and the lane's two key rows are requested in one round (keys past nk from a
    // clamped, always valid row, their scores masked), every piece in hand before any is
    // converted: a conversion right after a load makes the compiler wait for that load there.
    u32x4 qr[16], kr[2][16];
#pragma unroll
    for (int c = 0; c < 16; ++c) qr[c] = *(const u32x4*)(qrow + 8 * c);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int j = min(lane + 64 * u, nk - 1);
        const size_t row = j < W ? (size_t)b * W + j : (size_t)nb * W + (size_t)b * gamma + (j - W);
        const uint16_t* krow = qkv + (rows + row) * d + h * DH;
#pragma unroll
        for (int c = 0; c < 16; ++c) kr[u][c] = *(const u32x4*)(krow + 8 * c);
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) asm volatile("" : "+v"(qr[c].x), "+v"(qr[c].y), "+v"(qr[c].z), "+v"(qr[c].w));
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < 16; ++c)
            asm volatile("" : "+v"(kr[u][c].x), "+v"(kr[u][c].y), "+v"(kr[u][c].z), "+v"(kr[u][c].w));
    float q[128];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const uint32_t w[4] = {qr[c].x, qr[c].y, qr[c].z, qr[c].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            q[8 * c + 2 * t] = __uint_as_float(w[t] << 16);
            q[8 * c + 2 * t + 1] = __uint_as_float(w[t] & 0xffff0000u);
        }
    }
    float mloc = -INFINITY;
    float sc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int j = lane + 64 * u;
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const uint32_t w[4] = {kr[u][c].x, kr[u][c].y, kr[u][c].z, kr[u][c].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                s = fmaf(q[8 * c + 2 * t], __uint_as_float(w[t] << 16), s);
                s = fmaf(q[8 * c + 2 * t + 1], __uint_as_float(w[t] & 0xffff0000u), s);
            }
        }
        sc[u] = j < nk ? s * scale : -INFINITY;
        if (j < nk) mloc = fmaxf(mloc, sc[u]);
    }
    for (int off = 32; off >= 1; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int j = lane + 64 * u;
        const float p = j < nk ? __expf(sc[u] - mloc) : 0.f;
        sc[u] = p;
        sum += p;
    }
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int u = 0; u < 2; ++u)
        if (lane + 64 * u < nk) pr[lane + 64 * u] = sc[u] * inv;
    __syncthreads();
    // the value rows 32 at a time, each batch requested in one round (rows past nk from a
    // clamped row, not used), then summed in key order
    constexpr int VB = 32;
    float a0 = 0.f, a1 = 0.f;
    for (int j0 = 0; j0 < nk; j0 += VB) {
        uint32_t vv[VB];
#pragma unroll
        for (int t = 0; t < VB; ++t) {
            const int j = min(j0 + t, nk - 1);
            const size_t row = j < W ? (size_t)b * W + j : (size_t)nb * W + (size_t)b * gamma + (j - W);
            vv[t] = *(const uint32_t*)(qkv + (2 * rows + row) * d + h * DH + 2 * lane);
        }
#pragma unroll
        for (int t = 0; t < VB; ++t) asm volatile("" : "+v"(vv[t]));
#pragma unroll
        for (int t = 0; t < VB; ++t) {
            if (j0 + t < nk) {
                const float p = pr[j0 + t];
                a0 = fmaf(p, __uint_as_float(vv[t] << 16), a0);
                a1 = fmaf(p, __uint_as_float(vv[t] & 0xffff0000u), a1);
            }
        }
    }
    const uint32_t packed = (uint32_t)f2bf(a0) | ((uint32_t)f2bf(a1) << 16);
    *(uint32_t*)(o + ((size_t)b * gamma + i) * d + h * DH + 2 * lane) = packed;
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
    const float scale = 1.0f / sqrtf((float)D->head_dim);
    for (int l = 0; l < D->n_layers; ++l) {
        const hci_drafter_layer& L = D->layers[l];
        if ((e = launch_rmsnorm((int)rows, d, h, L.g1, D->eps, a, st)) != hipSuccess) return e;
        if ((e = launch_linear((int)rows, d, 3 * d, 3, a, L.w_qkv, nullptr, qkv, false, st)) != hipSuccess) return e;
        hipLaunchKernelGGL(k_draft_attn, dim3(gamma, D->heads, nb), dim3(64), p.attn_lds, st, qkv, o, nb, W, gamma,
                           D->heads, D->head_dim, scale);
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
