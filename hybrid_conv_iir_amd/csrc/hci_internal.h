// Internal helpers shared by the libhci kernels and host code (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "hci.h"

namespace hci {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal: streamed data that is read exactly once
// (the KV prefix) bypasses cache retention, which lifts the sustained read
// rate of a full-chip stream by about 15% on gfx950.
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

constexpr int kTile = HCI_KV_TILE;   // keys per KV tile

// ORs HCI_DS_* bits into sequence b's status word; no-op when the caller passed no status
// array.  A vector atomic from the calling lane.
__device__ __forceinline__ void report(uint32_t* status, size_t b, uint32_t bits) {
    if (status != nullptr && bits != 0u) atomicOr(status + b, bits);
}

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN (a select, not a branch)
__device__ __forceinline__ uint16_t f2bf(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t nan = (u >> 16) | 0x40u;
    return (uint16_t)((u & 0x7fffffffu) > 0x7f800000u ? nan : rne);
}

template <int ACT> struct Act;
template <> struct Act<HCI_F32> {
    typedef float T;
    __device__ static __forceinline__ float load(const T* p, size_t i) { return p[i]; }
    __device__ static __forceinline__ void store(T* p, size_t i, float v) { p[i] = v; }
};
template <> struct Act<HCI_BF16> {
    typedef uint16_t T;
    __device__ static __forceinline__ float load(const T* p, size_t i) { return bf2f(p[i]); }
    __device__ static __forceinline__ void store(T* p, size_t i, float v) { p[i] = f2bf(v); }
};

// ------------------------------------------------------------- KV layout
//
// A cache holds, per (sequence, head), kv_cap/32 tiles of 32 keys x Dh.
// Inside a tile the element order is the register order of the attention
// kernel's matrix-core operands, so that every wave-wide 16-byte load reads
// one contiguous kilobyte:
//   K: [u<2][j<Dh/32][g<4][m<16][e<8]  holds K[16u+m][32j+8g+e]
//   V: [t<Dh/16][g<4][m<16][i<8]       holds V[kmap(g,i)][16t+m]
// with kmap(g,i) = 4g+i for i<4 and 16+4g+(i-4) for i>=4: the keys a lane
// holds after the score product (4 per 16-key half) are the keys it must
// supply to the value product.

__host__ __device__ __forceinline__ size_t k_tile_offset(int w, int dd, int Dh) {
    const int u = w >> 4, m = w & 15;
    const int j = dd >> 5, g = (dd >> 3) & 3, e = dd & 7;
    return ((((size_t)(u * (Dh >> 5) + j) * 4 + g) * 16 + m) * 8 + e);
}

__host__ __device__ __forceinline__ size_t v_tile_offset(int w, int dd, int Dh) {
    (void)Dh;
    const int half = w >> 4, r = w & 15;
    const int g = r >> 2, i = (r & 3) + 4 * half;
    const int t = dd >> 4, m = dd & 15;
    return ((((size_t)t * 4 + g) * 16 + m) * 8 + i);
}

// element offset of (row, dd) inside one (sequence, head) cache slab
__host__ __device__ __forceinline__ size_t k_elem(int row, int dd, int Dh) {
    return (size_t)(row >> 5) * kTile * Dh + k_tile_offset(row & 31, dd, Dh);
}
__host__ __device__ __forceinline__ size_t v_elem(int row, int dd, int Dh) {
    return (size_t)(row >> 5) * kTile * Dh + v_tile_offset(row & 31, dd, Dh);
}

// ----------------------------------------------------------- launch API

// Split-K plan for the attention prefix: the same function sizes the
// workspace and launches the kernels, so both always agree.
struct AttnPlan {
    int nq;            // queries per sequence = nc * P
    int resident;      // streaming workgroups kept resident (the work list is cut for this many)
    int items_cap;     // bound on the prefix work items; 0 when max_kv_len is 0, -1 when too many
    int kv_lim;        // prefix lengths are read clamped to [0, kv_lim] (= max_kv_len)
    size_t header_bytes;   // first section of the workspace: the job queue's counter (bytes 0..3)
                           // and, from byte kWsTableOff, the work-list table (worklist.h)
    size_t part_o_elems, part_ml_elems;
    size_t bytes;      // workspace bytes (256-aligned sections)
};
AttnPlan plan_attention(const hci_layer* L, int nb, int nc, int gamma, int max_kv_len, int num_cus);
int device_cu_count();

// dynamic LDS bytes of the verify's finish kernel (conv/IIR scan and combine; at most kMaxLds)
size_t stream_lds_bytes(const hci_layer* L, int nc, int P);
constexpr size_t kMaxLds = 160 * 1024;

// the whole verify: the prefix stream then the finish kernel; ev (may be null)
// = 4 events recorded before the set-up kernel, before and after the streaming kernel, and at
// the end
// parent: a token tree per sequence ([nb][P] parents, nc = 1) instead of chains of candidate positions
hipError_t launch_verify(const hci_layer* L, const hci_state* S, const hci_block* blk,
                         int nb, int nc, int P, const AttnPlan& plan, void* ws, hipStream_t st, hipEvent_t* ev,
                         bool conv = true, const int32_t* parent = nullptr);
// dynamic LDS bytes of the finish kernel of a tree verify (tree conv role and combine role)
size_t tree_finish_lds_bytes(const hci_layer* L, int n);
hipError_t launch_accept(int mode, int nb, int nc, int gamma, int V, float temperature,
                         const float* zt, const float* zd, const int32_t* drafts, const double* u,
                         int32_t* n_acc, int32_t* next, int32_t* best, double* margin, uint32_t* status,
                         hipStream_t st);
// lim: the host's bound on kv_len (max_kv_len); a sequence outside [0, lim] is left unchanged
// path / parent (token trees, nc = 1, P = nodes): commit the accepted path's nodes as rows 0..k
hipError_t launch_slice(const hci_layer* L, const hci_state* S, const hci_block* blk,
                        int nb, int nc, int P, int lim, const int32_t* n_acc, const int32_t* best, hipStream_t st,
                        const int32_t* path = nullptr, const int32_t* parent = nullptr);
hipError_t launch_accept_tree(int mode, int nb, int n, int V, float temperature, const int32_t* parent,
                              const int32_t* tokens, const float* zt, const float* zd, const double* u, int32_t* n_acc,
                              int32_t* path, int32_t* next, double* margin, uint32_t* status, hipStream_t st);
hipError_t launch_kv_copy(const hci_layer* L, const hci_state* S, int b, int row0, int nrows,
                          const void* k_rows, const void* v_rows, void* k_out, void* v_out,
                          bool write, hipStream_t st);
// row0 < 0: append at kv_len[b] (read on the device), skipped when kv_len[b] is outside [0, lim]
hipError_t launch_kv_pack(const hci_layer* L, const hci_state* S, int b, int row0, int nrows, const void* k_rows,
                          const void* v_rows, size_t row_stride, size_t head_stride, hipStream_t st, int lim = 0);
// kv_len += add for every sequence whose kv_len is inside [0, lim]; the others are reported
hipError_t launch_len_add(const hci_state* S, int nb, int add, int lim, hipStream_t st);

// prefill of a prompt into the committed state
struct PrefillPlan {
    bool state_only;             // folded FIR/IIR path for the state (T >= To)
    bool y_mfma;                 // outputs y by the matrix-core pass (bf16), next to the state path
    int sub_len, chunk_len;      // state path: positions per scan thread and per chunk
    int nchunks;                 // chunks (256 positions on the output path, chunk_len on the state path)
    size_t s_elems, ftail_elems, yloc_elems;
    size_t bytes;                // workspace bytes (256-aligned sections)
};
PrefillPlan plan_prefill(const hci_layer* L, int nb, int T, bool want_y);
size_t prefill_lds_bytes(int To);
bool prefill_state_path(const hci_layer* L, int T, bool want_y);
size_t prefill_state_lds_bytes(const hci_layer* L);
size_t prefill_y_lds_bytes(int To);
hipError_t launch_prefill(const hci_layer* L, const hci_state* S, int nb, int T, int lim, const void* x,
                          const void* k, const void* v, void* y, const PrefillPlan& plan, void* ws, hipStream_t st);

// dense projections
struct LinearPlan {
    int ct, mt, kw, kspw;        // column strips and 16-row tiles per workgroup, waves splitting K, K steps per wave
    int grid_x, grid_y;
    size_t lds;
};
LinearPlan plan_linear(int M, int K, int N);
// act: 0 none, 1 SiLU (applied after the residual)
hipError_t launch_linear(int M, int K, int N, int parts, const void* x, const void* wp, const void* res, void* y,
                         bool out_f32, hipStream_t st, int act = 0);
hipError_t launch_linear_pack(int K, int N, const void* w, void* wp, hipStream_t st);
hipError_t launch_rmsnorm(int M, int K, const void* x, const float* g, float eps, void* y, hipStream_t st);

// full layer stack
struct ModelPlan {
    size_t rows;                 // nb * nc * P
    size_t a_off, y_off, attn_off, bytes;
    bool has_attn;
    AttnPlan attn;
};
size_t mixer_lds_bytes(int kind, int Tl, int P);
ModelPlan plan_model(const hci_model* M, int nb, int nc, int gamma, int max_kv_len, int num_cus);
hipError_t launch_model_verify(const hci_model* M, const hci_model_state* S, const hci_model_block* blk, int nb,
                               int nc, int P, const ModelPlan& plan, void* ws, hipStream_t st);
hipError_t launch_model_slice(const hci_model* M, const hci_model_state* S, const hci_model_block* blk, int nb,
                              int nc, int P, const int32_t* n_acc, const int32_t* best, hipStream_t st);

// drafter trunk and sampling
struct DraftPlan {
    size_t rows;                 // nb * (W + gamma)
    size_t h_off, a_off, qkv_off, o_off, m_off, bytes;
    size_t attn_lds;
};
size_t draft_attn_lds(int W, int gamma, int DH);
DraftPlan plan_draft(const hci_drafter* D, int nb, int gamma);
hipError_t launch_draft_logits(const hci_drafter* D, int nb, int gamma, const void* window, const int32_t* anchor,
                               float* z, const DraftPlan& p, void* ws, hipStream_t st);
hipError_t launch_draft_sample(int nb, int gamma, int V, float temperature, const float* z, const float* markov,
                               const int32_t* anchor, const double* u, int32_t* drafts, float* dl, double* margin,
                               hipStream_t st);

hipError_t launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t st);
hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t st);
int probe_blocks();

}  // namespace hci
