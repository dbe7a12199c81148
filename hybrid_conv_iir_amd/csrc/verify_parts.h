// Arguments and launchers of the verify's finish kernel, shared by its
// translation unit and the verify's host code.
#pragma once

#include "hci_internal.h"

namespace hci {

constexpr int kCombT = 256;
constexpr int kCombW = kCombT / 64;
// finish workgroups resident per CU as far as registers go (the kernel's launch bound: four
// waves per SIMD, one wave of each workgroup on each SIMD)
constexpr int kFinishPerCu = 4;

struct FinishArgs {
    // conv / IIR
    const float *w_short, *w_outer, *lam, *beta, *cc;
    const void* short_win; const float* outer_win; const float* iir; const void* x;
    float* f_out; float* s_out; void* y_out;
    int d, Ts, To, N, nc, n_conv;
    int comb_first;                    // 1: the combine workgroups take the grid's low indices
    // combine
    const int32_t* kv_len; const float *part_o, *part_ml;
    const int32_t* table;              // the work-list table written by the set-up kernel
    const void *q, *kb, *vb; void* o;
    int nb, H, DH, nq, P, kv_lim, resident, rg_count;
    float scale_log2;
    // token trees (nc = 1, P = nodes): parent [nb][P], or nullptr for chains of candidate blocks
    const int32_t* parent;
    uint32_t* status;                  // HCI_DS_* per sequence (may be nullptr)
};

// LDS row stride (bytes) of the combine role's block K and V rows: Dh activations and 16
// bytes of padding
__host__ __device__ inline int combine_row_bytes(int DH, int act_bytes) { return DH * act_bytes + 16; }

// dynamic LDS floats of the combine role: the candidate's block K and V rows (raw
// activations, padded rows), then per row and state (four waves + the block part) O [Dh] and
// (m, l), then 64 block weights per wave, then (token trees) 64 ancestor masks and 64 jump
// entries
constexpr int kCombTreeFloats = 64 * 2 + 32;      // 64 masks (8-byte aligned) + 64 jump bytes
__host__ __device__ inline size_t combine_lds_floats(int P, int DH, int act_bytes, int RG) {
    return (size_t)2 * P * combine_row_bytes(DH, act_bytes) / 4 + (size_t)(kCombW + 1) * RG * (DH + 2) + 64 * kCombW +
           kCombTreeFloats;
}

// rows per combine workgroup for these sizes (1, 2, 4, 8 or 16)
int combine_rows(int nb, int nc, int H, int P, int num_cus, bool tree);
// the finish kernel: grid = F.n_conv + F.rg_count * nc * H * nb workgroups of kCombT threads
hipError_t launch_finish(const FinishArgs& F, int act_dtype, int rg, int blocks, size_t lds, hipStream_t st);

}  // namespace hci
