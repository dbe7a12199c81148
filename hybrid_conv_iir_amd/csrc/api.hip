// Host side of the C ABI: argument validation, launch planning, launches.
// Every check runs before the first launch, so a rejected call enqueues
// nothing; no call allocates, frees, synchronises or keeps a pointer.
#include "hci_internal.h"

#include <atomic>
#include <stdio.h>
#include <string.h>

namespace hci {

static std::atomic<int> g_cu_cache[64];

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < 64) {
        const int c = g_cu_cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (dev >= 0 && dev < 64) g_cu_cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static int check_layer(const hci_layer* L) {
    if (!L) return HCI_EINVAL;
    if (L->d < 1 || L->taps_short < 1 || L->taps_outer < 1 || L->poles < 1 || L->heads < 1 || L->head_dim < 1)
        return HCI_EINVAL;
    if (L->act_dtype != HCI_F32 && L->act_dtype != HCI_BF16) return HCI_EINVAL;
    if (L->poles > 64 || L->heads > 65535) return HCI_EUNSUPPORTED;
    if (L->act_dtype == HCI_BF16 && L->head_dim != 64 && L->head_dim != 128) return HCI_EUNSUPPORTED;
    if (L->act_dtype == HCI_F32 && (L->head_dim % 32 != 0 || L->head_dim > 128)) return HCI_EUNSUPPORTED;
    if (!L->w_short || !L->w_outer || !L->lambda || !L->beta || !L->c) return HCI_EINVAL;
    return HCI_OK;
}

static int check_state(const hci_layer* L, const hci_state* S, int nb, long long need_rows) {
    if (!S) return HCI_EINVAL;
    if (S->kv_cap < kTile || S->kv_cap % kTile != 0) return HCI_EINVAL;
    if (!S->k_cache || !S->v_cache || !S->kv_len || !S->iir) return HCI_EINVAL;
    if (L->taps_short > 1 && !S->short_win) return HCI_EINVAL;
    if (L->taps_outer > 1 && !S->outer_win) return HCI_EINVAL;
    if (!aligned(S->k_cache, 16) || !aligned(S->v_cache, 16)) return HCI_EINVAL;
    if (nb < 1 || nb > 65535) return HCI_EINVAL;
    if (need_rows > S->kv_cap) return HCI_ECAPACITY;
    return HCI_OK;
}

static int check_block(const hci_block* blk) {
    if (!blk || !blk->x || !blk->q || !blk->k || !blk->v || !blk->f || !blk->s || !blk->y || !blk->o)
        return HCI_EINVAL;
    if (!aligned(blk->q, 16)) return HCI_EINVAL;
    return HCI_OK;
}

}  // namespace hci

using namespace hci;

extern "C" {

static const char* status_name(int status) {
    switch (status) {
        case HCI_OK: return "HCI_OK";
        case HCI_EINVAL: return "HCI_EINVAL: invalid argument";
        case HCI_ECAPACITY: return "HCI_ECAPACITY: KV cache capacity exceeded";
        case HCI_EUNSUPPORTED: return "HCI_EUNSUPPORTED: shape or dtype not supported";
        case HCI_EDEVICE: return "HCI_EDEVICE: HIP launch error";
        case HCI_EWORKSPACE: return "HCI_EWORKSPACE: workspace missing or too small";
        default: return "HCI: unknown status";
    }
}

// copies text into buf the way snprintf does (truncated, NUL-terminated when n > 0) and
// returns the full length
static int put_text(const char* text, char* buf, size_t n) {
    const size_t len = strlen(text);
    if (n > 0) {
        const size_t m = len < n - 1 ? len : n - 1;
        memcpy(buf, text, m);
        buf[m] = '\0';
    }
    return (int)len;
}

int hci_status_string(int status, char* buf, size_t n) {
    if (!buf && n > 0) return HCI_EINVAL;
    return put_text(status_name(status), buf, n);
}

int hci_device_status_string(uint32_t bits, char* buf, size_t n) {
    if (!buf && n > 0) return HCI_EINVAL;
    static const struct { uint32_t bit; const char* name; } names[] = {
        {HCI_DS_NONFINITE, "HCI_DS_NONFINITE"}, {HCI_DS_K_RANGE, "HCI_DS_K_RANGE"},
        {HCI_DS_CAND_RANGE, "HCI_DS_CAND_RANGE"}, {HCI_DS_KV_LEN, "HCI_DS_KV_LEN"},
        {HCI_DS_DRAFT_ID, "HCI_DS_DRAFT_ID"}, {HCI_DS_TREE, "HCI_DS_TREE"}};
    char text[160];
    size_t used = 0;
    text[0] = '\0';
    for (const auto& e : names) {
        if (!(bits & e.bit)) continue;
        used += (size_t)snprintf(text + used, sizeof(text) - used, "%s%s", used ? "|" : "", e.name);
        bits &= ~e.bit;
    }
    if (bits) used += (size_t)snprintf(text + used, sizeof(text) - used, "%sunknown 0x%x", used ? "|" : "", bits);
    return put_text(used ? text : "none", buf, n);
}

int hci_version(void) { return 200; }

size_t hci_verify_workspace_bytes(const hci_layer* L, int nb, int nc, int gamma, int max_kv_len) {
    if (check_layer(L) != HCI_OK || nb < 1 || nc < 1 || gamma < 0 || max_kv_len < 0) return 0;
    return plan_attention(L, nb, nc, gamma, max_kv_len, device_cu_count()).bytes;
}

static int verify_impl(const hci_layer* L, const hci_state* S, const hci_block* blk,
                       int nb, int nc, int gamma, int max_kv_len,
                       void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t* ev) {
    int rc = check_layer(L);
    if (rc) return rc;
    if (nc < 1 || gamma < 0 || max_kv_len < 0) return HCI_EINVAL;
    const int P = gamma + 1;
    if (P > 64 || (long long)nc * P > 64) return HCI_EUNSUPPORTED;
    rc = check_state(L, S, nb, (long long)max_kv_len + gamma + 1);
    if (rc) return rc;
    rc = check_block(blk);
    if (rc) return rc;
    if (stream_lds_bytes(L, nc, P) > kMaxLds)
        return HCI_EUNSUPPORTED;
    const AttnPlan plan = plan_attention(L, nb, nc, gamma, max_kv_len, device_cu_count());
    if (plan.items_cap < 0) return HCI_EUNSUPPORTED;
    if (plan.bytes > 0 && (!ws || ws_bytes < plan.bytes || !aligned(ws, 256))) return HCI_EWORKSPACE;

    if (launch_verify(L, S, blk, nb, nc, P, plan, ws, stream, ev) != hipSuccess) return HCI_EDEVICE;
    return HCI_OK;
}

int hci_verify_block(const hci_layer* L, const hci_state* S, const hci_block* blk,
                     int nb, int nc, int gamma, int max_kv_len,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
    return verify_impl(L, S, blk, nb, nc, gamma, max_kv_len, ws, ws_bytes, stream, nullptr);
}

int hci_verify_block_timed(const hci_layer* L, const hci_state* S, const hci_block* blk,
                           int nb, int nc, int gamma, int max_kv_len,
                           void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t* events) {
    if (!events) return HCI_EINVAL;
    return verify_impl(L, S, blk, nb, nc, gamma, max_kv_len, ws, ws_bytes, stream, events);
}

int hci_accept(int mode, int nb, int nc, int gamma, int vocab, float temperature,
               const float* target_logits, const float* draft_logits,
               const int32_t* draft_tokens, const double* uniforms,
               int32_t* n_accepted, int32_t* next_token, int32_t* best_cand,
               double* margin, uint32_t* status, hipStream_t stream) {
    if (mode != HCI_GREEDY && mode != HCI_SAMPLE && mode != HCI_SAMPLE_RECURSIVE) return HCI_EINVAL;
    if (nb < 1 || nb > 2147483647 || nc < 1 || nc > 64 || gamma < 0 || vocab < 1) return HCI_EINVAL;
    if (vocab > 65536 || (long long)nb * nc > 2147483647LL) return HCI_EUNSUPPORTED;
    if (!target_logits || !n_accepted || !next_token) return HCI_EINVAL;
    if (gamma > 0 && !draft_tokens) return HCI_EINVAL;
    if (mode != HCI_GREEDY) {
        if (!(temperature > 0.f) || temperature == INFINITY) return HCI_EINVAL;
        if (!uniforms || (gamma > 0 && !draft_logits)) return HCI_EINVAL;
    }
    if (launch_accept(mode, nb, nc, gamma, vocab, temperature, target_logits, draft_logits, draft_tokens,
                      uniforms, n_accepted, next_token, best_cand, margin, status, stream) != hipSuccess)
        return HCI_EDEVICE;
    return HCI_OK;
}

int hci_slice_state(const hci_layer* L, const hci_state* S, const hci_block* blk,
                    int nb, int nc, int gamma, int max_kv_len,
                    const int32_t* n_accepted, const int32_t* best_cand, hipStream_t stream) {
    int rc = check_layer(L);
    if (rc) return rc;
    if (nc < 1 || gamma < 0 || max_kv_len < 0 || !n_accepted) return HCI_EINVAL;
    if (nc > 1 && !best_cand) return HCI_EINVAL;
    if (gamma + 1 > 64 || (long long)nc * (gamma + 1) > 64) return HCI_EUNSUPPORTED;
    rc = check_state(L, S, nb, (long long)max_kv_len + gamma + 1);
    if (rc) return rc;
    if (!blk || !blk->x || !blk->k || !blk->v || !blk->f || !blk->s) return HCI_EINVAL;
    if (launch_slice(L, S, blk, nb, nc, gamma + 1, max_kv_len, n_accepted, best_cand, stream) != hipSuccess)
        return HCI_EDEVICE;
    return HCI_OK;
}

static hci_block tree_block(const hci_tree* t) {
    hci_block blk{};
    blk.x = t->x; blk.q = t->q; blk.k = t->k; blk.v = t->v;
    blk.f = t->f; blk.s = t->s; blk.y = t->y; blk.o = t->o;
    return blk;
}

int hci_verify_tree(const hci_layer* L, const hci_state* S, const hci_tree* tree,
                    int nb, int n, int max_kv_len, void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc = check_layer(L);
    if (rc) return rc;
    if (!tree || !tree->parent || n < 1 || max_kv_len < 0) return HCI_EINVAL;
    if (n > 64 || L->poles > 16) return HCI_EUNSUPPORTED;
    rc = check_state(L, S, nb, (long long)max_kv_len + n);
    if (rc) return rc;
    const hci_block blk = tree_block(tree);
    rc = check_block(&blk);
    if (rc) return rc;
    if (tree_finish_lds_bytes(L, n) > kMaxLds) return HCI_EUNSUPPORTED;
    const AttnPlan plan = plan_attention(L, nb, 1, n - 1, max_kv_len, device_cu_count());
    if (plan.items_cap < 0) return HCI_EUNSUPPORTED;
    if (!ws || ws_bytes < plan.bytes || !aligned(ws, 256)) return HCI_EWORKSPACE;
    if (launch_verify(L, S, &blk, nb, 1, n, plan, ws, stream, nullptr, true, tree->parent) != hipSuccess)
        return HCI_EDEVICE;
    return HCI_OK;
}

int hci_accept_tree(int mode, int nb, int n, int vocab, float temperature, const int32_t* parent,
                    const int32_t* tokens, const float* target_logits, const float* draft_logits,
                    const double* uniforms, int32_t* n_accepted, int32_t* path, int32_t* next_token,
                    double* margin, uint32_t* status, hipStream_t stream) {
    if (mode != HCI_GREEDY && mode != HCI_SAMPLE) return HCI_EINVAL;
    if (nb < 1 || nb > 2147483647 || n < 1 || vocab < 1) return HCI_EINVAL;
    if (n > 64 || vocab > 65536) return HCI_EUNSUPPORTED;
    if (!parent || !tokens || !target_logits || !n_accepted || !path || !next_token) return HCI_EINVAL;
    if (mode == HCI_SAMPLE) {
        if (!(temperature > 0.f) || temperature == INFINITY) return HCI_EINVAL;
        if (!uniforms || !draft_logits) return HCI_EINVAL;
    }
    if (launch_accept_tree(mode, nb, n, vocab, temperature, parent, tokens, target_logits,
                           mode == HCI_SAMPLE ? draft_logits : nullptr, uniforms, n_accepted, path, next_token, margin,
                           status, stream) != hipSuccess)
        return HCI_EDEVICE;
    return HCI_OK;
}

int hci_slice_tree(const hci_layer* L, const hci_state* S, const hci_tree* tree, int nb, int n, int max_kv_len,
                   const int32_t* n_accepted, const int32_t* path, hipStream_t stream) {
    int rc = check_layer(L);
    if (rc) return rc;
    if (!tree || !tree->parent || !tree->x || !tree->k || !tree->v || !tree->f || !tree->s) return HCI_EINVAL;
    if (n < 1 || max_kv_len < 0 || !n_accepted || !path) return HCI_EINVAL;
    if (n > 64) return HCI_EUNSUPPORTED;
    rc = check_state(L, S, nb, (long long)max_kv_len + n);
    if (rc) return rc;
    const hci_block blk = tree_block(tree);
    if (launch_slice(L, S, &blk, nb, 1, n, max_kv_len, n_accepted, nullptr, stream, path, tree->parent) != hipSuccess)
        return HCI_EDEVICE;
    return HCI_OK;
}

size_t hci_prefill_workspace_bytes(const hci_layer* L, int nb, int T, int want_y) {
    if (check_layer(L) != HCI_OK || nb < 1 || T < 1) return 0;
    return plan_prefill(L, nb, T, want_y != 0).bytes;
}

int hci_prefill(const hci_layer* L, const hci_state* S, int nb, int T, int max_kv_len,
                const void* x, const void* k, const void* v, void* y,
                void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc = check_layer(L);
    if (rc) return rc;
    if (T < 1 || max_kv_len < 0 || !x || !k || !v) return HCI_EINVAL;
    if (!aligned(x, 16) || !aligned(k, 16) || !aligned(v, 16) || (y && !aligned(y, 16))) return HCI_EINVAL;
    if (L->poles > 16) return HCI_EUNSUPPORTED;
    rc = check_state(L, S, nb, (long long)max_kv_len + T);
    if (rc) return rc;
    const PrefillPlan plan = plan_prefill(L, nb, T, y != nullptr);
    if (plan.state_only ? prefill_state_lds_bytes(L) > 65536 : prefill_lds_bytes(L->taps_outer) > kMaxLds)
        return HCI_EUNSUPPORTED;
    if (plan.y_mfma && prefill_y_lds_bytes(L->taps_outer) > kMaxLds) return HCI_EUNSUPPORTED;
    if (plan.nchunks > 65535) return HCI_EUNSUPPORTED;
    if (!ws || ws_bytes < plan.bytes || !aligned(ws, 256)) return HCI_EWORKSPACE;
    if (launch_prefill(L, S, nb, T, max_kv_len, x, k, v, y, plan, ws, stream) != hipSuccess) return HCI_EDEVICE;
    return HCI_OK;
}

size_t hci_kv_cache_elems(const hci_layer* L, int nb, int kv_cap) {
    if (check_layer(L) != HCI_OK || nb < 1 || kv_cap < kTile || kv_cap % kTile) return 0;
    return (size_t)nb * L->heads * (size_t)kv_cap * L->head_dim;
}

static int kv_access(const hci_layer* L, const hci_state* S, int nb, int b, int row0, int nrows,
                     const void* a, const void* c, bool write, hipStream_t stream, void* oa, void* oc) {
    int rc = check_layer(L);
    if (rc) return rc;
    if (!S || !S->k_cache || !S->v_cache || S->kv_cap < kTile || S->kv_cap % kTile) return HCI_EINVAL;
    if (nb < 1 || b < 0 || b >= nb || row0 < 0 || nrows < 0) return HCI_EINVAL;
    if ((long long)row0 + nrows > S->kv_cap) return HCI_ECAPACITY;
    if (write ? (!a || !c) : (!oa || !oc)) return HCI_EINVAL;
    if (write && (!aligned(a, 16) || !aligned(c, 16))) return HCI_EINVAL;
    if (launch_kv_copy(L, S, b, row0, nrows, a, c, oa, oc, write, stream) != hipSuccess) return HCI_EDEVICE;
    return HCI_OK;
}

int hci_kv_write(const hci_layer* L, const hci_state* S, int nb, int b, int row0, int nrows,
                 const void* k_rows, const void* v_rows, hipStream_t stream) {
    return kv_access(L, S, nb, b, row0, nrows, k_rows, v_rows, true, stream, nullptr, nullptr);
}

int hci_kv_read(const hci_layer* L, const hci_state* S, int nb, int b, int row0, int nrows,
                void* k_rows, void* v_rows, hipStream_t stream) {
    return kv_access(L, S, nb, b, row0, nrows, nullptr, nullptr, false, stream, k_rows, v_rows);
}

static bool linear_shape_ok(int K, int N) {
    return K >= 32 && N >= 16 && K % 32 == 0 && N % 16 == 0 && N / 16 <= 2147483647 / 16 && K <= (1 << 20) &&
           N <= (1 << 20);
}

size_t hci_linear_packed_elems(int K, int N) {
    return linear_shape_ok(K, N) ? (size_t)K * N : 0;
}

int hci_linear_pack(int K, int N, const void* w, void* w_packed, hipStream_t stream) {
    if (!linear_shape_ok(K, N)) return HCI_EUNSUPPORTED;
    if (!w || !w_packed || !aligned(w_packed, 16)) return HCI_EINVAL;
    return launch_linear_pack(K, N, w, w_packed, stream) == hipSuccess ? HCI_OK : HCI_EDEVICE;
}

int hci_linear(int M, int K, int N, const void* x, const void* w_packed, const void* residual, void* y,
               int out_f32, hipStream_t stream) {
    if (!linear_shape_ok(K, N)) return HCI_EUNSUPPORTED;
    if (M < 1 || M > 65535 * 64) return HCI_EINVAL;
    if (!x || !w_packed || !y || !aligned(x, 16) || !aligned(w_packed, 16) || !aligned(y, 16)) return HCI_EINVAL;
    if (residual && !aligned(residual, 16)) return HCI_EINVAL;
    return launch_linear(M, K, N, 1, x, w_packed, residual, y, out_f32 != 0, stream) == hipSuccess ? HCI_OK
                                                                                                : HCI_EDEVICE;
}

int hci_rmsnorm(int M, int K, const void* x, const float* gamma, float eps, void* y, hipStream_t stream) {
    if (M < 1 || K < 1 || !x || !gamma || !y || !(eps >= 0.f)) return HCI_EINVAL;
    return launch_rmsnorm(M, K, x, gamma, eps, y, stream) == hipSuccess ? HCI_OK : HCI_EDEVICE;
}

static int check_model(const hci_model* M) {
    if (!M || !M->layers || M->n_layers < 1 || M->n_layers > 1024) return HCI_EINVAL;
    if (M->d < 32 || M->d % 32 || M->heads < 1 || M->head_dim < 1 || M->heads * M->head_dim != M->d)
        return HCI_EINVAL;
    if (M->head_dim != 64 && M->head_dim != 128) return HCI_EUNSUPPORTED;
    if (M->feature_layer < 0 || M->feature_layer >= M->n_layers || M->feature_window < 1) return HCI_EINVAL;
    if (!(M->eps >= 0.f)) return HCI_EINVAL;
    for (int l = 0; l < M->n_layers; ++l) {
        const hci_mixer& x = M->layers[l];
        if (!x.norm || !x.w_in || !x.w_out || !aligned(x.w_in, 16) || !aligned(x.w_out, 16)) return HCI_EINVAL;
        if (x.kind == HCI_MIX_ATTN) continue;
        if (x.kind != HCI_MIX_FIR && x.kind != HCI_MIX_IIR) return HCI_EINVAL;
        if (x.taps_short < 1 || x.taps_short > 8 || !x.w_short) return HCI_EUNSUPPORTED;
        if (x.kind == HCI_MIX_FIR && (x.taps_long < 1 || x.taps_long > 256 || !x.w_long)) return HCI_EUNSUPPORTED;
        if (x.kind == HCI_MIX_IIR && (x.poles < 1 || x.poles > 16 || !x.lambda || !x.beta || !x.c))
            return HCI_EUNSUPPORTED;
    }
    return HCI_OK;
}

static int check_model_io(const hci_model* M, const hci_model_state* S, const hci_model_block* blk, int nb, int nc,
                          int gamma, int max_kv_len) {
    int rc = check_model(M);
    if (rc) return rc;
    if (nb < 1 || nb > 65535 || nc < 1 || gamma < 0 || max_kv_len < 0) return HCI_EINVAL;
    const int P = gamma + 1;
    if (P > 64 || (long long)nc * P > 64 || (long long)nb * nc * P > 65535) return HCI_EUNSUPPORTED;
    if (!S || !S->layers || !S->kv_len || !S->feature || !blk || !blk->x || !blk->layers) return HCI_EINVAL;
    if (!aligned(blk->x, 16)) return HCI_EINVAL;
    bool attn = false;
    for (int l = 0; l < M->n_layers; ++l) {
        const hci_mixer& x = M->layers[l];
        const hci_layer_state& ls = S->layers[l];
        const hci_layer_block& lb = blk->layers[l];
        if (!lb.z || !aligned(lb.z, 16)) return HCI_EINVAL;
        if (x.kind == HCI_MIX_ATTN) {
            attn = true;
            if (!ls.k_cache || !ls.v_cache || !aligned(ls.k_cache, 16) || !aligned(ls.v_cache, 16)) return HCI_EINVAL;
            continue;
        }
        if (x.taps_short > 1 && !ls.short_win) return HCI_EINVAL;
        if (x.kind == HCI_MIX_FIR && (!lb.u || (x.taps_long > 1 && !ls.long_win))) return HCI_EINVAL;
        if (x.kind == HCI_MIX_IIR && (!lb.s || !ls.iir)) return HCI_EINVAL;
    }
    if (attn) {
        if (S->kv_cap < kTile || S->kv_cap % kTile) return HCI_EINVAL;
        if ((long long)max_kv_len + P > S->kv_cap) return HCI_ECAPACITY;
    }
    return HCI_OK;
}

size_t hci_model_workspace_bytes(const hci_model* M, int nb, int nc, int gamma, int max_kv_len) {
    if (check_model(M) != HCI_OK || nb < 1 || nc < 1 || gamma < 0 || max_kv_len < 0) return 0;
    return plan_model(M, nb, nc, gamma, max_kv_len, device_cu_count()).bytes;
}

int hci_model_verify(const hci_model* M, const hci_model_state* S, const hci_model_block* blk,
                     int nb, int nc, int gamma, int max_kv_len, void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc = check_model_io(M, S, blk, nb, nc, gamma, max_kv_len);
    if (rc) return rc;
    const int P = gamma + 1;
    const ModelPlan plan = plan_model(M, nb, nc, gamma, max_kv_len, device_cu_count());
    if (plan.has_attn && plan.attn.items_cap < 0) return HCI_EUNSUPPORTED;
    if (!ws || ws_bytes < plan.bytes || !aligned(ws, 256)) return HCI_EWORKSPACE;
    if (plan.has_attn) {
        const hci_layer L{M->d, 1, 1, 1, M->heads, M->head_dim, HCI_BF16, nullptr, nullptr, nullptr, nullptr, nullptr};
        if (stream_lds_bytes(&L, nc, P) > kMaxLds) return HCI_EUNSUPPORTED;
    }
    if (launch_model_verify(M, S, blk, nb, nc, P, plan, ws, stream) != hipSuccess) return HCI_EDEVICE;
    return HCI_OK;
}

int hci_model_slice(const hci_model* M, const hci_model_state* S, const hci_model_block* blk,
                    int nb, int nc, int gamma, int max_kv_len,
                    const int32_t* n_accepted, const int32_t* best_cand, hipStream_t stream) {
    int rc = check_model_io(M, S, blk, nb, nc, gamma, max_kv_len);
    if (rc) return rc;
    if (!n_accepted || (nc > 1 && !best_cand)) return HCI_EINVAL;
    if (launch_model_slice(M, S, blk, nb, nc, gamma + 1, n_accepted, nc > 1 ? best_cand : nullptr, stream) !=
        hipSuccess)
        return HCI_EDEVICE;
    return HCI_OK;
}

static int check_drafter(const hci_drafter* D) {
    if (!D || !D->layers || D->n_layers < 1 || D->n_layers > 64) return HCI_EINVAL;
    if (D->d < 32 || D->d % 32 || D->head_dim != 128 || D->heads * D->head_dim != D->d) return HCI_EUNSUPPORTED;
    if (D->d_target < 32 || D->d_target % 32 || D->ffn < 32 || D->ffn % 32 || D->vocab < 16 || D->vocab % 16)
        return HCI_EUNSUPPORTED;
    if (D->window < 1 || D->window > 64 || !(D->eps >= 0.f)) return HCI_EINVAL;
    if (!D->w_proj || !D->emb || !D->emb_t || !D->mask || !D->g_f) return HCI_EINVAL;
    if (!aligned(D->w_proj, 16) || !aligned(D->emb_t, 16)) return HCI_EINVAL;
    for (int l = 0; l < D->n_layers; ++l) {
        const hci_drafter_layer& L = D->layers[l];
        if (!L.g1 || !L.g2 || !L.w_qkv || !L.w_o || !L.w_up || !L.w_down) return HCI_EINVAL;
        if (!aligned(L.w_qkv, 16) || !aligned(L.w_o, 16) || !aligned(L.w_up, 16) || !aligned(L.w_down, 16))
            return HCI_EINVAL;
    }
    return HCI_OK;
}

size_t hci_draft_workspace_bytes(const hci_drafter* D, int nb, int gamma) {
    if (check_drafter(D) != HCI_OK || nb < 1 || gamma < 1 || gamma > 32) return 0;
    return plan_draft(D, nb, gamma).bytes;
}

int hci_draft_logits(const hci_drafter* D, int nb, int gamma, const void* window, const int32_t* anchor,
                     float* z, void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc = check_drafter(D);
    if (rc) return rc;
    if (nb < 1 || nb > 65535 || gamma < 1 || gamma > 32) return HCI_EINVAL;
    if (!window || !anchor || !z || !aligned(window, 16) || !aligned(z, 16)) return HCI_EINVAL;
    const DraftPlan p = plan_draft(D, nb, gamma);
    if (p.attn_lds > kMaxLds) return HCI_EUNSUPPORTED;
    if (!ws || ws_bytes < p.bytes || !aligned(ws, 256)) return HCI_EWORKSPACE;
    return launch_draft_logits(D, nb, gamma, window, anchor, z, p, ws, stream) == hipSuccess ? HCI_OK : HCI_EDEVICE;
}

int hci_draft_sample(int nb, int gamma, int vocab, float temperature, const float* z, const float* markov,
                     const int32_t* anchor, const double* uniforms, int32_t* drafts, float* draft_logits,
                     double* margin, hipStream_t stream) {
    if (nb < 1 || nb > 2147483647 || gamma < 1 || vocab < 1) return HCI_EINVAL;
    if (vocab > 4096) return HCI_EUNSUPPORTED;
    if (!(temperature > 0.f) || temperature == INFINITY) return HCI_EINVAL;
    if (!z || !markov || !anchor || !uniforms || !drafts || !draft_logits) return HCI_EINVAL;
    return launch_draft_sample(nb, gamma, vocab, temperature, z, markov, anchor, uniforms, drafts, draft_logits,
                               margin, stream) == hipSuccess ? HCI_OK : HCI_EDEVICE;
}

int hci_probe_sink_words(void) { return probe_blocks(); }

int hci_probe_read(const void* src, size_t bytes, float* sink, hipStream_t stream) {
    if (!src || !sink || bytes % 16 || !aligned(src, 16)) return HCI_EINVAL;
    return launch_probe_read(src, bytes, sink, stream) == hipSuccess ? HCI_OK : HCI_EDEVICE;
}

int hci_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
    if (!src || !dst || bytes % 16 || !aligned(src, 16) || !aligned(dst, 16)) return HCI_EINVAL;
    return launch_probe_copy(dst, src, bytes, stream) == hipSuccess ? HCI_OK : HCI_EDEVICE;
}

}  // extern "C"
