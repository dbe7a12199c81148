// hci_verify_block for callers that cannot allocate device memory: the
// verify's workspace (the job queue's counter, the work-list table and the
// split-K partials) lives in a file-scope device array instead of a buffer the
// caller passes.  Every GPU the library runs on holds its own copy of the
// array until the process ends; its device address is looked up once per
// device, with that device current, and kept.
#include "hci_internal.h"

#include <atomic>
#include <mutex>

namespace hci {

constexpr size_t kScratchBytes = HCI_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// In host code this name is only a stand-in for the symbol; kernels receive the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static std::atomic<void*> g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

// The current device's copy of the scratch array (nullptr if the lookup fails).
static void* scratch_ptr(int dev) {
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace hci

extern "C" int hci_verify_block_noalloc(const hci_layer* L, const hci_state* S, const hci_block* blk,
                                        int nb, int nc, int gamma, int max_kv_len, hipStream_t stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= hci::kMaxDevices) return HCI_EDEVICE;
    void* ws = hci::scratch_ptr(dev);
    if (!ws) return HCI_EDEVICE;
    // the verify's own checks reject a call whose workspace would exceed the array
    // (HCI_EWORKSPACE) before anything is enqueued; its set-up kernel re-initialises the queue
    // counter and the work list on every call, whatever an earlier call left behind
    return hci_verify_block(L, S, blk, nb, nc, gamma, max_kv_len, ws, hci::kScratchBytes, stream);
}
