// gdn_chunk_fwd_noalloc: gdn_chunk_fwd with its workspace in a static device
// array instead of caller memory, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  It runs exactly the kernels of gdn_chunk_fwd.
//
// The array lives in this translation unit's code object: every GPU the
// library runs this entry point on holds its own copy (kScratchBytes) until
// the process ends.  Host code never uses the array's name as a device
// address (in host code it names a host-side stand-in): on its first call on
// a device, with that device current, the entry point asks the runtime for
// the array's device address and keeps it per device.
#include <atomic>

#include "gdn_internal.h"
#include "../../include/gdn.h"

namespace {

constexpr size_t kScratchBytes = (size_t)128 << 20;  // GDN_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == GDN_NOALLOC_SCRATCH_BYTES, "header and library agree");
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The array's device address on each device, filled on the first call there
// (the only state the library keeps between calls; every thread that fills a
// slot stores the same address).
std::atomic<void*> g_scratch_addr[kMaxDevices];

void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_addr[dev].store(ptr, std::memory_order_release);
    return ptr;
}

}  // namespace

extern "C" int gdn_chunk_fwd_noalloc(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                     int32_t chunk, int32_t dtype, int32_t gate, int32_t order,
                                     float scale, const void* q, const void* k, const void* v,
                                     const float* alpha, const float* beta, const float* state0,
                                     float* out, float* state_out, void* stream) {
    const int s = gdn_validate(B, T, H, dk, dv, chunk, dtype, gate, order, 1);
    if (s != GDN_OK) return s;
    // gdn_chunk_fwd's own workspace size for these arguments (host only)
    const size_t need = gdn_workspace_bytes(B, T, H, dk, dv, chunk, dtype, gate, 1);
    if (need > kScratchBytes) return GDN_E_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        ws = scratch_on_current_device();
        if (!ws) return GDN_E_HIP;
    }
    // nothing in the workspace needs to start at zero: every kernel writes
    // what it later reads (the last call's contents are overwritten)
    return gdn_chunk_fwd(B, T, H, dk, dv, chunk, dtype, gate, order, scale, q, k, v, alpha, beta,
                         state0, out, state_out, ws, need > 0 ? kScratchBytes : 0, stream);
}
