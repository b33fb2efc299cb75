// moe_permute_noalloc: moe_permute for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation).  Its scratch -- the per-assignment local ranks and the
// per-segment expert counts the grouping passes exchange -- lives in a
// file-scope device array of fixed size instead of a caller workspace.
//
// Each device holds its own copy of `scratch` (loaded with the library's code
// object, kept until the process ends).  In host code the array's name is only
// a host-side stand-in, so its device address is taken once per device, with
// that device current, by hipGetSymbolAddress, and only that address is handed
// to the kernels.  All calls on one device share its copy: calls that overlap
// on one device (different streams, or threads) race on it.  Nothing in it must
// start at zero: the grouping writes every local rank and segment count before
// it reads them.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = MOE_PERMUTE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];   // the current device's address of `scratch`, once known

// The device address of the current device's scratch, looked up on the first
// call on that device; nullptr if the lookup fails.
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" {

moe_status moe_permute_noalloc(const int32_t* ids, int64_t n_assign, int32_t E,
                               int64_t capacity, const void* src, moe_dtype dt, int64_t width,
                               int32_t src_div, void* dst, int64_t R_phys, int32_t* slot_row,
                               int32_t* row_src, int32_t* counts, int32_t* offsets,
                               int64_t* n_dropped, moe_stream stream) {
    using namespace moe;
    const moe_status st = permute_check(ids, n_assign, E, capacity, src, dt, width, src_div, dst,
                                        R_phys, slot_row, row_src, counts, offsets, n_dropped);
    if (st != MOE_OK) return st;
    if (permute_ws_bytes(n_assign, E) > kScratchBytes) return MOE_EWORKSPACE;
    void* ws = device_scratch();
    if (!ws) return MOE_ELAUNCH;
    const int es = dt == MOE_BF16 ? 2 : 4;
    if (launch_permute(ids, n_assign, E, capacity, src, src ? es : 0, width, src_div, dst, R_phys,
                       slot_row, row_src, counts, offsets, n_dropped, nullptr, 0, ws,
                       (hipStream_t)stream) != hipSuccess)
        return MOE_ELAUNCH;
    return MOE_OK;
}

}  // extern "C"
