// noalloc.hip -- the fixed scratch of zero_shard_step_noalloc, the shard step
// for callers that cannot allocate device or pinned memory.
//
// zero_shard_step keeps its flag word, blocks-done counter and the host word
// the pass's last block writes the decision into in a workspace it allocates
// on a device's first call.  The no-allocation variant keeps the same three
// words in this file-scope device array instead, one copy per device, held
// until the process ends; its decision word is device memory, which the call
// copies back after the pass.
#include <mutex>

#include "zp_internal.hpp"

namespace zp {

// Word 0: the flag word; words 16-17: the 64-bit blocks-done counter; words
// 32-33: the decision word ((epoch << 1) | flag).  256 bytes in all.
static __device__ __align__(256) uint32_t scratch[kStaticScratchWords];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
uint32_t* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

namespace {
// Zeroes n words at w (one block; n <= 64 * 4).  A kernel rather than a
// memset node, so the clear is an ordinary launch on the caller's stream.
__global__ void clear_words_kernel(uint32_t* w, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) w[i] = 0u;
}
}  // namespace

hipError_t clear_scratch(uint32_t* w, hipStream_t stream) {
    hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(64), 0, stream, w, kStaticScratchWords);
    return hipGetLastError();
}

int static_scratch(int dev, uint32_t** out) {
    if (dev < 0 || dev >= kMaxScratchDevices) return fail(ZERO_ERR_INVALID_ARG, "device index out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        // device `dev` is current: this is its copy of the array
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress (scratch)");
        g_scratch_ptr[dev] = static_cast<uint32_t*>(p);
    }
    *out = g_scratch_ptr[dev];
    return ZERO_OK;
}

}  // namespace zp
