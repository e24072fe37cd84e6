// launch_stubs.cpp -- stand-ins for the kernel launchers of libpkv, so that
// the host code of the library (argument checks, work-split and workspace
// sizing, the block pool, the table helpers) builds and runs under the
// address and undefined-behaviour sanitizers on a machine without a GPU.
// Test infrastructure only: each launcher records that it was reached and
// launches nothing.
#include <hip/hip_runtime_api.h>

#include "pkv_internal.h"

namespace pkv {

int g_launches = 0;  // launchers reached (the driver checks valid calls get here)

hipError_t launch_store(const StoreArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_store_fp8(const StoreFp8Args &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode(const DecodeArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prefill(const PrefillArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_mixed(const MixedArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_cascade(const CascadeArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
int32_t compute_units() { return 256; }
hipError_t launch_copy_blocks(const CopyArgs &) { ++g_launches; return hipSuccess; }
hipError_t launch_read_probe(const void *, size_t, uint32_t *, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t noalloc_scratch(void **ptr) {
    static char fake[256] __attribute__((aligned(256)));
    *ptr = fake;  // never dereferenced: the stub launchers read nothing
    return hipSuccess;
}

}  // namespace pkv

extern "C" const char *hipGetErrorString(hipError_t) { return "hip error (stub)"; }

namespace pkv {
// the status words of a build without PKV_DEBUG_BOUNDS: always zero
#define PKV_STUB_WORD(name)                                \
    hipError_t debug_word_##name(uint32_t *out, bool) {    \
        out[0] = out[1] = out[2] = out[3] = 0u;            \
        return hipSuccess;                                 \
    }
PKV_STUB_WORD(store)
PKV_STUB_WORD(decode)
PKV_STUB_WORD(prefill)
PKV_STUB_WORD(mixed)
PKV_STUB_WORD(cascade)
PKV_STUB_WORD(copy)
}  // namespace pkv
