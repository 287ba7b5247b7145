// Kernel-launcher stand-ins for the host-only sanitizer build of the library (no HIP, no
// GPU): host.cpp is compiled with AddressSanitizer and UndefinedBehaviorSanitizer and
// linked against these, so the CPU tests exercise every validation path, the descriptor
// builders and the Variable Block expansion under the sanitizers. Every argument error is
// detected before a launch, so no test reaches a launcher; one that did aborts the process.
#include <stdio.h>
#include <stdlib.h>

#include "../../masked_long_context_tiled_amd/csrc/host.h"

namespace mlct {

[[noreturn]] static void no_gpu(const char* fn) {
    fprintf(stderr, "%s reached in the host-only sanitizer build (no GPU here)\n", fn);
    abort();
}

int launch_desc(const attn_mask_params&, int32_t, int32_t*, void*) { no_gpu(__func__); }
int launch_index_dense(const Problem&, const int32_t*, void*, void*) { no_gpu(__func__); }
int launch_index_sparse(const Problem&, const uint8_t*, void*, void*) { no_gpu(__func__); }
int launch_fwd(const Problem&, const void*, const void*, const void*, void*, void*, float*, const int32_t*,
               const void*, void*) { no_gpu(__func__); }
int launch_bwd_pre(const Problem&, const void*, const void*, const void*, const void*, const void*, const void*,
                   float*, void*) { no_gpu(__func__); }
int launch_bwd_main(const Problem&, const void*, const void*, const void*, const float*, const void*, float*,
                    float*, float*, const int32_t*, const void*, float*, int, void*) { no_gpu(__func__); }
int launch_cast_bf16(const float*, void*, size_t, void*) { no_gpu(__func__); }
int launch_block_select(const Problem&, int, int, float, int, const void*, const void*, float*, uint8_t*, void*,
                        void*) { no_gpu(__func__); }
int launch_block_select_scratch(const Problem&, int, int, float, int, const void*, const void*, float*, uint8_t*,
                                void*) { no_gpu(__func__); }
int launch_lse_merge(const Problem&, void*, void*, float*, const void*, const void*, const float*, void*) {
    no_gpu(__func__);
}

}  // namespace mlct
