// The full pass's 8-wavefront ping-pong instantiations of the flash kernel
// (attn_flash_kernel.h), plain and with RoPE inside, at head_dim 64 and 128.
// This file is compiled on its own with LLVM's maximum-ILP machine scheduler
// (-amdgpu-sched-strategy=max-ilp): on the ping-pong phases it gave the same
// instructions in an order that ran 0.6-1.5% faster at 480p and 0.7% at
// 720p, side by side, with bit-identical output, while the 4-wavefront
// pipelined tile of the other passes ran 0.5% slower with it.
#include "attn_flash_kernel.h"

namespace vdit {

hipError_t launch_flash_full_bf16(const void *q, const void *k, const void *v, void *o, int B, int N, int heads,
                                  int D, float scale_log2e, const FlashRope *rope, hipStream_t s) {
    const float c = scale_log2e;
    if (D == 128)
        return rope ? launch<128, 1, kFullWaves, 4>(q, k, v, o, B, N, N, heads, c, s, WinGeom{}, *rope)
                    : launch<128, 1, kFullWaves, 0>(q, k, v, o, B, N, N, heads, c, s);
    if (D == 64)
        return rope ? launch<64, 1, kFullWaves, 4>(q, k, v, o, B, N, N, heads, c, s, WinGeom{}, *rope)
                    : launch<64, 1, kFullWaves, 0>(q, k, v, o, B, N, N, heads, c, s);
    return hipErrorInvalidValue;
}

}  // namespace vdit
