// Launchers of the flash attention kernel (attn_flash_kernel.h) for the
// spatial, cross and window passes, and for every pass at head_dim 32. The
// full pass at head_dim 64 and 128 runs the 8-wavefront ping-pong
// instantiations, which attn_flash_full.hip builds with a scheduler of
// their own.
#include "attn_flash_kernel.h"

namespace vdit {
hipError_t launch_flash_bf16(const void *q, const void *k, const void *v, void *o, int nseg, int L,
                             int Lk, int heads, int D, float scale_log2e, int pass, hipStream_t s) {
    if (pass == 0 && (D == 128 || D == 64))
        return launch_flash_full_bf16(q, k, v, o, nseg, L, heads, D, scale_log2e, nullptr, s);
    if (D == 128) {
        if (pass == 1) return launch<128, 1, kSpatialWaves, 1>(q, k, v, o, nseg, L, Lk, heads, scale_log2e, s);
        return launch<128, 1, kSpatialWaves, 2>(q, k, v, o, nseg, L, Lk, heads, scale_log2e, s);
    }
    if (D == 64) {
        if (pass == 1) return launch<64, 1, kSpatialWaves, 1>(q, k, v, o, nseg, L, Lk, heads, scale_log2e, s);
        return launch<64, 1, kSpatialWaves, 2>(q, k, v, o, nseg, L, Lk, heads, scale_log2e, s);
    }
    if (D == 32) {
        // A 64-key tile of 32-wide rows is 4 KB, half a 1 KB load per wave of
        // the 8-wave ping-pong; every pass takes the 4-wave pipelined tile.
        if (pass == 0) return launch<32, 1, kSpatialWaves, 0>(q, k, v, o, nseg, L, Lk, heads, scale_log2e, s);
        if (pass == 1) return launch<32, 1, kSpatialWaves, 1>(q, k, v, o, nseg, L, Lk, heads, scale_log2e, s);
        return launch<32, 1, kSpatialWaves, 2>(q, k, v, o, nseg, L, Lk, heads, scale_log2e, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_flash_rope_bf16(const void *q, const void *k, const void *v, void *o, int nseg, int L, int Lk,
                                  int heads, int D, float scale_log2e, int pass, const FlashRope &rope,
                                  hipStream_t s) {
    const float c = scale_log2e;
    if (pass == 0 && (D == 128 || D == 64))
        return launch_flash_full_bf16(q, k, v, o, nseg, L, heads, D, c, &rope, s);
    if (D == 128) {
        if (pass == 1) return launch<128, 1, kSpatialWaves, 5>(q, k, v, o, nseg, L, Lk, heads, c, s, WinGeom{}, rope);
    }
    if (D == 64) {
        if (pass == 1) return launch<64, 1, kSpatialWaves, 5>(q, k, v, o, nseg, L, Lk, heads, c, s, WinGeom{}, rope);
    }
    if (D == 32) {
        if (pass == 0) return launch<32, 1, kSpatialWaves, 4>(q, k, v, o, nseg, L, Lk, heads, c, s, WinGeom{}, rope);
        if (pass == 1) return launch<32, 1, kSpatialWaves, 5>(q, k, v, o, nseg, L, Lk, heads, c, s, WinGeom{}, rope);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_window_bf16(const void *q, const void *k, const void *v, void *o, int B, int heads, int D,
                              const WinGeom &g, float scale_log2e, hipStream_t s) {
    WinGeom wg = g;
    wg.nwt = (g.T + g.wt - 1) / g.wt;
    wg.nwh = (g.Hp + g.wh - 1) / g.wh;
    wg.nww = (g.Wp + g.ww - 1) / g.ww;
    const int nseg = B * wg.nwt * wg.nwh * wg.nww;
    const int Lmax = g.wt * g.wh * g.ww;  // extents are already clipped to the grid
    if (D == 128) return launch<128, 1, kSpatialWaves, 3>(q, k, v, o, nseg, Lmax, Lmax, heads, scale_log2e, s, wg);
    if (D == 64) return launch<64, 1, kSpatialWaves, 3>(q, k, v, o, nseg, Lmax, Lmax, heads, scale_log2e, s, wg);
    if (D == 32) return launch<32, 1, kSpatialWaves, 3>(q, k, v, o, nseg, Lmax, Lmax, heads, scale_log2e, s, wg);
    return hipErrorInvalidValue;
}

}  // namespace vdit
