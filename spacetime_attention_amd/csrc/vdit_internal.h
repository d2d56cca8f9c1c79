// Internal declarations shared by the HIP translation units of libvdit.
// Not part of the public ABI (include/vdit.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vdit {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 <-> fp32 on raw bits. Round-to-nearest-even; NaN stays NaN.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// acc + lo + hi of a packed bf16 pair (lo in bits 0..15), in fp32: one
// v_dot2c_f32_bf16 against the pair (1, 1). The probabilities of a softmax
// are summed this way from the same bf16 values the V product consumes, so
// the normalisation divides exactly the weights that were applied.
__device__ __forceinline__ float add_bf16_pair(uint32_t pk, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                           acc, false);
}

// Maps a hardware workgroup id to a logical tile id so that the workgroups
// one XCD receives (ids congruent mod 8, dispatched round-robin) form one
// contiguous run of logical tiles and so share K/V in that XCD's L2.
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t hw_id, uint32_t total) {
    const uint32_t nx = 8;
    const uint32_t xcd = hw_id % nx, local = hw_id / nx;
    const uint32_t per = total / nx, extra = total % nx;
    return xcd < extra ? xcd * (per + 1) + local : extra * (per + 1) + (xcd - extra) * per + local;
}

// ---- launchers (each returns hipGetLastError() after its launch) ----------

// Softmax attention over contiguous segments: segment s has L query rows
// [s*L, (s+1)*L) of q/o and Lk key rows [s*Lk, (s+1)*Lk) of k/v, all arrays
// [rows, heads, D]; its queries attend to exactly its keys. Full attention is
// nseg = B, L = Lk = N; the spatial pass nseg = B*T, L = Lk = Hp*Wp;
// cross-attention nseg = B, L = Nq, Lk = Nk. pass: 0 full, 1 spatial,
// 2 cross (selects the tuned instantiation).
hipError_t launch_flash_bf16(const void *q, const void *k, const void *v, void *o, int nseg,
                             int L, int Lk, int heads, int D, float scale_log2e, int pass,
                             hipStream_t s);

// 3D RoPE applied inside an attention kernel (the flash kernel: to the
// queries once, and to each K tile as it lands in LDS; the temporal kernel:
// to each sequence's Q and K rows in LDS). Token n of a clip sits at grid position
// (n / (Hp*Wp), (n / Wp) % Hp, n % Wp) of a T x Hp x Wp grid; pair j
// (< D/2) turns with t below b1, with h below b2 and with w above, at
// freq_rev[j] = theta^(-2jj/d_a) / (2 pi) revolutions per grid step.
struct FlashRope {
    int T, Hp, Wp, b1, b2;
    float freq_rev[64];
};
// As launch_flash_bf16 for pass 0 (full) or 1 (spatial), with q and k
// rotated by `rope` on the fly (q and k in memory stay unrotated).
hipError_t launch_flash_rope_bf16(const void *q, const void *k, const void *v, void *o, int nseg, int L, int Lk,
                                  int heads, int D, float scale_log2e, int pass, const FlashRope &rope,
                                  hipStream_t s);
// Full attention at head_dim 64 or 128 (nseg = B clips of N tokens) on the
// 8-wavefront ping-pong kernel; rope as launch_flash_rope_bf16, or null.
hipError_t launch_flash_full_bf16(const void *q, const void *k, const void *v, void *o, int B, int N, int heads,
                                  int D, float scale_log2e, const FlashRope *rope, hipStream_t s);

// Non-overlapping spacetime windows over a (T, Hp, Wp) token grid: window
// (iwt, iwh, iww) holds tokens t in [iwt*wt, min((iwt+1)*wt, T)) and likewise
// for h and w; its queries attend to exactly its tokens. wt/wh/ww are clipped
// to the grid by the caller; nwt/nwh/nww (windows per axis) and nqb (query
// blocks per window) are filled in by the launcher.
struct WinGeom {
    int T, Hp, Wp, wt, wh, ww, nwt, nwh, nww, nqb;
};
hipError_t launch_window_bf16(const void *q, const void *k, const void *v, void *o, int B, int heads, int D,
                              const WinGeom &g, float scale_log2e, hipStream_t s);
hipError_t launch_window_f32(const float *q, const float *k, const float *v, float *o, int B, int heads, int D,
                             const WinGeom &g, float scale, hipStream_t s);

// fp32 attention with a generic key set: query token n of batch b has keys
// key(m) = kbase(n) + m*kstride, m < nkeys, where for mode 0 (full)
// kbase = b*N, kstride = 1, nkeys = N; mode 1 (spatial) kbase = b*N + t*HW,
// kstride = 1, nkeys = HW; mode 2 (temporal) kbase = b*N + p, kstride = HW,
// nkeys = T.
hipError_t launch_attn_f32(const float *q, const float *k, const float *v, float *o, int B,
                           int heads, int T, int HW, int D, int mode, float scale, hipStream_t s);
// fp32 cross-attention: q/o [B, Nq, heads, D], k/v [B, Nk, heads, D].
hipError_t launch_cross_f32(const float *q, const float *k, const float *v, float *o, int B,
                            int heads, int Nq, int Nk, int D, float scale, hipStream_t s);

// Temporal pass in bf16: one wavefront per (b, position, head) sequence of T
// tokens at stride HW tokens.
hipError_t launch_temporal_bf16(const void *q, const void *k, const void *v, void *o, int B,
                                int heads, int T, int HW, int D, float scale_log2e, hipStream_t s);

// The temporal pass with q and k rotated by `rope` (FlashRope, above) in
// on-chip memory; q and k in memory stay unrotated.
hipError_t launch_temporal_rope_bf16(const void *q, const void *k, const void *v, void *o, int B, int heads, int T,
                                     int HW, int D, float scale_log2e, const FlashRope &rope, hipStream_t s);

// Patchify as an implicit-im2col GEMM.
struct PatchGeom {
    int B, C, pt, ph, pw, Tl, Hl, Wl, T, Hp, Wp, Dout;
};
hipError_t launch_patchify_bf16(const void *x, const void *w, const void *bias, void *tok,
                                const PatchGeom &g, hipStream_t s);
hipError_t launch_patchify_f32(const float *x, const float *w, const float *bias, float *tok,
                               const PatchGeom &g, hipStream_t s);

// 3D RoPE: per pair j (< D/2) its axis (0 t, 1 h, 2 w) and frequency
// (fp64 so that the angle can be formed and reduced in fp64).
struct RopeTable {
    double freq[128];
    unsigned char axis[128];
};
hipError_t launch_rope_bf16(const void *x, void *y, int B, int heads, int T, int Hp, int Wp, int D,
                            const RopeTable &tab, hipStream_t s);
hipError_t launch_rope_f32(const float *x, float *y, int B, int heads, int T, int Hp, int Wp, int D,
                           const RopeTable &tab, hipStream_t s);

// QKV projection: tokens x [M][dim] (M = B*N, batch-major), fused weight
// [3*dim][dim], outputs [M][dim] each; token m sits at grid index m % N of a
// (T, Hp, Wp) grid. D is head_dim.
struct QkvGeom {
    int M, N, Hp, Wp, dim, D;
    float eps;
};
// Rotation for the bf16 kernel: per pair j (< 64) its frequency in
// revolutions per grid step (theta^(-2jj/d_a) / (2 pi)); pairs j < b1 turn
// with t, b1 <= j < b2 with h, the rest with w; on = 0 disables it.
struct QkvRope {
    float freq_rev[64];
    int b1, b2;
    int on;
};
hipError_t launch_qkv_proj_bf16(const void *x, const void *w, const void *bias, const void *gq, const void *gk,
                                void *q, void *k, void *v, const QkvGeom &g, const QkvRope &rope, hipStream_t s);
hipError_t launch_qkv_proj_f32(const float *x, const float *w, const float *bias, const float *gq, const float *gk,
                               float *q, float *k, float *v, const QkvGeom &g, const RopeTable &tab, int rope_on,
                               hipStream_t s);

}  // namespace vdit
