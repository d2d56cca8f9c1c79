// Temporal pass of divided attention (bf16, gfx950).
//
// Each query (t, h, w) attends to the T tokens (t', h, w) at its own patch
// position: the "temporal pass across frames at each position" of "Video as a
// 3D signal" ("Patches and attention"), the (HW)*T^2 term of the divided cost
// in the "Video and 3D Generation" cheatsheet. With T = 21 latent frames
// ("Video Diffusion Models, in depth", Step 1) a sequence is 21 x 21 scores,
// so the pass moves 4 bytes of Q/K/V/O per ~10 FLOP and is bound by HBM.
//
// One wavefront owns one (b, position, head) sequence; a workgroup's four
// wavefronts take four consecutive heads of one position, so every token row
// they touch is one contiguous 4*head_dim*2-byte run. The sequence's frames
// are HW tokens apart; the kernel addresses them in place, so the
// time<->space permute is never materialised.
//  * V rows of the sequence are staged into the wave's LDS slice with 16-byte
//    loads, zero-filled past T; K and Q are read straight into their MFMA
//    operand registers (each lane one 16-byte piece of a row per k-step), so
//    a workgroup needs only 4 x 8 KB of LDS and more of them fit on a CU.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (32x32 covers T <= 32; T <= 64
//    uses 2x2 blocks): the matrix-core work is ~2% of the time the pass's
//    bytes need at HBM speed, and it frees the vector ALUs, which would
//    otherwise need ~60 TFLOP/s of fp32 FMA for the same products.
//  * An exact softmax per query column (one exchange with lane^32), then
//    O^T = V^T P^T with V^T read through ds_read_b64_tr_b16.
//  * O is staged through LDS and written back as whole 16-byte row chunks.
#include "vdit_internal.h"

namespace vdit {
namespace {

constexpr int kWaves = 4;

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <int D>
__device__ __forceinline__ int swz_k(int r, int c) { return c ^ (r % (D / 8)); }
template <int D>
__device__ __forceinline__ int swz_v(int r, int c) {
    constexpr int CH = D / 8;
    constexpr int RPP = 256 / (2 * D);
    return c ^ (4 * ((r / RPP) % (CH / 4)));
}

__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int KB>
__global__ __launch_bounds__(kWaves * 64, 4) void temporal_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    uint16_t *__restrict__ o, int B, int heads, int T, int HW, float c)
{
    constexpr int TP = 32 * KB;      // padded sequence length
    constexpr int CH = D / 8;        // 16-byte chunks per row
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int TILE = TP * D * 2; // bytes of one V slice
    __shared__ __attribute__((aligned(16))) unsigned char smem[kWaves * TILE];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, col = lane & 31;
    lds_u8 *vs_ = (lds_u8 *)smem + wave * TILE;

    const int64_t total = (int64_t)B * HW * heads;
    const int64_t sid = (int64_t)blockIdx.x * kWaves + wave;  // head fastest, then position, then b
    const bool active = sid < total;
    const int hd = (int)(sid % heads);
    const int64_t bp = sid / heads;
    const int64_t p = bp % HW;
    const int64_t b = bp / HW;
    const int64_t fs = (int64_t)HW * heads * D;  // elements between frames of one sequence
    const int64_t base = ((b * T * HW + p) * heads + hd) * D;

    // Stage V rows, zero past T.
    for (int ci = lane; ci < TP * CH; ci += 64) {
        const int r = ci / CH, ch = ci % CH;
        u32x4 vv = {0u, 0u, 0u, 0u};
        if (active && r < T) vv = *(const u32x4 *)(v + base + r * fs + ch * 8);
        *(__attribute__((address_space(3))) u32x4 *)(vs_ + r * D * 2 + swz_v<D>(r, ch) * 16) = vv;
    }
    // Queries as B operands and keys as A operands, zero past T.
    bf16x8 qop[KB][KS], kop[KB][KS];
#pragma unroll
    for (int qb = 0; qb < KB; ++qb) {
        const int qi = qb * 32 + col;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bool in = active && qi < T;
            qop[qb][s] = in ? *(const bf16x8 *)(q + base + qi * fs + 16 * s + 8 * half) : (bf16x8){};
            kop[qb][s] = in ? *(const bf16x8 *)(k + base + qi * fs + 16 * s + 8 * half) : (bf16x8){};
        }
    }
    __syncthreads();

    // S^T = K Q^T.
    f32x16 sacc[KB][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int qb = 0; qb < KB; ++qb) sacc[kb][qb] = (f32x16){};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int qb = 0; qb < KB; ++qb)
                sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kb][s], qop[qb][s], sacc[kb][qb], 0, 0, 0);

    // Exact softmax over the T keys of each query column.
    bf16x8 pop[KB][KB][2];
    float lsum[KB];
#pragma unroll
    for (int qb = 0; qb < KB; ++qb) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (key >= T) sacc[kb][qb][r] = -INFINITY;
            }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
        const float nm = -pair_max(mx) * c;
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                float pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][qb][8 * s2 + e], c, nm));
                    ls += pv[e];
                }
                u32x4 pk;
                pk[0] = pack_bf16x2(pv[0], pv[1]);
                pk[1] = pack_bf16x2(pv[2], pv[3]);
                pk[2] = pack_bf16x2(pv[4], pv[5]);
                pk[3] = pack_bf16x2(pv[6], pv[7]);
                pop[qb][kb][s2] = __builtin_bit_cast(bf16x8, pk);
            }
        lsum[qb] = pair_sum(ls);
    }

    // O^T = V^T P^T.
    const int grp = lane >> 4, gl = lane & 15;
    const int vrow = 4 * (grp >> 1) + (gl >> 2);
    const int vcol = 16 * (grp & 1) + 4 * (gl & 3);
    f32x16 oacc[DB][KB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < KB; ++qb) oacc[db][qb] = (f32x16){};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int r0 = kb * 32 + 16 * s2 + vrow;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int dc = db * 32 + vcol;
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_bf16x4 *)(vs_ + r0 * D * 2 + swz_v<D>(r0, dc >> 3) * 16 + (dc & 7) * 2));
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_bf16x4 *)(vs_ + (r0 + 8) * D * 2 + swz_v<D>(r0 + 8, dc >> 3) * 16 + (dc & 7) * 2));
                const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int qb = 0; qb < KB; ++qb)
                    oacc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop[qb][kb][s2], oacc[db][qb], 0, 0, 0);
            }
        }
    __syncthreads();  // every wave is done reading its V slice

    // Normalise into the V slice as row-major O rows, then write whole chunks.
#pragma unroll
    for (int qb = 0; qb < KB; ++qb) {
        const float inv = 1.0f / lsum[qb];
        const int qi = qb * 32 + col;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = db * 32 + 8 * r4 + 4 * half;
                u32x2 w;
                w[0] = pack_bf16x2(oacc[db][qb][4 * r4 + 0] * inv, oacc[db][qb][4 * r4 + 1] * inv);
                w[1] = pack_bf16x2(oacc[db][qb][4 * r4 + 2] * inv, oacc[db][qb][4 * r4 + 3] * inv);
                *(__attribute__((address_space(3))) u32x2 *)(vs_ + qi * D * 2 + swz_k<D>(qi, d >> 3) * 16 +
                                                              (d & 7) * 2) = w;
            }
    }
    __syncthreads();
    if (active)
        for (int ci = lane; ci < T * CH; ci += 64) {
            const int r = ci / CH, ch = ci % CH;
            *(u32x4 *)(o + base + r * fs + ch * 8) =
                *(const __attribute__((address_space(3))) u32x4 *)(vs_ + r * D * 2 + swz_k<D>(r, ch) * 16);
        }
}

template <int D, int KB>
hipError_t launch(const void *q, const void *k, const void *v, void *o, int B, int heads, int T, int HW,
                  float c, hipStream_t s) {
    const int64_t total = (int64_t)B * HW * heads;
    const uint32_t grid = (uint32_t)((total + kWaves - 1) / kWaves);
    hipLaunchKernelGGL((temporal_bf16<D, KB>), dim3(grid), dim3(kWaves * 64), 0, s, (const uint16_t *)q,
                       (const uint16_t *)k, (const uint16_t *)v, (uint16_t *)o, B, heads, T, HW, c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_temporal_bf16(const void *q, const void *k, const void *v, void *o, int B, int heads, int T,
                                int HW, int D, float scale_log2e, hipStream_t s) {
    if (T <= 32) {
        if (D == 128) return launch<128, 1>(q, k, v, o, B, heads, T, HW, scale_log2e, s);
        if (D == 64) return launch<64, 1>(q, k, v, o, B, heads, T, HW, scale_log2e, s);
    } else if (T <= 64) {
        if (D == 128) return launch<128, 2>(q, k, v, o, B, heads, T, HW, scale_log2e, s);
        if (D == 64) return launch<64, 2>(q, k, v, o, B, heads, T, HW, scale_log2e, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace vdit
