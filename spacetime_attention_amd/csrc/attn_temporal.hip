// Temporal pass of divided attention (bf16, gfx950).
//
// Each query (t, h, w) attends to the T tokens (t', h, w) at its own patch
// position: the "temporal pass across frames at each position" of "Video as a
// 3D signal" ("Patches and attention"), the (HW)*T^2 term of the divided cost
// in the "Video and 3D Generation" cheatsheet. With T = 21 latent frames
// ("Video Diffusion Models, in depth", Step 1) a sequence is 21 x 21 scores,
// so the pass moves 4 bytes of Q/K/V/O per ~10 FLOP and is bound by HBM.
//
// One wavefront owns one (b, position, head) sequence; a workgroup's
// wavefronts take consecutive heads of one position. The sequence's frames
// are HW tokens apart; the kernel addresses them in place, so the
// time<->space permute is never materialised.
//  * Q, K and V rows of the sequence go straight from HBM into the wave's
//    own LDS slice with non-temporal buffer loads that write LDS (each 1 KB
//    load covers four whole 256-byte rows, so every request is a full
//    cache line). The buffer descriptors end at row T-1, so the padding rows
//    read as zeros.
//    Each wave only ever reads its own slice, so waves never wait for each
//    other: no workgroup barrier.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (32x32 covers T <= 32; T <= 64
//    uses 2x2 blocks): the matrix-core work is ~2% of the time the pass's
//    bytes need at HBM speed, and it frees the vector ALUs, which would
//    otherwise need ~60 TFLOP/s of fp32 FMA for the same products.
//  * An exact softmax per query column (one exchange with lane^32), then
//    O^T = V^T P^T with V^T read through ds_read_b64_tr_b16.
//  * O is staged through the Q slice and written back as whole 16-byte row
//    chunks.
//  * The RoPE instantiation rotates the sequence's Q and K rows in the LDS
//    slice once they have landed: each lane rewrites the 16-byte chunks its
//    own loads wrote. A Q chunk and the K chunk at the same place belong to
//    the same frame and feature pairs, so they share their angles; every
//    row is rotated exactly once, as the separate RoPE pass would.
#include "vdit_internal.h"

namespace vdit {
namespace {

constexpr int kWaves = 2;  // wavefronts per workgroup (each on its own LDS slice)

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Buffer descriptor word 3 for gfx9-family raw (unswizzled) buffers.
constexpr int kBufferFlags = 0x00020000;
// Cache policy of the Q/K/V loads: non-temporal (the NT bit). Every byte of
// Q, K and V is read exactly once, and marked as streaming data the pass
// runs at 5.8 TB/s instead of 5.1 (plain or non-temporal stores of O make no
// difference, and non-temporal stores on top of these loads cost some of
// the gain).
constexpr int kStreamLoad = 2;
// s_waitcnt vmcnt(N): at most N of this wave's vector-memory loads
// (including the ones that write LDS directly) are still outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem_upto() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 0..63");
    // vmcnt is split over bits [3:0] and [15:14]; expcnt and lgkmcnt stay at
    // their maximum (no wait).
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

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

// QKR: rows of the Q and K slices. With T <= 24, 24 rows suffice: the
// operand reads of rows 24..31 then fall into the next slice of the same
// wave (finite data), and land only in key rows that the mask overwrites
// with -inf and in query columns that are never stored. V always has TP
// rows, zero past T, because a zero weight times non-finite padding would
// not be zero.
template <int D, int KB, int QKR, bool ROPE>
__global__ __launch_bounds__(kWaves * 64) void temporal_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    uint16_t *__restrict__ o, int B, int heads, int T, int HW, float c, FlashRope fr)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    constexpr int TP = 32 * KB;      // padded sequence length
    constexpr int CH = D / 8;        // 16-byte chunks per row
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int VT = TP * D * 2;   // bytes of the V slice
    constexpr int QT = QKR * D * 2;  // bytes of the Q and of the K slice
    constexpr int RPL = 64 / CH;     // rows per wave-wide 1 KB load
    static_assert(QKR % RPL == 0 && QKR <= TP, "slice rows must be whole 1 KB loads");
    __shared__ __attribute__((aligned(16))) unsigned char smem[kWaves * (2 * QT + VT)];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5, col = lane & 31;
    lds_u8 *qs_ = (lds_u8 *)smem + wave * (2 * QT + VT);
    lds_u8 *ks_ = qs_ + QT;
    lds_u8 *vs_ = ks_ + QT;

    const int64_t total = (int64_t)B * HW * heads;
    // Workgroups are renumbered so that each XCD walks a contiguous run of
    // sequences: the heads of neighbouring positions, whose rows of a frame
    // are contiguous in memory, are then read by one XCD at about the same
    // time (2% faster than the round-robin order, same-box A/B).
    const uint32_t wg = xcd_contiguous(blockIdx.x, gridDim.x);
    const int64_t sid = (int64_t)wg * kWaves + wave;  // head fastest, then position, then b
    if (sid >= total) return;  // whole wave leaves; no barrier follows
    const int hd = (int)(sid % heads);
    const int64_t bp = sid / heads;
    const int64_t p = bp % HW;
    const int64_t b = bp / HW;
    const int64_t fs = (int64_t)HW * heads * D;  // elements between frames of one sequence
    const int64_t base = ((b * T * HW + p) * heads + hd) * D;

    // Descriptors over this sequence's rows: the size ends at row T-1.
    const int nrec = (int)(((int64_t)(T - 1) * fs + D) * 2);
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc((void *)(q + base), 0, nrec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void *)(k + base), 0, nrec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void *)(v + base), 0, nrec, kBufferFlags);
    // RoPE: the frequencies of the four pairs in each chunk this lane loads,
    // read from the kernel arguments before any tile load is issued. Loads
    // complete in issue order, so reading them after the V loads would make
    // the rotation wait for all of V.
    f32x4 fq[ROPE ? QKR / RPL : 1];
    if constexpr (ROPE) {
#pragma unroll
        for (int i = 0; i < QKR / RPL; ++i) {
            const int r = RPL * i + lane / CH;
            const int lc = (lane % CH) ^ swz_k<D>(r, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) fq[i][e] = fr.freq_rev[4 * lc + e];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // Q and K first, V last: the score products only wait for Q and K, and
    // V's loads keep streaming under them.
#pragma unroll
    for (int i = 0; i < QKR / RPL; ++i) {
        const int r = RPL * i + lane / CH, pc = lane % CH;
        const uint32_t off = (uint32_t)(r * fs * 2) + (pc ^ swz_k<D>(r, 0)) * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_void *)(qs_ + i * 1024), 16, off, 0, 0, kStreamLoad);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void *)(ks_ + i * 1024), 16, off, 0, 0, kStreamLoad);
    }
#pragma unroll
    for (int i = 0; i < TP / RPL; ++i) {
        const int r = RPL * i + lane / CH, pc = lane % CH;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void *)(vs_ + i * 1024), 16,
                                                 (uint32_t)(r * fs * 2) + (pc ^ swz_v<D>(r, 0)) * 16, 0, 0,
                                                 kStreamLoad);
    }
    // Loads complete in issue order: with only the TP/RPL V loads still
    // outstanding, this wave's Q and K rows are in its LDS slice.
    wait_vmem_upto<TP / RPL>();

    if constexpr (ROPE) {
        // Row r of the slices is frame r at patch position p = (h, w). Pair j
        // turns with t below b1, with h below b2 and with w above; the angle
        // is taken in revolutions, reduced to [0, 1) for v_sin/v_cos.
        const float fh = (float)(int)(p / fr.Wp), fw = (float)(int)(p % fr.Wp);
#pragma unroll
        for (int i = 0; i < QKR / RPL; ++i) {
            const int r = RPL * i + lane / CH;
            const int lc = (lane % CH) ^ swz_k<D>(r, 0);
            auto *qp = (__attribute__((address_space(3))) u32x4 *)(qs_ + i * 1024 + 16 * lane);
            auto *kp = (__attribute__((address_space(3))) u32x4 *)(ks_ + i * 1024 + 16 * lane);
            u32x4 xq = *qp, xk = *kp;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * lc + e;
                const float pos = j < fr.b1 ? (float)r : (j < fr.b2 ? fh : fw);
                const float rev = __builtin_amdgcn_fractf(pos * fq[i][e]);
                const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
                float x0 = __uint_as_float(xq[e] << 16), x1 = __uint_as_float(xq[e] & 0xffff0000u);
                xq[e] = pack_bf16x2(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
                x0 = __uint_as_float(xk[e] << 16);
                x1 = __uint_as_float(xk[e] & 0xffff0000u);
                xk[e] = pack_bf16x2(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
            }
            *qp = xq;
            *kp = xk;
        }
    }

    // S^T = K Q^T: K rows as A operands, Q rows as B operands.
    f32x16 sacc[KB][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int qb = 0; qb < KB; ++qb) sacc[kb][qb] = (f32x16){};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        bf16x8 kop[KB], qop[KB];
#pragma unroll
        for (int xb = 0; xb < KB; ++xb) {
            const int r = xb * 32 + col;
            const int off = r * D * 2 + swz_k<D>(r, 2 * s + half) * 16;
            kop[xb] = *(const __attribute__((address_space(3))) bf16x8 *)(ks_ + off);
            qop[xb] = *(const __attribute__((address_space(3))) bf16x8 *)(qs_ + off);
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int qb = 0; qb < KB; ++qb)
                sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kb], qop[qb], sacc[kb][qb], 0, 0, 0);
    }

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
                for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][qb][8 * s2 + e], c, nm));
                u32x4 pk;
                pk[0] = pack_bf16x2(pv[0], pv[1]);
                pk[1] = pack_bf16x2(pv[2], pv[3]);
                pk[2] = pack_bf16x2(pv[4], pv[5]);
                pk[3] = pack_bf16x2(pv[6], pv[7]);
                pop[qb][kb][s2] = __builtin_bit_cast(bf16x8, pk);
                // The sum takes the same bf16 weights the V product applies.
#pragma unroll
                for (int e = 0; e < 4; ++e) ls = add_bf16_pair(pk[e], ls);
            }
        lsum[qb] = pair_sum(ls);
    }

    // O^T = V^T P^T.
    wait_vmem_upto<0>();  // V has landed
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

    // Normalise into the Q slice (fully consumed above, and LDS accesses of
    // one wave complete in order) as row-major O rows, then store whole rows.
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
                *(__attribute__((address_space(3))) u32x2 *)(qs_ + qi * D * 2 + swz_k<D>(qi, d >> 3) * 16 +
                                                              (d & 7) * 2) = w;
            }
    }
    for (int ci = lane; ci < T * CH; ci += 64) {
        const int r = ci / CH, ch = ci % CH;
        *(u32x4 *)(o + base + r * fs + ch * 8) =
            *(const __attribute__((address_space(3))) u32x4 *)(qs_ + r * D * 2 + swz_k<D>(r, ch) * 16);
    }
#endif
}

template <int D, int KB, int QKR, bool ROPE>
hipError_t launch(const void *q, const void *k, const void *v, void *o, int B, int heads, int T, int HW,
                  float c, hipStream_t s, const FlashRope &fr) {
    const int64_t total = (int64_t)B * HW * heads;
    const uint32_t grid = (uint32_t)((total + kWaves - 1) / kWaves);
    hipLaunchKernelGGL((temporal_bf16<D, KB, QKR, ROPE>), dim3(grid), dim3(kWaves * 64), 0, s, (const uint16_t *)q,
                       (const uint16_t *)k, (const uint16_t *)v, (uint16_t *)o, B, heads, T, HW, c, fr);
    return hipGetLastError();
}

template <bool ROPE>
hipError_t dispatch(const void *q, const void *k, const void *v, void *o, int B, int heads, int T, int HW, int D,
                    float c, hipStream_t s, const FlashRope &fr) {
    if (T <= 24) {
        if (D == 128) return launch<128, 1, 24, ROPE>(q, k, v, o, B, heads, T, HW, c, s, fr);
        if (D == 64) return launch<64, 1, 24, ROPE>(q, k, v, o, B, heads, T, HW, c, s, fr);
        // 32-wide rows: one 1 KB load is 16 rows, so the Q and K slices are 32.
        if (D == 32) return launch<32, 1, 32, ROPE>(q, k, v, o, B, heads, T, HW, c, s, fr);
    } else if (T <= 32) {
        if (D == 128) return launch<128, 1, 32, ROPE>(q, k, v, o, B, heads, T, HW, c, s, fr);
        if (D == 64) return launch<64, 1, 32, ROPE>(q, k, v, o, B, heads, T, HW, c, s, fr);
        if (D == 32) return launch<32, 1, 32, ROPE>(q, k, v, o, B, heads, T, HW, c, s, fr);
    } else if (T <= 64) {
        if (D == 128) return launch<128, 2, 64, ROPE>(q, k, v, o, B, heads, T, HW, c, s, fr);
        if (D == 64) return launch<64, 2, 64, ROPE>(q, k, v, o, B, heads, T, HW, c, s, fr);
        if (D == 32) return launch<32, 2, 64, ROPE>(q, k, v, o, B, heads, T, HW, c, s, fr);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_temporal_bf16(const void *q, const void *k, const void *v, void *o, int B, int heads, int T,
                                int HW, int D, float scale_log2e, hipStream_t s) {
    return dispatch<false>(q, k, v, o, B, heads, T, HW, D, scale_log2e, s, FlashRope{});
}

hipError_t launch_temporal_rope_bf16(const void *q, const void *k, const void *v, void *o, int B, int heads, int T,
                                     int HW, int D, float scale_log2e, const FlashRope &rope, hipStream_t s) {
    return dispatch<true>(q, k, v, o, B, heads, T, HW, D, scale_log2e, s, rope);
}

}  // namespace vdit
