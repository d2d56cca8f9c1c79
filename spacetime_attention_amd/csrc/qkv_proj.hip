// QKV projection of a DiT block's attention input (bf16, gfx950), with the
// per-head RMSNorm of Q and K and their 3D rotation fused into the epilogue.
//
// "How AI Generates Video: Inside Sora and Wan2.1 on a Real GPU", section 5
// (attn1): the block projects its tokens into heads of 128-wide queries, keys
// and values, applies RMSNorm to Q and K, and rotates Q and K with the
// [44, 42, 42] factorised RoPE of section 4. With a fused weight W
// [3*dim][dim] (rows 0..dim-1 make Q, then K, then V) and tokens x [M][dim]:
//   y[m][c] = bias[c] + sum_k W[c][k] x[m][k]
//   Q, K: each head's head_dim values scaled by 1/sqrt(mean(y^2) + eps) and
//         by the per-channel gain, then rotated by the token's (t, h, w);
//   V:    y as is.
//
// The product is formed transposed, out^T = W x^T, on
// v_mfma_f32_32x32x16_bf16: the A operand is a 32-channel block of W, the B
// operand a 32-token block of x, both K-contiguous rows read from LDS. In the
// result a lane owns one token and 16 channels per block; over a head's four
// blocks, lanes l and l^32 together hold the token's 128 channels, so the
// head's mean square is a register sum plus one v_permlane32_swap, and each
// RoPE pair (2j, 2j+1) sits in one lane's consecutive registers.
//
// Work layout: a workgroup owns a 256-channel x 256-token tile with 8
// wavefronts, two per SIMD, so that one's LDS reads, waits and epilogue
// overlap the other's MFMAs; a wavefront owns 128 channels (one head) x 64
// tokens, i.e. 4 x 2 blocks and 8 accumulators. K advances in stages of 64: W and x
// tiles of [256][64] bf16 are filled by buffer loads that write LDS directly
// and are double-buffered; a chunk-XOR swizzle keeps the operand reads
// (32 rows, one 16-byte chunk each) free of bank conflicts. Rows past the end
// of W or x read as zero through the buffer descriptors' sizes.
#include "vdit_internal.h"

#include <type_traits>

namespace vdit {
namespace {

constexpr int kTileC = 256;  // channels per workgroup
constexpr int kTileT = 256;  // tokens per workgroup
constexpr int kBK = 64;      // k per LDS stage
constexpr int kThreads = 512;
constexpr int kGroupT = 8;   // token tiles per ordering group
constexpr int kRowBytes = kBK * 2;                  // 128 bytes of one tile row
constexpr int kTileBytes = kTileC * kRowBytes;      // 32 KB (W or x tile)
constexpr int kStageBytes = 2 * kTileBytes;         // W tile then x tile
constexpr int kStagesBytes = 2 * kStageBytes;       // two stages: 128 KB
// After the stages: the tile's 256 biases and gains as fp32, and the RoPE
// frequency of each (axis, lane half, register pair) slot of the epilogue,
// zero where the pair turns with another axis.
constexpr int kTabBytes = (2 * kTileC + 3 * 64) * 4;
constexpr int kLdsBytes = kStagesBytes + kTabBytes;
constexpr int kLoads = kTileBytes / 1024 / (kThreads / 64);  // 1 KB loads per wave per tile

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Physical 16-byte chunk of logical chunk c in tile row r: rows are 128
// bytes, two per 256-byte bank period, so XOR with (r/2) % 8 spreads the 16
// rows one b128 read pass touches over all banks.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__global__ __launch_bounds__(kThreads, 1) void qkv_proj_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const uint16_t *__restrict__ bias,
    const uint16_t *__restrict__ gq, const uint16_t *__restrict__ gk, uint16_t *__restrict__ q,
    uint16_t *__restrict__ k, uint16_t *__restrict__ v, QkvGeom g, QkvRope rope)
{
#if defined(__HIP_DEVICE_COMPILE__)
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];
    lds_u8 *lds = (lds_u8 *)dyn_lds;
    const int dim = g.dim;
    const int nct = (3 * dim + kTileC - 1) / kTileC;
    const int ntt = (g.M + kTileT - 1) / kTileT;
    const uint32_t id = xcd_contiguous(blockIdx.x, (uint32_t)(nct * ntt));
    // Tiles are taken in groups of kGroupT token tiles: within a group the
    // token tile varies fastest, then the channel tile, so the workgroups
    // one XCD runs together (a contiguous run of ids) cover a few channel
    // tiles of several token tiles and share both operands' rows in its L2.
    const int grp = (int)(id / (uint32_t)(kGroupT * nct));
    const int gt0 = grp * kGroupT;
    const int gsz = min(kGroupT, ntt - gt0);
    const int rem = (int)(id - (uint32_t)grp * kGroupT * nct);
    const int ct = rem / gsz, tt = gt0 + rem % gsz;
    const int c0 = ct * kTileC, t0 = tt * kTileT;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, col = lane & 31;
    const int wc = wave & 1, wt = wave >> 1;  // channel half, token quarter of the tile

    // Epilogue tables (published by the first barrier below). Slot j of a
    // lane half h is register pair rp = j % 8 of channel block cb = j / 8,
    // i.e. pair cb*16 + 4*(rp/2) + rp%2 + 2h of the head; its angle is
    // t*ft + h*fh + w*fw with two of the three frequencies zero.
    lds_f32 *tbias = (lds_f32 *)(lds + kStagesBytes);
    lds_f32 *tgain = tbias + kTileC;
    lds_f32 *tfreq = tgain + kTileC;  // [axis][half][32]
    {
        const int c = tid & (kTileC - 1), cc = c0 + c;
        if (tid < kTileC) {
            tbias[c] = bias && cc < 3 * dim ? __uint_as_float((uint32_t)bias[cc] << 16) : 0.f;
        } else {
            float gv = 1.f;
            if (cc < dim) {
                if (gq) gv = __uint_as_float((uint32_t)gq[cc] << 16);
            } else if (cc < 2 * dim) {
                if (gk) gv = __uint_as_float((uint32_t)gk[cc - dim] << 16);
            }
            tgain[c] = gv;
        }
        if (tid < 3 * 64) {
            const int ax = tid >> 6, h = (tid >> 5) & 1, j = tid & 31;
            const int pr = (j >> 3) * 16 + 4 * ((j & 7) >> 1) + (j & 1) + 2 * h;
            const bool on = ax == 0 ? pr < rope.b1 : (ax == 1 ? pr >= rope.b1 && pr < rope.b2 : pr >= rope.b2);
            tfreq[tid] = on ? rope.freq_rev[pr] : 0.f;
        }
    }

    // Buffer descriptors from the tile's first W row and first x row; the
    // sizes end at the last row of each matrix.
    const uint32_t rowb = (uint32_t)dim * 2;
    const int nrec_w = (int)((int64_t)(3 * dim - c0) * rowb);
    const int nrec_x = (int)((int64_t)(g.M - t0) * rowb);
    const __amdgpu_buffer_rsrc_t wrs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(w + (int64_t)c0 * dim), 0, nrec_w, kBufferFlags);
    const __amdgpu_buffer_rsrc_t xrs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(x + (int64_t)t0 * dim), 0, nrec_x, kBufferFlags);
    // Load i of this wave fills tile rows 8*(wave*kLoads + i) + lane/8,
    // physical chunk lane%8, which holds logical chunk (lane%8) ^ swz.
    uint32_t goff[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int r = 8 * (wave * kLoads + i) + (lane >> 3);
        goff[i] = (uint32_t)r * rowb + (uint32_t)swz(r, lane & 7) * 16;
    }
    auto load_stage = [&](int kt, int st) {
        lds_u8 *wb = lds + st * kStageBytes;
        lds_u8 *xb = wb + kTileBytes;
        const uint32_t so = (uint32_t)kt * kRowBytes;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_void *)(wb + (wave * kLoads + i) * 1024), 16,
                                                     goff[i], so, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_void *)(xb + (wave * kLoads + i) * 1024), 16,
                                                     goff[i], so, 0, 0);
        }
    };

    // Operand read offsets for k-step 0 of stage 0: W row wc*128 + col (+32
    // per channel block), x row wt*64 + col (+32 per token block); the
    // swizzle depends on the row only through col.
    uint32_t aofs[4], bofs[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        aofs[ks] = (uint32_t)((wc * 128 + col) * kRowBytes + swz(col, 2 * ks + half) * 16);
        bofs[ks] = (uint32_t)(kTileBytes + (wt * 64 + col) * kRowBytes + swz(col, 2 * ks + half) * 16);
    }

    f32x16 acc[4][2];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) acc[cb][tb] = (f32x16){};

    const int nk = dim / kBK;
    auto stage = [&](auto stc) {
        constexpr uint32_t S0 = decltype(stc)::value * kStageBytes;
        bf16x8 a[2][4], b[2][2];
        auto rd = [&](int ks, int slot) {
#pragma unroll
            for (int i = 0; i < 4; ++i) a[slot][i] = *(const lds_bf16x8 *)(lds + aofs[ks] + (S0 + i * 32 * kRowBytes));
#pragma unroll
            for (int i = 0; i < 2; ++i) b[slot][i] = *(const lds_bf16x8 *)(lds + bofs[ks] + (S0 + i * 32 * kRowBytes));
        };
        rd(0, 0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) rd(ks + 1, (ks + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
                    acc[cb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks & 1][cb], b[ks & 1][tb],
                                                                         acc[cb][tb], 0, 0, 0);
        }
    };

    // Stages alternate between the two LDS buffers; the loop takes them in
    // pairs so the buffer is a compile-time constant, and an odd last stage
    // (already loaded into buffer 0) follows it.
    load_stage(0, 0);
    wait_vmem();
    __syncthreads();
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        load_stage(kt + 1, 1);
        stage(std::integral_constant<int, 0>{});
        wait_vmem();
        __syncthreads();
        if (kt + 2 < nk) load_stage(kt + 2, 0);
        stage(std::integral_constant<int, 1>{});
        wait_vmem();
        __syncthreads();
    }
    if (kt < nk) {
        stage(std::integral_constant<int, 0>{});
        // The epilogue stages through LDS that other waves may still be
        // reading in this stage. (dim is a multiple of 128, so nk is even and
        // this branch does not run; the barrier keeps it safe if it does.)
        __syncthreads();
    }

    // Epilogue: this wave's 128 channels are one head of one of Q, K, V.
    // Lane channels within the head: cb*32 + 8*r4 + 4*half + e, e < 4 (the
    // accumulator register 4*r4 + e of block cb). Every 32-token block is
    // finished in registers, staged through this wave's own LDS region and
    // written as whole 256-byte token rows. Bias, gain and the RoPE
    // frequencies come from the fp32 tables in LDS, four per read.
    const int cw = c0 + wc * 128;
    if (cw >= 3 * dim) return;
    const int which = cw / dim;             // 0 Q, 1 K, 2 V
    const int hc = cw - which * dim;        // first channel of the head within its tensor
    uint16_t *out = which == 0 ? q : (which == 1 ? k : v);
    const bool norm = which == 0 ? gq != nullptr : (which == 1 ? gk != nullptr : false);
    const bool rot = which < 2 && rope.on;
    const int HW = g.Hp * g.Wp;
    constexpr int kPitch = 272;  // bytes per staged token row (256 + 16 keeps writes conflict-free)
    lds_u8 *stg = lds + wave * 32 * kPitch;
    const lds_f32 *wbias = tbias + wc * 128 + 4 * half, *wgain = tgain + wc * 128 + 4 * half;
    const lds_f32 *wfreq = tfreq + 32 * half;

#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int mt = t0 + wt * 64 + tb * 32;  // first token row of the block
        const int m = mt + col;
        float y[4][16];
        float ss = 0.f;
        // Lane channels of block cb, registers 4*r4 .. 4*r4+3: head channels
        // cb*32 + 8*r4 + 4*half .. +3.
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 b4 = *(const lds_f32x4 *)(wbias + cb * 32 + 8 * r4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    y[cb][4 * r4 + e] = acc[cb][tb][4 * r4 + e] + b4[e];
                    ss = fmaf(y[cb][4 * r4 + e], y[cb][4 * r4 + e], ss);
                }
            }
        // RMSNorm: the gain now, the token's 1/rms after the rotation
        // (which is linear and acts within the token).
        float rs = 1.f;
        if (norm) {
            rs = __builtin_amdgcn_rsqf(pair_sum(ss) * (1.0f / 128.0f) + g.eps);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const f32x4 g4 = *(const lds_f32x4 *)(wgain + cb * 32 + 8 * r4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[cb][4 * r4 + e] *= g4[e];
                }
        }
        if (rot) {
            const int n = m % g.N;
            const float pt = (float)(n / HW), ph = (float)((n / g.Wp) % g.Hp), pw = (float)(n % g.Wp);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int rq = 0; rq < 2; ++rq) {
                    const int j = cb * 8 + 4 * rq;
                    const f32x4 ft = *(const lds_f32x4 *)(wfreq + j);
                    const f32x4 fh = *(const lds_f32x4 *)(wfreq + 64 + j);
                    const f32x4 fw = *(const lds_f32x4 *)(wfreq + 128 + j);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // Angle in revolutions, reduced to [0, 1) for v_sin/v_cos.
                        const float rev = __builtin_amdgcn_fractf(fmaf(pw, fw[i], fmaf(ph, fh[i], pt * ft[i])));
                        const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
                        const int r = 2 * (4 * rq + i);
                        const float re = y[cb][r], im = y[cb][r + 1];
                        y[cb][r] = re * cs - im * sn;
                        y[cb][r + 1] = re * sn + im * cs;
                    }
                }
        }
        if (norm) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) y[cb][r] *= rs;
        }
        // Stage: token col's row, channels cb*32 + 8*r4 + 4*half .. +3.
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                u32x2 st;
                st[0] = pack_bf16x2(y[cb][4 * r4 + 0], y[cb][4 * r4 + 1]);
                st[1] = pack_bf16x2(y[cb][4 * r4 + 2], y[cb][4 * r4 + 3]);
                *(__attribute__((address_space(3))) u32x2 *)(stg + col * kPitch + (cb * 32 + 8 * r4 + 4 * half) * 2) =
                    st;
            }
        // The region is this wave's own: its LDS writes complete in order
        // before the reads below.
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        // Rows back out: 16 lanes per 256-byte row, 4 rows per read.
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = 4 * i + (lane >> 4);
            const u32x4 d = *(const __attribute__((address_space(3))) u32x4 *)(stg + row * kPitch + (lane & 15) * 16);
            // Non-temporal stores: the outputs are not read again here
            // (1.2-1.5% faster than plain stores, side by side).
            if (mt + row < g.M)
                __builtin_nontemporal_store(d, (u32x4 *)(out + (int64_t)(mt + row) * dim + hc + (lane & 15) * 8));
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
    }
#endif
}

// fp32: one thread per (token, tensor, head), fp32 dot products, fp64
// angles; for small workloads checked against fp64 at 1e-5.
__global__ __launch_bounds__(128) void qkv_proj_f32(const float *__restrict__ x, const float *__restrict__ w,
                                                    const float *__restrict__ bias, const float *__restrict__ gq,
                                                    const float *__restrict__ gk, float *__restrict__ q,
                                                    float *__restrict__ k, float *__restrict__ v, QkvGeom g,
                                                    RopeTable tab, int rope_on)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int heads = g.dim / g.D;
    if (idx >= (int64_t)g.M * 3 * heads) return;
    const int hd = (int)(idx % heads);
    const int which = (int)((idx / heads) % 3);
    const int64_t m = idx / (3 * heads);
    const float *xr = x + m * g.dim;
    float y[256];
    const int D = g.D;
    for (int d = 0; d < D; ++d) {
        const int c = which * g.dim + hd * D + d;
        const float *wr = w + (int64_t)c * g.dim;
        float s = 0.f;
        for (int kk = 0; kk < g.dim; ++kk) s = fmaf(wr[kk], xr[kk], s);
        y[d] = s + (bias ? bias[c] : 0.f);
    }
    const float *gain = which == 0 ? gq : (which == 1 ? gk : nullptr);
    if (gain) {
        float ss = 0.f;
        for (int d = 0; d < D; ++d) ss = fmaf(y[d], y[d], ss);
        const float sc = 1.0f / sqrtf(ss / (float)D + g.eps);
        for (int d = 0; d < D; ++d) y[d] = y[d] * sc * gain[hd * D + d];
    }
    if (which < 2 && rope_on) {
        const int n = (int)(m % g.N);
        const int pos[3] = {n / (g.Hp * g.Wp), (n / g.Wp) % g.Hp, n % g.Wp};
        for (int j = 0; j < D / 2; ++j) {
            double ang = (double)pos[tab.axis[j]] * tab.freq[j];
            ang -= 6.283185307179586476925286766559 * rint(ang * 0.15915494309189533576888376337251);
            float sn, cs;
            sincosf((float)ang, &sn, &cs);
            const float re = y[2 * j], im = y[2 * j + 1];
            y[2 * j] = re * cs - im * sn;
            y[2 * j + 1] = re * sn + im * cs;
        }
    }
    float *out = which == 0 ? q : (which == 1 ? k : v);
    for (int d = 0; d < D; ++d) out[m * g.dim + hd * D + d] = y[d];
}

}  // namespace

hipError_t launch_qkv_proj_bf16(const void *x, const void *w, const void *bias, const void *gq, const void *gk,
                                void *q, void *k, void *v, const QkvGeom &g, const QkvRope &rope, hipStream_t s) {
    const int64_t nct = (3 * (int64_t)g.dim + kTileC - 1) / kTileC;
    const int64_t ntt = ((int64_t)g.M + kTileT - 1) / kTileT;
    const int64_t grid = nct * ntt;
    if (grid <= 0 || grid > UINT32_MAX) return hipErrorInvalidConfiguration;
    hipError_t e = hipFuncSetAttribute((const void *)qkv_proj_bf16, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       kLdsBytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(qkv_proj_bf16, dim3((uint32_t)grid), dim3(kThreads), kLdsBytes, s, (const uint16_t *)x,
                       (const uint16_t *)w, (const uint16_t *)bias, (const uint16_t *)gq, (const uint16_t *)gk,
                       (uint16_t *)q, (uint16_t *)k, (uint16_t *)v, g, rope);
    return hipGetLastError();
}

hipError_t launch_qkv_proj_f32(const float *x, const float *w, const float *bias, const float *gq, const float *gk,
                               float *q, float *k, float *v, const QkvGeom &g, const RopeTable &tab, int rope_on,
                               hipStream_t s) {
    const int64_t n = (int64_t)g.M * 3 * (g.dim / g.D);
    const int64_t blocks = (n + 127) / 128;
    if (blocks <= 0 || blocks > UINT32_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(qkv_proj_f32, dim3((uint32_t)blocks), dim3(128), 0, s, x, w, bias, gq, gk, q, k, v, g, tab,
                       rope_on);
    return hipGetLastError();
}

}  // namespace vdit
