// Spacetime tube patchify: a Conv3d whose stride equals its kernel, computed
// as a GEMM with the im2col folded into the load addressing.
//
// "Video and 3D Generation" cheatsheet, "Tiny video DiT" (Conv3d with stride
// equal to kernel); "How AI Generates Video: Inside Sora and Wan2.1 on a Real
// GPU", section 4 (each 16-channel 1x2x2 brick, 64 numbers, becomes one
// 1,536-wide token). With K = C*pt*ph*pw patch values per token:
//   tokens[m][o] = bias[o] + sum_k W[o][k] * A[m][k],
//   A[m][k] = latent[b][c][t*pt+i][h*ph+j][w*pw+kw], k = ((c*pt+i)*ph+j)*pw+kw,
// which is the Conv3d weight [Dout][C][pt][ph][pw] read as a [Dout][K]
// row-major matrix. Output rows are token-major, m = b*N + (t*Hp+h)*Wp + w.
//
// bf16 path (v_mfma_f32_32x32x16_bf16, fp32 accumulation): a workgroup owns
// 64 tokens; it gathers their [64][K] patch matrix into LDS once and sweeps
// all output channels in chunks of 128, each wave computing a 32-channel x
// 64-token block of C^T = W A^T with W read straight from global (it is small
// and stays in L2). Each output chunk is staged through LDS and written as
// whole 256-byte row runs: at K = 64 the kernel writes 24x more bytes than it
// reads, so coalesced stores set its speed.
//
// fp32 path: one thread per output element, a plain dot product (for the
// small fp32 workloads that must agree with fp64 to 1e-5).
#include "vdit_internal.h"

namespace vdit {
namespace {

constexpr int kTok = 64;   // tokens per workgroup
constexpr int kOut = 128;  // output channels per chunk
constexpr int kMaxK = 512; // padded patch length the LDS tile holds

typedef __attribute__((address_space(3))) unsigned char lds_u8;

__global__ __launch_bounds__(256) void patchify_bf16_kernel(const uint16_t *__restrict__ x,
                                                            const uint16_t *__restrict__ w,
                                                            const uint16_t *__restrict__ bias,
                                                            uint16_t *__restrict__ tok, PatchGeom g, int K,
                                                            int Kp)
{
    // A tile: [kTok][Kp + 8] bf16 (the 16-byte pad staggers rows over banks).
    __shared__ __attribute__((aligned(16))) unsigned char a_lds[kTok * (kMaxK + 8) * 2];
    // Output chunk: [kTok][kOut + 8] bf16.
    __shared__ __attribute__((aligned(16))) unsigned char o_lds[kTok * (kOut + 8) * 2];
    lds_u8 *al = (lds_u8 *)a_lds;
    lds_u8 *ol = (lds_u8 *)o_lds;
    const int arow = (Kp + 8) * 2;     // bytes per A row
    const int orow = (kOut + 8) * 2;   // bytes per output-chunk row

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int64_t N = (int64_t)g.T * g.Hp * g.Wp;
    const int64_t M = (int64_t)g.B * N;
    const int64_t m0 = (int64_t)blockIdx.x * kTok;

    // Gather the patch matrix (zero past K and past the last token).
    for (int idx = tid; idx < kTok * Kp; idx += 256) {
        const int r = idx / Kp, kk = idx % Kp;
        const int64_t m = m0 + r;
        uint16_t val = 0;
        if (m < M && kk < K) {
            const int kw = kk % g.pw, j = (kk / g.pw) % g.ph, i = (kk / (g.pw * g.ph)) % g.pt;
            const int c = kk / (g.pw * g.ph * g.pt);
            const int64_t b = m / N, n = m % N;
            const int64_t t = n / ((int64_t)g.Hp * g.Wp);
            const int64_t hh = (n / g.Wp) % g.Hp, ww = n % g.Wp;
            val = x[(((b * g.C + c) * g.Tl + t * g.pt + i) * g.Hl + hh * g.ph + j) * g.Wl + ww * g.pw + kw];
        }
        *(__attribute__((address_space(3))) uint16_t *)(al + r * arow + kk * 2) = val;
    }
    __syncthreads();

    const bool kvec = (K % 8) == 0;  // W rows can be read as 16-byte vectors
    for (int oc = 0; oc < g.Dout; oc += kOut) {
        f32x16 acc[2] = {(f32x16){}, (f32x16){}};
        const int orow_w = oc + wave * 32 + col;  // W row this lane feeds
        for (int s = 0; s < Kp / 16; ++s) {
            const int k0 = 16 * s + 8 * half;
            bf16x8 wa = (bf16x8){};
            if (orow_w < g.Dout) {
                if (kvec) {
                    if (k0 < K) wa = *(const bf16x8 *)(w + (int64_t)orow_w * K + k0);
                } else {
                    uint16_t e8[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) e8[e] = (k0 + e < K) ? w[(int64_t)orow_w * K + k0 + e] : 0;
                    wa = __builtin_bit_cast(bf16x8, e8);
                }
            }
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const bf16x8 bt = *(const __attribute__((address_space(3))) bf16x8 *)(
                    al + (tb * 32 + col) * arow + k0 * 2);
                acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, bt, acc[tb], 0, 0, 0);
            }
        }
        // acc[tb]: lane holds token tb*32+col, channels wave*32 + 8*(r/4) + 4*half + r%4.
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int oo = wave * 32 + 8 * r4 + 4 * half;  // channel within the chunk
                float vals[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float bv = 0.f;
                    if (bias && oc + oo + e < g.Dout) bv = bf16_bits_to_f32(bias[oc + oo + e]);
                    vals[e] = acc[tb][4 * r4 + e] + bv;
                }
                u32x2 pk;
                pk[0] = pack_bf16x2(vals[0], vals[1]);
                pk[1] = pack_bf16x2(vals[2], vals[3]);
                *(__attribute__((address_space(3))) u32x2 *)(ol + (tb * 32 + col) * orow + oo * 2) = pk;
            }
        __syncthreads();
        for (int idx = tid; idx < kTok * (kOut / 8); idx += 256) {
            const int r = idx / (kOut / 8), ch = idx % (kOut / 8);
            const int64_t m = m0 + r;
            const int o0 = oc + ch * 8;
            if (m < M && o0 < g.Dout)
                *(u32x4 *)(tok + m * g.Dout + o0) = *(const __attribute__((address_space(3))) u32x4 *)(
                    ol + r * orow + ch * 16);
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void patchify_f32_kernel(const float *__restrict__ x, const float *__restrict__ w,
                                                           const float *__restrict__ bias, float *__restrict__ tok,
                                                           PatchGeom g)
{
    const int64_t N = (int64_t)g.T * g.Hp * g.Wp;
    const int64_t total = (int64_t)g.B * N * g.Dout;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int o = (int)(idx % g.Dout);
    const int64_t m = idx / g.Dout;
    const int64_t b = m / N, n = m % N;
    const int64_t t = n / ((int64_t)g.Hp * g.Wp), hh = (n / g.Wp) % g.Hp, ww = n % g.Wp;
    float acc = bias ? bias[o] : 0.f;
    const float *wr = w + (int64_t)o * g.C * g.pt * g.ph * g.pw;
    int kk = 0;
    for (int c = 0; c < g.C; ++c)
        for (int i = 0; i < g.pt; ++i)
            for (int j = 0; j < g.ph; ++j)
                for (int kw = 0; kw < g.pw; ++kw, ++kk)
                    acc = fmaf(wr[kk],
                               x[(((b * g.C + c) * g.Tl + t * g.pt + i) * g.Hl + hh * g.ph + j) * g.Wl + ww * g.pw + kw],
                               acc);
    tok[idx] = acc;
}

}  // namespace

hipError_t launch_patchify_bf16(const void *x, const void *w, const void *bias, void *tok, const PatchGeom &g,
                                hipStream_t s) {
    const int K = g.C * g.pt * g.ph * g.pw;
    const int Kp = (K + 15) / 16 * 16;
    if (Kp > kMaxK || g.Dout % 8) return hipErrorInvalidValue;
    const int64_t M = (int64_t)g.B * g.T * g.Hp * g.Wp;
    const uint32_t grid = (uint32_t)((M + kTok - 1) / kTok);
    hipLaunchKernelGGL(patchify_bf16_kernel, dim3(grid), dim3(256), 0, s, (const uint16_t *)x,
                       (const uint16_t *)w, (const uint16_t *)bias, (uint16_t *)tok, g, K, Kp);
    return hipGetLastError();
}

hipError_t launch_patchify_f32(const float *x, const float *w, const float *bias, float *tok, const PatchGeom &g,
                               hipStream_t s) {
    const int64_t total = (int64_t)g.B * g.T * g.Hp * g.Wp * g.Dout;
    const uint32_t grid = (uint32_t)((total + 255) / 256);
    hipLaunchKernelGGL(patchify_f32_kernel, dim3(grid), dim3(256), 0, s, x, w, bias, tok, g);
    return hipGetLastError();
}

}  // namespace vdit
