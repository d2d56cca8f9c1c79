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
// bf16 paths (fp32 accumulation). At K = 64 the kernel writes 24x more
// bytes than it reads, so the store stream sets its speed.
//  - K <= 64 (patchify_ldsw_bf16, below): W and bias in LDS, each wavefront
//    free of barriers after start-up, so stores stream without a break.
//  - Longer patches (patchify_bf16_kernel, v_mfma_f32_32x32x16_bf16): a
//    workgroup owns kTok tokens; it gathers their [kTok][K] patch matrix
//    into LDS once and
//    sweeps all output channels in chunks of 128, each wave computing a
//    32-channel x kTok-token block of C^T = W A^T with W and the bias read
//    straight from global (they are small and stay in L2), one chunk ahead.
//    Each chunk is staged through LDS (two alternating buffers, one barrier
//    per chunk) and written as whole 256-byte row runs. LDS is sized to the
//    actual patch length so several workgroups share a CU.
//
// fp32 path: one thread per output element, a plain dot product (for the
// small fp32 workloads that must agree with fp64 to 1e-5).
#include "vdit_internal.h"

#include <type_traits>

namespace vdit {
namespace {

constexpr int kTok = 64;   // tokens per workgroup
constexpr int kTB = kTok / 32;  // 32-token MFMA blocks per workgroup
constexpr int kChunkSplit = 1;  // workgroups that share one token block's channel chunks
constexpr int kOut = 128;  // output channels per chunk
constexpr int kMaxK = 512; // padded patch length the LDS tile holds

typedef __attribute__((address_space(3))) unsigned char lds_u8;

// KSC: the number of 16-wide k-steps (Kp/16) when it is at most 8, so the W
// operands of a chunk sit in registers and the next chunk's can be
// prefetched; 0 selects a generic path that loads W step by step.
template <int KSC>
__global__ __launch_bounds__(512) void patchify_bf16_kernel(const uint16_t *__restrict__ x,
                                                            const uint16_t *__restrict__ w,
                                                            const uint16_t *__restrict__ bias,
                                                            uint16_t *__restrict__ tok, PatchGeom g, int K,
                                                            int Kp)
{
    // Dynamic LDS, sized to the patch length: two output chunks
    // [kTok][kOut + 8] bf16 (alternate chunks use alternate buffers), then
    // the A tile [kTok][Kp + 8] bf16 (the 16-byte pads stagger rows over
    // banks).
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];
    const int arow = (Kp + 8) * 2;     // bytes per A row
    const int orow = (kOut + 8) * 2;   // bytes per output-chunk row
    lds_u8 *ol0 = (lds_u8 *)dyn_lds;
    lds_u8 *al = ol0 + 4 * kTok * orow;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int64_t N = (int64_t)g.T * g.Hp * g.Wp;
    const int64_t M = (int64_t)g.B * N;
    const int64_t m0 = (int64_t)blockIdx.x * kTok;

    // Gather the patch matrix (zero past K and past the last token): all
    // eight wavefronts on the fast path for two-wide bricks, the first four
    // on the general one.
    const bool fast_gather = g.pw == 2 && (g.Wl & 1) == 0 && kTok == 64;
    if (!fast_gather && tid >= 256) {
    } else if (fast_gather) {
        // Bricks two wide (an even latent width keeps every pair 4-byte
        // aligned): lane l of each wave owns token m0 + l, and the waves take
        // the token's (c, i, j) rows in turn, one 4-byte (kw = 0, 1) pair per
        // load. The 64 lanes of a load read neighbouring tokens of one latent
        // row, so each load instruction covers one or two contiguous runs.
        const int64_t m = m0 + lane;
        lds_u8 *arow_p = al + lane * arow;
        const int rows = g.C * g.pt * g.ph;  // K / 2 pairs
        if (m < M) {
            const int64_t b = m / N, n = m % N;
            const int t = (int)(n / ((int64_t)g.Hp * g.Wp));
            const int hh = (int)((n / g.Wp) % g.Hp), ww = (int)(n % g.Wp);
            const uint16_t *xb = x + (((b * g.C) * g.Tl + (int64_t)t * g.pt) * g.Hl + (int64_t)hh * g.ph) * g.Wl +
                                 (int64_t)ww * 2;
            for (int cij = wave; cij < rows; cij += 8) {
                const int j = cij % g.ph, i = (cij / g.ph) % g.pt, c = cij / (g.ph * g.pt);
                const uint32_t v2 = *(const uint32_t *)(xb + (((int64_t)c * g.Tl + i) * g.Hl + j) * g.Wl);
                *(__attribute__((address_space(3))) uint32_t *)(arow_p + cij * 4) = v2;
            }
        } else {
            for (int cij = wave; cij < rows; cij += 8)
                *(__attribute__((address_space(3))) uint32_t *)(arow_p + cij * 4) = 0u;
        }
        // Padding columns K .. Kp-1 (K is even here).
        for (int kk = K + 2 * wave; kk < Kp; kk += 16)
            *(__attribute__((address_space(3))) uint32_t *)(arow_p + kk * 2) = 0u;
    } else {
        // Any brick: each thread owns one token and a run of KR = Kp / (256 /
        // kTok) consecutive patch indices: the token's (b, t, h, w) is
        // decomposed once and the patch index (c, i, j, kw) advances by
        // carries, so the index math is a few adds per element.
        constexpr int TPT = 256 / kTok;  // threads per token
        const int r = tid / TPT;
        const int KR = Kp / TPT;
        const int kk0 = (tid % TPT) * KR;
        const int64_t m = m0 + r;
        lds_u8 *arow_p = al + r * arow;
        if (m < M) {
            const int64_t b = m / N, n = m % N;
            const int t = (int)(n / ((int64_t)g.Hp * g.Wp));
            const int hh = (int)((n / g.Wp) % g.Hp), ww = (int)(n % g.Wp);
            const uint16_t *xb = x + (((b * g.C) * g.Tl + (int64_t)t * g.pt) * g.Hl + (int64_t)hh * g.ph) * g.Wl +
                                 (int64_t)ww * g.pw;
            int kw = kk0 % g.pw, j = (kk0 / g.pw) % g.ph, i = (kk0 / (g.pw * g.ph)) % g.pt;
            int c = kk0 / (g.pw * g.ph * g.pt);
            for (int e = 0; e < KR; ++e) {
                const int kk = kk0 + e;
                uint16_t val = 0;
                if (kk < K) val = xb[(((int64_t)c * g.Tl + i) * g.Hl + j) * g.Wl + kw];
                *(__attribute__((address_space(3))) uint16_t *)(arow_p + kk * 2) = val;
                if (++kw == g.pw) {
                    kw = 0;
                    if (++j == g.ph) {
                        j = 0;
                        if (++i == g.pt) {
                            i = 0;
                            ++c;
                        }
                    }
                }
            }
        } else {
            for (int e = 0; e < KR; ++e) *(__attribute__((address_space(3))) uint16_t *)(arow_p + (kk0 + e) * 2) = 0;
        }
    }
    __syncthreads();

    const bool kvec = (K % 8) == 0;  // W rows can be read as 16-byte vectors
    // Two groups of four wavefronts take alternate channel chunks: group grp
    // does chunks c0 + grp, c0 + grp + 2, ..., each wave 32 of a chunk's 128
    // channels, and both groups meet one barrier per step.
    // This workgroup's channel chunks: kOut-wide chunks c0, c0 + 1, ..., c1 - 1.
    const int nchunks = (g.Dout + kOut - 1) / kOut;
    const int per = (nchunks + gridDim.y - 1) / gridDim.y;
    const int c0 = blockIdx.y * per, c1 = min(nchunks, c0 + per);
    const int grp = wave >> 2, gw = wave & 3, gtid = tid & 255;
    const int nsteps = (c1 - c0 + 1) / 2;
    // W operands (A of C^T = W A^T) of chunk oc, step s2: lane row
    // oc + wave*32 + col, features 16*s2 + 8*half .. +8.
    auto w_op = [&](int oc, int s2) {
        const int orow_w = oc + gw * 32 + col;
        const int k0 = 16 * s2 + 8 * half;
        bf16x8 v8 = (bf16x8){};
        if (orow_w < g.Dout) {
            if (kvec) {
                if (k0 < K) v8 = *(const bf16x8 *)(w + (int64_t)orow_w * K + k0);
            } else {
                uint16_t e8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) e8[e] = (k0 + e < K) ? w[(int64_t)orow_w * K + k0 + e] : 0;
                v8 = __builtin_bit_cast(bf16x8, e8);
            }
        }
        return v8;
    };
    // Bias of chunk oc for this lane's rows: channels oc + wave*32 + 8*r4 +
    // 4*half .. +4, one 8-byte load each (Dout is a multiple of 8 and bias is
    // 16-byte aligned, so a run of 4 never straddles the end).
    auto b_op = [&](int oc, int r4) {
        const int ch = oc + gw * 32 + 8 * r4 + 4 * half;
        u32x2 v = (u32x2){0u, 0u};
        if (bias && ch < g.Dout) v = *(const u32x2 *)(bias + ch);
        return v;
    };
    constexpr int NS = KSC > 0 ? KSC : 1;
    bf16x8 wcur[NS], wnext[NS];
    u32x2 bcur[4], bnext[4];
    if (c0 + grp < c1) {
        if constexpr (KSC > 0) {
#pragma unroll
            for (int s2 = 0; s2 < KSC; ++s2) wcur[s2] = w_op((c0 + grp) * kOut, s2);
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) bcur[r4] = b_op((c0 + grp) * kOut, r4);
    }
    for (int st = 0; st < nsteps; ++st) {
        const int ci = c0 + 2 * st + grp;
        const bool live = ci < c1;
        const int oc = ci * kOut;
        lds_u8 *ol = ol0 + (2 * grp + (st & 1)) * kTok * orow;
        if (live) {
            // The group's next chunk's bias loads are in flight during this chunk.
            if (ci + 2 < c1)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) bnext[r4] = b_op(oc + 2 * kOut, r4);
            f32x16 acc[kTB];
#pragma unroll
            for (int tb = 0; tb < kTB; ++tb) acc[tb] = (f32x16){};
            auto step = [&](int s2, const bf16x8 &wa) {
                const int k0 = 16 * s2 + 8 * half;
#pragma unroll
                for (int tb = 0; tb < kTB; ++tb) {
                    const bf16x8 bt = *(const __attribute__((address_space(3))) bf16x8 *)(
                        al + (tb * 32 + col) * arow + k0 * 2);
                    acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, bt, acc[tb], 0, 0, 0);
                }
            };
            if constexpr (KSC > 0) {
                // The group's next chunk's W loads are in flight during this chunk.
                if (ci + 2 < c1)
#pragma unroll
                    for (int s2 = 0; s2 < KSC; ++s2) wnext[s2] = w_op(oc + 2 * kOut, s2);
#pragma unroll
                for (int s2 = 0; s2 < KSC; ++s2) step(s2, wcur[s2]);
#pragma unroll
                for (int s2 = 0; s2 < KSC; ++s2) wcur[s2] = wnext[s2];
            } else {
                for (int s2 = 0; s2 < Kp / 16; ++s2) step(s2, w_op(oc, s2));
            }
            // acc[tb]: lane holds token tb*32+col, channels gw*32 + 8*(r/4) + 4*half + r%4.
#pragma unroll
            for (int tb = 0; tb < kTB; ++tb)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int oo = gw * 32 + 8 * r4 + 4 * half;  // channel within the chunk
                    float vals[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t bw = bcur[r4][e >> 1];
                        const float bv = __uint_as_float((e & 1) ? (bw & 0xFFFF0000u) : (bw << 16));
                        vals[e] = acc[tb][4 * r4 + e] + bv;
                    }
                    u32x2 pk;
                    pk[0] = pack_bf16x2(vals[0], vals[1]);
                    pk[1] = pack_bf16x2(vals[2], vals[3]);
                    *(__attribute__((address_space(3))) u32x2 *)(ol + (tb * 32 + col) * orow + oo * 2) = pk;
                }
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) bcur[r4] = bnext[r4];
        }
        // One barrier per step: it orders each group's LDS writes of this
        // step before its reads below, and its reads of the step before
        // (other buffer) ahead of its writes to that buffer in the next step.
        // It orders LDS only, so the global stores stay in flight across it.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        if (live)
            for (int idx = gtid; idx < kTok * (kOut / 8); idx += 256) {
                const int r = idx / (kOut / 8), ch = idx % (kOut / 8);
                const int64_t m = m0 + r;
                const int o0 = oc + ch * 8;
                if (m < M && o0 < g.Dout)
                    *(u32x4 *)(tok + m * g.Dout + o0) = *(const __attribute__((address_space(3))) u32x4 *)(
                        ol + r * orow + ch * 16);
            }
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

// ---- Patch lengths up to 64: W in LDS, wavefronts without barriers ----
//
// A workgroup owns kPWaves * 64 tokens (64 per wavefront) x kPCh output
// channels.
// It copies its kPCh rows of W and their bias into LDS once, while each
// wavefront gathers its 64 tokens' patch values straight into the B operands
// of v_mfma_f32_16x16x32_bf16 (tokens as columns); after one barrier no
// wavefront touches global memory again except to store. A wavefront sweeps
// the channels 64 at a time: A operands (channels as rows) and bias come
// from LDS, the 16 x 16 results start from the bias, go to bf16, are staged
// through the wavefront's own LDS rows and leave as 128-byte row pieces.
// Vector-memory completions are counted in issue order, so loads issued
// after stores would wait for those stores; with no loads after the first
// store, the stores stream out at the rate HBM takes them, which at K = 64
// (24x more bytes written than read) sets the kernel's pace.
//
// 16x16x32 operand layout: lane l holds 8 consecutive-k values of row
// (A) or column (B) l % 16, k group l / 16; the result lane l holds rows
// 4*(l/16) .. +3 of column l % 16.
constexpr int kPTok = 64;       // tokens per wavefront: four 16-token blocks
constexpr int kPWaves = 8;      // wavefronts per workgroup, two per SIMD
constexpr int kPCh = 384;       // output channels per workgroup: six 64-channel steps
constexpr int kPPitch = 144;    // bytes per LDS row of W and of the staged output (128 + 16: no bank conflicts)
constexpr int kPLdsW = kPCh * kPPitch;
constexpr int kPLdsBias = kPCh * 2;
constexpr int kPLdsStage = kPWaves * kPTok * kPPitch;
constexpr int kPLds = kPLdsW + kPLdsBias + kPLdsStage;
constexpr int kPThreads = 64 * kPWaves;

// KS: 32-wide k steps (1 or 2). FAST: bricks two wide with an even latent
// width, so each (kw = 0, 1) pair is one aligned 4-byte load. KVEC: K a
// multiple of 8, so W rows are read in 16-byte pieces.
//
// The start-up loads are unconditional (addresses clamped into range, the
// values zeroed afterwards where they fall outside), so that no lane-
// dependent branch separates them and each wait covers exactly the loads it
// needs.
template <int KS, bool FAST, bool KVEC>
__global__ __launch_bounds__(kPThreads) void patchify_ldsw_bf16(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ w,
                                                          const uint16_t *__restrict__ bias,
                                                          uint16_t *__restrict__ tok, PatchGeom g, int K,
                                                          int ngroups)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];
    lds_u8 *wl = (lds_u8 *)dyn_lds;
    lds_u8 *bl = wl + kPLdsW;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, kg = lane >> 4;
    lds_u8 *stg = bl + kPLdsBias + wave * kPTok * kPPitch;
    const int64_t N = (int64_t)g.T * g.Hp * g.Wp;
    const int64_t M = (int64_t)g.B * N;
    // Workgroups are numbered so that the channel groups of one token block
    // run on one XCD (ids congruent mod 8 share an XCD): the latent rows the
    // first of them gathers are then in that XCD's L2 for the others.
    const uint32_t wid = xcd_contiguous(blockIdx.x, gridDim.x);
    const int64_t sb = wid / ngroups;
    const int ch0 = (int)(wid % ngroups) * kPCh;
    const int64_t m0 = (sb * kPWaves + wave) * kPTok;

    // W rows ch0 .. ch0 + kPCh - 1 for LDS: 16-byte chunk q of row r holds
    // k = 8q .. 8q+7 (zero past K and past Dout); eight threads per row. All
    // loads are issued before any LDS write (and before the gather's loads),
    // so their latencies overlap.
    constexpr int kFill = kPCh * 8 / kPThreads;
    static_assert(kPCh * 8 % kPThreads == 0 && kPCh <= kPThreads,
                  "W rows fill whole rounds of the workgroup; one bias per thread");
    u32x4 wv[kFill];
    if constexpr (KVEC) {
#pragma unroll
        for (int it = 0; it < kFill; ++it) {
            const int c = tid + kPThreads * it, r = c >> 3, q = c & 7, ch = ch0 + r;
            const bool in = ch < g.Dout && 8 * q < K;
            wv[it] = *(const u32x4 *)(w + (int64_t)min(ch, g.Dout - 1) * K + (in ? 8 * q : 0));
            if (!in) wv[it] = (u32x4){0u, 0u, 0u, 0u};
        }
    } else {
        // W rows not 16-byte aligned: element by element, straight to LDS.
        for (int c = tid; c < kPCh * 8; c += kPThreads) {
            const int r = c >> 3, q = c & 7, ch = ch0 + r;
            uint16_t e8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                e8[e] = (ch < g.Dout && 8 * q + e < K) ? w[(int64_t)ch * K + 8 * q + e] : 0;
            *(__attribute__((address_space(3))) u32x4 *)(wl + r * kPPitch + q * 16) = __builtin_bit_cast(u32x4, e8);
        }
    }


    // B operands: token block tb, k step s holds patch values k = 32*s +
    // 8*kg .. +8 of token m0 + 16*tb + col (zero past K and past M).
    //
    // Patch value k sits at latent offset poff(k) from the token's brick
    // corner; the lane's offsets are the same for all four tokens it
    // gathers, so they are formed once, by carrying through (c, i, j, kw)
    // rather than dividing. FAST reads (kw = 0, 1) pairs: pair index
    // r = k / 2 = (c*pt + i)*ph + j.
    constexpr int NV = FAST ? 4 : 8;  // loads per k step
    int poff[KS][NV];
    {
        const int64_t sc = (int64_t)g.Tl * g.Hl * g.Wl, si = (int64_t)g.Hl * g.Wl;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
            // First index of this lane's run, split once.
            int k0 = 32 * s2 + 8 * kg;
            int kw = 0, j, ii, c;
            if constexpr (FAST) {
                const int r0 = k0 / 2;
                j = r0 % g.ph;
                ii = (r0 / g.ph) % g.pt;
                c = r0 / (g.ph * g.pt);
            } else {
                kw = k0 % g.pw;
                j = (k0 / g.pw) % g.ph;
                ii = (k0 / (g.pw * g.ph)) % g.pt;
                c = k0 / (g.pw * g.ph * g.pt);
            }
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int kk = FAST ? k0 + 2 * v : k0 + v;
                poff[s2][v] = kk < K ? (int)(c * sc + ii * si + (int64_t)j * g.Wl + kw) : -1;
                if (!FAST && ++kw < g.pw) continue;
                kw = 0;
                if (++j == g.ph) {
                    j = 0;
                    if (++ii == g.pt) {
                        ii = 0;
                        ++c;
                    }
                }
            }
        }
    }
    // The wavefront's first token is split once (uniform); the lane's tokens
    // m0 + col + 16*tb then follow by carrying through (w, h, t, b).
    int64_t bb = m0 / N;
    int nn = (int)(m0 - bb * N) + col;
    while (nn >= N) {
        nn -= (int)N;
        ++bb;
    }
    const int HWp = g.Hp * g.Wp;
    int tt = nn / HWp, hh = (nn - tt * HWp) / g.Wp;
    int ww = nn - tt * HWp - hh * g.Wp;
    // Brick corners of the lane's four tokens, then every load, then the
    // operands: no load waits on another.
    const uint16_t *xbs[4];
    bool live[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        live[tb] = m0 + 16 * tb + col < M;
        // Tokens past the end read from the start of the latent (one clip
        // spans every patch offset) and are zeroed below.
        xbs[tb] = live[tb] ? x + (((bb * g.C) * g.Tl + (int64_t)tt * g.pt) * g.Hl + (int64_t)hh * g.ph) * g.Wl +
                                 (int64_t)ww * g.pw
                           : x;
        // Next token of this lane: 16 further along w.
        ww += 16;
        while (ww >= g.Wp) {
            ww -= g.Wp;
            if (++hh == g.Hp) {
                hh = 0;
                if (++tt == g.T) {
                    tt = 0;
                    ++bb;
                }
            }
        }
    }
    // Offsets past K (marked -1) read the brick corner and are zeroed
    // below, so no load is branched around.
    // This thread's bias value for LDS (read now, zeroed at its LDS write).
    const uint16_t bv16 = bias ? bias[min(ch0 + tid, g.Dout - 1)] : (uint16_t)0;
    using raw_t = std::conditional_t<FAST, uint32_t, uint16_t>;
    raw_t raw[4][KS][NV];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int o = poff[s2][v];
                raw[tb][s2][v] = *(const raw_t *)(xbs[tb] + (o < 0 ? 0 : o));
            }
    if constexpr (KVEC) {
#pragma unroll
        for (int it = 0; it < kFill; ++it) {
            const int c = tid + kPThreads * it;
            *(__attribute__((address_space(3))) u32x4 *)(wl + (c >> 3) * kPPitch + (c & 7) * 16) = wv[it];
        }
    }
    if (tid < kPCh)
        *(__attribute__((address_space(3))) uint16_t *)(bl + 2 * tid) = ch0 + tid < g.Dout ? bv16 : (uint16_t)0;
    __syncthreads();
    if (m0 >= M) return;  // past the last token; no barrier follows
    bf16x8 bop[4][KS];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
            if constexpr (FAST) {
                u32x4 u;
#pragma unroll
                for (int v = 0; v < 4; ++v) u[v] = (poff[s2][v] < 0 || !live[tb]) ? 0u : raw[tb][s2][v];
                bop[tb][s2] = __builtin_bit_cast(bf16x8, u);
            } else {
                uint16_t e16[8];
#pragma unroll
                for (int v = 0; v < 8; ++v) e16[v] = (poff[s2][v] < 0 || !live[tb]) ? (uint16_t)0 : raw[tb][s2][v];
                bop[tb][s2] = __builtin_bit_cast(bf16x8, e16);
            }
        }

    const int nsteps = min(kPCh / 64, (g.Dout - ch0 + 63) / 64);
    for (int st = 0; st < nsteps; ++st) {
        // Result (cb, tb): lane holds channels 64*st + 16*cb + 4*kg + e of
        // token 16*tb + col; staged at that token's row, byte 32*cb + 8*kg.
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int r = 64 * st + 16 * cb;
            bf16x8 a[KS];
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2)
                a[s2] = *(const __attribute__((address_space(3))) bf16x8 *)(wl + (r + col) * kPPitch +
                                                                             (4 * s2 + kg) * 16);
            const u32x2 bw = *(const __attribute__((address_space(3))) u32x2 *)(bl + 2 * (r + 4 * kg));
            const f32x4 acc0 = (f32x4){__uint_as_float(bw[0] << 16), __uint_as_float(bw[0] & 0xffff0000u),
                                       __uint_as_float(bw[1] << 16), __uint_as_float(bw[1] & 0xffff0000u)};
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                f32x4 acc = acc0;
#pragma unroll
                for (int s2 = 0; s2 < KS; ++s2)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s2], bop[tb][s2], acc, 0, 0, 0);
                u32x2 pk;
                pk[0] = pack_bf16x2(acc[0], acc[1]);
                pk[1] = pack_bf16x2(acc[2], acc[3]);
                *(__attribute__((address_space(3))) u32x2 *)(stg + (16 * tb + col) * kPPitch + 32 * cb + 8 * kg) = pk;
            }
        }
        // The rows are this wavefront's own: its LDS writes complete in
        // order before the reads below.
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        // Rows back out: 8 lanes per 128-byte row piece, 8 rows per read.
        const int chs = ch0 + 64 * st + 8 * (lane & 7);
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int row = 8 * it + (lane >> 3);
            const u32x4 d = *(const __attribute__((address_space(3))) u32x4 *)(stg + row * kPPitch + (lane & 7) * 16);
            const int64_t m = m0 + row;
            if (m < M && chs < g.Dout) *(u32x4 *)(tok + m * g.Dout + chs) = d;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace

hipError_t launch_patchify_bf16(const void *x, const void *w, const void *bias, void *tok, const PatchGeom &g,
                                hipStream_t s) {
    const int K = g.C * g.pt * g.ph * g.pw;
    const int Kp = (K + 15) / 16 * 16;
    if (Kp > kMaxK || g.Dout % 8) return hipErrorInvalidValue;
    const int64_t M = (int64_t)g.B * g.T * g.Hp * g.Wp;
    if (K <= 64 && (int64_t)g.T * g.Hp * g.Wp < INT32_MAX && (int64_t)g.C * g.Tl * g.Hl * g.Wl < INT32_MAX) {
        // One workgroup per kPWaves * 64 tokens x kPCh channels (clip length and one
        // clip's latent addressed with 32-bit offsets).
        const int ngroups = (g.Dout + kPCh - 1) / kPCh;
        const int64_t wgs = (M + kPTok * kPWaves - 1) / (kPTok * kPWaves) * ngroups;
        if (wgs > 0 && wgs <= UINT32_MAX) {
            const bool fast = g.pw == 2 && (g.Wl & 1) == 0;
            auto go_w = [&](auto kernel) {
                const hipError_t e =
                    hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kPLds);
                if (e != hipSuccess) return e;
                hipLaunchKernelGGL(kernel, dim3((uint32_t)wgs), dim3(kPThreads), kPLds, s, (const uint16_t *)x,
                                   (const uint16_t *)w, (const uint16_t *)bias, (uint16_t *)tok, g, K, ngroups);
                return hipGetLastError();
            };
            const bool kvec = K % 8 == 0;
            if (K <= 32) {
                if (fast) return kvec ? go_w(patchify_ldsw_bf16<1, true, true>) : go_w(patchify_ldsw_bf16<1, true, false>);
                return kvec ? go_w(patchify_ldsw_bf16<1, false, true>) : go_w(patchify_ldsw_bf16<1, false, false>);
            }
            if (fast) return kvec ? go_w(patchify_ldsw_bf16<2, true, true>) : go_w(patchify_ldsw_bf16<2, true, false>);
            return kvec ? go_w(patchify_ldsw_bf16<2, false, true>) : go_w(patchify_ldsw_bf16<2, false, false>);
        }
    }
    const dim3 grid((uint32_t)((M + kTok - 1) / kTok), kChunkSplit);
    const size_t lds = (size_t)kTok * (4 * (kOut + 8) + (Kp + 8)) * 2;
    auto go = [&](auto kernel) {
        if (lds > 65536) {  // above the default dynamic-LDS limit (up to 99 KB at Kp = 512)
            const hipError_t e =
                hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(kernel, grid, dim3(512), lds, s, (const uint16_t *)x, (const uint16_t *)w,
                           (const uint16_t *)bias, (uint16_t *)tok, g, K, Kp);
        return hipGetLastError();
    };
    switch (Kp / 16) {
        case 1: return go(patchify_bf16_kernel<1>);
        case 2: return go(patchify_bf16_kernel<2>);
        case 3: return go(patchify_bf16_kernel<3>);
        case 4: return go(patchify_bf16_kernel<4>);
        case 5: return go(patchify_bf16_kernel<5>);
        case 6: return go(patchify_bf16_kernel<6>);
        case 7: return go(patchify_bf16_kernel<7>);
        case 8: return go(patchify_bf16_kernel<8>);
        default: return go(patchify_bf16_kernel<0>);
    }
}

hipError_t launch_patchify_f32(const float *x, const float *w, const float *bias, float *tok, const PatchGeom &g,
                               hipStream_t s) {
    const int64_t total = (int64_t)g.B * g.T * g.Hp * g.Wp * g.Dout;
    const uint32_t grid = (uint32_t)((total + 255) / 256);
    hipLaunchKernelGGL(patchify_f32_kernel, dim3(grid), dim3(256), 0, s, x, w, bias, tok, g);
    return hipGetLastError();
}

}  // namespace vdit
