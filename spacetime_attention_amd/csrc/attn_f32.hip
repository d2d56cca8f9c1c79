// fp32 attention for all three key sets (full, spatial, temporal).
//
// The fp32 path serves fp32 workloads such as the tiny video DiT of the
// "Video and 3D Generation" cheatsheet ("Tiny video DiT": 256 tokens, 2 heads
// of 32), where results must agree with fp64 to 1e-5. One thread owns one
// (batch, token, head) query: its row of Q and its output accumulator live in
// registers, and an online softmax in fp32 runs over the query's key set,
// read through the workgroup's LDS in tiles shared by the 64 queries of a
// wavefront-sized group. Keys of query n = (b, t, p), p = h*Wp + w:
//   full      m = 0..N-1             at token b*N + m
//   spatial   m = 0..HW-1            at token b*N + t*HW + m
//   temporal  m = 0..T-1             at token b*N + m*HW + p
// Queries of one workgroup share (b, head) and, for the spatial and temporal
// passes, are grouped so that they share one key set.
#include "vdit_internal.h"

namespace vdit {
namespace {

constexpr int kQ = 64;     // queries per workgroup (one wavefront)
constexpr int kTile = 32;  // keys staged per step

template <int D>
__global__ __launch_bounds__(kQ) void attn_f32_kernel(const float *__restrict__ q, const float *__restrict__ k,
                                                      const float *__restrict__ v, float *__restrict__ o,
                                                      int B, int heads, int T, int HW, int mode, float scale)
{
    __shared__ float ks[kTile][D];
    __shared__ float vs[kTile][D];
    const int64_t N = (int64_t)T * HW;
    // Query groups: a group is a set of up to kQ queries with one key set.
    //   full: groups of kQ consecutive tokens of one (b, head).
    //   spatial: groups of kQ consecutive tokens within one frame.
    //   temporal: the kQ-token group is a run of positions p within one
    //   frame t; every query of it has its own key set (its column), so the
    //   temporal mode reads keys per thread instead of through LDS.
    const int64_t L = (mode == 0) ? N : (mode == 1 ? HW : HW);
    const int64_t groups_per_seg = (L + kQ - 1) / kQ;
    const int64_t nseg_per_b = (mode == 0) ? 1 : T;
    int64_t g = blockIdx.x;
    const int64_t gi = g % groups_per_seg;
    g /= groups_per_seg;
    const int64_t segi = g % nseg_per_b;
    g /= nseg_per_b;
    const int hd = (int)(g % heads);
    const int b = (int)(g / heads);
    const int64_t within = gi * kQ + threadIdx.x;  // index inside the segment
    const bool valid = within < L;
    const int64_t n = (mode == 0) ? within : segi * HW + within;  // query token
    const int64_t rs = (int64_t)heads * D;
    const int64_t bbase = (int64_t)b * N;

    float qr[D], acc[D];
    if (valid) {
        const float *qp = q + ((bbase + n) * heads + hd) * D;
#pragma unroll
        for (int d = 0; d < D; ++d) qr[d] = qp[d];
    } else {
#pragma unroll
        for (int d = 0; d < D; ++d) qr[d] = 0.f;
    }
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = 0.f;
    float mx = -INFINITY, l = 0.f;

    auto consume = [&](const float *kr, const float *vr) {
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) s = fmaf(qr[d], kr[d], s);
        s *= scale;
        if (s > mx) {
            const float corr = expf(mx - s);
            l *= corr;
#pragma unroll
            for (int d = 0; d < D; ++d) acc[d] *= corr;
            mx = s;
        }
        const float p = expf(s - mx);
        l += p;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vr[d], acc[d]);
    };

    if (mode == 2) {
        // Temporal: keys at stride HW tokens from the query's own position.
        const int64_t p = n % HW;
        if (valid)
            for (int m = 0; m < T; ++m) {
                const int64_t key = bbase + (int64_t)m * HW + p;
                consume(k + (key * heads + hd) * D, v + (key * heads + hd) * D);
            }
    } else {
        const int64_t kbase = (mode == 0) ? bbase : bbase + segi * HW;
        for (int64_t m0 = 0; m0 < L; m0 += kTile) {
            const int nk = (int)((L - m0) < kTile ? (L - m0) : kTile);
            for (int i = threadIdx.x; i < nk * D; i += kQ) {
                const int r = i / D, d = i % D;
                const int64_t key = kbase + m0 + r;
                ks[r][d] = k[(key * heads + hd) * D + d];
                vs[r][d] = v[(key * heads + hd) * D + d];
            }
            __syncthreads();
            if (valid)
                for (int r = 0; r < nk; ++r) consume(ks[r], vs[r]);
            __syncthreads();
        }
    }
    if (valid) {
        float *op = o + ((bbase + n) * heads + hd) * D;
        const float inv = 1.0f / l;
#pragma unroll
        for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
    }
}

// Cross-attention in fp32: one thread per (b, query, head); the Nk keys of
// batch b are staged through LDS in tiles shared by the workgroup's queries.
template <int D>
__global__ __launch_bounds__(kQ) void cross_f32_kernel(const float *__restrict__ q, const float *__restrict__ k,
                                                       const float *__restrict__ v, float *__restrict__ o, int B,
                                                       int heads, int Nq, int Nk, float scale)
{
    __shared__ float ks[kTile][D];
    __shared__ float vs[kTile][D];
    const int64_t groups = (Nq + kQ - 1) / kQ;
    const int64_t gi = blockIdx.x % groups;
    const int hd = (int)((blockIdx.x / groups) % heads);
    const int b = (int)(blockIdx.x / (groups * heads));
    const int64_t n = gi * kQ + threadIdx.x;
    const bool valid = n < Nq;

    float qr[D], acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        qr[d] = valid ? q[(((int64_t)b * Nq + n) * heads + hd) * D + d] : 0.f;
        acc[d] = 0.f;
    }
    float mx = -INFINITY, l = 0.f;
    for (int m0 = 0; m0 < Nk; m0 += kTile) {
        const int nk = (Nk - m0) < kTile ? (Nk - m0) : kTile;
        for (int i = threadIdx.x; i < nk * D; i += kQ) {
            const int r = i / D, d = i % D;
            const int64_t key = (int64_t)b * Nk + m0 + r;
            ks[r][d] = k[(key * heads + hd) * D + d];
            vs[r][d] = v[(key * heads + hd) * D + d];
        }
        __syncthreads();
        if (valid)
            for (int r = 0; r < nk; ++r) {
                float sc = 0.f;
#pragma unroll
                for (int d = 0; d < D; ++d) sc = fmaf(qr[d], ks[r][d], sc);
                sc *= scale;
                if (sc > mx) {
                    const float corr = expf(mx - sc);
                    l *= corr;
#pragma unroll
                    for (int d = 0; d < D; ++d) acc[d] *= corr;
                    mx = sc;
                }
                const float p = expf(sc - mx);
                l += p;
#pragma unroll
                for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[r][d], acc[d]);
            }
        __syncthreads();
    }
    if (valid) {
        const float inv = 1.0f / l;
#pragma unroll
        for (int d = 0; d < D; ++d) o[(((int64_t)b * Nq + n) * heads + hd) * D + d] = acc[d] * inv;
    }
}

// Windowed attention in fp32: one thread per (b, window-local query j,
// head), 64 queries of one window per workgroup; the window's keys are
// gathered into LDS in tiles. Window-local index j maps to the token
// (t0 + j/(ch*cw), h0 + (j/cw)%ch, w0 + j%cw) of the window's clipped
// extents ct x ch x cw.
template <int D>
__global__ __launch_bounds__(kQ) void window_f32_kernel(const float *__restrict__ q, const float *__restrict__ k,
                                                        const float *__restrict__ v, float *__restrict__ o,
                                                        int heads, WinGeom g, float scale)
{
    __shared__ float ks[kTile][D];
    __shared__ float vs[kTile][D];
    const int nwin = g.nwt * g.nwh * g.nww;
    const int qblk = (int)(blockIdx.x % g.nqb);
    const int hd = (int)((blockIdx.x / g.nqb) % heads);
    const int seg = (int)(blockIdx.x / ((uint32_t)g.nqb * heads));
    const int b = seg / nwin, w = seg % nwin;
    const int iww = w % g.nww, iwh = (w / g.nww) % g.nwh, iwt = w / (g.nww * g.nwh);
    const int t0 = iwt * g.wt, h0 = iwh * g.wh, w0 = iww * g.ww;
    const int ct = min(g.wt, g.T - t0), ch = min(g.wh, g.Hp - h0), cw = min(g.ww, g.Wp - w0);
    const int Lw = ct * ch * cw;
    if (qblk * kQ >= Lw) return;
    const int64_t HW = (int64_t)g.Hp * g.Wp;
    const int64_t org = (int64_t)b * g.T * HW + ((int64_t)t0 * g.Hp + h0) * g.Wp + w0;
    auto tok = [&](int j) -> int64_t { return org + (j / (ch * cw)) * HW + ((j / cw) % ch) * g.Wp + j % cw; };

    const int j = qblk * kQ + threadIdx.x;
    const bool valid = j < Lw;
    float qr[D], acc[D];
    const float *qp = q + (tok(valid ? j : 0) * heads + hd) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) {
        qr[d] = valid ? qp[d] : 0.f;
        acc[d] = 0.f;
    }
    float mx = -INFINITY, l = 0.f;
    for (int m0 = 0; m0 < Lw; m0 += kTile) {
        const int nk = (Lw - m0) < kTile ? (Lw - m0) : kTile;
        for (int i = threadIdx.x; i < nk * D; i += kQ) {
            const int r = i / D, d = i % D;
            const int64_t key = tok(m0 + r);
            ks[r][d] = k[(key * heads + hd) * D + d];
            vs[r][d] = v[(key * heads + hd) * D + d];
        }
        __syncthreads();
        if (valid)
            for (int r = 0; r < nk; ++r) {
                float sc = 0.f;
#pragma unroll
                for (int d = 0; d < D; ++d) sc = fmaf(qr[d], ks[r][d], sc);
                sc *= scale;
                if (sc > mx) {
                    const float corr = expf(mx - sc);
                    l *= corr;
#pragma unroll
                    for (int d = 0; d < D; ++d) acc[d] *= corr;
                    mx = sc;
                }
                const float p = expf(sc - mx);
                l += p;
#pragma unroll
                for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[r][d], acc[d]);
            }
        __syncthreads();
    }
    if (valid) {
        float *op = o + (tok(j) * heads + hd) * D;
        const float inv = 1.0f / l;
#pragma unroll
        for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
    }
}

template <int D>
hipError_t launch_window(const float *q, const float *k, const float *v, float *o, int B, int heads,
                         WinGeom g, float scale, hipStream_t s) {
    g.nwt = (g.T + g.wt - 1) / g.wt;
    g.nwh = (g.Hp + g.wh - 1) / g.wh;
    g.nww = (g.Wp + g.ww - 1) / g.ww;
    g.nqb = (g.wt * g.wh * g.ww + kQ - 1) / kQ;
    const uint64_t grid = (uint64_t)B * g.nwt * g.nwh * g.nww * heads * g.nqb;
    if (grid == 0 || grid > UINT32_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(window_f32_kernel<D>, dim3((uint32_t)grid), dim3(kQ), 0, s, q, k, v, o, heads, g, scale);
    return hipGetLastError();
}

template <int D>
hipError_t launch_cross(const float *q, const float *k, const float *v, float *o, int B, int heads, int Nq,
                        int Nk, float scale, hipStream_t s) {
    const int64_t groups = (int64_t)((Nq + kQ - 1) / kQ) * heads * B;
    hipLaunchKernelGGL(cross_f32_kernel<D>, dim3((uint32_t)groups), dim3(kQ), 0, s, q, k, v, o, B, heads, Nq, Nk,
                       scale);
    return hipGetLastError();
}

template <int D>
hipError_t launch(const float *q, const float *k, const float *v, float *o, int B, int heads, int T,
                  int HW, int mode, float scale, hipStream_t s) {
    const int64_t N = (int64_t)T * HW;
    const int64_t L = (mode == 0) ? N : HW;
    const int64_t groups = ((L + kQ - 1) / kQ) * ((mode == 0) ? 1 : T) * heads * B;
    hipLaunchKernelGGL(attn_f32_kernel<D>, dim3((uint32_t)groups), dim3(kQ), 0, s, q, k, v, o, B, heads, T,
                       HW, mode, scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_window_f32(const float *q, const float *k, const float *v, float *o, int B, int heads, int D,
                             const WinGeom &g, float scale, hipStream_t s) {
    switch (D) {
        case 32: return launch_window<32>(q, k, v, o, B, heads, g, scale, s);
        case 64: return launch_window<64>(q, k, v, o, B, heads, g, scale, s);
        case 128: return launch_window<128>(q, k, v, o, B, heads, g, scale, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_cross_f32(const float *q, const float *k, const float *v, float *o, int B, int heads, int Nq,
                            int Nk, int D, float scale, hipStream_t s) {
    switch (D) {
        case 32: return launch_cross<32>(q, k, v, o, B, heads, Nq, Nk, scale, s);
        case 64: return launch_cross<64>(q, k, v, o, B, heads, Nq, Nk, scale, s);
        case 128: return launch_cross<128>(q, k, v, o, B, heads, Nq, Nk, scale, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attn_f32(const float *q, const float *k, const float *v, float *o, int B, int heads,
                           int T, int HW, int D, int mode, float scale, hipStream_t s) {
    switch (D) {
        case 32: return launch<32>(q, k, v, o, B, heads, T, HW, mode, scale, s);
        case 64: return launch<64>(q, k, v, o, B, heads, T, HW, mode, scale, s);
        case 128: return launch<128>(q, k, v, o, B, heads, T, HW, mode, scale, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace vdit
