// 3D factorised rotary position embedding (bf16 or fp32 storage, fp32 math).
//
// "How AI Generates Video: Inside Sora and Wan2.1 on a Real GPU", section 4
// ("How 3D Factorized RoPE Encodes (t', h, w)"): a head vector is cut into
// three consecutive segments (44, 42, 42 of 128); in segment a the pair
// (x[2j], x[2j+1]) is rotated by p_a * theta^(-2j/d_a), p_a being the token's
// t, h or w index. The angle depends on the token and the pair, not on the
// head, so a thread computes the sin/cos of its four pairs once and applies
// them to every head of its token. The angle is formed and reduced to
// [-pi, pi] in fp64 before the fp32 sin/cos, so its error does not grow with
// the position. The pass is elementwise and bound by HBM: each thread moves
// whole 16-byte (bf16) or 32-byte (fp32) groups of 8 elements.
#include "vdit_internal.h"

namespace vdit {
namespace {

template <typename Elem>
struct Vec8;
template <>
struct Vec8<uint16_t> {
    u32x4 raw;
    __device__ void load(const uint16_t *p) { raw = *(const u32x4 *)p; }
    __device__ void store(uint16_t *p) const { *(u32x4 *)p = raw; }
    __device__ float get(int i) const { return bf16_bits_to_f32((raw[i >> 1] >> (16 * (i & 1))) & 0xffffu); }
    __device__ void set_pair(int j, float a, float b) { raw[j] = pack_bf16x2(a, b); }
};
template <>
struct Vec8<float> {
    f32x4 lo, hi;
    __device__ void load(const float *p) { lo = *(const f32x4 *)p; hi = *(const f32x4 *)(p + 4); }
    __device__ void store(float *p) const { *(f32x4 *)p = lo; *(f32x4 *)(p + 4) = hi; }
    __device__ float get(int i) const { return i < 4 ? lo[i] : hi[i - 4]; }
    __device__ void set_pair(int j, float a, float b) {
        if (j < 2) { lo[2 * j] = a; lo[2 * j + 1] = b; } else { hi[2 * j - 4] = a; hi[2 * j - 3] = b; }
    }
};

template <typename Elem>
__global__ __launch_bounds__(256) void rope_kernel(const Elem *x, Elem *y, int B, int heads, int T,
                                                   int Hp, int Wp, int D, RopeTable args)
{
    const int gpt = D / 8;  // 8-element groups per head vector
    const int64_t N = (int64_t)T * Hp * Wp;
    const int64_t total = (int64_t)B * N * gpt;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int grp = (int)(idx % gpt);
    const int64_t token = idx / gpt;
    const int64_t n = token % N;
    const int pos[3] = {(int)(n / ((int64_t)Hp * Wp)), (int)((n / Wp) % Hp), (int)(n % Wp)};

    float cs[4], sn[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int j = grp * 4 + e;
        const double a = (double)pos[args.axis[j]] * args.freq[j];
        const double two_pi = 6.283185307179586476925286766559;
        const float r = (float)(a - rint(a / two_pi) * two_pi);
        sincosf(r, &sn[e], &cs[e]);
    }
    const Elem *xp = x + token * heads * D + grp * 8;
    Elem *yp = y + token * heads * D + grp * 8;
    for (int hd = 0; hd < heads; ++hd) {
        Vec8<Elem> in;
        in.load(xp + (int64_t)hd * D);
        Vec8<Elem> out = in;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x0 = in.get(2 * e), x1 = in.get(2 * e + 1);
            out.set_pair(e, x0 * cs[e] - x1 * sn[e], x0 * sn[e] + x1 * cs[e]);
        }
        out.store(yp + (int64_t)hd * D);
    }
}

template <typename Elem>
hipError_t launch(const Elem *x, Elem *y, int B, int heads, int T, int Hp, int Wp, int D, const RopeTable &tab,
                  hipStream_t s) {
    const int64_t total = (int64_t)B * T * Hp * Wp * (D / 8);
    const uint32_t grid = (uint32_t)((total + 255) / 256);
    hipLaunchKernelGGL(rope_kernel<Elem>, dim3(grid), dim3(256), 0, s, x, y, B, heads, T, Hp, Wp, D,
                       tab);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_bf16(const void *x, void *y, int B, int heads, int T, int Hp, int Wp, int D,
                            const RopeTable &tab, hipStream_t s) {
    return launch<uint16_t>((const uint16_t *)x, (uint16_t *)y, B, heads, T, Hp, Wp, D, tab, s);
}
hipError_t launch_rope_f32(const float *x, float *y, int B, int heads, int T, int Hp, int Wp, int D,
                           const RopeTable &tab, hipStream_t s) {
    return launch<float>(x, y, B, heads, T, Hp, Wp, D, tab, s);
}

}  // namespace vdit
