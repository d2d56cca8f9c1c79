// C ABI of libvdit: argument checks, then one kernel launch per call.
// Every check runs before anything is enqueued; the library allocates
// nothing and keeps no state between calls.
#include "vdit.h"
#include "vdit_internal.h"

#include <cmath>
#include <cstdint>

using namespace vdit;

namespace {

constexpr double kLog2e = 1.4426950408889634073599246810019;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void *a, uint64_t na, const void *b, uint64_t nb) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

// a*b*... as uint64 with overflow detection against 2^62.
bool mul_ok(uint64_t &acc, int64_t f) {
    if (f <= 0) return false;
    if (acc > (uint64_t(1) << 62) / (uint64_t)f) return false;
    acc *= (uint64_t)f;
    return true;
}

int esize(vdit_dtype_t dt) { return dt == VDIT_F32 ? 4 : 2; }

vdit_status_t launch_status(hipError_t e) { return e == hipSuccess ? VDIT_OK : VDIT_E_LAUNCH; }

enum Mode { kFull = 0, kSpatial = 1, kTemporal = 2 };

// RoPE split of a head vector into (d_t, d_h, d_w): nonnegative even parts
// that add up to head_dim.
bool split_ok(int D, int d_t, int d_h, int d_w) {
    return d_t >= 0 && d_h >= 0 && d_w >= 0 && !(d_t & 1) && !(d_h & 1) && !(d_w & 1) &&
           (int64_t)d_t + d_h + d_w == D;
}

// Rotation parameters of the attention kernels that apply RoPE themselves
// (rope != nullptr selects them; `split` = {d_t, d_h, d_w}).
struct AttnRope {
    int split[3];
    float theta;
};

vdit_status_t attn(const void *q, const void *k, const void *v, void *o, int B, int heads, int T, int Hp, int Wp,
                   int D, float scale, vdit_dtype_t dt, void *stream, Mode mode, const AttnRope *rope = nullptr) {
    if (!q || !k || !v || !o) return VDIT_E_NULL;
    if (dt != VDIT_BF16 && dt != VDIT_F32) return VDIT_E_DTYPE;
    if (rope && dt != VDIT_BF16) return VDIT_E_DTYPE;
    if (B <= 0 || heads <= 0 || T <= 0 || Hp <= 0 || Wp <= 0 || D <= 0) return VDIT_E_SHAPE;
    uint64_t n_tok = 1;
    if (!mul_ok(n_tok, T) || !mul_ok(n_tok, Hp) || !mul_ok(n_tok, Wp)) return VDIT_E_SHAPE;
    if (n_tok > (uint64_t)INT32_MAX) return VDIT_E_SHAPE;
    uint64_t elems = n_tok;
    if (!mul_ok(elems, B) || !mul_ok(elems, heads) || !mul_ok(elems, D)) return VDIT_E_SHAPE;
    const uint64_t bytes = elems * (uint64_t)esize(dt);
    if (D != 32 && D != 64 && D != 128) return VDIT_E_HEAD_DIM;
    if (mode == kTemporal && T > (dt == VDIT_BF16 ? 64 : 256)) return VDIT_E_SHAPE;
    // Workgroup counts must fit a 1-D grid.
    if ((uint64_t)B * heads * n_tok > (uint64_t)UINT32_MAX * 32) return VDIT_E_SHAPE;
    // The bf16 kernels address one batch's tokens through buffer descriptors
    // whose byte range is a signed 32-bit value.
    if (dt == VDIT_BF16 && n_tok * (uint64_t)heads * (uint64_t)D * 2u >= (uint64_t(1) << 31)) return VDIT_E_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return VDIT_E_ALIGN;
    if (rope && !split_ok(D, rope->split[0], rope->split[1], rope->split[2])) return VDIT_E_ROPE_SPLIT;
    if (rope && (!(rope->theta > 0.f) || !std::isfinite(rope->theta))) return VDIT_E_SHAPE;
    if (overlap(o, bytes, q, bytes) || overlap(o, bytes, k, bytes) || overlap(o, bytes, v, bytes))
        return VDIT_E_ALIAS;

    const float s = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)D));
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int HW = Hp * Wp;
    if (rope) {
        FlashRope fr{};
        fr.T = T;
        fr.Hp = Hp;
        fr.Wp = Wp;
        fr.b1 = rope->split[0] / 2;
        fr.b2 = (rope->split[0] + rope->split[1]) / 2;
        int j = 0;
        for (int a = 0; a < 3; ++a)
            for (int jj = 0; jj < rope->split[a] / 2; ++jj, ++j)
                fr.freq_rev[j] = (float)(std::pow((double)rope->theta, -2.0 * jj / (double)rope->split[a]) /
                                         6.283185307179586476925286766559);
        const float c = (float)((double)s * kLog2e);
        if (mode == kFull)
            return launch_status(launch_flash_rope_bf16(q, k, v, o, B, T * HW, T * HW, heads, D, c, 0, fr, st));
        if (mode == kSpatial)
            return launch_status(launch_flash_rope_bf16(q, k, v, o, B * T, HW, HW, heads, D, c, 1, fr, st));
        return launch_status(launch_temporal_rope_bf16(q, k, v, o, B, heads, T, HW, D, c, fr, st));
    }
    if (dt == VDIT_F32)
        return launch_status(launch_attn_f32((const float *)q, (const float *)k, (const float *)v, (float *)o, B,
                                             heads, T, HW, D, (int)mode, s, st));
    const float c = (float)((double)s * kLog2e);
    switch (mode) {
        case kFull: return launch_status(launch_flash_bf16(q, k, v, o, B, T * HW, T * HW, heads, D, c, 0, st));
        case kSpatial: return launch_status(launch_flash_bf16(q, k, v, o, B * T, HW, HW, heads, D, c, 1, st));
        default: return launch_status(launch_temporal_bf16(q, k, v, o, B, heads, T, HW, D, c, st));
    }
}

}  // namespace

extern "C" {

const char *vdit_status_str(vdit_status_t status) {
    switch (status) {
        case VDIT_OK: return "VDIT_OK";
        case VDIT_E_NULL: return "VDIT_E_NULL: a required pointer is NULL";
        case VDIT_E_SHAPE: return "VDIT_E_SHAPE: invalid or overflowing sizes";
        case VDIT_E_HEAD_DIM: return "VDIT_E_HEAD_DIM: unsupported head_dim";
        case VDIT_E_ROPE_SPLIT: return "VDIT_E_ROPE_SPLIT: d_t + d_h + d_w != head_dim or an odd part";
        case VDIT_E_ALIGN: return "VDIT_E_ALIGN: pointer not 16-byte aligned";
        case VDIT_E_ALIAS: return "VDIT_E_ALIAS: output overlaps an input";
        case VDIT_E_DTYPE: return "VDIT_E_DTYPE: unknown dtype";
        case VDIT_E_LAUNCH: return "VDIT_E_LAUNCH: kernel launch failed";
    }
    return "unknown vdit status";
}

vdit_status_t vdit_attn_full(const void *q, const void *k, const void *v, void *o, int B, int heads, int T, int Hp,
                             int Wp, int head_dim, float scale, vdit_dtype_t dtype, void *stream) {
    return attn(q, k, v, o, B, heads, T, Hp, Wp, head_dim, scale, dtype, stream, kFull);
}

vdit_status_t vdit_attn_spatial(const void *q, const void *k, const void *v, void *o, int B, int heads, int T,
                                int Hp, int Wp, int head_dim, float scale, vdit_dtype_t dtype, void *stream) {
    return attn(q, k, v, o, B, heads, T, Hp, Wp, head_dim, scale, dtype, stream, kSpatial);
}

vdit_status_t vdit_attn_full_rope(const void *q, const void *k, const void *v, void *o, int B, int heads, int T,
                                  int Hp, int Wp, int head_dim, int d_t, int d_h, int d_w, float theta, float scale,
                                  vdit_dtype_t dtype, void *stream) {
    const AttnRope r{{d_t, d_h, d_w}, theta};
    return attn(q, k, v, o, B, heads, T, Hp, Wp, head_dim, scale, dtype, stream, kFull, &r);
}

vdit_status_t vdit_attn_spatial_rope(const void *q, const void *k, const void *v, void *o, int B, int heads, int T,
                                     int Hp, int Wp, int head_dim, int d_t, int d_h, int d_w, float theta,
                                     float scale, vdit_dtype_t dtype, void *stream) {
    const AttnRope r{{d_t, d_h, d_w}, theta};
    return attn(q, k, v, o, B, heads, T, Hp, Wp, head_dim, scale, dtype, stream, kSpatial, &r);
}

vdit_status_t vdit_attn_temporal_rope(const void *q, const void *k, const void *v, void *o, int B, int heads,
                                      int T, int Hp, int Wp, int head_dim, int d_t, int d_h, int d_w, float theta,
                                      float scale, vdit_dtype_t dtype, void *stream) {
    const AttnRope r{{d_t, d_h, d_w}, theta};
    return attn(q, k, v, o, B, heads, T, Hp, Wp, head_dim, scale, dtype, stream, kTemporal, &r);
}

vdit_status_t vdit_attn_temporal(const void *q, const void *k, const void *v, void *o, int B, int heads, int T,
                                 int Hp, int Wp, int head_dim, float scale, vdit_dtype_t dtype, void *stream) {
    return attn(q, k, v, o, B, heads, T, Hp, Wp, head_dim, scale, dtype, stream, kTemporal);
}

vdit_status_t vdit_attn_cross(const void *q, const void *k, const void *v, void *o, int B, int heads, int Nq,
                              int Nk, int head_dim, float scale, vdit_dtype_t dtype, void *stream) {
    if (!q || !k || !v || !o) return VDIT_E_NULL;
    if (dtype != VDIT_BF16 && dtype != VDIT_F32) return VDIT_E_DTYPE;
    if (B <= 0 || heads <= 0 || Nq <= 0 || Nk <= 0 || head_dim <= 0) return VDIT_E_SHAPE;
    const int D = head_dim;
    if (D != 32 && D != 64 && D != 128) return VDIT_E_HEAD_DIM;
    uint64_t qe = 1, ke = 1;
    if (!mul_ok(qe, B) || !mul_ok(qe, Nq) || !mul_ok(qe, heads) || !mul_ok(qe, D)) return VDIT_E_SHAPE;
    if (!mul_ok(ke, B) || !mul_ok(ke, Nk) || !mul_ok(ke, heads) || !mul_ok(ke, D)) return VDIT_E_SHAPE;
    if ((uint64_t)B * heads * (uint64_t)Nq > (uint64_t)UINT32_MAX * 32) return VDIT_E_SHAPE;
    if (dtype == VDIT_BF16 && ((uint64_t)Nk * heads * D * 2u >= (uint64_t(1) << 31) ||
                               (uint64_t)Nq * heads * D * 2u >= (uint64_t(1) << 31)))
        return VDIT_E_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return VDIT_E_ALIGN;
    const uint64_t es = (uint64_t)esize(dtype);
    if (overlap(o, qe * es, q, qe * es) || overlap(o, qe * es, k, ke * es) || overlap(o, qe * es, v, ke * es))
        return VDIT_E_ALIAS;
    const float s = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)D));
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dtype == VDIT_F32)
        return launch_status(launch_cross_f32((const float *)q, (const float *)k, (const float *)v, (float *)o, B,
                                              heads, Nq, Nk, D, s, st));
    return launch_status(launch_flash_bf16(q, k, v, o, B, Nq, Nk, heads, D, (float)((double)s * kLog2e), 2, st));
}

vdit_status_t vdit_attn_window(const void *q, const void *k, const void *v, void *o, int B, int heads, int T,
                               int Hp, int Wp, int head_dim, int wt, int wh, int ww, float scale, vdit_dtype_t dtype,
                               void *stream) {
    if (!q || !k || !v || !o) return VDIT_E_NULL;
    if (dtype != VDIT_BF16 && dtype != VDIT_F32) return VDIT_E_DTYPE;
    if (B <= 0 || heads <= 0 || T <= 0 || Hp <= 0 || Wp <= 0 || head_dim <= 0 || wt <= 0 || wh <= 0 || ww <= 0)
        return VDIT_E_SHAPE;
    const int D = head_dim;
    if (D != 32 && D != 64 && D != 128) return VDIT_E_HEAD_DIM;
    uint64_t n_tok = 1;
    if (!mul_ok(n_tok, T) || !mul_ok(n_tok, Hp) || !mul_ok(n_tok, Wp)) return VDIT_E_SHAPE;
    if (n_tok > (uint64_t)INT32_MAX) return VDIT_E_SHAPE;
    uint64_t elems = n_tok;
    if (!mul_ok(elems, B) || !mul_ok(elems, heads) || !mul_ok(elems, D)) return VDIT_E_SHAPE;
    const uint64_t bytes = elems * (uint64_t)esize(dtype);
    // Windows larger than the grid are clipped to it.
    WinGeom g{T, Hp, Wp, wt < T ? wt : T, wh < Hp ? wh : Hp, ww < Wp ? ww : Wp, 0, 0, 0, 0};
    const uint64_t nwin = (uint64_t)((T + g.wt - 1) / g.wt) * ((Hp + g.wh - 1) / g.wh) * ((Wp + g.ww - 1) / g.ww);
    const uint64_t lw = (uint64_t)g.wt * g.wh * g.ww;
    // Workgroups (at most 64 queries of one window and head each) must fit a
    // 1-D grid; windows per batch times B must fit an int.
    if ((uint64_t)B * nwin > (uint64_t)INT32_MAX || (uint64_t)B * nwin * heads * ((lw + 63) / 64) > UINT32_MAX)
        return VDIT_E_SHAPE;
    if (dtype == VDIT_BF16 && n_tok * (uint64_t)heads * (uint64_t)D * 2u >= (uint64_t(1) << 31)) return VDIT_E_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return VDIT_E_ALIGN;
    if (overlap(o, bytes, q, bytes) || overlap(o, bytes, k, bytes) || overlap(o, bytes, v, bytes))
        return VDIT_E_ALIAS;
    const float s = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)D));
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dtype == VDIT_F32)
        return launch_status(
            launch_window_f32((const float *)q, (const float *)k, (const float *)v, (float *)o, B, heads, D, g, s, st));
    return launch_status(launch_window_bf16(q, k, v, o, B, heads, D, g, (float)((double)s * kLog2e), st));
}

vdit_status_t vdit_qkv_proj(const void *x, const void *w, const void *bias, const void *gamma_q,
                            const void *gamma_k, void *q, void *k, void *v, int B, int T, int Hp, int Wp, int heads,
                            int head_dim, int d_t, int d_h, int d_w, float theta, float eps, vdit_dtype_t dtype,
                            void *stream) {
    if (!x || !w || !q || !k || !v) return VDIT_E_NULL;
    if (dtype != VDIT_BF16 && dtype != VDIT_F32) return VDIT_E_DTYPE;
    if (B <= 0 || T <= 0 || Hp <= 0 || Wp <= 0 || heads <= 0 || head_dim <= 0) return VDIT_E_SHAPE;
    const int D = head_dim;
    if (dtype == VDIT_BF16 && D != 128) return VDIT_E_HEAD_DIM;
    if (dtype == VDIT_F32 && (D > 256 || D % 2)) return VDIT_E_HEAD_DIM;
    const bool rope_on = d_t != 0 || d_h != 0 || d_w != 0;
    if (rope_on && !split_ok(D, d_t, d_h, d_w)) return VDIT_E_ROPE_SPLIT;
    if (rope_on && (!(theta > 0.f) || !std::isfinite(theta))) return VDIT_E_SHAPE;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return VDIT_E_SHAPE;
    uint64_t n_tok = 1, dim = 1;
    if (!mul_ok(n_tok, B) || !mul_ok(n_tok, T) || !mul_ok(n_tok, Hp) || !mul_ok(n_tok, Wp)) return VDIT_E_SHAPE;
    if (!mul_ok(dim, heads) || !mul_ok(dim, D)) return VDIT_E_SHAPE;
    if (n_tok > (uint64_t)INT32_MAX || dim * 3 > (uint64_t)INT32_MAX) return VDIT_E_SHAPE;
    uint64_t xel = n_tok, wel = dim * 3;
    if (!mul_ok(xel, (int64_t)dim) || !mul_ok(wel, (int64_t)dim)) return VDIT_E_SHAPE;
    const uint64_t es = (uint64_t)esize(dtype);
    if (dtype == VDIT_BF16) {
        // K advances 64 at a time and the epilogue takes whole heads; the
        // buffer descriptors' byte ranges are signed 32-bit values.
        if (dim % 128) return VDIT_E_SHAPE;
        if (xel * 2 >= (uint64_t(1) << 31) || wel * 2 >= (uint64_t(1) << 31)) return VDIT_E_SHAPE;
    }
    if (!aligned16(x) || !aligned16(w) || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
        (bias && !aligned16(bias)) || (gamma_q && !aligned16(gamma_q)) || (gamma_k && !aligned16(gamma_k)))
        return VDIT_E_ALIGN;
    const uint64_t ob = xel * es;
    const void *outs[3] = {q, k, v};
    for (int i = 0; i < 3; ++i) {
        if (overlap(outs[i], ob, x, xel * es) || overlap(outs[i], ob, w, wel * es) ||
            (bias && overlap(outs[i], ob, bias, dim * 3 * es)) || (gamma_q && overlap(outs[i], ob, gamma_q, dim * es)) ||
            (gamma_k && overlap(outs[i], ob, gamma_k, dim * es)))
            return VDIT_E_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], ob, outs[j], ob)) return VDIT_E_ALIAS;
    }
    QkvGeom g{(int)n_tok, T * Hp * Wp, Hp, Wp, (int)dim, D, eps};
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int width[3] = {d_t, d_h, d_w};
    if (dtype == VDIT_F32) {
        RopeTable tab{};
        int j = 0;
        if (rope_on)
            for (int a = 0; a < 3; ++a)
                for (int jj = 0; jj < width[a] / 2; ++jj, ++j) {
                    tab.axis[j] = (unsigned char)a;
                    tab.freq[j] = std::pow((double)theta, -2.0 * jj / (double)width[a]);
                }
        return launch_status(launch_qkv_proj_f32((const float *)x, (const float *)w, (const float *)bias,
                                                 (const float *)gamma_q, (const float *)gamma_k, (float *)q,
                                                 (float *)k, (float *)v, g, tab, rope_on ? 1 : 0, st));
    }
    QkvRope rope{};
    rope.on = rope_on ? 1 : 0;
    if (rope_on) {
        int j = 0;
        for (int a = 0; a < 3; ++a)
            for (int jj = 0; jj < width[a] / 2; ++jj, ++j)
                rope.freq_rev[j] = (float)(std::pow((double)theta, -2.0 * jj / (double)width[a]) /
                                           6.283185307179586476925286766559);
        rope.b1 = d_t / 2;
        rope.b2 = (d_t + d_h) / 2;
    }
    return launch_status(launch_qkv_proj_bf16(x, w, bias, gamma_q, gamma_k, q, k, v, g, rope, st));
}

vdit_status_t vdit_patchify(const void *latent, const void *weight, const void *bias, void *tokens, int B, int C,
                            int pt, int ph, int pw, int Tl, int Hl, int Wl, int heads, int T, int Hp, int Wp,
                            int head_dim, vdit_dtype_t dtype, void *stream) {
    if (!latent || !weight || !tokens) return VDIT_E_NULL;
    if (dtype != VDIT_BF16 && dtype != VDIT_F32) return VDIT_E_DTYPE;
    if (B <= 0 || C <= 0 || pt <= 0 || ph <= 0 || pw <= 0 || Tl <= 0 || Hl <= 0 || Wl <= 0 || heads <= 0 ||
        T <= 0 || Hp <= 0 || Wp <= 0 || head_dim <= 0)
        return VDIT_E_SHAPE;
    if (T != Tl / pt || Hp != Hl / ph || Wp != Wl / pw) return VDIT_E_SHAPE;
    uint64_t dout = 1, kdim = 1, lat = 1, tok = 1;
    if (!mul_ok(dout, heads) || !mul_ok(dout, head_dim)) return VDIT_E_SHAPE;
    if (!mul_ok(kdim, C) || !mul_ok(kdim, pt) || !mul_ok(kdim, ph) || !mul_ok(kdim, pw)) return VDIT_E_SHAPE;
    if (!mul_ok(lat, B) || !mul_ok(lat, C) || !mul_ok(lat, Tl) || !mul_ok(lat, Hl) || !mul_ok(lat, Wl))
        return VDIT_E_SHAPE;
    if (!mul_ok(tok, B) || !mul_ok(tok, T) || !mul_ok(tok, Hp) || !mul_ok(tok, Wp) || !mul_ok(tok, (int64_t)dout))
        return VDIT_E_SHAPE;
    if (dout > (uint64_t)INT32_MAX || dout % 8) return VDIT_E_SHAPE;
    if (dtype == VDIT_BF16 && (kdim + 15) / 16 * 16 > 512) return VDIT_E_SHAPE;
    if (tok / dout > (uint64_t)UINT32_MAX * 64 / 2) return VDIT_E_SHAPE;
    if (!aligned16(latent) || !aligned16(weight) || !aligned16(tokens) || (bias && !aligned16(bias)))
        return VDIT_E_ALIGN;
    const uint64_t es = (uint64_t)esize(dtype);
    if (overlap(tokens, tok * es, latent, lat * es) || overlap(tokens, tok * es, weight, dout * kdim * es) ||
        (bias && overlap(tokens, tok * es, bias, dout * es)))
        return VDIT_E_ALIAS;
    PatchGeom g{B, C, pt, ph, pw, Tl, Hl, Wl, T, Hp, Wp, (int)dout};
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dtype == VDIT_F32)
        return launch_status(
            launch_patchify_f32((const float *)latent, (const float *)weight, (const float *)bias, (float *)tokens, g, st));
    return launch_status(launch_patchify_bf16(latent, weight, bias, tokens, g, st));
}

vdit_status_t vdit_rope3d(const void *x, void *y, int B, int heads, int T, int Hp, int Wp, int head_dim, int d_t,
                          int d_h, int d_w, float theta, vdit_dtype_t dtype, void *stream) {
    if (!x || !y) return VDIT_E_NULL;
    if (dtype != VDIT_BF16 && dtype != VDIT_F32) return VDIT_E_DTYPE;
    if (B <= 0 || heads <= 0 || T <= 0 || Hp <= 0 || Wp <= 0 || head_dim <= 0) return VDIT_E_SHAPE;
    if (head_dim % 8 || head_dim > 256) return VDIT_E_HEAD_DIM;
    if (!split_ok(head_dim, d_t, d_h, d_w)) return VDIT_E_ROPE_SPLIT;
    if (!(theta > 0.f) || !std::isfinite(theta)) return VDIT_E_SHAPE;
    uint64_t elems = 1;
    if (!mul_ok(elems, B) || !mul_ok(elems, T) || !mul_ok(elems, Hp) || !mul_ok(elems, Wp) || !mul_ok(elems, heads) ||
        !mul_ok(elems, head_dim))
        return VDIT_E_SHAPE;
    if (elems / heads / 8 > (uint64_t)UINT32_MAX * 256) return VDIT_E_SHAPE;
    if (!aligned16(x) || !aligned16(y)) return VDIT_E_ALIGN;
    const uint64_t bytes = elems * (uint64_t)esize(dtype);
    if (x != y && overlap(x, bytes, y, bytes)) return VDIT_E_ALIAS;

    RopeTable tab{};
    const int width[3] = {d_t, d_h, d_w};
    int j = 0;
    for (int a = 0; a < 3; ++a)
        for (int jj = 0; jj < width[a] / 2; ++jj, ++j) {
            tab.axis[j] = (unsigned char)a;
            tab.freq[j] = std::pow((double)theta, -2.0 * jj / (double)width[a]);
        }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dtype == VDIT_F32)
        return launch_status(launch_rope_f32((const float *)x, (float *)y, B, heads, T, Hp, Wp, head_dim, tab, st));
    return launch_status(launch_rope_bf16(x, y, B, heads, T, Hp, Wp, head_dim, tab, st));
}

}  // extern "C"
