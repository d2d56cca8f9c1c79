// Flash-style fused attention for the full and spatial passes (bf16, gfx950).
//
// Computes o = softmax(scale * q k^T) v per (segment, head) without forming
// the score matrix: the tiled form that "Video Diffusion Models, in depth"
// (Step 3) calls mandatory, with an online softmax in fp32 (its "Failure
// modes" keep softmax in FP32). A segment is a run of L consecutive query
// tokens whose keys are the segment's Lk consecutive key tokens: the whole
// clip for full 3D attention, one latent frame (Hp*Wp tokens) for the
// spatial pass (Lk = L for both), and the whole text prompt for
// cross-attention ("How AI Generates Video ...", section 5, attn2).
// Windowed attention ("Video Diffusion Models, in depth", "Inference: where
// the time goes": attention restricted to local spacetime windows) runs the
// same tile loop over one wt x wh x ww box of the token grid: its queries and
// keys are gathered by window-local index j, whose token is found by a
// mixed-radix decomposition of j over the box's clipped extents, and key
// rows are advanced by that radix from one 64-key tile to the next.
//
// Layout of the work (one workgroup = 4 or 8 wavefronts of 32 queries):
//  * Scores are formed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16:
//    the A operand is a 32-key block of K read from LDS, the B operand the
//    wave's queries kept in registers for the whole pass. In the result each
//    lane owns one query column and 16 of its keys, so a row max and a row
//    sum are register reductions plus one exchange with lane^32
//    (v_permlane32_swap).
//  * The probabilities are reused in place as the B operand of
//    O^T = V^T P^T: the contraction runs over keys, and the order in which
//    keys feed it is free as long as both operands agree, so the S^T result
//    registers already hold a valid B operand (no shuffles). V^T comes from
//    a row-major V tile in LDS through ds_read_b64_tr_b16, which hands each
//    lane four consecutive keys of one feature column.
//  * K and V tiles of 64 keys are buffered in LDS and filled by
//    buffer loads that write LDS directly (no staging registers): lane l of a
//    load lands at byte 16*l of the wave's 1 KB destination, so each lane
//    fetches the global chunk that belongs at that swizzled LDS slot. The
//    buffer descriptor's size ends at the segment's last key, so loads past
//    it return zeros and need no bounds checks. The next tile's loads are
//    issued before the current tile's products. Chunk-XOR swizzles keep the
//    K reads (32 rows, one 16-byte chunk each) and the transposed V reads
//    (8 rows x 64 bytes) free of bank conflicts.
//  * Full attention (8 wavefronts, two per SIMD: waves w and w+4 share one)
//    runs a ping-pong schedule: each wave alternates an all-MFMA phase
//    (V^T P^T of the previous tile, then S^T of the current one) with an
//    all-VALU phase (the current tile's softmax), with a workgroup barrier
//    after every phase, and waves 4..7 run one phase behind waves 0..3, so
//    one wave's exponentials always run under the other's matrix products.
//  * The other passes (4 wavefronts, two workgroups per compute unit) run
//    each tile as a pipeline over its two 32-key blocks inside the wave:
//    S^T of the second block between the first block's exponentials, and
//    V^T P^T of the first block between the second's. Their two K/V buffer
//    pairs live in two distinct LDS arrays, so the compiler can see that the
//    transposed V reads of one pair do not alias the loads filling the other
//    and does not wait for those loads before the reads.
//  * The reference maximum of the online softmax is raised lazily: a tile's
//    probabilities are formed against the current reference, and only when
//    a lane's tile sum exceeds 256 (or is not finite, as on the first tile)
//    does the wave take the row maximum, raise the reference, rescale O^T
//    and form them again. Most tiles skip the row maximum and the rescale;
//    normalising by the sum taken against the same reference keeps the
//    result exactly softmax, and the reference, always an actual score,
//    never exceeds the true maximum.
//  * Workgroups are numbered so that each XCD gets a contiguous run of
//    (segment, head, query block) tiles and so shares K/V in its own L2.
//
// This header holds the kernel template and its launch helper; attn_flash.hip
// and attn_flash_full.hip instantiate it.
#pragma once

#include "vdit_internal.h"

#include <type_traits>

namespace vdit {
namespace {

constexpr int kBN = 64;                // keys per LDS tile
// Wavefronts per workgroup (32 queries each). Every workgroup streams its
// segment's whole K/V through L2, so more queries per workgroup means fewer
// re-reads: full attention (long segments) uses 8; the spatial pass (1,560-
// token frames that stay in L2) uses 4, which wastes less on the ragged
// last query block.
constexpr int kFullWaves = 8;
constexpr int kSpatialWaves = 4;
// A tile's probabilities against the reference maximum may sum to at most
// this before the reference is raised: every probability then stays below
// 256, so fp32 sums and accumulators over any key count stay finite. A
// small budget keeps the reference close behind a row's largest score, so a
// key that dominates its row soon carries probability exactly 1 (held
// exactly in bf16); on N(0,1) data the reference is still raised only on
// the first tile of a row.
constexpr float kTileSumBudget = 256.0f;

template <int D, int QB, int NW>
struct FlashShape {
    static constexpr int THREADS = NW * 64;
    static constexpr int BM = NW * 32 * QB;      // queries per workgroup
    static constexpr int CH = D / 8;             // 16-byte chunks per row
    static constexpr int KS = D / 16;            // k-steps of S^T = K Q^T
    static constexpr int DB = D / 32;            // 32-row blocks of O^T
    static constexpr int TILE = kBN * D * 2;     // bytes of one K or V tile
    static constexpr int LOADS = kBN * CH / THREADS;  // 1 KB LDS loads per wave per tensor
    static_assert(kBN * CH % THREADS == 0, "tile must split evenly over the threads");
};

// Physical 16-byte chunk of logical chunk c in row r of a K tile: XOR with
// the row index spreads the 16 rows one b128 read touches over all banks.
template <int D>
__device__ __forceinline__ int swz_k(int r, int c) { return c ^ (r % (D / 8)); }

// Same for a V tile, read transposed: a ds_read_b64_tr_b16 covers 4
// consecutive rows x 4 chunks per half-wave, so rows are moved apart by
// multiples of 4 chunks within each 256-byte bank period.
template <int D>
__device__ __forceinline__ int swz_v(int r, int c) {
    constexpr int CH = D / 8;
    constexpr int RPP = 256 / (2 * D);  // rows per 256-byte bank period
    return c ^ (4 * ((r / RPP) % (CH / 4)));
}

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Buffer descriptor word 3 for gfx9-family raw (unswizzled) buffers.
constexpr int kBufferFlags = 0x00020000;

// Wait until this wave's outstanding vector-memory loads (including the
// ones that write LDS directly) have completed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier that orders LDS accesses only: vector-memory loads that
// are still in flight stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ bf16x4 lds_read_tr(const lds_u8 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
}

// max and sum of x over the lane pair (l, l^32).
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __attribute__((address_space(3))) float lds_f32;

// RoPE on one 16-byte chunk of a head vector: its eight bf16 values are
// logical chunk lc, i.e. pairs 4*lc .. 4*lc+3, of a token at grid position
// (pt, ph, pw). The angle is taken in revolutions and reduced to [0, 1)
// for v_sin_f32 / v_cos_f32; rtab holds the pairs' frequencies.
__device__ __forceinline__ u32x4 rope_chunk(u32x4 x, int lc, float pt, float ph, float pw, const lds_f32 *rtab,
                                            int b1, int b2)
{
    const f32x4 fq = *(const __attribute__((address_space(3))) f32x4 *)(rtab + 4 * lc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int p = 4 * lc + e;
        const float pos = p < b1 ? pt : (p < b2 ? ph : pw);
        const float rev = __builtin_amdgcn_fractf(pos * fq[e]);
        const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
        const float x0 = __uint_as_float(x[e] << 16), x1 = __uint_as_float(x[e] & 0xffff0000u);
        x[e] = pack_bf16x2(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
    }
    return x;
}

// The three parts of one 64-key tile, which the full pass's ping-pong
// phases issue separately. flash_s forms S^T = K Q^T for both
// 32-key blocks from the K tile at LDS byte offset KB0; flash_softmax takes
// the online softmax over those scores (kvalid = number of the tile's keys
// that exist) and leaves the probabilities P^T as bf16 MFMA operands;
// flash_pv adds V^T P^T to O^T from the V tile VB0 bytes past the per-lane
// read bases vbase (row and column of the lane's transposed reads, plus
// the start of the V buffers).
template <int D, int QB>
__device__ __forceinline__ void flash_s(const lds_u8 *lds, uint32_t KB0, const uint32_t (&kofs)[D / 16],
                                        const bf16x8 (&qop)[QB][D / 16], f32x16 (&sacc)[2][QB])
{
    constexpr int KS = D / 16;
    constexpr int RB = D * 2;  // bytes per row
    // LDS operand reads run one step ahead of the MFMAs that use them,
    // in a second set of registers; scheduling fences keep the compiler
    // from sinking them back to their uses.
    bf16x8 ka[2][2];
    auto rdk = [&](int ks, int slot) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
            ka[slot][kb2] = *(const __attribute__((address_space(3))) bf16x8 *)(
                lds + kofs[ks] + (KB0 + kb2 * 32 * RB));
    };
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[kb2][qb] = (f32x16){};
    rdk(0, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) rdk(ks + 1, (ks + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                sacc[kb2][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks & 1][kb2], qop[qb][ks], sacc[kb2][qb], 0, 0, 0);
    }
}

template <int D, int QB>
__device__ __forceinline__ void flash_softmax(f32x16 (&sacc)[2][QB], bf16x8 (&pop)[QB][2][2],
                                              f32x16 (&oacc)[D / 32][QB], float (&mref)[QB], float (&lsum)[QB],
                                              float c, int kvalid, int half, bool first)
{
    constexpr int DB = D / 32;
    // Keys past the end of the segment (last tile only).
    if (kvalid < kBN) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kb2 * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (key >= kvalid)
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) sacc[kb2][qb][r] = -INFINITY;
            }
    }

    // Online softmax in the exp2 domain: x = s * scale * log2(e).
    // Probabilities are first formed against the current reference
    // maximum; only if a lane's tile sum leaves the budget (or is not
    // finite, as on the first tile) does the wave take the row maximum,
    // raise the reference, rescale and form them again.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        float ls = 0.f;
        // A 32-key block at a time: its 16 exponents, then the 16
        // exponentials, then a pairwise sum and the bf16 packing, each group
        // fenced so that the wave issues independent instructions back to
        // back instead of waiting on each result in turn.
        auto probs = [&]() {
            const float nm = -mref[qb];
            ls = 0.f;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                float p[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) p[r] = fmaf(sacc[kb2][qb][r], c, nm);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(p[r]);
                __builtin_amdgcn_sched_barrier(0);
                // The row sum takes the fp32 probabilities (a tree of adds):
                // summing the bf16 values the V product applies costs this
                // phase 2-8% (v_dot2c_f32_bf16 issues slowly here). The
                // reference is raised whenever a tile's sum passes the budget,
                // so a key that dominates a row soon carries probability 1,
                // which bf16 holds exactly.
                float t[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) t[i] = p[2 * i] + p[2 * i + 1];
#pragma unroll
                for (int i = 0; i < 4; ++i) t[i] = t[2 * i] + t[2 * i + 1];
                ls += (t[0] + t[1]) + (t[2] + t[3]);
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    u32x4 pk;
                    pk[0] = pack_bf16x2(p[8 * s2 + 0], p[8 * s2 + 1]);
                    pk[1] = pack_bf16x2(p[8 * s2 + 2], p[8 * s2 + 3]);
                    pk[2] = pack_bf16x2(p[8 * s2 + 4], p[8 * s2 + 5]);
                    pk[3] = pack_bf16x2(p[8 * s2 + 6], p[8 * s2 + 7]);
                    pop[qb][kb2][s2] = __builtin_bit_cast(bf16x8, pk);
                }
            }
        };
        if (first) {
            // Tile 0: the reference starts at the row maximum, so the
            // probabilities are formed once (against -inf they would all be
            // infinite and take the slow path below).
            float mx = sacc[0][qb][0];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb2][qb][r]);
            mref[qb] = pair_max(mx) * c;
        }
        probs();
        if (__builtin_amdgcn_ballot_w64(!(ls <= kTileSumBudget))) {
            float mx = sacc[0][qb][0];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb2][qb][r]);
            mx = pair_max(mx) * c;
            const float mnew = fmaxf(mx, mref[qb]);
            const float alpha = __builtin_amdgcn_exp2f(mref[qb] - mnew);
            mref[qb] = mnew;
            lsum[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db][qb] *= alpha;
            probs();
        }
        lsum[qb] += ls;
    }
}

template <int D, int QB>
__device__ __forceinline__ void flash_pv(const lds_u8 *lds, uint32_t VB0, const uint32_t (&vbase)[D / 32],
                                         const bf16x8 (&pop)[QB][2][2], f32x16 (&oacc)[D / 32][QB])
{
    constexpr int DB = D / 32;
    constexpr int RB = D * 2;  // bytes per row
    bf16x4 va[2][DB][2];
    auto rdv = [&](int st, int slot) {
        const uint32_t off = VB0 + ((st >> 1) * 32 + 16 * (st & 1)) * RB;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            va[slot][db][0] = lds_read_tr(lds + vbase[db] + off);
            va[slot][db][1] = lds_read_tr(lds + vbase[db] + (off + 8 * RB));
        }
    };
    rdv(0, 0);
    // O^T += V^T P^T over the tile's four 16-key steps.
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        if (st + 1 < 4) rdv(st + 1, (st + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const bf16x8 a = __builtin_shufflevector(va[st & 1][db][0], va[st & 1][db][1], 0, 1, 2, 3, 4,
                                                     5, 6, 7);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                oacc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop[qb][st >> 1][st & 1], oacc[db][qb], 0, 0, 0);
        }
    }
}

// One 64-key tile of the 4-wave passes, as a pipeline over its two 32-key
// blocks inside one wave: S^T of block 1 is issued between the softmax
// steps of block 0, and V^T P^T of block 0 between those of block 1, so the
// wave's own exponentials run under its own matrix products. The lazy
// reference of flash_softmax is kept per block: a block whose probabilities
// against the current reference sum past the budget (or are not finite)
// raises it, rescales O^T and the running sum (which already hold the
// earlier blocks) and forms that block again.
//
// On a row's first tile (first) the reference starts at block 0's row
// maximum instead of -inf. HALF is the form for a last tile whose keys all
// lie in block 0 (kvalid <= 32): block 1's products and probabilities, all of
// them for keys past the segment, are left out.
template <int D, bool HALF>
__device__ __forceinline__ void flash_tile_pipe(const lds_u8 *lds, uint32_t B0, const uint32_t (&kofs)[D / 16],
                                                const uint32_t (&vofs)[D / 32], const bf16x8 (&qop)[1][D / 16],
                                                f32x16 (&oacc)[D / 32][1], float (&mref)[1], float (&lsum)[1],
                                                float c, int kvalid, int half, bool first)
{
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int RB = D * 2;
    constexpr int TILE = kBN * RB;
    f32x16 sb[2] = {(f32x16){}, (f32x16){}};
    bf16x8 pb[2][2];
    auto kread = [&](int kb2, int ks) {
        return *(const __attribute__((address_space(3))) bf16x8 *)(lds + kofs[ks] + (B0 + kb2 * 32 * RB));
    };
    // V^T operand of 16-key step st and feature block db.
    auto vread = [&](int st, int db) {
        const uint32_t off = B0 + TILE + ((st >> 1) * 32 + 16 * (st & 1)) * RB;
        const bf16x4 lo = lds_read_tr(lds + (vofs[db] - TILE) + off);
        const bf16x4 hi = lds_read_tr(lds + (vofs[db] - TILE) + (off + 8 * RB));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto mask = [&](int kb2) {
        if (kvalid < kBN) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kb2 * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (key >= kvalid) sb[kb2][r] = -INFINITY;
            }
        }
    };
    // Probabilities r in [i*n, (i+1)*n) of block kb2 against the current reference.
    float p[16];
    auto prob_slice = [&](int kb2, int i, int n) {
        const float nm = -mref[0];
#pragma unroll
        for (int r = i * n; r < (i + 1) * n; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(sb[kb2][r], c, nm));
    };
    // Pack block kb2's probabilities and sum the packed values; if the sum leaves the budget,
    // raise the reference and form them again.
    auto finish_block = [&](int kb2) {
        auto sum_pack = [&]() {
            float ls = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                u32x4 pk;
                pk[0] = pack_bf16x2(p[8 * s2 + 0], p[8 * s2 + 1]);
                pk[1] = pack_bf16x2(p[8 * s2 + 2], p[8 * s2 + 3]);
                pk[2] = pack_bf16x2(p[8 * s2 + 4], p[8 * s2 + 5]);
                pk[3] = pack_bf16x2(p[8 * s2 + 6], p[8 * s2 + 7]);
                pb[kb2][s2] = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
                for (int e = 0; e < 4; ++e) ls = add_bf16_pair(pk[e], ls);
            }
            return ls;
        };
        float ls = sum_pack();
        if (__builtin_amdgcn_ballot_w64(!(ls <= kTileSumBudget))) {
            float mx = sb[kb2][0];
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sb[kb2][r]);
            mx = pair_max(mx) * c;
            const float mnew = fmaxf(mx, mref[0]);
            const float alpha = __builtin_amdgcn_exp2f(mref[0] - mnew);
            mref[0] = mnew;
            lsum[0] *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db][0] *= alpha;
            prob_slice(kb2, 0, 16);
            ls = sum_pack();
        }
        lsum[0] += ls;
    };

    // Stage 1: S^T of block 0.
    {
        bf16x8 ka[2];
        ka[0] = kread(0, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) ka[(ks + 1) & 1] = kread(0, ks + 1);
            __builtin_amdgcn_sched_barrier(0);
            sb[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks & 1], qop[0][ks], sb[0], 0, 0, 0);
        }
    }
    mask(0);
    if (first) {
        float mx = sb[0][0];
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sb[0][r]);
        mref[0] = pair_max(mx) * c;
    }
    // Stage 2: S^T of block 1 under block 0's exponentials.
    if constexpr (HALF) {
        prob_slice(0, 0, 16);
    } else {
        constexpr int n = 16 / KS;
        bf16x8 ka[2];
        ka[0] = kread(1, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) ka[(ks + 1) & 1] = kread(1, ks + 1);
            __builtin_amdgcn_sched_barrier(0);
            sb[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks & 1], qop[0][ks], sb[1], 0, 0, 0);
            prob_slice(0, ks, n);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    finish_block(0);
    if constexpr (!HALF) mask(1);
    // Stage 3: V^T P^T of block 0 (steps 0, 1) under block 1's exponentials.
    {
        constexpr int NM = 2 * DB;
        constexpr int n = 16 / NM;
        bf16x8 va[2];
        va[0] = vread(0, 0);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const int st = m / DB, db = m % DB;
            if (m + 1 < NM) va[(m + 1) & 1] = vread((m + 1) / DB, (m + 1) % DB);
            __builtin_amdgcn_sched_barrier(0);
            oacc[db][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[m & 1], pb[0][st], oacc[db][0], 0, 0, 0);
            if constexpr (!HALF) prob_slice(1, m, n);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if constexpr (HALF) return;
    finish_block(1);
    // Stage 4: V^T P^T of block 1 (steps 2, 3).
    {
        constexpr int NM = 2 * DB;
        bf16x8 va[2];
        va[0] = vread(2, 0);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const int st = 2 + m / DB, db = m % DB;
            if (m + 1 < NM) va[(m + 1) & 1] = vread(2 + (m + 1) / DB, (m + 1) % DB);
            __builtin_amdgcn_sched_barrier(0);
            oacc[db][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[m & 1], pb[1][st - 2], oacc[db][0], 0, 0, 0);
        }
    }
}

// PASS (0 full, 1 spatial, 2 cross, 3 window, 4 full with RoPE, 5 spatial
// with RoPE) names the instantiation, so that profiles attribute the passes
// separately; the first three run the same code. The RoPE passes rotate the
// queries in registers after they are read, and each wave rotates its own
// share of every K tile in LDS once its loads of that tile have landed and
// before the barrier that hands the tile to the other waves, so the barrier
// protocol is the same as without RoPE. L is the number of queries and Lk the number of keys per
// segment (equal for self-attention; the text length for cross-attention);
// the window pass takes both from the window it works on and nseg = B times
// the number of windows.
template <int D, int QB, int NW, int PASS>
__global__ __launch_bounds__(NW * 64, 8 / NW) void flash_fwd_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    uint16_t *__restrict__ o, int nseg, int L, int Lk, int heads, float c, WinGeom wg, FlashRope fr)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    using S = FlashShape<D, QB, NW>;
    constexpr bool WIN = PASS == 3;
    // The full pass (8 waves) runs two 4-wave groups out of phase over three
    // K and three V buffers; the other passes alternate two K/V pairs.
    constexpr bool PP = NW == 8 && !WIN;
    __shared__ __attribute__((aligned(16))) unsigned char smem[(PP ? 6 : 2) * S::TILE];
    // The other passes keep their second K/V buffer pair in an array of its
    // own. With the two pairs in distinct arrays the compiler can tell that
    // the transposed V reads of one pair do not alias the LDS-direct loads
    // filling the other, and adds no wait for those loads before the reads.
    // The RoPE passes keep their 64 pair frequencies after it.
    constexpr bool ROPE = PASS >= 4;
    __shared__ __attribute__((aligned(16))) unsigned char smem1[(PP ? 0 : 2 * S::TILE) + (ROPE ? 256 : (PP ? 16 : 0))];
    lds_u8 *lds = (lds_u8 *)smem;
    lds_u8 *lds1 = (lds_u8 *)smem1;
    lds_f32 *rtab = (lds_f32 *)(lds1 + (PP ? 0 : 2 * S::TILE));
    if constexpr (ROPE) {
        if (threadIdx.x < D / 2) rtab[threadIdx.x] = fr.freq_rev[threadIdx.x];
        __syncthreads();
    }

    const int nqb = WIN ? wg.nqb : (L + S::BM - 1) / S::BM;
    const uint32_t id = xcd_contiguous(blockIdx.x, (uint32_t)nseg * (uint32_t)heads * (uint32_t)nqb);
    const int qblk = (int)(id % nqb);
    const int hd = (int)((id / nqb) % heads);
    const int seg = (int)(id / ((uint32_t)nqb * heads));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
    const int half = lane >> 5, col = lane & 31;
    const int64_t rs = (int64_t)heads * D;  // elements between consecutive tokens

    // Token rows of the queries (qorg) and keys (korg) of this workgroup,
    // and, for a window, its clipped extents ct x chh x cww and the token
    // strides of its frame and row.
    int64_t qorg, korg;
    int ct = 0, chh = 1, cww = 1, HWt = 0, Wpt = 0;
    if constexpr (WIN) {
        const int nwin = wg.nwt * wg.nwh * wg.nww;
        const int b = seg / nwin, w = seg % nwin;
        const int iww = w % wg.nww, iwh = (w / wg.nww) % wg.nwh, iwt = w / (wg.nww * wg.nwh);
        const int t0 = iwt * wg.wt, h0 = iwh * wg.wh, w0 = iww * wg.ww;
        ct = min(wg.wt, wg.T - t0);
        chh = min(wg.wh, wg.Hp - h0);
        cww = min(wg.ww, wg.Wp - w0);
        HWt = wg.Hp * wg.Wp;
        Wpt = wg.Wp;
        L = Lk = ct * chh * cww;
        if (qblk * S::BM >= L) return;  // a block past the end of a clipped window
        qorg = korg = (int64_t)b * wg.T * HWt + ((int64_t)t0 * wg.Hp + h0) * wg.Wp + w0;
    } else {
        qorg = (int64_t)seg * L;
        korg = (int64_t)seg * Lk;
    }
    // Token (relative to the origin) of window-local index j.
    auto tok = [&](int j) -> int {
        if constexpr (WIN)
            return (j / (chh * cww)) * HWt + ((j / cww) % chh) * Wpt + j % cww;
        else
            return j;
    };
    const int64_t base = (qorg * heads + hd) * D;    // query / output rows
    const int64_t kvbase = (korg * heads + hd) * D;  // key / value rows
    const uint16_t *qp = q + base, *kp = k + kvbase, *vp = v + kvbase;
    uint16_t *op = o + base;

    // This wave's queries, as B operands of S^T = K Q^T.
    const int q0 = qblk * S::BM + wave * 32 * QB;
    // A wave whose queries all lie past the end of the segment (in the last,
    // ragged query block) still loads its share of every K/V tile and meets
    // every barrier, but skips the products and the softmax.
    const bool busy = q0 < L;
    bf16x8 qop[QB][S::KS];
    // The 4-wave passes stage the queries through LDS (below); the full pass
    // reads them straight into registers, once for its whole key loop.
    constexpr bool QSTAGE = !PP && QB == 1 && NW == 4;
    // RoPE: token rows are batch-major, so a row's index within its clip
    // (and with it the row's grid position) is the row modulo T*Hp*Wp.
    const int HWg = fr.Hp * fr.Wp;
    const int64_t Ng = (int64_t)fr.T * HWg;
    auto rope_q = [&]() {
        const int n = (int)((qorg + q0 + col) % Ng);
        const float pt = (float)(n / HWg), ph = (float)((n / fr.Wp) % fr.Hp), pw = (float)(n % fr.Wp);
#pragma unroll
        for (int ks = 0; ks < S::KS; ++ks)
            qop[0][ks] = __builtin_bit_cast(
                bf16x8, rope_chunk(__builtin_bit_cast(u32x4, qop[0][ks]), 2 * ks + half, pt, ph, pw, rtab, fr.b1,
                                   fr.b2));
    };
    if constexpr (!QSTAGE) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int qi = q0 + qb * 32 + col;
            const int64_t qrow = (int64_t)tok(qi < L ? qi : 0) * rs;
#pragma unroll
            for (int ks = 0; ks < S::KS; ++ks) {
                if (qi < L)
                    qop[qb][ks] = *(const bf16x8 *)(qp + qrow + 16 * ks + 8 * half);
                else
                    qop[qb][ks] = (bf16x8){};
            }
        }
        if constexpr (ROPE) rope_q();
    }

    // Buffer descriptors over this (segment, head)'s keys and values: the
    // size stops at the end of key Lk-1's row, so any row >= Lk reads as zero.
    const int nrec = (int)(((int64_t)tok(Lk - 1) * rs + D) * 2);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)kp, 0, nrec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)vp, 0, nrec, kBufferFlags);
    // Per-lane byte offsets (within a tile) of the chunks this lane fetches:
    // the wave's i-th load fills LDS rows RPL*(wave*LOADS + i) + lane/CH,
    // physical chunk lane%CH, which holds logical chunk (lane%CH) ^ swizzle.
    constexpr int RPL = 64 / S::CH;  // rows per wave-wide 1 KB load
    uint32_t koff[S::LOADS], voff[S::LOADS];
#pragma unroll
    for (int i = 0; i < S::LOADS; ++i) {
        const int r = RPL * (wave * S::LOADS + i) + lane / S::CH;
        const int pc = lane % S::CH;
        koff[i] = (uint32_t)(r * rs * 2 + (pc ^ (swz_k<D>(r, 0))) * 16);
        voff[i] = (uint32_t)(r * rs * 2 + (pc ^ (swz_v<D>(r, 0))) * 16);
    }
    // Window pass: the key index j of each load's row is carried as mixed-
    // radix digits (jt, jh, jw) over the extents (ct, chh, cww); koff/voff
    // then hold only the chunk parts, and one tile step adds 64 = dt*chh*cww
    // + dh*cww + dw with single carries (every digit sum stays below twice
    // its radix). Rows with jt >= ct (j >= Lk) get an offset past the
    // descriptor's size and read as zeros.
    int jt[S::LOADS], jh[S::LOADS], jw[S::LOADS];
    int dt = 0, dh = 0, dw = 0;
    if constexpr (WIN) {
        const int plane = chh * cww;
        dt = kBN / plane;
        dh = (kBN % plane) / cww;
        dw = (kBN % plane) % cww;
#pragma unroll
        for (int i = 0; i < S::LOADS; ++i) {
            const int r = RPL * (wave * S::LOADS + i) + lane / S::CH;
            koff[i] -= (uint32_t)(r * rs * 2);
            voff[i] -= (uint32_t)(r * rs * 2);
            jt[i] = r / plane;
            jh[i] = (r / cww) % chh;
            jw[i] = r % cww;
        }
    }
    const uint32_t rsb = (uint32_t)(rs * 2), HWb = (uint32_t)HWt * rsb, Wpb = (uint32_t)Wpt * rsb;
    // RoPE: grid position (rt, rh, rw) of the key row each of this wave's
    // loads fills in the next K tile to be rotated. Tiles are rotated in
    // order, and one tile step adds 64 = rdt*Hp*Wp + rdh*Wp + rdw with single
    // carries, as for the window digits above.
    int rt[S::LOADS], rh[S::LOADS], rw[S::LOADS];
    int rdt = 0, rdh = 0, rdw = 0;
    if constexpr (ROPE) {
        rdt = kBN / HWg;
        rdh = (kBN % HWg) / fr.Wp;
        rdw = kBN % fr.Wp;
#pragma unroll
        for (int i = 0; i < S::LOADS; ++i) {
            const int r = RPL * (wave * S::LOADS + i) + lane / S::CH;
            const int n = (int)((korg + r) % Ng);
            rt[i] = n / HWg;
            rh[i] = (n / fr.Wp) % fr.Hp;
            rw[i] = n % fr.Wp;
        }
    }
    // Rotates this wave's share of the K tile at kb: each lane rewrites the
    // 16 bytes its own load wrote (row r, physical chunk lane % CH, which
    // holds logical chunk (lane % CH) ^ (r % CH)).
    auto rope_k = [&](lds_u8 *kb) {
#pragma unroll
        for (int i = 0; i < S::LOADS; ++i) {
            const int r = RPL * (wave * S::LOADS + i) + lane / S::CH;
            const int lc = (lane % S::CH) ^ (r % S::CH);
            auto *p = (__attribute__((address_space(3))) u32x4 *)(kb + (wave * S::LOADS + i) * 1024 + 16 * lane);
            *p = rope_chunk(*p, lc, (float)rt[i], (float)rh[i], (float)rw[i], rtab, fr.b1, fr.b2);
            rw[i] += rdw;
            const int cw1 = rw[i] >= fr.Wp;
            rw[i] -= cw1 ? fr.Wp : 0;
            rh[i] += rdh + cw1;
            const int ch1 = rh[i] >= fr.Hp;
            rh[i] -= ch1 ? fr.Hp : 0;
            rt[i] += rdt + ch1;
        }
    };
    auto load_tile = [&](int t0, int buf) {
        lds_u8 *kb = buf ? lds1 : lds;
        lds_u8 *vb = kb + S::TILE;
        if constexpr (WIN) {
#pragma unroll
            for (int i = 0; i < S::LOADS; ++i) {
                const uint32_t row =
                    jt[i] < ct ? (uint32_t)jt[i] * HWb + (uint32_t)jh[i] * Wpb + (uint32_t)jw[i] * rsb : 0x80000000u;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void *)(kb + (wave * S::LOADS + i) * 1024), 16,
                                                         row + koff[i], 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void *)(vb + (wave * S::LOADS + i) * 1024), 16,
                                                         row + voff[i], 0, 0, 0);
                jw[i] += dw;
                const int cw1 = jw[i] >= cww;
                jw[i] -= cw1 ? cww : 0;
                jh[i] += dh + cw1;
                const int ch1 = jh[i] >= chh;
                jh[i] -= ch1 ? chh : 0;
                jt[i] += dt + ch1;
            }
        } else {
            const uint32_t so = (uint32_t)((int64_t)t0 * rs * 2);
#pragma unroll
            for (int i = 0; i < S::LOADS; ++i) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void *)(kb + (wave * S::LOADS + i) * 1024), 16,
                                                         koff[i], so, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void *)(vb + (wave * S::LOADS + i) * 1024), 16,
                                                         voff[i], so, 0, 0);
            }
        }
    };

    // K or V alone (full pass): tile at key t0 into LDS byte offset dst.
    auto load_one = [&](__amdgpu_buffer_rsrc_t rs_, const uint32_t (&off)[S::LOADS], int t0, uint32_t dst) {
        const uint32_t so = (uint32_t)((int64_t)t0 * rs * 2);
#pragma unroll
        for (int i = 0; i < S::LOADS; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_, (lds_void *)(lds + dst + (wave * S::LOADS + i) * 1024), 16,
                                                     off[i], so, 0, 0);
    };

    // Per-lane LDS byte offsets of the operand reads, for buffer 0 and key
    // block 0. Every other read adds a compile-time constant (buffer, key
    // block, 16-key step, upper 8 rows), which the ds_read offset field holds:
    //  * K (A of S^T): row col, logical chunk 2*ks + half;
    //  * V (A of O^T, transposed read): 16-lane group g reads rows
    //    4*(g/2) + lane%16/4 at feature column db*32 + 16*(g%2) + 4*(lane%4).
    // The swizzles depend on the row only through bits the constants leave
    // unchanged, so the constant parts stay additive.
    uint32_t kofs[S::KS], vofs[S::DB];
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) kofs[ks] = col * D * 2 + swz_k<D>(col, 2 * ks + half) * 16;
    {
        const int grp = lane >> 4, gl = lane & 15;
        const int vrow = 4 * (grp >> 1) + (gl >> 2);
        const int vcol = 16 * (grp & 1) + 4 * (gl & 3);
#pragma unroll
        for (int db = 0; db < S::DB; ++db) {
            const int dc = db * 32 + vcol;
            vofs[db] = S::TILE + vrow * D * 2 + swz_v<D>(vrow, dc >> 3) * 16 + (dc & 7) * 2;
        }
    }

    f32x16 oacc[S::DB][QB];
#pragma unroll
    for (int db = 0; db < S::DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = (f32x16){};
    float mref[QB], lsum[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        mref[qb] = -INFINITY;
        lsum[qb] = 0.f;
    }

    const int ntiles = (Lk + kBN - 1) / kBN;

    auto tile = [&](auto bufc, int j) {
        static_assert(PP || QB == 1, "the pipelined tile holds one 32-query block per wave");
        const lds_u8 *tb = decltype(bufc)::value ? lds1 : lds;
        flash_tile_pipe<D, false>(tb, 0, kofs, vofs, qop, oacc, mref, lsum, c, Lk - j * kBN, half, j == 0);
    };

    if constexpr (PP) {
        // Each wave alternates an MFMA phase X(j) = [O^T += V^T P^T for tile
        // j-1, then S^T for tile j] with a VALU phase Y(j) = the softmax of
        // tile j, and a barrier ends every phase. Waves 4..7 start one
        // barrier late, so while waves 0..3 run X they run Y and the other
        // way round: each SIMD holds one wave of each group (waves w and w+4
        // share a SIMD), so one wave's softmax runs under the other's MFMAs.
        // That placement only decides the overlap; the barrier protocol below
        // is correct for any placement. K(j) is read in X(j) and V(j)
        // in X(j+1); each sits in buffer j % 3 of its kind. Y(j) loads K(j+2)
        // and V(j+1), whose buffers (those of K(j-1) and V(j-2)) both groups
        // left at the latest in X(j-1), and each wave waits for its share
        // before the barrier that ends Y(j), ahead of their first reader.
        const bool late = wave >= 4;
        constexpr uint32_t VB = 3 * S::TILE;  // V buffers follow the K buffers
        // Per-lane bases of the transposed V reads, including the start of
        // the V buffers, kept opaque so that the compiler leaves the buffer
        // and row constants (all below 64 KB from here) in the reads'
        // offset fields instead of forming an address per read.
        uint32_t vbase[S::DB];
#pragma unroll
        for (int db = 0; db < S::DB; ++db) {
            vbase[db] = vofs[db] - S::TILE + VB;
            asm volatile("" : "+v"(vbase[db]));
        }
        f32x16 sacc[2][QB];
        bf16x8 pop[QB][2][2];
        load_one(krs, koff, 0, 0);
        if (ntiles > 1) load_one(krs, koff, kBN, S::TILE);
        load_one(vrs, voff, 0, VB);
        wait_vmem();
        if constexpr (ROPE) {
            rope_k(lds);
            if (ntiles > 1) rope_k(lds + S::TILE);
        }
        __syncthreads();
        if (late) lds_barrier();
        auto phase = [&](auto bufc, int j) {
            constexpr uint32_t b = decltype(bufc)::value;
            constexpr uint32_t bp = (b + 2) % 3, b1 = (b + 1) % 3, b2 = (b + 2) % 3;
            // X(j)
            if (busy) {
                if (j > 0) flash_pv<D, QB>(lds, bp * S::TILE, vbase, pop, oacc);
                if (j < ntiles) flash_s<D, QB>(lds, b * S::TILE, kofs, qop, sacc);
            }
            lds_barrier();
            if (j >= ntiles) return false;
            // Y(j)
            if (j + 2 < ntiles) load_one(krs, koff, (j + 2) * kBN, b2 * S::TILE);
            if (j + 1 < ntiles) load_one(vrs, voff, (j + 1) * kBN, VB + b1 * S::TILE);
            if (busy) flash_softmax<D, QB>(sacc, pop, oacc, mref, lsum, c, Lk - j * kBN, half, j == 0);
            wait_vmem();
            if constexpr (ROPE)
                if (j + 2 < ntiles) rope_k(lds + b2 * S::TILE);
            lds_barrier();
            return true;
        };
        for (int j = 0;; j += 3) {
            if (!phase(std::integral_constant<uint32_t, 0>{}, j)) break;
            if (!phase(std::integral_constant<uint32_t, 1>{}, j + 1)) break;
            if (!phase(std::integral_constant<uint32_t, 2>{}, j + 2)) break;
        }
        if (!late) lds_barrier();
    } else {
    if constexpr (QSTAGE) {
        // The wave's 32 query rows go through LDS-direct loads (whole rows,
        // four per instruction) into exactly the bytes its own loads of tile
        // 1 fill later: rows 0-15 where its share of that K tile goes, rows
        // 16-31 where its share of that V tile goes, chunk-swizzled like a K
        // tile. Rows past the segment read as zeros.
        static_assert(RPL * S::LOADS == 16, "a wave's share of one K or V tile is 16 rows");
        const int nrecq = (int)(((int64_t)tok(L - 1) * rs + D) * 2);
        const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void *)qp, 0, nrecq, kBufferFlags);
#pragma unroll
        for (int i = 0; i < 2 * S::LOADS; ++i) {
            const int r = RPL * i + lane / S::CH, qi = q0 + r;
            const uint32_t off = qi < L ? (uint32_t)((int64_t)tok(qi) * rs * 2) +
                                              (uint32_t)(((lane % S::CH) ^ swz_k<D>(r, 0)) * 16)
                                        : 0x80000000u;
            const uint32_t dst = (i < S::LOADS ? 0 : 1) * S::TILE + (wave * S::LOADS + i % S::LOADS) * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lds_void *)(lds1 + dst), 16, off, 0, 0, 0);
        }
    }
    load_tile(0, 0);
    wait_vmem();
    if constexpr (ROPE) rope_k(lds);
    __syncthreads();
    if constexpr (QSTAGE) {
        const uint32_t qb0 = (col < 16 ? 0 : S::TILE - 16 * D * 2) + wave * S::LOADS * 1024;
#pragma unroll
        for (int ks = 0; ks < S::KS; ++ks)
            qop[0][ks] = *(const __attribute__((address_space(3))) bf16x8 *)(lds1 + qb0 + kofs[ks]);
        // The first tile-1 load below overwrites these bytes.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if constexpr (ROPE) rope_q();
    }
    // Tiles alternate between the two LDS buffers; the loop body takes one
    // tile from each so that the buffer is a compile-time constant. The
    // other buffer was released by the barrier that ended the previous tile,
    // so the next tile's loads start before this tile's products.
    // A last tile whose keys all lie in its first 32-key block (the
    // 1,560-key frames of the spatial pass end with 24) is taken out of the
    // loop and run in the half form; the loop has already loaded it.
    const int nmain = Lk - (ntiles - 1) * kBN <= 32 ? ntiles - 1 : ntiles;
    for (int j = 0; j < nmain; j += 2) {
        if (j + 1 < ntiles) load_tile((j + 1) * kBN, 1);
        if (busy) tile(std::integral_constant<int, 0>{}, j);
        wait_vmem();
        if constexpr (ROPE)
            if (j + 1 < ntiles) rope_k(lds1);
        __syncthreads();
        if (j + 1 >= nmain) break;
        if (j + 2 < ntiles) load_tile((j + 2) * kBN, 0);
        if (busy) tile(std::integral_constant<int, 1>{}, j + 1);
        wait_vmem();
        if constexpr (ROPE)
            if (j + 2 < ntiles) rope_k(lds);
        __syncthreads();
    }
    if (nmain < ntiles) {
        const int jl = ntiles - 1;
        if (busy)
            flash_tile_pipe<D, true>((jl & 1) ? lds1 : lds, 0, kofs, vofs, qop, oacc, mref, lsum, c, Lk - jl * kBN,
                                     half, jl == 0);
        __syncthreads();  // every wave is done with the tile before the buffers stage the output
    }
    }

    // Normalise and store: lane holds query column `col`, features
    // db*32 + 8*(r/4) + 4*half + r%4. The 32 rows are staged through this
    // wave's own stretch of the (now idle) K/V buffers and written as whole
    // rows, 16 bytes per lane, so every store instruction covers four
    // contiguous rows instead of 16-byte pieces of 32.
    {
        constexpr int OP = D * 2 + 16;  // staging pitch (bytes): rows 16 bytes apart in the banks
        static_assert(PP ? NW * 32 * OP <= 6 * S::TILE : 2 * 32 * OP <= 2 * S::TILE, "staging fits the K/V buffers");
        lds_u8 *st = PP ? lds + wave * 32 * OP : (wave < 2 ? lds : lds1) + (wave & 1) * 32 * OP;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float inv = 1.0f / pair_sum(lsum[qb]);
#pragma unroll
            for (int db = 0; db < S::DB; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int d = db * 32 + 8 * r4 + 4 * half;
                    u32x2 w;
                    w[0] = pack_bf16x2(oacc[db][qb][4 * r4 + 0] * inv, oacc[db][qb][4 * r4 + 1] * inv);
                    w[1] = pack_bf16x2(oacc[db][qb][4 * r4 + 2] * inv, oacc[db][qb][4 * r4 + 3] * inv);
                    *(__attribute__((address_space(3))) u32x2 *)(st + col * OP + d * 2) = w;
                }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's rows are in LDS
            __builtin_amdgcn_wave_barrier();
            constexpr int CPR = D * 2 / 16;  // 16-byte chunks per row
#pragma unroll
            for (int i = 0; i < 32 * CPR / 64; ++i) {
                const int idx = lane + 64 * i;
                const int r = idx / CPR, ch = idx % CPR;
                const int qi = q0 + qb * 32 + r;
                const u32x4 val = *(const __attribute__((address_space(3))) u32x4 *)(st + r * OP + ch * 16);
                if (qi < L) *(u32x4 *)(op + (int64_t)tok(qi) * rs + ch * 8) = val;
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
        }
    }
#endif
}

template <int D, int QB, int NW, int PASS>
hipError_t launch(const void *q, const void *k, const void *v, void *o, int nseg, int L, int Lk,
                  int heads, float c, hipStream_t s, WinGeom wg = WinGeom{}, FlashRope fr = FlashRope{}) {
    using S = FlashShape<D, QB, NW>;
    if (PASS == 3) {
        // L is the largest window's token count; nseg = B * windows.
        wg.nqb = (L + S::BM - 1) / S::BM;
    }
    const int nqb = (L + S::BM - 1) / S::BM;
    const uint64_t grid = (uint64_t)nseg * heads * nqb;
    if (grid == 0 || grid > UINT32_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((flash_fwd_bf16<D, QB, NW, PASS>), dim3((uint32_t)grid), dim3(S::THREADS), 0, s,
                       (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (uint16_t *)o,
                       nseg, L, Lk, heads, c, wg, fr);
    return hipGetLastError();
}

}  // namespace
}  // namespace vdit
